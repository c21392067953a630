// pa_device.h -- device helpers shared by the gfx950 kernels of libpa.
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   ToPG     = «ToPG框架解析：大模型推理性能优化与三阶段流水线设计»
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ----------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__host__ __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ----------------------------------------------------------------- fp8 e4m3fn
//
// OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities, S.1111.111 is NaN, largest finite magnitude 448, smallest
// subnormal 2^-9. The KV cache stores code = Q(x / scale) and reads code *
// scale back (Tutorial §3.1 "量化基础": symmetric_quantize and dequantize;
// ToPG §3 names fp8 as the KV-cache compression format).

// Encode one float32 (already divided by the scale): nearest code, ties to
// the even code, magnitudes above 448 saturate to 448, NaN -> NaN.
__host__ __device__ __forceinline__ uint8_t fp8_e4m3fn_encode(float y) {
    uint32_t u;
    __builtin_memcpy(&u, &y, 4);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu);   // NaN
    if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);  // |y| >= 448 (and inf)
    if (a < 0x3c800000u) {                                  // |y| < 2^-6: subnormal codes
        // |y| * 2^9 is exact; round it to an integer, ties to even. The code
        // of m * 2^-9 is m for m = 0..7, and m = 8 is code 0x08 = 2^-6.
        float ay;
        __builtin_memcpy(&ay, &a, 4);
        const float m = __builtin_rintf(ay * 512.0f);
        return (uint8_t)(sign | (uint32_t)m);
    }
    // Normal range [2^-6, 448): round the 23-bit mantissa to 3 bits, ties to
    // even; a carry moves into the exponent field, which is what we want.
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const uint32_t e = (r >> 23) - 127u + 7u;
    const uint32_t m = (r >> 20) & 7u;
    return (uint8_t)(sign | (e << 3) | m);
}

// ----------------------------------------------------------------- loads

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource for `bytes` bytes from a wave-uniform base. Offsets at or
// past `bytes` read as zero instead of touching memory. The last word is the
// gfx9-family default (untyped, 32-bit data format field set).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy bits of a buffer load on gfx950: bit 1 = nt (non-temporal).
constexpr int kCachePolicyDefault = 0;
constexpr int kCachePolicyStream = 2;

// 16-byte buffer load at voff (per-lane, VGPR) + soff (wave-uniform, SGPR).
// Keeping the uniform part in soff lets per-lane offsets stay loop-invariant,
// so issuing a tile's loads needs no vector temporaries.
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicyDefault);
}

// A load of data read once (the KV cache in decode): marked non-temporal, so
// that the caches treat the lines as streaming. On MI355X a plain streaming
// read reaches ~6.25 TB/s with default loads and ~7.0 TB/s with nt loads.
__device__ __forceinline__ u32x4 buf_load_b128_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicyStream);
}

__device__ __forceinline__ u32x2 buf_load_b64(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
}

// ----------------------------------------------------------------- cross-lane

// Sum over the 16 lanes of each DPP row (every lane gets the row's sum).
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
    return x;
}

// Sum over each aligned group of 8 lanes.
__device__ __forceinline__ float row8_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
    return x;
}

// Sum over each aligned group of 4 lanes.
__device__ __forceinline__ float row4_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
    return x;
}

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group size");
    if constexpr (LANES == 16) return row16_sum(x);
    else if constexpr (LANES == 8) return row8_sum(x);
    else return row4_sum(x);
}

// Lane exchange with lane ^ mask (ds_bpermute; any mask < 64).
__device__ __forceinline__ float xor_shfl(float x, int mask) {
    const int lane = (int)__lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa
