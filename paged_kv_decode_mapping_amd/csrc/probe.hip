// probe.hip -- a plain streaming-read kernel: the read bandwidth a kernel of
// this library can reach on the current GPU, the practical ceiling that the
// decode kernels' achieved bandwidth is compared with (next to the
// published HBM peak).
//
// Each thread issues kUnroll independent 16-byte loads per step over a
// grid-stride loop, so every byte of the buffer is read exactly once, with
// either the default cache policy or the non-temporal one the decode kernels
// use for the KV cache. The loaded words are folded into one value per
// thread, written only if it equals a constant that the data never produces
// in practice, so that the loads cannot be dropped.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void pa_probe_read_kernel(const u32x4* p, int64_t n, uint32_t* sink) {
    const int64_t per_step = (int64_t)kProbeThreads * kUnroll;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * per_step; base < n; base += (int64_t)gridDim.x * per_step) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads + threadIdx.x;
            v[u] = i < n ? (NT ? __builtin_nontemporal_load(p + i) : p[i]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x5a17c0deu) sink[threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t bytes, bool nontemporal, uint32_t* sink, int cus,
                             hipStream_t s) {
    const int64_t n = bytes / 16;
    // 8 workgroups per compute unit: enough loads in flight to saturate HBM
    const int64_t want = (n + (int64_t)kProbeThreads * kUnroll - 1) / ((int64_t)kProbeThreads * kUnroll);
    int64_t blocks = (int64_t)cus * 8;
    if (blocks > want) blocks = want;
    if (blocks < 1) blocks = 1;
    const u32x4* p = static_cast<const u32x4*>(buf);
    if (nontemporal) hipLaunchKernelGGL(pa_probe_read_kernel<true>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, p, n, sink);
    else hipLaunchKernelGGL(pa_probe_read_kernel<false>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, p, n, sink);
    return hipGetLastError();
}

}  // namespace pa
