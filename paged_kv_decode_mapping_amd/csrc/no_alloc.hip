// no_alloc.hip -- pa_decode_no_alloc: the decode step for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The call is pa_decode with its workspace -- the device-built work list and
// the split-K partial states -- placed in `scratch`, a static array of this
// library's code object, instead of a buffer the caller passes. The HIP
// runtime allocates the array on each device when it loads the library's
// code there, and it lives until the process ends. In host code `scratch`
// names a host-side stand-in, not the device array: its device address
// comes from hipGetSymbolAddress, once per device (on that device's first
// call, with the device current), and only that address is ever passed on.
//
// Nothing in the array needs clearing between calls: the work-list builder
// writes the item count before the decode kernel reads it, and every partial
// state the merge reads was written by the same call's decode kernel. All
// calls on one device share its array, so calls that may overlap there
// (streams without ordering, concurrent host threads) race on it.
#include <mutex>

#include "pa_abi.h"

namespace {

constexpr size_t kScratchBytes = PA_NO_ALLOC_SCRATCH;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once).
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" int pa_decode_no_alloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                  const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                                  const pa_tensor* out, float k_scale, float v_scale, const pa_decode_opts* opts,
                                  void* stream) {
    // The plan's workspace need (0 also when the arguments are invalid:
    // pa_decode then reports why).
    const size_t need = pa_decode_workspace_size(q, k_cache, block_tables, opts);
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    void* ws = nullptr;
    const int st = scratch_on_current_device(&ws);
    if (st != PA_OK) return st;
    return pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale, v_scale, ws, kScratchBytes,
                     opts, stream);
}
