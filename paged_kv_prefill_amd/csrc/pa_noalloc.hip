// pa_noalloc.hip -- pa_prefill_bf16_noalloc: pa_prefill_bf16 for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that must not call the allocator, harnesses that forbid it).
//
// The call's tile images and work schedule (the workspace of pa_prefill_bf16)
// live in `scratch`, a file-scope device array of PA_NOALLOC_SCRATCH_BYTES
// that every GPU the library runs on holds from the module's load until the
// process ends.  In host code the array's name stands for a host-side shadow,
// not a device address, so the device address is looked up once per device
// with hipGetSymbolAddress (that device current) and kept; only that address
// ever reaches a kernel.  The entry point then runs pa_prefill_bf16 with it --
// the same checks, kernels and results.  It calls no allocator.
//
// Every call on a GPU shares that GPU's array and finds it as the last call
// left it.  Nothing in it needs clearing: each call writes every byte it reads
// (the images of its requests' tiles, then the schedule) before reading it.
// Calls that overlap on one GPU (other streams, other host threads) race.
#include "../../include/paged_kv_prefill.h"

#include <hip/hip_runtime.h>
#include <mutex>

#include "pa_kernels.h"

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];   // device address of `scratch`, per device

// the current device's scratch address, looked up on its first use
int device_scratch(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
    if (dev < 0 || dev >= MAX_DEVICES) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" int pa_prefill_bf16_noalloc(const pa_paged_args *a, const void *q, const void *k_pool,
                                       const void *v_pool, void *out, int32_t out_dtype,
                                       hipStream_t stream) {
    int rc = pa::prefill_bf16_check(a, q, k_pool, v_pool, out, out_dtype);
    if (rc) return rc;
    // the array is shared by every call: no call may rely on what an earlier one left
    if (a->flags) return PA_ERR_SHAPE;
    const size_t need = pa_workspace_bytes(a, PA_ENTRY_PREFILL_BF16);
    if (need == 0) return PA_ERR_SHAPE;
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_TOO_LARGE;
    void *ws = nullptr;
    if ((rc = device_scratch(&ws))) return rc;
    return pa_prefill_bf16(a, q, k_pool, v_pool, out, out_dtype, ws, PA_NOALLOC_SCRATCH_BYTES, stream);
}
