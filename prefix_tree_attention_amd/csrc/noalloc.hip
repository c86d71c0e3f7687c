// The backward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// tree_attn_bwd with its workspace -- -Delta and -LSE / scale for bf16, Delta
// for fp32 -- taken from a fixed-size array the library owns on each device,
// instead of a caller-provided buffer.  The kernels are tree_attn_bwd's.

#include <mutex>

#include "device.h"
#include "status.h"

namespace {

// One array per device, held from the first call on that device until the
// process ends.  Every call on a device shares it.
static __device__ __align__(256) unsigned char scratch[TREE_BWD_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.  The host-side name of the array is only a
// stand-in for registration; kernels must be given this address.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return treeattn::set_error(TREE_E_HIP, "tree_attn_bwd_noalloc: hipGetDevice failed (%s)",
                                   hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return treeattn::set_error(TREE_E_ARG, "tree_attn_bwd_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return treeattn::set_error(TREE_E_HIP, "tree_attn_bwd_noalloc: hipGetSymbolAddress failed (%s)",
                                       hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TREE_OK;
}

}  // namespace

extern "C" int tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv, const int32_t* d_se,
                                     const void* d_meta_ws, int64_t L, int32_t Hq, int32_t Hkv, int32_t D,
                                     float scale, int32_t dtype, void* stream) {
    // arguments and the size limit first, so a bad call fails before any
    // device call
    if (int rc = treeattn::check_attn("tree_attn_bwd_noalloc", L, Hq, Hkv, D, scale, dtype)) return rc;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !d_se || !d_meta_ws)
        return treeattn::set_error(TREE_E_ARG, "tree_attn_bwd_noalloc: NULL device pointer");
    const size_t need = tree_attn_bwd_workspace_bytes(L, Hq, D, dtype);
    if (need > size_t(TREE_BWD_STATIC_SCRATCH_BYTES))
        return treeattn::set_error(TREE_E_ARG,
                                   "tree_attn_bwd_noalloc: L * Hq = %lld needs %zu bytes of workspace, more than "
                                   "the %zu-byte static scratch (L * Hq <= %zu)",
                                   (long long)(L * int64_t(Hq)), need, size_t(TREE_BWD_STATIC_SCRATCH_BYTES),
                                   size_t(TREE_BWD_STATIC_SCRATCH_BYTES) / 8);
    void* ws = nullptr;
    if (int rc = scratch_address(&ws)) return rc;
    // tree_attn_bwd_phase validates the rest and launches; nothing in the
    // scratch has to start at zero (every word the kernels read is written
    // earlier in the same call)
    return tree_attn_bwd_phase(TREE_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, d_se, d_meta_ws, ws,
                               size_t(TREE_BWD_STATIC_SCRATCH_BYTES), L, Hq, Hkv, D, scale, dtype, stream);
}
