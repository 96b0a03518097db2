// fa_bwd_noalloc: the backward pass with its scratch (D = rowsum(dO o O), one
// float per query row) in a static device array instead of a caller
// workspace, for callers that cannot allocate.  The kernels are fa_bwd's.
//
// The array's name is a host-side stand-in in this file: host code uses only
// the device address hipGetSymbolAddress returns for it, looked up once per
// device (with that device current) and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[FA_BWD_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES];   // device address of `scratch` on each device (null until looked up)

// Device address of the scratch array on the current device.
hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                    const float* LSE, void* dQ, void* dK, void* dV, int32_t B, int32_t H,
                                    int32_t N, int32_t d, fa_dtype dtype, float scale, int32_t causal,
                                    float dropout_p, uint64_t seed, const uint8_t* block_mask, const fa_opts* opts,
                                    hipStream_t stream) {
    fa::BwdArgs a;
    fa_status st = fa::bwd_prepare(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, d, dtype, scale, causal, dropout_p,
                                   seed, block_mask, opts, &a);
    if (st != FA_OK) return st;
    if (fa_bwd_workspace_bytes(B, H, N, d) > FA_BWD_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return fa::set_hip_error(e);
    a.delta = static_cast<float*>(ws);
    e = fa::launch_bwd(a, dtype, d, stream);
    return e == hipSuccess ? FA_OK : fa::set_hip_error(e);
}
