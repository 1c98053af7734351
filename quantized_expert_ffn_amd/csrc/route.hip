// Router kernels for the two-launch path (logits, then selection); the
// device routines are in router.h.
#include "device_common.h"
#include "kernels.h"
#include "router.h"

namespace coli {

// One wavefront per (token, expert).  Grid: (E, S), 64 threads.
template <int MAXJ>
__global__ __launch_bounds__(64) void k_router_logits(const float *__restrict__ x,
                                                      const float *__restrict__ W,
                                                      float *__restrict__ logits,
                                                      uint32_t *__restrict__ status, int H,
                                                      int E) {
    const int e = blockIdx.x;
    const int t = blockIdx.y;
    bool ok;
    const float p = logit_wave<MAXJ>(x + (size_t)t * H, W + (size_t)e * H, H, &ok);
    if (status && !ok) raise_status(status, ST_NONFINITE);
    if (threadIdx.x == 0) logits[(size_t)t * E + e] = p;
}

// One wavefront per token.
__global__ __launch_bounds__(64) void k_router_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias,
                                                      int32_t *__restrict__ idx_out,
                                                      float *__restrict__ w_out,
                                                      uint32_t *__restrict__ status, int E, int K,
                                                      float rsf, int norm) {
    __shared__ float sig_s[1024];
    __shared__ float sel_sig[32];
    const int t = blockIdx.x;
    const float *lg = logits + (size_t)t * E;
    const bool ok = select_wave([&](int e) { return lg[e]; }, bias, E, K, rsf, norm,
                                idx_out + (size_t)t * K, w_out + (size_t)t * K, sig_s, sel_sig);
    if (!ok && threadIdx.x == 0) raise_status(status, ST_NONFINITE);
}

hipError_t launch_router_logits(const float *x, const float *W, float *logits, uint32_t *status,
                                int S, int H, int E, hipStream_t st) {
    if (H <= 24 * 256)
        hipLaunchKernelGGL(k_router_logits<24>, dim3(E, S), dim3(64), 0, st, x, W, logits, status, H, E);
    else
        hipLaunchKernelGGL(k_router_logits<16>, dim3(E, S), dim3(64), 0, st, x, W, logits, status, H, E);
    return hipGetLastError();
}

hipError_t launch_router_select(const float *logits, const float *bias, int32_t *idx, float *w,
                                uint32_t *status, int S, int E, int K, float rsf, int norm,
                                hipStream_t st) {
    hipLaunchKernelGGL(k_router_select, dim3(S), dim3(64), 0, st, logits, bias, idx, w, status, E,
                       K, rsf, norm);
    return hipGetLastError();
}

}  // namespace coli
