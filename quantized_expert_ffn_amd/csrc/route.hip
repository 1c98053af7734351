// Router kernels for the two-launch path (logits, then selection); the
// device routines are in router.h.
#include "device_common.h"
#include "kernels.h"
#include "router.h"

namespace coli {

// Q8_0 of the hidden states, one 32-value block per lane (blocks
// 64 * qblk + lane of token t).
__device__ __forceinline__ void quant_x_wave(const float *__restrict__ x, int8_t *__restrict__ qx,
                                             float *__restrict__ dx, uint32_t *__restrict__ status,
                                             int H, int t, int qblk) {
    const int nbx = H / 32;
    const int b = qblk * 64 + (int)(threadIdx.x & 63);
    if (b < nbx) {
        bool ok;
        const float d = q8_0_block_lane(x + (size_t)t * H + 32 * b, qx + (size_t)t * H + 32 * b, &ok);
        dx[(size_t)t * nbx + b] = d;
        if (!ok && status) raise_status(status, ST_NONFINITE);
    }
}

// One wavefront per (token, expert); with qx, the workgroups past the E
// experts quantise the token's hidden state (64 blocks each).
// Grid: (E + ceil(H / 2048) if qx else E, S), 64 threads.
template <int MAXJ>
__global__ __launch_bounds__(64) void k_router_logits(const float *__restrict__ x,
                                                      const float *__restrict__ W,
                                                      float *__restrict__ logits,
                                                      uint32_t *__restrict__ status, int H,
                                                      int E, int8_t *__restrict__ qx,
                                                      float *__restrict__ dx) {
    const int e = blockIdx.x;
    const int t = blockIdx.y;
    if (e >= E) {
        quant_x_wave(x, qx, dx, status, H, t, e - E);
        return;
    }
    bool ok;
    const float p = logit_wave<MAXJ>(x + (size_t)t * H, W + (size_t)e * H, H, &ok);
    if (status && !ok) raise_status(status, ST_NONFINITE);
    if (threadIdx.x == 0) logits[(size_t)t * E + e] = p;
}

// One wavefront per token.
template <int MAXM>
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
    const bool ok = select_wave<MAXM>([&](int e) { return lg[e]; }, bias, E, K, rsf, norm,
                                idx_out + (size_t)t * K, w_out + (size_t)t * K, sig_s, sel_sig);
    if (!ok && threadIdx.x == 0) raise_status(status, ST_NONFINITE);
}

// Q8_0 of the hidden states alone.  Grid: (ceil(H / 2048), S), 64 threads.
__global__ __launch_bounds__(64) void k_quant_x(const float *__restrict__ x, int8_t *__restrict__ qx,
                                                float *__restrict__ dx, uint32_t *__restrict__ status,
                                                int H) {
    quant_x_wave(x, qx, dx, status, H, blockIdx.y, blockIdx.x);
}

hipError_t launch_router_logits(const float *x, const float *W, float *logits, uint32_t *status,
                                int S, int H, int E, int8_t *qx, float *dx, hipStream_t st) {
    const int gx = E + (qx ? (H / 32 + 63) / 64 : 0);
    if (H <= 24 * 256) return launch(k_router_logits<24>, dim3(gx, S), dim3(64), 0, st, x, W, logits, status, H, E, qx, dx);
    return launch(k_router_logits<16>, dim3(gx, S), dim3(64), 0, st, x, W, logits, status, H, E, qx, dx);
}

hipError_t launch_quant_x(const float *x, int8_t *qx, float *dx, uint32_t *status, int S, int H,
                          hipStream_t st) {
    return launch(k_quant_x, dim3((H / 32 + 63) / 64, S), dim3(64), 0, st, x, qx, dx, status, H);
}

hipError_t launch_router_select(const float *logits, const float *bias, int32_t *idx, float *w,
                                uint32_t *status, int S, int E, int K, float rsf, int norm,
                                hipStream_t st) {
    if (E <= 256)
        return launch(k_router_select<4>, dim3(S), dim3(64), 0, st, logits, bias, idx, w, status, E, K, rsf, norm);
    return launch(k_router_select<16>, dim3(S), dim3(64), 0, st, logits, bias, idx, w, status, E, K, rsf, norm);
}

}  // namespace coli
