// Router kernels: logits of the hidden states against the router gate, then
// sigmoid + bias-corrected top-K and renormalised gate weights
// ("Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM", "How it
// works (validated core mechanics)"; colibrì README v1.0 "What's
// implemented": DeepSeek-V3-style sigmoid router with routed_scaling_factor).
#include "device_common.h"
#include "kernels.h"

namespace coli {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One wavefront per (token, expert).  Lane l accumulates, with fmaf from 0,
// the elements h = 256 j + 4 l + c for j ascending and c = 0..3 (a float4
// per lane per step, so each step reads 1 KB of the gate row coalesced);
// then six xor-butterfly additions p_l + p_{l^o}, o = 32..1, leave the logit
// in every lane.  Grid: (E, S), 64 threads.
__global__ __launch_bounds__(64) void k_router_logits(const float *__restrict__ x,
                                                      const float *__restrict__ W,
                                                      float *__restrict__ logits,
                                                      uint32_t *__restrict__ status, int H,
                                                      int E) {
    const int lane = threadIdx.x;
    const int e = blockIdx.x;
    const int t = blockIdx.y;
    const f32x4 *xr = reinterpret_cast<const f32x4 *>(x + (size_t)t * H);
    const f32x4 *wr = reinterpret_cast<const f32x4 *>(W + (size_t)e * H);
    float p = 0.0f;
    bool ok = true;
    const int steps = H / 256;
#pragma unroll 8
    for (int j = 0; j < steps; ++j) {
        const f32x4 xv = xr[64 * j + lane];
        const f32x4 wv = wr[64 * j + lane];
        p = __builtin_fmaf(xv.x, wv.x, p);
        p = __builtin_fmaf(xv.y, wv.y, p);
        p = __builtin_fmaf(xv.z, wv.z, p);
        p = __builtin_fmaf(xv.w, wv.w, p);
        ok = ok && finite_f32(xv.x) && finite_f32(xv.y) && finite_f32(xv.z) && finite_f32(xv.w) &&
             finite_f32(wv.x) && finite_f32(wv.y) && finite_f32(wv.z) && finite_f32(wv.w);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o, 64);
    if (status && (!ok || !finite_f32(p))) raise_status(status, ST_NONFINITE);
    if (lane == 0) logits[(size_t)t * E + e] = p;
}

// One wavefront per token.  Lane l owns experts l, l+64, ...; sig = sigmoid,
// score = sig + bias.  K rounds of a wavefront argmax under the total order
// (score desc, id asc) pick the experts in rank order; the gate weights are
// (sig_k / ((sig_0 + sig_1) + ...)) * rsf, or sig_k * rsf without
// renormalisation.  E <= 1024, K <= 32.
__global__ __launch_bounds__(64) void k_router_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias,
                                                      int32_t *__restrict__ idx_out,
                                                      float *__restrict__ w_out,
                                                      uint32_t *__restrict__ status, int E, int K,
                                                      float rsf, int norm) {
    constexpr int MAXM = 16;
    __shared__ float sel_sig[32];
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    float sig[MAXM], score[MAXM];
    uint32_t taken = 0;
    bool ok = true;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int e = lane + 64 * m;
        sig[m] = 0.0f;
        score[m] = -__builtin_inff();
        if (e < E) {
            const float l = logits[(size_t)t * E + e];
            const float b = bias ? bias[e] : 0.0f;
            ok = ok && finite_f32(l) && finite_f32(b);
            sig[m] = sigmoid_f32(l);
            score[m] = sig[m] + b;
        }
    }
    if (!ok) raise_status(status, ST_NONFINITE);
    for (int k = 0; k < K; ++k) {
        float bs = -__builtin_inff();
        int be = 0x7fffffff;
        float bsig = 0.0f;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int e = lane + 64 * m;
            if (e < E && !((taken >> m) & 1u)) {
                if (score[m] > bs || (score[m] == bs && e < be)) {
                    bs = score[m];
                    be = e;
                    bsig = sig[m];
                }
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float os = __shfl_xor(bs, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            const float osig = __shfl_xor(bsig, o, 64);
            if (os > bs || (os == bs && oe < be)) {
                bs = os;
                be = oe;
                bsig = osig;
            }
        }
        if (be >= E) {  // only reachable with NaN scores, already flagged
            be = k;
            bsig = 0.0f;
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == 0) {
            idx_out[(size_t)t * K + k] = be;
            sel_sig[k] = bsig;
        }
    }
    __syncthreads();
    if (lane == 0) {
        if (norm) {
            float denom = sel_sig[0];
            for (int k = 1; k < K; ++k) denom = denom + sel_sig[k];
            if (!(denom > 0.0f) || !finite_f32(denom)) raise_status(status, ST_NONFINITE);
            for (int k = 0; k < K; ++k) w_out[(size_t)t * K + k] = (sel_sig[k] / denom) * rsf;
        } else {
            for (int k = 0; k < K; ++k) w_out[(size_t)t * K + k] = sel_sig[k] * rsf;
        }
    }
}

hipError_t launch_router_logits(const float *x, const float *W, float *logits, uint32_t *status,
                                int S, int H, int E, hipStream_t st) {
    hipLaunchKernelGGL(k_router_logits, dim3(E, S), dim3(64), 0, st, x, W, logits, status, H, E);
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
