// Router kernels: logits of the hidden states against the router gate, then
// sigmoid + bias-corrected top-K and renormalised gate weights
// ("Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM", "How it
// works (validated core mechanics)"; colibrì README v1.0 "What's
// implemented": DeepSeek-V3-style sigmoid router with routed_scaling_factor).
#include "device_common.h"
#include "kernels.h"

namespace coli {


// One wavefront per (token, expert).  Lane l accumulates, with fmaf from 0,
// the elements h = 256 j + 4 l + c for j ascending and c = 0..3 (a float4
// per lane per step, so each step reads 1 KB of the gate row coalesced);
// then six xor-butterfly additions p_l + p_{l^o}, o = 32..1, leave the logit
// in every lane.  Up to MAXJ steps the whole row is loaded before the chain;
// longer rows go in chunks of MAXJ.  Grid: (E, S), 64 threads.
template <int MAXJ>
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
    const int steps = H / 256;
    float p = 0.0f;
    bool ok = true;
    for (int j0 = 0; j0 < steps; j0 += MAXJ) {
        f32x4 xv[MAXJ], wv[MAXJ];
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj)
            if (j0 + jj < steps) {
                wv[jj] = __builtin_nontemporal_load(wr + 64 * (j0 + jj) + lane);
                xv[jj] = xr[64 * (j0 + jj) + lane];
            }
#pragma unroll
        for (int jj = 0; jj < MAXJ; ++jj) {
            if (j0 + jj < steps) {
                p = __builtin_fmaf(xv[jj].x, wv[jj].x, p);
                p = __builtin_fmaf(xv[jj].y, wv[jj].y, p);
                p = __builtin_fmaf(xv[jj].z, wv[jj].z, p);
                p = __builtin_fmaf(xv[jj].w, wv[jj].w, p);
                ok = ok && finite_f32(xv[jj].x) && finite_f32(xv[jj].y) && finite_f32(xv[jj].z) &&
                     finite_f32(xv[jj].w) && finite_f32(wv[jj].x) && finite_f32(wv[jj].y) &&
                     finite_f32(wv[jj].z) && finite_f32(wv[jj].w);
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o, 64);
    if (status && (!ok || !finite_f32(p))) raise_status(status, ST_NONFINITE);
    if (lane == 0) logits[(size_t)t * E + e] = p;
}

// ---- wavefront reductions through DPP (result uniform across the wave) ----
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}

__device__ __forceinline__ float wave_max_f32(float v) {
    int i = __float_as_int(v);
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0xB1>(i))));  // quad [1,0,3,2]
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0x4E>(i))));  // quad [2,3,0,1]
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0x141>(i)))); // row half mirror
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0x140>(i)))); // row mirror
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0x142, 0xA>(i))));  // row bcast 15
    i = __float_as_int(__builtin_fmaxf(__int_as_float(i), __int_as_float(dpp<0x143, 0xC>(i))));  // row bcast 31
    return __int_as_float(__builtin_amdgcn_readlane(i, 63));
}

__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, dpp<0xB1>(v));
    v = min(v, dpp<0x4E>(v));
    v = min(v, dpp<0x141>(v));
    v = min(v, dpp<0x140>(v));
    v = min(v, dpp<0x142, 0xA>(v));
    v = min(v, dpp<0x143, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// One wavefront per token.  Lane l owns experts l, l+64, ...; sig = sigmoid,
// score = sig + bias.  K rounds pick the experts in rank order under the
// total order (score desc, id asc): the wavefront maximum of the lanes' best
// remaining scores, then the smallest id holding that score.  The gate
// weights are (sig_k / ((sig_0 + sig_1) + ...)) * rsf, or sig_k * rsf
// without renormalisation.  E <= 1024, K <= 32.
__global__ __launch_bounds__(64) void k_router_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias,
                                                      int32_t *__restrict__ idx_out,
                                                      float *__restrict__ w_out,
                                                      uint32_t *__restrict__ status, int E, int K,
                                                      float rsf, int norm) {
    constexpr int MAXM = 16;
    __shared__ float sig_s[1024];
    __shared__ float sel_sig[32];
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const int mcount = (E + 63) / 64;
    float score[MAXM];
    uint32_t taken = 0;
    bool ok = true;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int e = lane + 64 * m;
        score[m] = -__builtin_inff();
        if (m < mcount && e < E) {
            const float l = logits[(size_t)t * E + e];
            const float b = bias ? bias[e] : 0.0f;
            ok = ok && finite_f32(l) && finite_f32(b);
            const float sg = sigmoid_f32(l);
            sig_s[e] = sg;
            score[m] = sg + b;
        }
    }
    if (!ok) raise_status(status, ST_NONFINITE);
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        float bs = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m < mcount && !((taken >> m) & 1u) && score[m] > bs) {
                bs = score[m];
                be = lane + 64 * m;
            }
        }
        const float M = wave_max_f32(bs);
        int sel = wave_min_i32(bs == M ? be : 0x7fffffff);
        if (sel >= E) {  // only reachable with NaN scores, already flagged
            sel = k;
        }
        if ((sel & 63) == lane) taken |= 1u << (sel >> 6);
        if (lane == 0) {
            idx_out[(size_t)t * K + k] = sel;
            sel_sig[k] = sig_s[sel];
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
