// Router device routines ("Colibri (colibrì): GLM-5.2 local inference on
// 25 GB of RAM", "How it works (validated core mechanics)"; colibrì README
// v1.0 "What's implemented": DeepSeek-V3-style sigmoid router with
// routed_scaling_factor): one router logit per wavefront in the layer's fixed
// order, and the bias-corrected top-K selection with renormalised weights.
#pragma once

#include "device_common.h"

namespace coli {

// Logit of one (token, expert) by one wavefront.  Lane l accumulates, with
// fmaf from 0, the elements h = 256 j + 4 l + c for j ascending and c = 0..3
// (a float4 per lane per step: each step reads 1 KB of the gate row
// coalesced); then six xor-butterfly additions p_l + p_{l^o}, o = 32..1,
// leave the logit in every lane.  Up to MAXJ steps of the row are loaded
// before the chain starts.  *ok is cleared on a non-finite input.
template <int MAXJ>
__device__ __forceinline__ float logit_wave(const float *__restrict__ xrow,
                                            const float *__restrict__ wrow, int H, bool *ok) {
    const int lane = threadIdx.x & 63;
    const f32x4 *xr = reinterpret_cast<const f32x4 *>(xrow);
    const f32x4 *wr = reinterpret_cast<const f32x4 *>(wrow);
    const int steps = H / 256;
    float p = 0.0f;
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
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o, 64);
    // a non-finite x or W_r element makes the logit non-finite (an infinity
    // times zero or an opposite infinity gives NaN; NaN and infinities
    // survive the chain and the sums), so this checks the inputs too
    *ok = finite_f32(p);
    return p;
}

// ---- wavefront reductions through DPP (result uniform across the wave) ----

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}

// Order-preserving map of non-NaN binary32 values to uint32 (sign-magnitude
// to offset binary; -0 sorts just below +0).
__device__ __forceinline__ uint32_t f32_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// DPP move whose disabled or out-of-row source lanes read 0 (the identity of
// an unsigned maximum), so that the compiler folds it into the v_max_u32.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u0(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// Wavefront maximum (uniform): each DPP step folds into one v_max_u32.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
    k = max(k, dpp_u0<0xB1>(k));        // quad [1,0,3,2]
    k = max(k, dpp_u0<0x4E>(k));        // quad [2,3,0,1]
    k = max(k, dpp_u0<0x141>(k));       // row half mirror
    k = max(k, dpp_u0<0x140>(k));       // row mirror
    k = max(k, dpp_u0<0x142, 0xA>(k));  // row bcast 15
    k = max(k, dpp_u0<0x143, 0xC>(k));  // row bcast 31
    return __builtin_amdgcn_readlane(k, 63);
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

// Selection for one token by one wavefront.  Lane l owns experts l, l+64,
// ...; sig = sigmoid(logit), score = sig + bias.  K rounds pick the experts
// in rank order under the total order (score desc, id asc): the wavefront
// maximum of the lanes' best remaining scores, then the smallest id holding
// it (a ballot settles the usual single-holder case; exact ties take a
// minimum reduction).  Gate weights: (sig_k / ((sig_0 + sig_1) + ...)) * rsf,
// or sig_k * rsf without renormalisation.  Lane k < K receives the k-th pick
// in *idx / *w.  load_logit(e) returns the token's logit e, load_bias(m, e)
// the bias of expert e = lane + 64 m.  E <= 64 * MAXM, K <= 32.  Returns false on a non-finite input or zero weights.
template <int MAXM, typename LoadLogit, typename LoadBias>
__device__ __forceinline__ bool select_wave_b(LoadLogit load_logit, LoadBias load_bias, int E, int K, float rsf,
                                              int norm, int32_t *idx, float *w) {
    const int lane = threadIdx.x & 63;
    const int mcount = (E + 63) / 64;
    float score[MAXM], sig[MAXM], lv[MAXM], bv[MAXM];
    bool ok = true;
    // all loads first (in flight together), then the arithmetic
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int e = min(lane + 64 * m, E - 1);
        if (m < mcount) {
            lv[m] = load_logit(e);
            bv[m] = load_bias(m, e);
        }
    }
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int e = lane + 64 * m;
        score[m] = -__builtin_inff();
        sig[m] = 0.0f;
        if (m < mcount && e < E) {
            ok = ok && finite_f32(lv[m]) && finite_f32(bv[m]);
            sig[m] = sigmoid_f32(lv[m]);
            score[m] = sig[m] + bv[m];
        }
    }
    // The rounds compare order-preserving keys of the scores (f32_key): a
    // candidate's key is 0 once taken, or when it is missing or its score is
    // not above -inf (NaN included), so it never wins a round, as a score
    // that is not above the running best never does.  Scores are never -0
    // (sig >= +0), so key order is score order.
    uint32_t key[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) key[m] = score[m] > -__builtin_inff() ? f32_key(score[m]) : 0u;
    int32_t my_idx = 0;
    float my_sig = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t bk = 0;
        float bsig = 0.0f;
        int be = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (key[m] > bk) {
                bk = key[m];
                bsig = sig[m];
                be = lane + 64 * m;
            }
        }
        const uint32_t M = wave_max_u32(bk);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(bk == M);
        int sel;
        if (__builtin_popcountll(hit) == 1)
            sel = __builtin_amdgcn_readlane(be, (int)__builtin_ctzll(hit));
        else
            sel = wave_min_i32(bk == M ? be : 0x7fffffff);
        if (sel >= E) sel = k;  // only reachable with NaN scores, flagged below
        const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bsig), sel & 63));
        if ((sel & 63) == lane) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                if (m == (sel >> 6)) key[m] = 0u;
        }
        if (lane == k) {
            my_idx = sel;
            my_sig = s;
        }
    }
    bool wok = true;
    float denom = 1.0f;
    if (norm) {
        denom = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_sig), 0));
        for (int k = 1; k < K; ++k)
            denom = denom + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_sig), k));
        wok = denom > 0.0f && finite_f32(denom);
    }
    *idx = my_idx;
    *w = norm ? (my_sig / denom) * rsf : my_sig * rsf;
    return __builtin_amdgcn_readfirstlane((int)(ok && wok)) != 0;
}

// select_wave_b with the bias read from memory (null: no bias).
template <int MAXM, typename LoadLogit>
__device__ __forceinline__ bool select_wave(LoadLogit load_logit, const float *__restrict__ bias, int E, int K,
                                            float rsf, int norm, int32_t *idx, float *w) {
    return select_wave_b<MAXM>(load_logit, [&](int, int e) { return bias ? bias[e] : 0.0f; }, E, K, rsf, norm, idx,
                               w);
}

}  // namespace coli
