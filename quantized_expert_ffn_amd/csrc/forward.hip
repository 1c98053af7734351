// Expert FFN kernels of the MoE layer for decode and speculative-verify
// batches (colibrì README v1.0, "What's implemented": SwiGLU experts over
// int8 / packed int4 / packed int2 weights with per-row scales, integer dots
// over Q8_0 activations, batch-union MoE with each unique expert read once).
//
// Work decomposition.  A "unit" is one unique routed expert of the call (in
// ascending id) or the shared expert (last).  A workgroup takes unit
// blockIdx.y and a tile of weight rows blockIdx.x, and streams those rows
// once for all tokens routed to the unit; the unit table comes from the
// router launch (the workspace) or is rebuilt from topk_idx in LDS (a few
// hundred integer operations).
//
//   k_gateup:  32 gate rows + the 32 matching up rows (rows i0..i0+31) ->
//              SwiGLU -> one Q8_0 block of h per token, written to the
//              workspace slot of the (token, rank) pair.
//   k_down:    64 down rows -> y per pair slot in the workspace (Y).
//   k_combine: out[t] = rank-order fmaf chain over the routed y of token t,
//              plus its shared y, once k_down has finished: each output
//              element has exactly one writer; no floating-point atomics.
// Batches whose down+combine tile fits 80 KiB of LDS take k_down_rows
// (down_rows.hip) instead of k_down + k_combine.
//
// Inner loop (both kernels).  Wave w owns 16 rows.  A row is read in chunks
// of 64 Q8_0 blocks: lane l loads block 64c+l of each of its 16 rows
// (contiguous across lanes: 1 KB per row per load for int4), forms the exact
// int32 block dots against the LDS-staged activation codes, and writes them
// to LDS.  Then thread (row, token) runs the binary32 chain
// acc = fmaf(d_b, isum_b, acc) over the chunk's blocks in ascending order —
// the layer's defined order — and finally multiplies by the row scale.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "gateup.h"
#include "kernels.h"
#include "stream.h"

namespace coli {

// Copies the unit table of the call (workspace, built by the router
// launch) into LDS words at `tab`; returns the blob pointer of unit u (or
// null when u is past the table).  One memory latency.
__device__ __forceinline__ const uint8_t *load_unit_table(const uint8_t *units, const UnitTable &U, int *tab,
                                                          int u) {
    const int32_t *src = reinterpret_cast<const int32_t *>(units);
    for (int q = threadIdx.x; q < U.words; q += blockDim.x) tab[q] = src[q];
    const uint8_t *blob = u < U.umax ? reinterpret_cast<const uint8_t *const *>(units + U.ublob)[u] : nullptr;
    __syncthreads();
    return blob;
}

// Gate/up of one (32-row tile, unit).  With TABLE the units come from the
// call's unit table (coli_moe_layer): row y = 0 is the shared expert (its
// pairs do not depend on the routing, so it needs no table) and row y > 0
// routed unit y - 1, where y = blockIdx.y + shared_done (the router launch
// may already have run the shared expert's gate/up: then the workgroups of
// grid row 0 first quantise its h, one 32-row block each, to Q8_0(h) in the
// shared expert's pair slots).  Otherwise every workgroup builds the unit
// table from topk_idx and takes unit blockIdx.y.
template <int BITS, int NT, bool TABLE, bool GROUPED, bool MX = false>
__global__ __launch_bounds__(256) void k_gateup(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I, P = S * K;
    const SmemPlan L = smem_plan(S, K, E, NT, H);
    const int *uexp = reinterpret_cast<const int *>(smem + L.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + L.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + L.pairs);
    const int y = (int)blockIdx.y + (TABLE ? a.shared_done : 0);
    if (TABLE && a.shared_done && blockIdx.y == 0 && wave == 0) {
        // half-wave t: block blockIdx.x of token t's h (S <= 2)
        const int t = lane >> 5, i = 32 * (int)blockIdx.x + (lane & 31);
        if (t < S) {
            float d;
            const int8_t q = q8_0_lane(a.hs[(size_t)t * I + i], &d);
            a.qh[(size_t)(P + t) * I + i] = q;
            if ((lane & 31) == 0) a.dh[(size_t)(P + t) * (I / 32) + blockIdx.x] = d;
        }
    }
    int u = y, e;
    const uint8_t *tblob = nullptr;
    if (TABLE && a.n_shared && y == 0) {
        int *pw = reinterpret_cast<int *>(smem + L.pairs);
        int *ow = reinterpret_cast<int *>(smem + L.uoff);
        for (int t = tid; t < S; t += 256) pw[t] = P + t;
        if (tid == 0) {
            ow[0] = 0;
            ow[1] = S;
        }
        __syncthreads();
        u = 0;
        e = -1;
        tblob = a.shared;
    } else if (TABLE) {
        // the table's words go to the start of LDS (the region this kernel
        // otherwise uses to build its unit table, which is at least as large)
        const UnitTable U = unit_table(S, K, E);
        int *tab = reinterpret_cast<int *>(smem);
        u = y - (a.n_shared ? 1 : 0);
        tblob = load_unit_table(a.units, U, tab, u);
        uexp = tab + U.uexp;
        uoff = tab + U.uoff;
        pairs = tab + U.pairs;
        if (u >= uniform(tab[1])) return;
        e = uniform(uexp[u]);
    } else {
        build_units(a.idx, S, K, E, a.n_shared, smem, L, a.status,
                    blockIdx.x == 0 && blockIdx.y == 0 && a.pend_mode != 2);
        const int n_units = uniform(reinterpret_cast<const int *>(smem + L.misc)[0]);
        if (u >= n_units) return;
        e = uniform(uexp[u]);
    }
    if (e >= 0 && a.pend_mode != 0) {
        const bool pend = (a.pend[e >> 5] >> (e & 31)) & 1u;
        if ((a.pend_mode == 1) == pend) return;
    }
    const uint8_t *blob = uniform_ptr(TABLE ? tblob : (e < 0 ? a.shared : a.blobs[e]));
    if (blob == nullptr) {
        if (tid == 0) raise_status(a.status, ST_NOTRESIDENT);
        return;
    }
    const int nb = H / 32, vds = vd_stride(nb);
    const int p0 = uniform(uoff[u]), np = uniform(uoff[u + 1]) - p0;
    // Q8_0(x) of a group's tokens (computed once per call) into LDS: direct
    // global-to-LDS loads (1 KB of codes or 64 scales per wavefront
    // instruction) when the rows split into whole chunks
    auto stage = [&](int g0, int ng) {
        int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
        float *vd = reinterpret_cast<float *>(smem + L.vd);
        if (H % 2048 == 0) {
            const int qch = H / 1024, dch = nb / 64;
            for (int j = wave; j < ng * (qch + dch); j += 4) {
                const int it = j / (qch + dch), ch = j - it * (qch + dch);
                const int v = pairs[p0 + g0 + it];
                const int t = v < P ? v / K : v - P;
                if (ch < qch)
                    lds_dma16(a.qx + (size_t)t * H + ch * 1024 + 16 * lane, vq + (size_t)it * H + ch * 1024);
                else
                    lds_dma4(a.dx + (size_t)t * nb + (ch - qch) * 64 + lane, vd + it * vds + (ch - qch) * 64);
            }
            drain_vm();
        } else {
            for (int it = 0; it < ng; ++it) {
                const int v = pairs[p0 + g0 + it];
                const int t = v < P ? v / K : v - P;
                const i32x4 *src = reinterpret_cast<const i32x4 *>(a.qx + (size_t)t * H);
                i32x4 *dst = reinterpret_cast<i32x4 *>(vq + (size_t)it * H);
                for (int q = tid; q < H / 16; q += 256) dst[q] = src[q];
                for (int q = tid; q < nb; q += 256) vd[it * vds + q] = a.dx[(size_t)t * nb + q];
            }
        }
        __syncthreads();
    };
    // (MXFP4 with one vector only: the f16 activation pairs of more do not
    // fit the registers beside two chunks of weights)
    if constexpr (BITS < 8 && (!MX || NT == 1)) {
        const int nch = (nb + 63) / 64;
        if (np <= NT && H <= 8192 && nch >= 2 && (!GROUPED || primed_scales_fit(H, a.group, MX))) {
            // all of the unit's vectors in one pass: their activations (and
            // the rows' group scales) are loaded ahead of the weights
            // (gateup_unit_primed)
            auto tok = [&](int it) {
                const int v = pairs[p0 + it];
                return v < P ? v / K : v - P;
            };
            auto go = [&](auto nch_c) {
                gateup_unit_primed<BITS, NT, decltype(nch_c)::value, decltype(tok), GROUPED, MX>(
                    blob, H, I, blockIdx.x * 32, pairs + p0, np, smem, L, a.qx, a.dx, tok, a.qh, a.dh, a.group,
                    L.total);
            };
            if (nch == 2)
                go(std::integral_constant<int, 2>());
            else if (nch == 3)
                go(std::integral_constant<int, 3>());
            else
                go(std::integral_constant<int, 4>());
            return;
        }
    }
    gateup_unit<BITS, NT, GROUPED, MX>(blob, H, I, a.group, blockIdx.x * 32, pairs + p0, np, smem, L, L.total, a.qh,
                                       a.dh, stage);
}

// Down projection: 64 rows of one unit per workgroup, y written to the
// pair's slot of the workspace (the combine kernel reads it after this
// kernel has finished, so no cross-workgroup signalling is needed).
template <int BITS, int NT, bool GROUPED, bool MX = false>
__global__ __launch_bounds__(256) void k_down(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I;
    const SmemPlan L = smem_plan(S, K, E, NT, I);
    build_units(a.idx, S, K, E, a.n_shared, smem, L, a.status, false);
    const int *uexp = reinterpret_cast<const int *>(smem + L.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + L.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + L.pairs);
    const int n_units = uniform(reinterpret_cast<const int *>(smem + L.misc)[0]);
    const int u = blockIdx.y;
    if (u >= n_units) return;
    const int e = uniform(uexp[u]);
    const uint8_t *blob = uniform_ptr(e < 0 ? a.shared : a.blobs[e]);
    const int r0 = blockIdx.x * 64;
    const int p0 = uniform(uoff[u]), np = uniform(uoff[u + 1]) - p0;
    if (blob == nullptr) {
        if (tid == 0) raise_status(a.status, ST_NOTRESIDENT);
        for (int q = tid; q < np * 64; q += 256) {
            const int slot = pairs[p0 + (q >> 6)];
            a.Y[(size_t)slot * H + r0 + (q & 63)] = 0.0f;
        }
        return;
    }
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * ROWS_PER_WAVE * ISUM_PITCH;
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED && !MX ? a.group : 0, MX);
    const size_t row_bytes = (size_t)I * BITS / 8;
    const int rw = r0 + wave * ROWS_PER_WAVE;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[ROWS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < ROWS_PER_WAVE; ++j) rowoff[j] = (uint32_t)(BL.down + (size_t)(rw + j) * row_bytes);
    const float *s_down = reinterpret_cast<const float *>(blob + BL.s_down);
    RowGroups G;
    G.lgb = GROUPED ? group_lgb(a.group) : -1;
    if (GROUPED) {
        G.rsrc = rsrc;
        G.row_stride = MX ? (uint32_t)(I / 32) : (uint32_t)(4 * (I / a.group));
        G.base = (uint32_t)(BL.s_down + (size_t)rw * G.row_stride);
        G.lds = reinterpret_cast<float *>(smem + L.total) + wave * ROWS_PER_WAVE * (64 >> G.lgb);
    }
    const int nb = I / 32;
    const int vds = vd_stride(nb);
    const int crow = lane & 15, cvec = lane >> 4;
    for (int g0 = 0; g0 < np; g0 += NT) {
        const int ng = min(NT, np - g0);
        auto stage = [&]() {
            for (int it = 0; it < ng; ++it) {
                const int slot = pairs[p0 + g0 + it];
                const i32x4 *src = reinterpret_cast<const i32x4 *>(a.qh + (size_t)slot * I);
                i32x4 *dst = reinterpret_cast<i32x4 *>(vq + (size_t)it * I);
                for (int q = tid; q < I / 16; q += 256) dst[q] = src[q];
                for (int q = tid; q < nb; q += 256) vd[it * vds + q] = a.dh[(size_t)slot * nb + q];
            }
            __syncthreads();
        };
        BlockBits<BITS> cur[ROWS_PER_WAVE];
        prime_rows<BITS, ROWS_PER_WAVE>(rsrc, rowoff, nb, cur);
        const float acc =
            stream_rows<BITS, NT, ROWS_PER_WAVE, GROUPED, MX>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, I, stage, cur, G);
        if (cvec < ng) {
            const int slot = pairs[p0 + g0 + cvec];
            a.Y[(size_t)slot * H + rw + crow] = GROUPED ? acc : acc * s_down[rw + crow];
        }
        __syncthreads();
    }
}

// Combine: out[t, r] = (fmaf chain over k in rank order of w[t,k] * y[t,k][r]
// from 0) + y_shared[t][r].  One writer per element, no atomics.  A thread
// owns 4 consecutive elements (16-byte loads) and issues the loads of 8
// ranks at a time before their chains.  Grid (ceil(H / 1024), S).
constexpr int CB_K = 8;
__global__ __launch_bounds__(256) void k_combine(const FwdArgs a) {
    const int t = blockIdx.y;
    const int r = 4 * (blockIdx.x * 256 + threadIdx.x);
    const int K = a.K, H = a.H, P = a.S * a.K;
    if (r >= H) return;
    const float *w = a.w + (size_t)t * K;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    bool ok = true;
    for (int k0 = 0; k0 < K; k0 += CB_K) {
        f32x4 y[CB_K];
#pragma unroll
        for (int k = 0; k < CB_K; ++k)
            if (k0 + k < K) y[k] = *reinterpret_cast<const f32x4 *>(a.Y + (size_t)(t * K + k0 + k) * H + r);
#pragma unroll
        for (int k = 0; k < CB_K; ++k) {
            if (k0 + k < K) {
                const float wk = w[k0 + k];
                ok = ok && finite_f32(wk);
                acc.x = __builtin_fmaf(wk, y[k].x, acc.x);
                acc.y = __builtin_fmaf(wk, y[k].y, acc.y);
                acc.z = __builtin_fmaf(wk, y[k].z, acc.z);
                acc.w = __builtin_fmaf(wk, y[k].w, acc.w);
            }
        }
    }
    if (a.n_shared) {
        const f32x4 ys = *reinterpret_cast<const f32x4 *>(a.Y + (size_t)(P + t) * H + r);
        acc.x = acc.x + ys.x;
        acc.y = acc.y + ys.y;
        acc.z = acc.z + ys.z;
        acc.w = acc.w + ys.w;
    }
    *reinterpret_cast<f32x4 *>(a.out + (size_t)t * H + r) = acc;
    if (!ok && r == 0) raise_status(a.status, ST_NONFINITE);
}

// ---- launchers -----------------------------------------------------------
static int pick_nt(int S) { return S >= 4 ? 4 : (S >= 2 ? 2 : 1); }

size_t forward_smem_max(int S, int H, int I, int E, int K, int n_shared, int group) {
    (void)n_shared;
    const int nt = pick_nt(S);
    // group scales staged a chunk at a time, or every chunk's at once by the
    // primed gate/up tile (group 32 may be MXFP4: one E8M0 byte per block)
    const size_t gs = group ? std::max({groups_lds_bytes(group, 4), primed_scales_lds_bytes(H, group, false),
                                        group == 32 ? primed_scales_lds_bytes(H, group, true) : (size_t)0})
                            : 0;
    return std::max(smem_plan(S, K, E, nt, H).total, smem_plan(S, K, E, nt, I).total) + gs;
}

template <typename F>
static hipError_t launch_dyn(F kern, dim3 grid, size_t smem, hipStream_t st, const FwdArgs &a) {
    const hipError_t err = ensure_dyn_smem(reinterpret_cast<const void *>(kern), smem);
    if (err != hipSuccess) return err;
    return launch(kern, grid, dim3(256), smem, st, a);
}

template <int BITS, bool TABLE, bool GROUPED = false, bool MX = false>
static hipError_t gateup_bits(const FwdArgs &a, hipStream_t st) {
    const int P = a.S * a.K;
    const int umax = std::min(P, a.E) + a.n_shared - (TABLE ? a.shared_done : 0);
    const dim3 grid(a.I / 32, umax);
    const int nt = pick_nt(a.S);
    // group scales: a chunk at a time, or every chunk's at once (primed tile)
    const size_t gs = GROUPED ? std::max(groups_lds_bytes(a.group, 4), primed_scales_lds_bytes(a.H, a.group, MX)) : 0;
    const size_t smem = smem_plan(a.S, a.K, a.E, nt, a.H).total + gs;
    if (nt == 1) return launch_dyn(k_gateup<BITS, 1, TABLE, GROUPED, MX>, grid, smem, st, a);
    if (nt == 2) return launch_dyn(k_gateup<BITS, 2, TABLE, GROUPED, MX>, grid, smem, st, a);
    return launch_dyn(k_gateup<BITS, 4, TABLE, GROUPED, MX>, grid, smem, st, a);
}

template <int BITS, bool GROUPED = false, bool MX = false>
static hipError_t down_bits(const FwdArgs &a, hipStream_t st) {
    const int P = a.S * a.K;
    const int umax = std::min(P, a.E) + a.n_shared;
    const dim3 grid(a.H / 64, umax);
    const int nt = pick_nt(a.S);
    const size_t smem = smem_plan(a.S, a.K, a.E, nt, a.I).total + groups_lds_bytes(a.group, 4);
    if (nt == 1) return launch_dyn(k_down<BITS, 1, GROUPED, MX>, grid, smem, st, a);
    if (nt == 2) return launch_dyn(k_down<BITS, 2, GROUPED, MX>, grid, smem, st, a);
    return launch_dyn(k_down<BITS, 4, GROUPED, MX>, grid, smem, st, a);
}

// Group-scaled and MXFP4 weights are 4-bit codes only (the dims check
// refuses the others).
hipError_t launch_gateup(const FwdArgs &a, int bits, hipStream_t st) {
    const bool table = a.units != nullptr;
    if (a.mx) return table ? gateup_bits<4, true, true, true>(a, st) : gateup_bits<4, false, true, true>(a, st);
    if (a.group) return table ? gateup_bits<4, true, true>(a, st) : gateup_bits<4, false, true>(a, st);
    if (bits == 8) return table ? gateup_bits<8, true>(a, st) : gateup_bits<8, false>(a, st);
    if (bits == 4) return table ? gateup_bits<4, true>(a, st) : gateup_bits<4, false>(a, st);
    return table ? gateup_bits<2, true>(a, st) : gateup_bits<2, false>(a, st);
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t st) {
    return launch(k_combine, dim3((a.H + 1023) / 1024, a.S), dim3(256), 0, st, a);
}

hipError_t launch_down(const FwdArgs &a, int bits, hipStream_t st) {
    if (a.mx) return down_bits<4, true, true>(a, st);
    if (a.group) return down_bits<4, true>(a, st);
    if (bits == 8) return down_bits<8>(a, st);
    if (bits == 4) return down_bits<4>(a, st);
    return down_bits<2>(a, st);
}

}  // namespace coli
