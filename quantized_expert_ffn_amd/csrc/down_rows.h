// Down projection and combine of one tile of 8 output rows for every unit of
// a decode / speculative-verify call (colibrì README v1.0, "What's
// implemented": SwiGLU experts on Q8_0 activations, shared expert,
// batch-union MoE).  Used by the down+combine kernel and by the down phase
// of the persistent layer kernel.
//
// The workgroup that owns rows r0 .. r0+7 (2 per wavefront) holds every term
// of those output elements and combines them itself: one writer per element,
// no floating-point atomics.  Per batch of units (up to UB units and
// DR_MAXPB pair slots): lane b loads block c*64 + b of its wavefront's two
// rows for each unit (one straight run of loads; slots past the batch read
// through an empty buffer resource, which returns zeros without touching
// memory), the batch's Q8_0(h) vectors and block scales are staged in LDS,
// the exact int32 block dots go to LDS, and lane (row, pair) runs the
// binary32 chain acc = fmaf(d_b, isum_b, acc) over the blocks in ascending
// order; y = acc * s_down[row].  The combine is the fmaf chain over k in rank
// order of w[t,k] * y[t,k][row] from 0, plus the shared expert's y.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "stream.h"

namespace coli {

constexpr int DR_T = 256;                // threads per workgroup
constexpr int DR_W = DR_T / 64;          // wavefronts
constexpr int DR_RPW = 2;                // rows per wavefront
constexpr int DR_ROWS = DR_W * DR_RPW;   // rows per workgroup
constexpr int DR_MAXPB = 16;             // pair slots per batch (chain lanes: DR_RPW x DR_MAXPB)
constexpr int DR_MQ = 5, DR_MD = 3;      // staging words per thread and round (codes, scales)
constexpr int CPOL_SC1 = 16;             // buffer cache policy: device-scope coherent

template <int BITS>
struct DownRowsBatch {
    static constexpr int UB = BITS == 8 ? 4 : (BITS == 4 ? 9 : 16);  // units per batch
};

// Whether the binary32 group scales (group > 0) of a wave's rows of a whole
// batch fit the staged tile's round of registers (DownTile::GW_GS words per
// lane) as whole 4-byte words.
__host__ __device__ inline bool down_staged_groups_fit(int I, int group, int bits) {
    const int ub = bits == 8 ? DownRowsBatch<8>::UB : (bits == 4 ? DownRowsBatch<4>::UB : DownRowsBatch<2>::UB);
    return group > 0 && I % group == 0 && ub * DR_RPW * (I / group) <= 64 * 9;
}

// Whether every pair slot of a call fits one batch and one staging round of
// a down tile whatever the routing (a unit has at least one pair, so there
// are no more units than slots), with rows of one 64-block chunk, and the
// unit table and routing weights one word per thread: the condition of
// slot-order staging (DownTile::slots_fetch / run_staged).
__host__ __device__ inline bool down_slots_fit(int S, int K, int E, int n_shared, int I, int bits) {
    const int slots = S * K + S * n_shared, nbi = I / 32;
    const int ub = bits == 8 ? DownRowsBatch<8>::UB : (bits == 4 ? DownRowsBatch<4>::UB : DownRowsBatch<2>::UB);
    const UnitTable U = unit_table(S, K, E);
    return nbi <= 64 && slots <= ub && slots <= DR_MAXPB && slots * (I / 16) <= DR_MQ * DR_T &&
           slots * nbi <= DR_MD * DR_T && U.words <= DR_T && U.umax <= DR_T && S * K <= DR_T;
}

// LDS of one down tile (from `base`).
struct DownTilePlan {
    size_t qh, dh, isum, sdn, y, gs, end;
    int mpb;   // pair slots per batch
};
// group > 0: room for the group scales of one batch of units (UB units x
// DR_ROWS rows x I / group scales).
// gs_bytes: bytes per staged scale (4: binary32 group scales; 1: raw E8M0
// bytes of the slot-staged MXFP4 tile).  A batch holds at most 2 ub pair
// slots (ub units of a batch, 0: no such bound): with int8 codes (4 units a
// batch) that keeps the tile of a 4-token verify step within a third of a
// CU's LDS, so all H / 8 workgroups are resident at once.
__host__ __device__ inline DownTilePlan down_tile_plan(size_t base, int S, int K, int E, int n_shared, int I,
                                                       int group = 0, int ub = 0, int gs_bytes = 4) {
    DownTilePlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    const int slots = P + S * n_shared;
    const int cap = ub > 0 && 2 * ub < DR_MAXPB ? 2 * ub : DR_MAXPB;
    const int mpb = slots < cap ? slots : cap;
    p.mpb = mpb;
    p.qh = a16(base);
    p.dh = a16(p.qh + (size_t)mpb * round_up(I, 1024));
    p.isum = a16(p.dh + 4 * (size_t)mpb * round_up(I / 32, 64));
    p.sdn = a16(p.isum + 4 * (size_t)DR_W * DR_RPW * mpb * ISUM_PITCH);
    p.y = a16(p.sdn + 4 * (size_t)umax * DR_ROWS);
    p.gs = a16(p.y + 4 * (size_t)slots * DR_ROWS);
    p.end = a16(p.gs + (group ? (size_t)gs_bytes * ub * DR_ROWS * (I / group) : 0));
    return p;
}

// The MXFP4 chain of one (row, pair) over nb blocks from 0 with the row's
// E8M0 bytes as raw words (4 blocks each): acc = fmaf(d_b * 2^(x_b - 128),
// S_b, acc), S_b the exact binary32 block sum stored as its bits; the same
// operations as chain_chunk_g<true> with group 32.
__device__ __forceinline__ float chain_mx_bytes(const int32_t *is, const float *dv, const uint32_t *xw, int nb) {
    float acc = 0.0f;
    for (int b = 0; b < nb; b += 4) {
        const i32x4 iv = *reinterpret_cast<const i32x4 *>(is + b);
        const f32x4 dd = *reinterpret_cast<const f32x4 *>(dv + b);
        const uint32_t x = xw[b / 4];
        acc = __builtin_fmaf(dd.x * e8m0_half(x & 0xFFu), __int_as_float(iv.x), acc);
        acc = __builtin_fmaf(dd.y * e8m0_half((x >> 8) & 0xFFu), __int_as_float(iv.y), acc);
        acc = __builtin_fmaf(dd.z * e8m0_half((x >> 16) & 0xFFu), __int_as_float(iv.z), acc);
        acc = __builtin_fmaf(dd.w * e8m0_half(x >> 24), __int_as_float(iv.w), acc);
    }
    return acc;
}

// One down tile.  COHERENT: Q8_0(h) was written earlier in the same launch
// by other workgroups, so it is read with device-scope loads.
// MX: MXFP4 down rows (4-bit E2M1 codes, one E8M0 byte per block; GROUPED
// with group 32).
template <int BITS, bool ONE_TOKEN, bool COHERENT, bool GROUPED = false, bool MX = false>
struct DownTile {
    static_assert(!MX || (BITS == 4 && GROUPED), "MXFP4 rows are 4-bit codes with a scale per block");
    static constexpr int UB = DownRowsBatch<BITS>::UB;
    // Staged tiles: units whose weights are in flight ahead of the block
    // dots.  Fewer loads out at once than the whole batch keeps the early
    // burst short; three cover the latency of the next (two for MXFP4 rows,
    // whose block dots take longer).
    static constexpr int AHEAD = MX ? 2 : 3;
    // Batched tiles with per-row scales (batch()): units of a batch whose
    // weights go out with its staged data; the rest follow one at a time
    // behind the block dots.
    static constexpr int BATCH_AHEAD = UB < 2 ? UB : 2;
    const FwdArgs &a;
    uint8_t *smem;
    DownTilePlan D;
    const int *uoff, *pairs;
    const uint8_t *const *ublob;   // LDS, [n_units]
    const float *w;                // routing weights [S*K] (LDS or device)
    int n_units, rt, mpb, nbi, nch, qpitch, dpitch;
    uint32_t m16, mnb;             // reciprocals for i / (I / 16) and i / nbi (fast_div)
    size_t ro, irow;
    BlobLayout BL;
    BlockBits<BITS> wv[UB][DR_RPW];

    __device__ __forceinline__ DownTile(const FwdArgs &a_, uint8_t *smem_, const DownTilePlan &D_, const int *uoff_,
                        const int *pairs_, const uint8_t *const *ublob_, const float *w_, int n_units_, int rt_)
        : a(a_), smem(smem_), D(D_), uoff(uoff_), pairs(pairs_), ublob(ublob_), w(w_), n_units(n_units_), rt(rt_) {
        mpb = D.mpb;
        nbi = a.I / 32;
        nch = (nbi + 63) / 64;
        qpitch = round_up(a.I, 1024);
        dpitch = round_up(nbi, 64);
        m16 = fast_div_magic(a.I / 16);
        mnb = fast_div_magic(nbi);
        BL = blob_layout(a.H, a.I, BITS, GROUPED && !MX ? a.group : 0, MX);
        irow = (size_t)a.I * BITS / 8;
        ro = BL.down + (size_t)(rt * DR_ROWS + uniform(threadIdx.x >> 6) * DR_RPW) * irow;
    }

    __device__ __forceinline__ int batch_end(int u0) const {
        int u1 = u0, npb = 0;
        while (u1 < n_units && u1 - u0 < UB) {
            const int np = uoff[u1 + 1] - uoff[u1];
            if (npb + np > mpb && u1 > u0) break;
            npb += np;
            ++u1;
        }
        return uniform(u1);
    }

    // All units in one batch, rows of one chunk, staging in one round: the
    // straight-line case (the weights can be issued ahead, see issue()).
    __device__ __forceinline__ bool single() const {
        const int all_pairs = uniform(uoff[n_units]) - uniform(uoff[0]);
        return nch == 1 && batch_end(0) == n_units && all_pairs * (a.I / 16) <= DR_MQ * DR_T &&
               all_pairs * nbi <= DR_MD * DR_T;
    }

    // Weight loads of units [u0, u1), chunk c, in one straight run.
    __device__ __forceinline__ void issue(int u0, int u1, int c) {
#pragma unroll
        for (int ui = 0; ui < UB; ++ui) {
            const int uu = u0 + ui;
            issue_unit(ui, uniform_ptr(ublob[min(uu, n_units - 1)]), uu < u1, c);
        }
    }
    // The loads of batch entry ui (unit blob, wave-uniform; live: part of
    // the batch; a null or dead blob reads zeros).
    __device__ __forceinline__ void issue_unit(int ui, const uint8_t *blob, bool live, int c) {
        const int b = c * 64 + (int)(threadIdx.x & 63);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(blob, (live && blob) ? (uint32_t)BL.total : 0u);
#pragma unroll
        for (int r = 0; r < DR_RPW; ++r) wv[ui][r] = load_block<BITS>(rs, (uint32_t)(ro + r * irow), b);
    }

    __device__ __forceinline__ i32x4 ld_qh(uint32_t off) const {
        if (COHERENT) {
            const uint32_t bytes = (uint32_t)(a.S * a.K + a.S * a.n_shared) * (uint32_t)a.I;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.qh, bytes);
            return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1));
        }
        return *reinterpret_cast<const i32x4 *>(a.qh + off);
    }
    __device__ __forceinline__ float ld_dh(size_t i) const { return COHERENT ? ld_dev(a.dh + i) : a.dh[i]; }

    // Group scales of this wave's DR_RPW rows for every unit of the batch
    // into the wave's LDS region of gsl (UB x DR_RPW x ngr floats).  In two
    // parts, so that the loads go out before the batch's weight loads and the
    // caller's wait for its staged data (loads complete in issue order) also
    // covers them: groups_issue sends direct global-to-LDS loads (f32 group
    // scales) or, for MXFP4, loads the first GW_MX words of E8M0 bytes per
    // lane into registers; groups_finish converts and stores those words
    // (2^(x - 128)) and does whatever did not fit, after the weights.  A unit
    // that is not resident leaves zeros (f32 scales: unset): its block dots
    // are zero and its rows' results are replaced by 0.
    static constexpr int GW_MX = 8;
    __device__ __forceinline__ int groups_ngr() const { return a.I / a.group; }
    __device__ __forceinline__ float *groups_dst(float *gsl) const {
        return gsl + uniform(threadIdx.x >> 6) * UB * DR_RPW * groups_ngr();
    }
    __device__ __forceinline__ int groups_row0() const { return rt * DR_ROWS + uniform(threadIdx.x >> 6) * DR_RPW; }
    __device__ __forceinline__ uint32_t mx_word(int u0, int w) const {
        const int wpr = groups_ngr() / 4, ur = w / wpr, p = w - ur * wpr;
        const uint8_t *blob = ublob[u0 + ur / DR_RPW];
        return blob ? *reinterpret_cast<const uint32_t *>(
                          blob + BL.s_down + (size_t)(groups_row0() + ur % DR_RPW) * groups_ngr() + 4 * p)
                    : 0u;
    }
    // Word w of the binary32 group scales of this wave's rows of units
    // u0 ..: row ur = w / ngr of them (unit u0 + ur / DR_RPW), scale w % ngr.
    static constexpr int GW_GS = 9;
    __device__ __forceinline__ uint32_t gs_word(int u0, int w) const {
        const int ngr = groups_ngr(), ur = w / ngr, p = w - ur * ngr;
        const uint8_t *blob = ublob[u0 + ur / DR_RPW];
        return blob ? *reinterpret_cast<const uint32_t *>(
                          blob + BL.s_down + ((size_t)(groups_row0() + ur % DR_RPW) * ngr + p) * 4)
                    : 0u;
    }
    __device__ __forceinline__ void mx_store(int u0, int w, uint32_t v, float *dst) const {
        const bool live = ublob[u0 + w / (groups_ngr() / 4) / DR_RPW] != nullptr;
        reinterpret_cast<f32x4 *>(dst)[w] = live ? f32x4{e8m0_half(v & 0xFFu), e8m0_half((v >> 8) & 0xFFu),
                                                         e8m0_half((v >> 16) & 0xFFu), e8m0_half(v >> 24)}
                                                 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    __device__ __forceinline__ void groups_issue(int u0, int u1, float *gsl, uint32_t (&mxv)[GW_MX]) {
        const int lane = threadIdx.x & 63, ngr = groups_ngr();
        const int nw = (u1 - u0) * DR_RPW * ngr / 4;
        if (MX) {
#pragma unroll
            for (int k = 0; k < GW_MX; ++k) {
                const int w = lane + 64 * k;
                mxv[k] = w < nw ? mx_word(u0, w) : 0u;
            }
        } else if ((ngr & 3) == 0) {
            float *dst = groups_dst(gsl);
            const int wpr = ngr / 4, rw0 = groups_row0();
            for (int w0 = 0; w0 < nw; w0 += 64) {
                const int w = w0 + lane;
                if (w < nw) {
                    const int ur = w / wpr, p = w - ur * wpr;
                    const uint8_t *blob = ublob[u0 + ur / DR_RPW];
                    if (blob)
                        lds_dma16(blob + BL.s_down + ((size_t)(rw0 + ur % DR_RPW) * ngr + 4 * p) * 4,
                                  dst + 4 * w0);
                }
            }
        }
    }

    __device__ __forceinline__ void groups_finish(int u0, int u1, float *gsl, const uint32_t (&mxv)[GW_MX]) {
        const int lane = threadIdx.x & 63, ngr = groups_ngr();
        float *dst = groups_dst(gsl);
        const int n = (u1 - u0) * DR_RPW * ngr, nw = n / 4;
        if (MX) {
#pragma unroll
            for (int k = 0; k < GW_MX; ++k) {
                const int w = lane + 64 * k;
                if (w < nw) mx_store(u0, w, mxv[k], dst);
            }
            for (int w0 = 64 * GW_MX; w0 < nw; w0 += 64 * GW_MX) {
                uint32_t v[GW_MX];
#pragma unroll
                for (int k = 0; k < GW_MX; ++k) {
                    const int w = w0 + lane + 64 * k;
                    v[k] = w < nw ? mx_word(u0, w) : 0u;
                }
#pragma unroll
                for (int k = 0; k < GW_MX; ++k) {
                    const int w = w0 + lane + 64 * k;
                    if (w < nw) mx_store(u0, w, v[k], dst);
                }
            }
        } else if ((ngr & 3) != 0) {
            const int rw0 = groups_row0();
            for (int i = lane; i < n; i += 64) {
                const int ur = i / ngr, g = i - ur * ngr;
                const uint8_t *blob = ublob[u0 + ur / DR_RPW];
                dst[i] = blob ? reinterpret_cast<const float *>(blob + BL.s_down)[(size_t)(rw0 + ur % DR_RPW) * ngr + g]
                              : 0.0f;
            }
        }
        // (f32 scales in whole 16-byte words: the direct loads of
        // groups_issue completed with the caller's wait)
    }

    // One batch of units [u0, u1); ONE: single() holds and, with issued,
    // the batch's weights were issued ahead by issue(0, n_units, 0).
    template <bool ONE>
    __device__ __forceinline__ int batch(int u0, bool issued) {
        const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
        const int I = a.I, r0 = rt * DR_ROWS;
        int8_t *qh_l = reinterpret_cast<int8_t *>(smem + D.qh);
        float *dh_l = reinterpret_cast<float *>(smem + D.dh);
        int32_t *isum = reinterpret_cast<int32_t *>(smem + D.isum) + wave * DR_RPW * mpb * ISUM_PITCH;
        float *sdn = reinterpret_cast<float *>(smem + D.sdn);
        float *y_l = reinterpret_cast<float *>(smem + D.y);
        const int u1 = ONE ? n_units : batch_end(u0);
        const int pbase = uniform(uoff[u0]);
        const int npb = uniform(uoff[u1]) - pbase;
        const int cr = lane >> 4 >= DR_RPW ? 0 : lane >> 4, cp = lane & 15;   // chain lane (row, pair)
        const bool chain_lane = lane < DR_RPW * 16;
        const int rl = wave * DR_RPW + cr;
        // the chain lane's unit: the last one whose first pair is at or before its pair
        auto unit_of_lane = [&]() {
            int u = u0;
            while (u + 1 < u1 && uoff[u + 1] <= pbase + cp) ++u;
            return u;
        };
        const int ug = GROUPED ? unit_of_lane() : 0;
        // group scales: one per 32 << lgb codes of a row, ngr per row
        const int lgb = GROUPED ? group_lgb(a.group) : -1, ngr = GROUPED ? I / a.group : 0;
        float *gsl = reinterpret_cast<float *>(smem + D.gs);
        float acc = 0.0f;
        // Q8_0(h) of the batch's pairs, their block scales and the down-row
        // scales of its units; the first round is issued before the weights
        // so that it arrives first (staged through registers: reading LDS
        // written by direct global-to-LDS loads would make the compiler wait
        // for every load)
        const int w16 = I / 16;
        const int nq = npb * w16, nd = npb * nbi, ns = (u1 - u0) * DR_ROWS;
        auto q_src = [&](int i) {
            const int pb = fast_div(i, m16);
            return ld_qh((uint32_t)pairs[pbase + pb] * (uint32_t)I + 16u * (uint32_t)(i - pb * w16));
        };
        auto q_dst = [&](int i) {
            const int pb = fast_div(i, m16);
            return reinterpret_cast<i32x4 *>(qh_l + (size_t)pb * qpitch) + (i - pb * w16);
        };
        auto d_src = [&](int i) {
            const int pb = fast_div(i, mnb);
            return ld_dh((size_t)pairs[pbase + pb] * nbi + (i - pb * nbi));
        };
        auto d_dst = [&](int i) {
            const int pb = fast_div(i, mnb);
            return dh_l + pb * dpitch + (i - pb * nbi);
        };
        auto s_src = [&](int i) {
            const uint8_t *blob = ublob[u0 + i / DR_ROWS];
            return blob ? reinterpret_cast<const float *>(blob + BL.s_down)[r0 + i % DR_ROWS] : 0.0f;
        };
        auto s_dst = [&](int i) { return sdn + u0 * DR_ROWS + i; };
        const int nr = max(stage_rounds(nq, DR_MQ * DR_T), max(stage_rounds(nd, DR_MD * DR_T), stage_rounds(ns, DR_T)));
        i32x4 qv[DR_MQ];
        float dv[DR_MD], sv[1];
        uint32_t mxv[GW_MX];
        stage_fetch(qv, 0, nq, q_src);
        stage_fetch(dv, 0, nd, d_src);
        stage_fetch(sv, 0, ns, s_src);
        if (GROUPED) groups_issue(u0, u1, gsl, mxv);
        __builtin_amdgcn_sched_barrier(0);
        for (int c = 0; c < (ONE ? 1 : nch); ++c) {
            const int b = c * 64 + lane;
            const bool act = b < nbi;
            if (!(ONE && issued)) {
                if constexpr (GROUPED) {
                    issue(u0, u1, c);
                } else {
#pragma unroll
                    for (int ui = 0; ui < BATCH_AHEAD; ++ui)
                        issue_unit(ui, uniform_ptr(ublob[min(u0 + ui, n_units - 1)]), u0 + ui < u1, c);
                }
            }
            if (c == 0) {
                // the staged data are in once no more than the weight loads
                // issued after them are outstanding
                __builtin_amdgcn_sched_barrier(0);
                if (ONE && issued)
                    wait_vm<0>();
                else
                    wait_vm<(GROUPED ? UB : BATCH_AHEAD) * DR_RPW * BlockLoads<BITS>::N>();
                stage_store(qv, 0, nq, q_dst);
                stage_store(dv, 0, nd, d_dst);
                stage_store(sv, 0, ns, s_dst);
                if (GROUPED) groups_finish(u0, u1, gsl, mxv);
                for (int rd = 1; !ONE && rd < nr; ++rd) {
                    stage_fetch(qv, rd, nq, q_src);
                    stage_fetch(dv, rd, nd, d_src);
                    stage_fetch(sv, rd, ns, s_src);
                    stage_store(qv, rd, nq, q_dst);
                    stage_store(dv, rd, nd, d_dst);
                    stage_store(sv, rd, ns, s_dst);
                }
                __syncthreads();
            }
#pragma unroll
            for (int ui = 0; ui < UB; ++ui) {
                if (u0 + ui < u1) {
                    const bool live = ublob[u0 + ui] != nullptr;
                    const int q0 = uniform(uoff[u0 + ui]);
                    const int q1 = ONE_TOKEN ? q0 + 1 : uniform(uoff[u0 + ui + 1]);
#pragma unroll
                    for (int q = q0; q < q1; ++q) {
                        int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                        if (act) load_act(qh_l + (size_t)(q - pbase) * qpitch, b, av);
                        if constexpr (MX) {
                            // exact block sums in binary32 (see block_dot_mx_f16)
                            f16x2 h[16];
                            mx_act_f16(av, h);
#pragma unroll
                            for (int r = 0; r < DR_RPW; ++r)
                                isum[(r * mpb + (q - pbase)) * ISUM_PITCH + lane] =
                                    (act && live) ? __float_as_int(block_dot_mx_f16(wv[ui][r].w, h)) : 0;
                        } else {
#pragma unroll
                            for (int r = 0; r < DR_RPW; ++r)
                                isum[(r * mpb + (q - pbase)) * ISUM_PITCH + lane] =
                                    (act && live) ? block_dot(wv[ui][r], av) : 0;
                        }
                    }
                }
                // unconditional within the batch (no records past u1), so
                // that no wait ahead of it covers the loads still in flight
                if constexpr (!GROUPED) {
                    if (!(ONE && issued) && ui + BATCH_AHEAD < UB) {
                        const int uj = ui + BATCH_AHEAD;
                        __builtin_amdgcn_sched_barrier(0);
                        issue_unit(uj, uniform_ptr(ublob[min(u0 + uj, n_units - 1)]), u0 + uj < u1, c);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            wave_lds_sync();
            if (chain_lane && cp < npb) {
                if (GROUPED)
                    acc = chain_chunk_g<MX>(acc, isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + cp * dpitch + c * 64,
                                        gsl + (wave * UB * DR_RPW + (ug - u0) * DR_RPW + cr) * ngr + c * (64 >> lgb),
                                        lgb,
                                        min(64, nbi - c * 64));
                else
                    acc = chain_chunk(acc, isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + cp * dpitch + c * 64,
                                      min(64, nbi - c * 64));
            }
            wave_lds_sync();
        }
        if (chain_lane && cp < npb) {
            const int ub = GROUPED ? ug : unit_of_lane();
            const int slot = pairs[pbase + cp];
            y_l[slot * DR_ROWS + rl] = ublob[ub] ? (GROUPED ? acc : acc * sdn[ub * DR_ROWS + rl]) : 0.0f;
        }
        __syncthreads();   // the next batch restages qh_l / dh_l
        return u1;
    }

    // Q8_0(h) codes and block scales of every pair slot, in slot order
    // (qh_l[slot], dh_l[slot]): the loads, then (after the caller's other
    // loads of the same round) the stores.
    __device__ __forceinline__ void slots_fetch(i32x4 (&qv)[DR_MQ], float (&dv)[DR_MD]) const {
        const int slots = a.S * a.K + a.S * a.n_shared, w16 = a.I / 16;
        stage_fetch(qv, 0, slots * w16, [&](int i) {
            const int sl = fast_div(i, m16);
            return ld_qh((uint32_t)sl * (uint32_t)a.I + 16u * (uint32_t)(i - sl * w16));
        });
        stage_fetch(dv, 0, slots * nbi, [&](int i) {
            const int sl = fast_div(i, mnb);
            return ld_dh((size_t)sl * nbi + (i - sl * nbi));
        });
    }
    __device__ __forceinline__ void slots_store(const i32x4 (&qv)[DR_MQ], const float (&dv)[DR_MD]) const {
        const int slots = a.S * a.K + a.S * a.n_shared, w16 = a.I / 16;
        int8_t *qh_l = reinterpret_cast<int8_t *>(smem + D.qh);
        float *dh_l = reinterpret_cast<float *>(smem + D.dh);
        stage_store(qv, 0, slots * w16, [&](int i) {
            const int sl = fast_div(i, m16);
            return reinterpret_cast<i32x4 *>(qh_l + (size_t)sl * qpitch) + (i - sl * w16);
        });
        stage_store(dv, 0, slots * nbi, [&](int i) {
            const int sl = fast_div(i, mnb);
            return dh_l + sl * dpitch + (i - sl * nbi);
        });
    }

    // Zeroes the per-slot results (a slot without a chain lane, as when a
    // non-finite routing left only the shared expert in the table, reads 0).
    __device__ __forceinline__ void zero_y() const {
        float *y_l = reinterpret_cast<float *>(smem + D.y);
        const int slots = a.S * a.K + a.S * a.n_shared;
        for (int q = threadIdx.x; q < slots * DR_ROWS; q += DR_T) y_l[q] = 0.0f;
    }

    // The whole tile when slots_fit() holds and the slots' Q8_0(h) is in LDS
    // (slots_store, then a workgroup barrier).  The weights of units [0,
    // AHEAD) go out first (per-row scales: the caller has issued them;
    // grouped and MXFP4 rows: here, behind the scale words), and unit ui +
    // AHEAD once unit ui's block dots are done.  The down-row scales come
    // right after the first loads (needed only at the end, so waiting for
    // them waits for nothing the block dots have not already waited for),
    // then the block dots, the chains and the combine.
    __device__ __forceinline__ void run_staged() {
        const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
        const int r0 = rt * DR_ROWS;
        const int8_t *qh_l = reinterpret_cast<const int8_t *>(smem + D.qh);
        const float *dh_l = reinterpret_cast<const float *>(smem + D.dh);
        int32_t *isum = reinterpret_cast<int32_t *>(smem + D.isum) + wave * DR_RPW * mpb * ISUM_PITCH;
        float *y_l = reinterpret_cast<float *>(smem + D.y);
        const int npb = uniform(uoff[n_units]);
        const int cr = lane >> 4 >= DR_RPW ? 0 : lane >> 4, cp = lane & 15;
        const bool chain = lane < DR_RPW * 16 && cp < npb;
        const int rl = wave * DR_RPW + cr;
        int ub = 0;
        while (ub + 1 < n_units && uoff[ub + 1] <= cp) ++ub;
        // MXFP4: the E8M0 bytes of this wave's rows of every unit (UB x
        // DR_RPW rows of nbi bytes, kept raw in LDS) go out first, the
        // weights right behind them; group scales (binary32, ngr a row:
        // down_staged_groups_fit) the same way, as raw words
        static_assert(!MX || UB * DR_RPW * 64 / 4 <= 64 * GW_MX, "one round of scale words");
        constexpr bool GS = GROUPED && !MX;
        const int ngr = GS ? groups_ngr() : 0;
        const int wrow = MX ? nbi / 4 : ngr;   // scale words per row
        uint32_t *gsw = reinterpret_cast<uint32_t *>(smem + D.gs) + wave * UB * DR_RPW * wrow;
        const int nsw = n_units * DR_RPW * wrow;
        uint32_t mxv[MX ? GW_MX : (GS ? GW_GS : 1)];
        if (MX) {
#pragma unroll
            for (int k = 0; k < GW_MX; ++k) {
                const int w = lane + 64 * k;
                mxv[k] = w < nsw ? mx_word(0, w) : 0u;
            }
        } else if (GS) {
#pragma unroll
            for (int k = 0; k < GW_GS; ++k) {
                const int w = lane + 64 * k;
                mxv[k] = w < nsw ? gs_word(0, w) : 0u;
            }
        }
        if constexpr (GROUPED) {
#pragma unroll
            for (int ui = 0; ui < (UB < AHEAD ? UB : AHEAD); ++ui)
                issue_unit(ui, uniform_ptr(ublob[min(ui, n_units - 1)]), ui < n_units, 0);
        }
        float sd = 0.0f;
        const uint8_t *my_blob = chain ? ublob[ub] : nullptr;
        if (!GROUPED && my_blob) sd = reinterpret_cast<const float *>(my_blob + BL.s_down)[r0 + rl];
        const int b = lane;
        const bool act = b < nbi;
#pragma unroll
        for (int ui = 0; ui < UB; ++ui) {
            if (ui < n_units) {
                const bool live = ublob[ui] != nullptr;
                const int q0 = uniform(uoff[ui]);
                const int q1 = ONE_TOKEN ? q0 + 1 : uniform(uoff[ui + 1]);
#pragma unroll
                for (int q = q0; q < q1; ++q) {
                    int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (act) load_act(qh_l + (size_t)pairs[q] * qpitch, b, av);
                    if constexpr (MX) {
                        // exact block sums in binary32 (see block_dot_mx_f16)
                        f16x2 h[16];
                        mx_act_f16(av, h);
#pragma unroll
                        for (int r = 0; r < DR_RPW; ++r)
                            isum[(r * mpb + q) * ISUM_PITCH + lane] =
                                (act && live) ? __float_as_int(block_dot_mx_f16(wv[ui][r].w, h)) : 0;
                    } else {
#pragma unroll
                        for (int r = 0; r < DR_RPW; ++r)
                            isum[(r * mpb + q) * ISUM_PITCH + lane] = (act && live) ? block_dot(wv[ui][r], av) : 0;
                    }
                }
            }
            // unconditional (a clamped index, no records past n_units), so
            // that no wait ahead of it covers the loads still in flight
            if (ui + AHEAD < UB) {
                const int uj = ui + AHEAD;
                __builtin_amdgcn_sched_barrier(0);
                issue_unit(uj, uniform_ptr(ublob[min(uj, n_units - 1)]), uj < n_units, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (GROUPED) {
#pragma unroll
            for (int k = 0; k < (MX ? GW_MX : GW_GS); ++k) {
                const int w = lane + 64 * k;
                if (w < nsw) gsw[w] = mxv[k];
            }
        }
        wave_lds_sync();
        if (chain) {
            const int slot = pairs[cp];
            if constexpr (GS) {
                // multiplier d_b * s_g per block, no row scale
                const float acc = chain_chunk_g(0.0f, isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + slot * dpitch,
                                                reinterpret_cast<const float *>(gsw) + (ub * DR_RPW + cr) * ngr,
                                                group_lgb(a.group), nbi);
                y_l[slot * DR_ROWS + rl] = my_blob ? acc : 0.0f;
            } else if constexpr (MX) {
                // multiplier d_b * 2^(x_b - 128) per block, no row scale
                const float acc = chain_mx_bytes(isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + slot * dpitch,
                                                 gsw + (ub * DR_RPW + cr) * (nbi / 4), nbi);
                y_l[slot * DR_ROWS + rl] = my_blob ? acc : 0.0f;
            } else {
                const float acc = chain_chunk(0.0f, isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + slot * dpitch, nbi);
                y_l[slot * DR_ROWS + rl] = my_blob ? acc * sd : 0.0f;
            }
        }
        __syncthreads();
        combine();
    }

    // Every unit of the tile, then the combine.  issued: single() holds and
    // issue(0, n_units, 0) was called.
    __device__ __forceinline__ void run(bool issued) {
        const int tid = threadIdx.x;
        const int S = a.S, K = a.K, P = S * K, slots = P + S * a.n_shared;
        float *y_l = reinterpret_cast<float *>(smem + D.y);
        __syncthreads();   // a previous tile's combine may still be reading y_l
        for (int q = tid; q < slots * DR_ROWS; q += DR_T) y_l[q] = 0.0f;
        if (issued) {
            batch<true>(0, true);
        } else if (single()) {
            batch<true>(0, false);
        } else {
            for (int u0 = 0; u0 < n_units;) u0 = batch<false>(u0, false);
        }
        const int r0 = rt * DR_ROWS;
        for (int q = tid; q < S * DR_ROWS; q += DR_T) {
            const int t = q / DR_ROWS, rl = q - t * DR_ROWS;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const float wk = w[t * K + k];
                if (rt == 0 && rl == 0 && !finite_f32(wk)) raise_status(a.status, ST_NONFINITE);
                acc = __builtin_fmaf(wk, y_l[(t * K + k) * DR_ROWS + rl], acc);
            }
            if (a.n_shared) acc = acc + y_l[(P + t) * DR_ROWS + rl];
            a.out[(size_t)t * a.H + r0 + rl] = acc;
        }
    }

    // out[t, rows] = rank-order fmaf chain of w[t, k] * y[t, k] from 0, plus
    // the shared expert's y (y_l complete, after a workgroup barrier).
    __device__ __forceinline__ void combine() {
        const int tid = threadIdx.x;
        const int S = a.S, K = a.K, P = S * K;
        const float *y_l = reinterpret_cast<const float *>(smem + D.y);
        const int r0 = rt * DR_ROWS;
        for (int q = tid; q < S * DR_ROWS; q += DR_T) {
            const int t = q / DR_ROWS, rl = q - t * DR_ROWS;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const float wk = w[t * K + k];
                if (rt == 0 && rl == 0 && !finite_f32(wk)) raise_status(a.status, ST_NONFINITE);
                acc = __builtin_fmaf(wk, y_l[(t * K + k) * DR_ROWS + rl], acc);
            }
            if (a.n_shared) acc = acc + y_l[(P + t) * DR_ROWS + rl];
            a.out[(size_t)t * a.H + r0 + rl] = acc;
        }
    }
};

}  // namespace coli
