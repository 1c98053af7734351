// Down projection and combine of a decode / speculative-verify batch in one
// launch (colibrì README v1.0, "What's implemented": SwiGLU experts on Q8_0
// activations, shared expert, batch-union MoE).
//
// Work decomposition.  Workgroup rt owns output rows 8 rt .. 8 rt + 7 of
// the layer (2 per wavefront) for every unit of the call, so it holds every
// term of those output elements and combines them itself: one writer per
// element, no cross-workgroup signalling, no floating-point atomics.  The
// grid is H / 8 workgroups of 256 threads, all resident at once on MI355X
// for H = 6144, and each reads 8 rows of every unique expert.
//
// Per batch of units (up to UB units and 16 pair slots): every lane loads
// block c*64 + lane of its wavefront's two rows for each unit of the batch
// (one 16-byte load per row and unit for int4, all in flight together), the
// batch's Q8_0(h) vectors are staged in LDS, the exact int32 block dots go
// to LDS, and lane (row, pair) runs the binary32 chain
// acc = fmaf(d_b, isum_b, acc) over the blocks in ascending order; the row
// result is acc * s_down[row].  The combine is the fmaf chain over k in rank
// order of w[t,k] * y[t,k][row] from 0, plus the shared expert's y.
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

template <int BITS>
struct DownRowsBatch {
    static constexpr int UB = BITS == 8 ? 4 : (BITS == 4 ? 9 : 16);  // units per batch
};

struct DownRowsPlan {
    SmemPlan T;                                      // unit table
    size_t ublob, w, qh, dh, isum, sdn, y, total;
};

__host__ __device__ inline DownRowsPlan down_rows_plan(int S, int K, int E, int n_shared, int I) {
    DownRowsPlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    const int slots = P + S * n_shared;
    const int mpb = slots < DR_MAXPB ? slots : DR_MAXPB;
    SmemPlan &T = p.T;
    T.cnt = 0;
    T.ustart = a16(T.cnt + 4 * (size_t)E);
    T.fill = a16(T.ustart + 4 * (size_t)E);
    T.uexp = a16(T.fill + 4 * (size_t)E);
    T.uoff = a16(T.uexp + 4 * (size_t)umax);
    T.pairs = a16(T.uoff + 4 * (size_t)(umax + 1));
    T.misc = a16(T.pairs + 4 * (size_t)(P + S));
    T.vq = T.vd = T.isum = T.gu = 0;
    p.ublob = a16(T.misc + 16);
    p.w = a16(p.ublob + 8 * (size_t)umax);
    p.qh = a16(p.w + 4 * (size_t)P);
    p.dh = a16(p.qh + (size_t)mpb * round_up(I, 1024));
    p.isum = a16(p.dh + 4 * (size_t)mpb * round_up(I / 32, 64));
    p.sdn = a16(p.isum + 4 * (size_t)DR_W * DR_RPW * mpb * ISUM_PITCH);
    p.y = a16(p.sdn + 4 * (size_t)umax * DR_ROWS);
    p.total = a16(p.y + 4 * (size_t)slots * DR_ROWS);
    T.total = p.total;
    return p;
}

// ONE_TOKEN: S == 1, so every unit has exactly one pair.
template <int BITS, bool ONE_TOKEN>
__global__ __launch_bounds__(DR_T) void k_down_rows(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int UB = DownRowsBatch<BITS>::UB;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I, P = S * K;
    const int slots = P + S * a.n_shared;
    const int mpb = slots < DR_MAXPB ? slots : DR_MAXPB;
    const DownRowsPlan D = down_rows_plan(S, K, E, a.n_shared, I);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(smem + D.ublob);
    float *w_l = reinterpret_cast<float *>(smem + D.w);
    int8_t *qh_l = reinterpret_cast<int8_t *>(smem + D.qh);
    float *dh_l = reinterpret_cast<float *>(smem + D.dh);
    int32_t *isum = reinterpret_cast<int32_t *>(smem + D.isum) + wave * DR_RPW * mpb * ISUM_PITCH;
    float *sdn = reinterpret_cast<float *>(smem + D.sdn);
    float *y_l = reinterpret_cast<float *>(smem + D.y);
    const int *uexp = reinterpret_cast<const int *>(smem + D.T.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + D.T.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + D.T.pairs);
    const int rt = blockIdx.x, r0 = rt * DR_ROWS;
    const BlobLayout BL = blob_layout(H, I, BITS);
    const int nbi = I / 32;
    const int nch = (nbi + 63) / 64;
    const int qpitch = round_up(I, 1024);       // LDS bytes per staged Q8_0(h) vector
    const int dpitch = round_up(nbi, 64);       // LDS floats per staged scale vector
    const size_t irow = (size_t)I * BITS / 8;

    for (int q = tid; q < P; q += DR_T) w_l[q] = a.w[q];
    for (int q = tid; q < slots * DR_ROWS; q += DR_T) y_l[q] = 0.0f;
    build_units(a.idx, S, K, E, a.n_shared, smem, D.T, a.status, false);
    const int n_units = uniform(reinterpret_cast<const int *>(smem + D.T.misc)[0]);
    for (int u = tid; u < n_units; u += DR_T) {
        const int e = uexp[u];
        ublob[u] = e < 0 ? a.shared : a.blobs[e];
    }
    __syncthreads();
    if (tid < n_units && ublob[tid] == nullptr) raise_status(a.status, ST_NOTRESIDENT);

    auto batch_end = [&](int u0) {
        int u1 = u0, npb = 0;
        while (u1 < n_units && u1 - u0 < UB) {
            const int np = uoff[u1 + 1] - uoff[u1];
            if (npb + np > mpb && u1 > u0) break;
            npb += np;
            ++u1;
        }
        return uniform(u1);
    };
    const int cr = lane >> 4 >= DR_RPW ? 0 : lane >> 4, cp = lane & 15;   // chain lane (row, pair)
    const bool chain_lane = lane < DR_RPW * 16;
    const size_t ro = BL.down + (size_t)(r0 + wave * DR_RPW) * irow;
    constexpr int MQ = 5, MD = 3;   // staging words per thread and round (codes, scales)
    BlockBits<BITS> wv[UB][DR_RPW];
    // One batch of units [u0, u1); returns u1.  ONE: a single chunk of blocks.
    auto batch = [&](int u0, auto one) -> int {
        constexpr bool ONE = decltype(one)::value;
        const int u1 = batch_end(u0);
        const int pbase = uniform(uoff[u0]);
        const int npb = uniform(uoff[u1]) - pbase;
        float acc = 0.0f;
        // Q8_0(h) of the batch's pairs (written by the gate/up kernel), their
        // block scales and the down-row scales of its units: the first round
        // of these loads is issued before the weights so that it arrives
        // first (staged through registers: reading LDS written by direct
        // global-to-LDS loads would make the compiler wait for every load)
        const int w16 = I / 16;
        const int nq = npb * w16, nd = npb * nbi, ns = (u1 - u0) * DR_ROWS;
        auto q_src = [&](int i) {
            const int pb = i / w16;
            return reinterpret_cast<const i32x4 *>(a.qh + (size_t)pairs[pbase + pb] * I) + (i - pb * w16);
        };
        auto q_dst = [&](int i) {
            const int pb = i / w16;
            return reinterpret_cast<i32x4 *>(qh_l + (size_t)pb * qpitch) + (i - pb * w16);
        };
        auto d_src = [&](int i) {
            const int pb = i / nbi;
            return a.dh + (size_t)pairs[pbase + pb] * nbi + (i - pb * nbi);
        };
        auto d_dst = [&](int i) {
            const int pb = i / nbi;
            return dh_l + pb * dpitch + (i - pb * nbi);
        };
        auto s_src = [&](int i) {
            const uint8_t *blob = ublob[u0 + i / DR_ROWS];
            return blob ? reinterpret_cast<const float *>(blob + BL.s_down) + r0 + i % DR_ROWS : &a.w[0];
        };
        auto s_dst = [&](int i) { return sdn + u0 * DR_ROWS + i; };

        const int nr = max(stage_rounds(nq, MQ * DR_T), max(stage_rounds(nd, MD * DR_T), stage_rounds(ns, DR_T)));
        i32x4 qv[MQ];
        float dv[MD], sv[1];
        stage_load(qv, 0, nq, q_src);
        stage_load(dv, 0, nd, d_src);
        stage_load(sv, 0, ns, s_src);
        __builtin_amdgcn_sched_barrier(0);
        for (int c = 0; c < (ONE ? 1 : nch); ++c) {
            const int b = c * 64 + lane;
            const bool act = b < nbi;
            // every unit slot of the batch loads in one straight run; slots
            // past the batch (or not resident) read through an empty buffer
            // resource, which returns zeros without touching memory
#pragma unroll
            for (int ui = 0; ui < UB; ++ui) {
                const int uu = u0 + ui;
                const uint8_t *blob = uniform_ptr(ublob[min(uu, n_units - 1)]);
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(blob, (uu < u1 && blob) ? (uint32_t)BL.total : 0u);
#pragma unroll
                for (int r = 0; r < DR_RPW; ++r) wv[ui][r] = load_block<BITS>(rs, (uint32_t)(ro + r * irow), b);
            }
            if (c == 0) {
                // the staged data are in once no more than the weight loads
                // just issued are outstanding
                __builtin_amdgcn_sched_barrier(0);
                wait_vm<UB * DR_RPW * BlockLoads<BITS>::N>();
                stage_store(qv, 0, nq, q_dst);
                stage_store(dv, 0, nd, d_dst);
                stage_store(sv, 0, ns, s_dst);
                for (int rd = 1; !ONE && rd < nr; ++rd) {
                    stage_load(qv, rd, nq, q_src);
                    stage_load(dv, rd, nd, d_src);
                    stage_load(sv, rd, ns, s_src);
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
#pragma unroll
                        for (int r = 0; r < DR_RPW; ++r)
                            isum[(r * mpb + (q - pbase)) * ISUM_PITCH + lane] =
                                (act && live) ? block_dot(wv[ui][r], av) : 0;
                    }
                }
            }
            wave_lds_sync();
            if (chain_lane && cp < npb)
                acc = chain_chunk(acc, isum + (cr * mpb + cp) * ISUM_PITCH, dh_l + cp * dpitch + c * 64,
                                  min(64, nbi - c * 64));
            wave_lds_sync();
        }
        if (chain_lane && cp < npb) {
            int ub = u0;   // the pair's unit: the last one whose first pair is at or before it
            while (ub + 1 < u1 && uoff[ub + 1] <= pbase + cp) ++ub;
            const int slot = pairs[pbase + cp];
            const int rl = wave * DR_RPW + cr;
            y_l[slot * DR_ROWS + rl] = ublob[ub] ? acc * sdn[ub * DR_ROWS + rl] : 0.0f;
        }
        __syncthreads();   // the next batch restages qh_l / dh_l
        return u1;
    };
    // The common decode case (every unit in one batch, rows of one chunk,
    // staging in one round) runs as straight-line code, so the compiler's
    // waits for the weight loads stay per unit; the general case loops.
    const int all_pairs = uniform(uoff[n_units]) - uniform(uoff[0]);
    if (nch == 1 && batch_end(0) == n_units && all_pairs * (I / 16) <= MQ * DR_T && all_pairs * nbi <= MD * DR_T) {
        batch(0, std::true_type{});
    } else {
        for (int u0 = 0; u0 < n_units;) u0 = batch(u0, std::false_type{});
    }
    for (int q = tid; q < S * DR_ROWS; q += DR_T) {
        const int t = q / DR_ROWS, rl = q - t * DR_ROWS;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            const float wk = w_l[t * K + k];
            if (rt == 0 && rl == 0 && !finite_f32(wk)) raise_status(a.status, ST_NONFINITE);
            acc = __builtin_fmaf(wk, y_l[(t * K + k) * DR_ROWS + rl], acc);
        }
        if (a.n_shared) acc = acc + y_l[(P + t) * DR_ROWS + rl];
        a.out[(size_t)t * H + r0 + rl] = acc;
    }
}

size_t down_rows_smem(int S, int I, int E, int K, int n_shared) {
    return down_rows_plan(S, K, E, n_shared, I).total;
}

hipError_t launch_down_rows(const FwdArgs &a, int bits, hipStream_t st) {
    const size_t smem = down_rows_plan(a.S, a.K, a.E, a.n_shared, a.I).total;
    const dim3 grid(a.H / DR_ROWS);
    auto go = [&](auto kern) {
        const hipError_t e = ensure_dyn_smem(reinterpret_cast<const void *>(kern), smem);
        if (e != hipSuccess) return e;
        return launch(kern, grid, dim3(DR_T), smem, st, a);
    };
    const bool one = a.S == 1;
    if (bits == 8) return one ? go(k_down_rows<8, true>) : go(k_down_rows<8, false>);
    if (bits == 4) return one ? go(k_down_rows<4, true>) : go(k_down_rows<4, false>);
    return one ? go(k_down_rows<2, true>) : go(k_down_rows<2, false>);
}

}  // namespace coli
