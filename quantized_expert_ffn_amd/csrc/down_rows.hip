// Down projection and combine of a decode / speculative-verify batch in one
// launch (colibrì README v1.0, "What's implemented": SwiGLU experts on Q8_0
// activations, shared expert, batch-union MoE): workgroup rt owns output
// rows 8 rt .. 8 rt + 7 for every unit of the call (the tile code is in
// down_rows.h).  The grid is H / 8 workgroups of 256 threads, all resident
// at once on MI355X for H = 6144.
#include "down_rows.h"

namespace coli {

// LDS: the unit table (or the table copied from the workspace), unit blob
// pointers, routing weights, then the down tile.
struct DownRowsPlan {
    SmemPlan T;
    size_t ublob, w;
    DownTilePlan tile;
    size_t total;
};

__host__ __device__ inline DownRowsPlan down_rows_plan(int S, int K, int E, int n_shared, int I, int group,
                                                       int bits, int gs_bytes = 4) {
    DownRowsPlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    p.T = smem_plan(S, K, E, 0, 0);
    p.ublob = a16(p.T.total);
    p.w = a16(p.ublob + 8 * (size_t)umax);
    const int ub = bits == 8 ? DownRowsBatch<8>::UB : (bits == 4 ? DownRowsBatch<4>::UB : DownRowsBatch<2>::UB);
    p.tile = down_tile_plan(p.w + 4 * (size_t)P, S, K, E, n_shared, I, group, ub, gs_bytes);
    p.total = p.tile.end;
    return p;
}

// ONE_TOKEN: S == 1, so every unit has exactly one pair.
// Three workgroups per CU except for MXFP4, whose f16 activation pairs do
// not fit 168 registers beside the batch's weights (two per CU, no spills).
template <int BITS, bool ONE_TOKEN, bool GROUPED, bool MX = false>
__global__ __launch_bounds__(DR_T) __attribute__((amdgpu_waves_per_eu(MX ? 2 : 3))) void k_down_rows(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int S = a.S, K = a.K, E = a.E, P = S * K;
    const DownRowsPlan D = down_rows_plan(S, K, E, a.n_shared, a.I, a.group, BITS);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(smem + D.ublob);
    float *w_l = reinterpret_cast<float *>(smem + D.w);
    const int *uexp = reinterpret_cast<const int *>(smem + D.T.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + D.T.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + D.T.pairs);
    for (int q = tid; q < P; q += DR_T) w_l[q] = a.w[q];
    int n_units;
    if (a.units) {
        // the call's unit table (workspace, built by the router launch), its
        // words at the start of LDS (the region build_units would use, which
        // is at least as large)
        const UnitTable U = unit_table(S, K, E);
        int *tab = reinterpret_cast<int *>(smem);
        const int32_t *src = reinterpret_cast<const int32_t *>(a.units);
        const uint8_t *const *tb = reinterpret_cast<const uint8_t *const *>(a.units + U.ublob);
        for (int q = tid; q < U.words; q += DR_T) tab[q] = src[q];
        for (int q = tid; q < U.umax; q += DR_T) ublob[q] = tb[q];
        __syncthreads();
        uoff = tab + U.uoff;
        pairs = tab + U.pairs;
        n_units = uniform(tab[0]);
    } else {
        build_units(a.idx, S, K, E, a.n_shared, smem, D.T, a.status, false);
        n_units = uniform(reinterpret_cast<const int *>(smem + D.T.misc)[0]);
        for (int u = tid; u < n_units; u += DR_T) {
            const int e = uexp[u];
            ublob[u] = e < 0 ? a.shared : a.blobs[e];
        }
        __syncthreads();
    }
    if (tid < n_units && ublob[tid] == nullptr) raise_status(a.status, ST_NOTRESIDENT);
    DownTile<BITS, ONE_TOKEN, false, GROUPED, MX> tile(a, smem, D.tile, uoff, pairs, ublob, w_l, n_units,
                                                      blockIdx.x);
    tile.run(false);
}

// The same tile when every pair slot of the call fits one staging round
// (down_slots_fit, per-row scales or MXFP4, the call's unit table in the
// workspace): the slots' Q8_0(h) is fetched in the same memory round trip as
// the table (in slot order: its addresses do not depend on the routing).
// With per-row scales every wave also reads the unit count and the blob
// pointers through the scalar cache and issues the weights of its first
// DownTile::AHEAD units as soon as those are in, before the staged data has
// arrived (loads complete in issue order, so storing the staged data to LDS
// then waits for none of the weights); the rest follow one unit at a time
// behind the block dots.  Grouped and MXFP4 tiles issue theirs the same way
// from LDS after the staging (DownTile::run_staged).
template <int BITS, bool ONE_TOKEN, bool GROUPED = false, bool MX = false>
__global__ __launch_bounds__(DR_T) __attribute__((amdgpu_waves_per_eu(3))) void k_down_rows_staged(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int S = a.S, K = a.K, E = a.E, P = S * K;
    const DownRowsPlan D = down_rows_plan(S, K, E, a.n_shared, a.I, GROUPED ? a.group : 0, BITS, MX ? 1 : 4);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(smem + D.ublob);
    float *w_l = reinterpret_cast<float *>(smem + D.w);
    const UnitTable U = unit_table(S, K, E);
    int *tab = reinterpret_cast<int *>(smem);
    DownTile<BITS, ONE_TOKEN, false, GROUPED, MX> tile(a, smem, D.tile, tab + U.uoff, tab + U.pairs, ublob, w_l, 0,
                                                       blockIdx.x);
    const int32_t tw = tid < U.words ? reinterpret_cast<const int32_t *>(a.units)[tid] : 0;
    const uint8_t *tb = tid < U.umax ? reinterpret_cast<const uint8_t *const *>(a.units + U.ublob)[tid] : nullptr;
    const float wt = tid < P ? a.w[tid] : 0.0f;
    i32x4 qv[DR_MQ];
    float dv[DR_MD];
    tile.slots_fetch(qv, dv);
    if constexpr (!GROUPED) {
        constexpr int UB = DownRowsBatch<BITS>::UB;   // units <= slots <= UB
        __builtin_amdgcn_sched_barrier(0);
        const int nu = ld_scalar<int32_t>(a.units);
        // every load unconditional (a clamped index), so that they go out
        // back to back behind one wait
        const uint8_t *bp[UB];
#pragma unroll
        for (int ui = 0; ui < UB; ++ui)
            bp[ui] = ld_scalar<const uint8_t *>(a.units + U.ublob + 8 * (size_t)min(ui, U.umax - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ui = 0; ui < (UB < tile.AHEAD ? UB : tile.AHEAD); ++ui)
            tile.issue_unit(ui, bp[ui], ui < nu, 0);   // past nu: no records
        __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < U.words) tab[tid] = tw;
    if (tid < U.umax) ublob[tid] = tb;
    if (tid < P) w_l[tid] = wt;
    tile.slots_store(qv, dv);
    tile.zero_y();
    if (GROUPED)
        __syncthreads();
    else
        lds_barrier();   // orders LDS only: the weights stay in flight
    tile.n_units = uniform(tab[0]);
    if (tid < tile.n_units && ublob[tid] == nullptr) raise_status(a.status, ST_NOTRESIDENT);
    tile.run_staged();
}

size_t down_rows_smem(int S, int I, int E, int K, int n_shared, int group, int bits) {
    return down_rows_plan(S, K, E, n_shared, I, group, bits).total;
}

hipError_t launch_down_rows(const FwdArgs &a, int bits, hipStream_t st) {
    const bool staged = a.units && (a.mx || !a.group || down_staged_groups_fit(a.I, a.group, bits)) &&
                        down_slots_fit(a.S, a.K, a.E, a.n_shared, a.I, bits);
    const size_t smem = down_rows_plan(a.S, a.K, a.E, a.n_shared, a.I, a.group, bits, staged && a.mx ? 1 : 4).total;
    const dim3 grid(a.H / DR_ROWS);
    auto go = [&](auto kern) {
        const hipError_t e = ensure_dyn_smem(reinterpret_cast<const void *>(kern), smem);
        if (e != hipSuccess) return e;
        return launch(kern, grid, dim3(DR_T), smem, st, a);
    };
    const bool one = a.S == 1;
    if (staged) {
        if (a.mx) return one ? go(k_down_rows_staged<4, true, true, true>) : go(k_down_rows_staged<4, false, true, true>);
        if (a.group) return one ? go(k_down_rows_staged<4, true, true>) : go(k_down_rows_staged<4, false, true>);
        if (bits == 8) return one ? go(k_down_rows_staged<8, true>) : go(k_down_rows_staged<8, false>);
        if (bits == 4) return one ? go(k_down_rows_staged<4, true>) : go(k_down_rows_staged<4, false>);
        return one ? go(k_down_rows_staged<2, true>) : go(k_down_rows_staged<2, false>);
    }
    if (a.mx) return one ? go(k_down_rows<4, true, true, true>) : go(k_down_rows<4, false, true, true>);
    if (a.group) return one ? go(k_down_rows<4, true, true>) : go(k_down_rows<4, false, true>);
    if (bits == 8) return one ? go(k_down_rows<8, true, false>) : go(k_down_rows<8, false, false>);
    if (bits == 4) return one ? go(k_down_rows<4, true, false>) : go(k_down_rows<4, false, false>);
    return one ? go(k_down_rows<2, true, false>) : go(k_down_rows<2, false, false>);
}

}  // namespace coli
