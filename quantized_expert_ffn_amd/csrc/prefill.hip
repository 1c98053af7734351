// Batch-union kernels for large batches (prefill): colibrì README v1.0,
// "What's implemented" (batch-union MoE, each unique expert read once and
// applied to every token routed to it; SwiGLU experts on packed int8 / int4 /
// int2 weights with per-row scales and integer dots on Q8_0 activations).
//
//   k_logits_tiled  router logits, one wavefront per 8 tokens x 8 experts,
//                   each logit in the fixed order of the decode router (lane
//                   partials over h = 256 j + 4 l + c by fmaf, xor butterfly);
//   k_group         the call's unit table (experts in ascending id, then the
//                   shared expert) and its tiles of up to PF_TOK pairs of a unit;
//   k_pf_gateup     per (rows, tile): int8 matrix-core products, one Q8_0
//                   block (K = 32) per instruction; each block's exact int32
//                   sums are folded into the binary32 chains
//                   acc = fmaf(d_b, isum_b, acc) in ascending b, then the row
//                   scales, SwiGLU and Q8_0(h) of 32 rows per token;
//   k_pf_down       the same for the down rows, into Y[slot][row].
// The combine kernel of the decode path finishes the layer.  The matrix-core
// lane layout is in mfma.h.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "mfma.h"
#include "stream.h"

namespace coli {

constexpr int PF_T = 256;            // threads per workgroup (4 waves)
constexpr int LG_TT = 8, LG_TE = 8;  // tokens x experts per router wavefront

// ---- router logits ------------------------------------------------------
// Grid (ceil(E / 32), ceil(S / 8)); wave w takes experts 32 x + 8 w .. +7.
__global__ __launch_bounds__(PF_T) void k_logits_tiled(const float *__restrict__ x, const float *__restrict__ W,
                                                      float *__restrict__ logits, uint32_t *__restrict__ status,
                                                      int S, int H, int E) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e0 = blockIdx.x * 32 + wave * LG_TE, t0 = blockIdx.y * LG_TT;
    if (e0 >= E) return;
    const f32x4 *xr[LG_TT];
    const f32x4 *wr[LG_TE];
#pragma unroll
    for (int i = 0; i < LG_TT; ++i) xr[i] = reinterpret_cast<const f32x4 *>(x + (size_t)min(t0 + i, S - 1) * H);
#pragma unroll
    for (int i = 0; i < LG_TE; ++i) wr[i] = reinterpret_cast<const f32x4 *>(W + (size_t)min(e0 + i, E - 1) * H);
    float acc[LG_TT][LG_TE];
#pragma unroll
    for (int a = 0; a < LG_TT; ++a)
#pragma unroll
        for (int b = 0; b < LG_TE; ++b) acc[a][b] = 0.0f;
    // A non-finite x or W_r element makes every logit it enters non-finite
    // (an infinity times zero or an opposite infinity gives NaN, and NaN and
    // infinities survive the fmaf chain and the sums), so checking the logits
    // checks the inputs too.
    const int steps = H / 256;
    for (int j = 0; j < steps; ++j) {
        f32x4 xv[LG_TT], wv[LG_TE];
#pragma unroll
        for (int i = 0; i < LG_TT; ++i) xv[i] = xr[i][64 * j + lane];
#pragma unroll
        for (int i = 0; i < LG_TE; ++i) wv[i] = wr[i][64 * j + lane];
#pragma unroll
        for (int a = 0; a < LG_TT; ++a)
#pragma unroll
            for (int b = 0; b < LG_TE; ++b) {
                acc[a][b] = __builtin_fmaf(xv[a].x, wv[b].x, acc[a][b]);
                acc[a][b] = __builtin_fmaf(xv[a].y, wv[b].y, acc[a][b]);
                acc[a][b] = __builtin_fmaf(xv[a].z, wv[b].z, acc[a][b]);
                acc[a][b] = __builtin_fmaf(xv[a].w, wv[b].w, acc[a][b]);
            }
    }
    // lane a * 8 + b keeps logit (t0 + a, e0 + b)
    float mine = 0.0f;
#pragma unroll
    for (int a = 0; a < LG_TT; ++a)
#pragma unroll
        for (int b = 0; b < LG_TE; ++b) {
            float p = acc[a][b];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o, 64);
            if (lane == a * LG_TE + b) mine = p;
        }
    const int t = t0 + lane / LG_TE, e = e0 + lane % LG_TE;
    if (t < S && e < E) {
        logits[(size_t)t * E + e] = mine;
        if (!finite_f32(mine)) raise_status(status, ST_NONFINITE);
    }
}

// ---- grouping -----------------------------------------------------------
// One workgroup of 1024 threads.  Writes the unit table in the layout of
// unit_table() and the tile list: word 0 the number of tiles, then from word
// 4 four words per tile (unit, first pair, pairs in 1 .. PF_TOK, 0), the
// tiles in unit order.
__global__ __launch_bounds__(1024) void k_group(const int32_t *__restrict__ idx, int S, int K, int E, int n_shared,
                                                uint8_t *__restrict__ units, int32_t *__restrict__ tiles,
                                                uint32_t *__restrict__ status) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const SmemPlan T = smem_plan(S, K, E, 0, 0);
    build_units(idx, S, K, E, n_shared, smem, T, status, true);
    const int *misc = reinterpret_cast<const int *>(smem + T.misc);
    const int *uexp = reinterpret_cast<const int *>(smem + T.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + T.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + T.pairs);
    const int n_units = misc[0];
    const UnitTable U = unit_table(S, K, E);
    int32_t *tab = reinterpret_cast<int32_t *>(units);
    const int tid = threadIdx.x;
    if (tid < 4) tab[tid] = tid < 3 ? misc[tid] : 0;
    for (int q = tid; q < n_units; q += blockDim.x) tab[U.uexp + q] = uexp[q];
    for (int q = tid; q <= n_units; q += blockDim.x) tab[U.uoff + q] = uoff[q];
    for (int q = tid; q < uoff[n_units]; q += blockDim.x) tab[U.pairs + q] = pairs[q];
    // tiles: lane l of wave 0 takes units l * per .. (l + 1) * per - 1
    if (tid < 64) {
        const int per = (n_units + 63) / 64, u0 = min(tid * per, n_units), u1 = min(u0 + per, n_units);
        int mine = 0;
        for (int u = u0; u < u1; ++u) mine += (uoff[u + 1] - uoff[u] + PF_TOK - 1) / PF_TOK;
        int incl = mine;
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (tid >= o) incl += v;
        }
        int q = incl - mine;
        for (int u = u0; u < u1; ++u)
            for (int p = uoff[u]; p < uoff[u + 1]; p += PF_TOK, ++q) {
                i32x4 d;
                d.x = u;
                d.y = p;
                d.z = min(PF_TOK, uoff[u + 1] - p);
                d.w = 0;
                reinterpret_cast<i32x4 *>(tiles + 4)[q] = d;
            }
        if (tid == 63) tiles[0] = incl;
    }
}

// ---- staging of weight rows and activations through LDS -----------------
// A workgroup computes PF_ROWS rows of each of its NM matrices (gate and up,
// or down) for the 32 pairs of a tile; wave w owns rows 32 w .. 32 w + 31.
// The K dimension advances in stages of 128 bytes of every weight row
// (C = 32 / BITS blocks): each stage is loaded with whole 128-byte segments
// per row (coalesced, every byte fetched once per workgroup) into registers
// while the previous stage is computed from LDS, then written to LDS.
//
// LDS rows (weight rows, activation vectors) are padded by 16 bytes, so the
// 16-byte pieces that 8 consecutive rows read at one block offset fall on 8
// different 16-byte bank groups and every block offset is an immediate.
// Scales are stored block-major, one word per column.
constexpr int PF_ROWS = 128;

template <int BITS, int NM>
struct PfStage {
    static constexpr int C = 32 / BITS;           // blocks per stage
    static constexpr int WPIECES = 8;             // 16-byte pieces of a row per stage
    static constexpr int APIECES = 2 * C;         // 16-byte pieces of a token per stage
    static constexpr int W_CHUNKS = NM * PF_ROWS * WPIECES / PF_T;   // per thread
    static constexpr int A_CHUNKS = 32 * APIECES / PF_T;             // per thread (1, 2, 4)
    static constexpr int D_WORDS = (32 * C + PF_T - 1) / PF_T;       // per thread (1, 1, 2)
    static constexpr int WS = 128 + 16;           // LDS bytes of a weight row
    static constexpr int AS = 32 * C + 16;        // LDS bytes of an activation vector
    static constexpr int W_BYTES = NM * PF_ROWS * WS;
    static constexpr int A_BYTES = 32 * AS;
    static constexpr int D_BYTES = 32 * C * 4;
    static constexpr int LDS = W_BYTES + A_BYTES + D_BYTES;
    static constexpr int SHIFT = BITS == 8 ? 0 : (BITS == 4 ? 4 : 6);
    // group scales (one per 64 codes of a row, int4 only): G_PER groups per
    // stage and matrix, stored group-major [m][g][row] after the scales
    static constexpr int G_PER = C / 2;
    static constexpr int GS_BYTES = NM * G_PER * PF_ROWS * 4;
};

// Weight operand of block j of the stage for lane half h, from the row's
// LDS bytes (lds_raw, unpack_raw below): 16 codes of the block, times
// 2^SHIFT, as signed bytes.  Inside
// a block the order of the 32 products is free (their sum is exact), so a
// lane half may take any 16 codes as long as its activation operand holds
// the matching activation codes in the same order:
//   int8: codes 16 h .. 16 h + 15 (bytes 16 h .. 16 h + 15), as they are;
//   int4: the low nibbles of bytes 8 h .. 8 h + 7 (codes 8 h .. 8 h + 7),
//         then their high nibbles (codes 16 + 8 h ..), each masked into the
//         top of a byte (16 * code); the activations of a block are stored
//         in LDS in the order 0-7, 16-23, 8-15, 24-31 to match;
//   int2: fields 2 h and 2 h + 1 of the block's 8 bytes (codes 16 h ..
//         16 h + 15), shifted into the top two bits (64 * code).
// The tile of workgroup row blockIdx.y: unit, first pair, pairs.
struct Tile {
    int u, p_first, n;
};

__device__ __forceinline__ int slot_token(int slot, int P, int K) { return slot < P ? slot / K : slot - P; }

// Whether d * 2^-SHIFT is exact for the nb block scales d[0 .. nb) of every
// lane of the wave (true unless some scale lies within 2^SHIFT of the
// denormal range).  Then d * 2^-SHIFT times the 2^SHIFT-scaled sum is the
// same product as d times the true sum, and the chain needs no shift.
// A scale that is 0 or at least 2^-120 qualifies (for SHIFT <= 6 its
// product with 2^-SHIFT is a normal number or 0); smaller ones take the
// shifting path, which is exact for every scale.
template <int SHIFT, bool GROUPED = false>
__device__ __forceinline__ bool scales_fold(const float *d, int nb) {
    if (SHIFT == 0 && !GROUPED) return true;
    constexpr float LOW = GROUPED ? 0x1p-60f : 0x1p-120f;
    bool ok = true;
    if ((nb & 3) == 0 && (reinterpret_cast<uintptr_t>(d) & 15) == 0) {
        const f32x4 *v4 = reinterpret_cast<const f32x4 *>(d);
#pragma unroll 8
        for (int b = 0; b < nb / 4; ++b) {
            const f32x4 v = v4[b];
            ok = ok && (v.x == 0.0f || v.x >= LOW) && (v.y == 0.0f || v.y >= LOW) && (v.z == 0.0f || v.z >= LOW) &&
                 (v.w == 0.0f || v.w >= LOW);
        }
    } else {
        for (int b = 0; b < nb; ++b) ok = ok && (d[b] == 0.0f || d[b] >= LOW);
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Operands of a tile: NM weight matrices at byte offsets mat[m] of the blob
// (rows of rb bytes, row0 = first row of the workgroup, n_rows valid rows of
// the matrix), the Q8_0 vectors of the tile's 32 columns (codes at
// voff[col] of ra, scales at doff[col] of rd, vec_bytes per vector).
template <int NM>
struct PfSrc {
    __amdgpu_buffer_rsrc_t rw, ra, rd;
    uint32_t mat[NM];
    uint32_t rb;
    int row0, n_rows, nb;
    uint32_t smat[NM];   // group-scaled: byte offsets of the scale sections
    uint32_t srow;       // and bytes of group scales per row
};

// Stage registers of one thread.
template <int BITS, int NM>
struct PfRegs {
    u32x4 w[PfStage<BITS, NM>::W_CHUNKS];
    u32x4 a[PfStage<BITS, NM>::A_CHUNKS];
    uint32_t d[PfStage<BITS, NM>::D_WORDS];
    u32x4 g;   // group-scaled: the stage's 4 group scales of one row (threads < NM * PF_ROWS)
};

template <int BITS, int NM, bool GROUPED = false>
__device__ __forceinline__ void pf_load(PfRegs<BITS, NM> &R, const PfSrc<NM> &src, const uint32_t *col_voff,
                                        const uint32_t *col_doff, int stage) {
    using ST = PfStage<BITS, NM>;
    const int tid = threadIdx.x;
    if constexpr (GROUPED) {
        static_assert(ST::G_PER == 4, "group-scaled stages hold 4 groups of 64 codes");
        if (tid < NM * PF_ROWS) {
            const int m = tid / PF_ROWS, row = tid % PF_ROWS;
            const int r = min(src.row0 + row, src.n_rows - 1);
            R.g = __builtin_amdgcn_raw_buffer_load_b128(src.rw, src.smat[m] + (uint32_t)r * src.srow + 16u * stage,
                                                        0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < ST::W_CHUNKS; ++i) {
        // a matrix spans PF_ROWS * 8 / PF_T = 4 chunks of every thread
        constexpr int PER_M = PF_ROWS * 8 / PF_T;
        const int m = i / PER_M, row = ((i % PER_M) * PF_T + tid) / 8, piece = tid % 8;
        const int r = min(src.row0 + row, src.n_rows - 1);
        const uint32_t off = src.mat[m] + (uint32_t)r * src.rb + 128u * stage + 16u * piece;
        // default cache policy: the tiles of one expert share these lines in L2
        R.w[i] = __builtin_amdgcn_raw_buffer_load_b128(src.rw, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < ST::A_CHUNKS; ++i) {
        const int g = i * PF_T + tid;
        const int col = g / ST::APIECES, piece = g % ST::APIECES;
        R.a[i] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, col_voff[col] + 32u * ST::C * stage + 16u * piece, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < ST::D_WORDS; ++i) {
        const int g = i * PF_T + tid;
        const int col = min(g / ST::C, 31), c = g % ST::C;
        R.d[i] = __builtin_amdgcn_raw_buffer_load_b32(src.rd, col_doff[col] + 4u * (ST::C * stage + c), 0, 0);
    }
}

// FOLD: the scales are stored times 2^-SHIFT.  GROUPED: the stage's group
// scales go to LDS too; with FOLD, a nonzero one below 2^-60 sets *refold
// (the folded chain is then not exact and the tile is recomputed).
template <int BITS, int NM, bool FOLD, bool GROUPED = false>
__device__ __forceinline__ void pf_store(const PfRegs<BITS, NM> &R, uint8_t *lds, int *refold = nullptr) {
    using ST = PfStage<BITS, NM>;
    const int tid = threadIdx.x;
    if constexpr (GROUPED) {
        if (tid < NM * PF_ROWS) {
            const int m = tid / PF_ROWS, row = tid % PF_ROWS;
            float *gs = reinterpret_cast<float *>(lds + ST::LDS) + m * ST::G_PER * PF_ROWS + row;
            // (the whole vector is reinterpreted: a bit cast of one element of a
            // vector register compiled to the first element for every one)
            const f32x4 v4 = __builtin_bit_cast(f32x4, R.g);
            const float v[4] = {v4.x, v4.y, v4.z, v4.w};
            bool small = false;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                gs[g * PF_ROWS] = v[g];
                small = small || (v[g] != 0.0f && __builtin_fabsf(v[g]) < 0x1p-60f);
            }
            if (FOLD && small) *refold = 1;
        }
    }
#pragma unroll
    for (int i = 0; i < ST::W_CHUNKS; ++i) {
        const int g = i * PF_T + tid;
        const int mrow = g / 8, piece = g % 8;  // row index over all matrices
        *reinterpret_cast<u32x4 *>(lds + ST::WS * mrow + 16 * piece) = R.w[i];
    }
    uint8_t *la = lds + ST::W_BYTES;
#pragma unroll
    for (int i = 0; i < ST::A_CHUNKS; ++i) {
        const int g = i * PF_T + tid;
        const int col = g / ST::APIECES, piece = g % ST::APIECES;
        uint8_t *dst = la + ST::AS * col + 16 * piece;
        if (BITS == 4) {
            // bytes 8 k .. 8 k + 7 of a block go to 8 (k / 2) + 16 (k % 2)
            uint8_t *blk = la + ST::AS * col + 32 * (piece >> 1) + 8 * (piece & 1);
            *reinterpret_cast<u32x2 *>(blk) = u32x2{R.a[i].x, R.a[i].y};
            *reinterpret_cast<u32x2 *>(blk + 16) = u32x2{R.a[i].z, R.a[i].w};
        } else {
            *reinterpret_cast<u32x4 *>(dst) = R.a[i];
        }
    }
    float *ld = reinterpret_cast<float *>(lds + ST::W_BYTES + ST::A_BYTES);
#pragma unroll
    for (int i = 0; i < ST::D_WORDS; ++i) {
        const int g = i * PF_T + tid;
        const float d = __builtin_bit_cast(float, R.d[i]);
        if (g < 32 * ST::C) ld[32 * (g % ST::C) + g / ST::C] = FOLD ? d * (1.0f / (float)(1 << ST::SHIFT)) : d;
    }
}

// Raw LDS words of a block's weight operand (8 or 16 bytes of the row).
template <int BITS>
struct RawW {
    typedef u32x2 T;
};
template <>
struct RawW<8> {
    typedef u32x4 T;
};

template <int BITS>
__device__ __forceinline__ typename RawW<BITS>::T lds_raw(const uint8_t *row_lds, int j, int h) {
    if constexpr (BITS == 8) return *reinterpret_cast<const u32x4 *>(row_lds + 32 * j + 16 * h);
    else if constexpr (BITS == 4) return *reinterpret_cast<const u32x2 *>(row_lds + 16 * j + 8 * h);
    else return *reinterpret_cast<const u32x2 *>(row_lds + 8 * j);
}

// The operand from the raw words (see lds_weight).
template <int BITS>
__device__ __forceinline__ i32x4 unpack_raw(typename RawW<BITS>::T w, int h) {
    i32x4 o;
    if constexpr (BITS == 8) {
        o = i32x4{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
    } else if constexpr (BITS == 4) {
        o.x = (int)((w.x << 4) & 0xF0F0F0F0u);
        o.y = (int)((w.y << 4) & 0xF0F0F0F0u);
        o.z = (int)(w.x & 0xF0F0F0F0u);
        o.w = (int)(w.y & 0xF0F0F0F0u);
    } else {
        const int s0 = 6 - 4 * h, s1 = 4 - 4 * h;
        o.x = (int)((w.x << s0) & 0xC0C0C0C0u);
        o.y = (int)((w.y << s0) & 0xC0C0C0C0u);
        o.z = (int)((w.x << s1) & 0xC0C0C0C0u);
        o.w = (int)((w.y << s1) & 0xC0C0C0C0u);
    }
    return o;
}

// Blocks 0 .. nblk - 1 of a stage in LDS (all C of them when FULL).  The
// raw operands of block j + 1 are read before the chains of block j and
// unpacked after them, so the LDS latency overlaps the chains.
// GROUPED: lg points at the lane's first row (32 w + 4 h) of group 0 of
// matrix 0 in the staged group scales; each block's multiplier is
// d_b * s[row][group] (one binary32 product).
template <int BITS, int NM, bool FOLD, int C, bool FULL, bool GROUPED = false>
__device__ __forceinline__ void pf_blocks(float (&acc)[NM][16], const uint8_t *lw, const uint8_t *la,
                                          const float *ld, int h, int nblk, const float *lg = nullptr) {
    using ST = PfStage<BITS, NM>;
    constexpr int SH = ST::SHIFT;
    float sg[NM][16];
    typename RawW<BITS>::T wr[NM];
    i32x4 xa;
    float da;
#pragma unroll
    for (int m = 0; m < NM; ++m) wr[m] = lds_raw<BITS>(lw + m * PF_ROWS * ST::WS, 0, h);
    xa = *reinterpret_cast<const i32x4 *>(la);
    da = ld[0];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        if (!FULL && j >= nblk) break;
        i32x16 c[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) c[m] = mfma_i8_32x32x32(unpack_raw<BITS>(wr[m], h), xa);
        const float d = da;
        if (j + 1 < C && (FULL || j + 1 < nblk)) {
#pragma unroll
            for (int m = 0; m < NM; ++m) wr[m] = lds_raw<BITS>(lw + m * PF_ROWS * ST::WS, j + 1, h);
            xa = *reinterpret_cast<const i32x4 *>(la + 32 * (j + 1));
            da = ld[32 * (j + 1)];
        }
        if constexpr (GROUPED) {
            if ((j & 1) == 0) {
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v =
                            *reinterpret_cast<const f32x4 *>(lg + (m * ST::G_PER + j / 2) * PF_ROWS + 8 * q);
                        sg[m][4 * q] = v.x;
                        sg[m][4 * q + 1] = v.y;
                        sg[m][4 * q + 2] = v.z;
                        sg[m][4 * q + 3] = v.w;
                    }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[m][r] = __builtin_fmaf(GROUPED ? d * sg[m][r] : d, (float)(FOLD ? c[m][r] : c[m][r] >> SH),
                                           acc[m][r]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The staged product loop: acc[m][r] = chain over the nb blocks of
// d_b * isum_b for row 32 w + mfma_c_row(lane, r) of matrix m and the lane's
// column.  Every wave runs the loads and barriers; `active` waves compute.
template <int BITS, int NM, bool FOLD, bool TAIL, bool GROUPED = false>
__device__ __forceinline__ void pf_run(float (&acc)[NM][16], uint8_t *lds, const PfSrc<NM> &src,
                                       const uint32_t *col_voff, const uint32_t *col_doff, bool active,
                                       int *refold = nullptr) {
    using ST = PfStage<BITS, NM>;
    constexpr int SH = ST::SHIFT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int n_stages = (src.nb + ST::C - 1) / ST::C;
    const float *lg = reinterpret_cast<const float *>(lds + ST::LDS) + 32 * wave + 4 * h;
    PfRegs<BITS, NM> R;
    pf_load<BITS, NM, GROUPED>(R, src, col_voff, col_doff, 0);
    const uint8_t *la = lds + ST::W_BYTES + ST::AS * n + 16 * h;
    const float *ld = reinterpret_cast<const float *>(lds + ST::W_BYTES + ST::A_BYTES) + n;
    const uint8_t *lw = lds + ST::WS * (32 * wave + n);
    // full stages; a short last stage (K no multiple of the stage) after the
    // loop, so that the loop body has a single path for the accumulators
    const int n_full = src.nb / ST::C;
    for (int s = 0; s < n_full; ++s) {
        if (s > 0) __syncthreads();  // every wave is done with the previous stage
        pf_store<BITS, NM, FOLD, GROUPED>(R, lds, refold);
        __syncthreads();
        if (s + 1 < n_stages) pf_load<BITS, NM, GROUPED>(R, src, col_voff, col_doff, s + 1);
        if (active) pf_blocks<BITS, NM, FOLD, ST::C, true, GROUPED>(acc, lw, la, ld, h, ST::C, lg);
    }
    if (TAIL && n_full < n_stages) {
        if (n_full > 0) __syncthreads();
        pf_store<BITS, NM, FOLD, GROUPED>(R, lds, refold);
        __syncthreads();
        const int nblk = src.nb - ST::C * n_full;
        if (active) {
            for (int j = 0; j < nblk; ++j) {
                const i32x4 xb = *reinterpret_cast<const i32x4 *>(la + 32 * j);
                const float d = ld[32 * j];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const i32x16 c = mfma_i8_32x32x32(
                        unpack_raw<BITS>(lds_raw<BITS>(lw + m * PF_ROWS * ST::WS, j, h), h), xb);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float dm = GROUPED ? d * lg[(m * ST::G_PER + j / 2) * PF_ROWS + mfma_c_row(lane, r) - 4 * h]
                                                 : d;
                        acc[m][r] = __builtin_fmaf(dm, (float)(FOLD ? c[r] : c[r] >> SH), acc[m][r]);
                    }
                }
            }
        }
    }
}

// pf_run with the folded or the shifting chain (FOLD is the same for every
// wave of a workgroup: they share the tile's columns).
template <int BITS, int NM, bool TAIL>
__device__ __forceinline__ void pf_dispatch(bool fold, float (&acc)[NM][16], uint8_t *lds, const PfSrc<NM> &src,
                                            const uint32_t *col_voff, const uint32_t *col_doff, bool active) {
    if (fold)
        pf_run<BITS, NM, true, TAIL>(acc, lds, src, col_voff, col_doff, active);
    else
        pf_run<BITS, NM, false, TAIL>(acc, lds, src, col_voff, col_doff, active);
}

// Group-scaled weights: the folded chain multiplies d * 2^-SHIFT by the group
// scale, which equals (d * s) * 2^-SHIFT while that product stays normal; the
// fold test admits block scales of at least 2^-60 and the stores check the
// group scales, so every product is at least 2^-120.  A tile whose group
// scales fail the check is recomputed with the shifting chain.
template <int BITS, int NM, bool TAIL>
__device__ __forceinline__ void pf_dispatch_grouped(bool fold, float (&acc)[NM][16], uint8_t *lds,
                                                    const PfSrc<NM> &src, const uint32_t *col_voff,
                                                    const uint32_t *col_doff, bool active, int *refold) {
    if (fold) {
        pf_run<BITS, NM, true, TAIL, true>(acc, lds, src, col_voff, col_doff, active, refold);
        __syncthreads();
        if (!*refold) return;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
    }
    pf_run<BITS, NM, false, TAIL, true>(acc, lds, src, col_voff, col_doff, active, refold);
}

// ---- tiles of at most 16 pairs -----------------------------------------
// The same stages, with two v_mfma_i32_16x16x32_i8 per block and matrix
// (rows 0-15 and 16-31 of the wave) over the tile's first 16 columns: half
// the conversions and chain steps of a 32-column product, the rest being
// padding.  Lane l takes column l % 16 and, of each block, the 8 codes of
// quarter q = l / 16: int8 codes 8 q .. 8 q + 7; int4 the low and high
// nibbles of bytes 4 q .. 4 q + 3 (codes 4 q .. 4 q + 3 and 16 + 4 q ..
// 16 + 4 q + 3, each as 16 * code), with the activations read in the
// matching order from their LDS order (0-7, 16-23, 8-15, 24-31).  A
// block's sum is exact whatever the order, so the chain is R-DOT's.
template <int BITS>
__device__ __forceinline__ int64_t narrow_w(const uint8_t *row_lds, int j, int q) {
    if constexpr (BITS == 8) {
        return *reinterpret_cast<const int64_t *>(row_lds + 32 * j + 8 * q);
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(row_lds + 16 * j + 4 * q);
        const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
        return (int64_t)(((uint64_t)hi << 32) | lo);
    }
}

template <int BITS>
__device__ __forceinline__ int64_t narrow_a(const uint8_t *col_lds, int j, int q) {
    if constexpr (BITS == 8) {
        return *reinterpret_cast<const int64_t *>(col_lds + 32 * j + 8 * q);
    } else {
        const int o = q < 2 ? 4 * q : 16 + 4 * (q - 2);
        const uint32_t lo = *reinterpret_cast<const uint32_t *>(col_lds + 32 * j + o);
        const uint32_t hi = *reinterpret_cast<const uint32_t *>(col_lds + 32 * j + o + 8);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    }
}

// Blocks 0 .. nblk - 1 of a stage in LDS (all C when FULL); acc[m][4 g + i]
// is row 16 g + 4 q + i of the wave's 32 rows of matrix m.  GROUPED: lg
// points at the lane's first row (32 w + 4 q) of group 0 of matrix 0 in the
// staged group scales, and each block's multiplier is d_b * s[row][group].
template <int BITS, int NM, bool FOLD, int C, bool FULL, bool GROUPED = false>
__device__ __forceinline__ void pf_blocks_narrow(float (&acc)[NM][8], const uint8_t *lw, const uint8_t *la,
                                                 const float *ld, int q, int nblk, const float *lg = nullptr) {
    using ST = PfStage<BITS, NM>;
    constexpr int SH = ST::SHIFT;
    float sg[NM][8];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        if (FULL || j < nblk) {
            const int64_t b = narrow_a<BITS>(la, j, q);
            const float d = ld[32 * j];
            if constexpr (GROUPED) {
                if ((j & 1) == 0) {
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int g = 0; g < 2; ++g) {
                            const f32x4 v =
                                *reinterpret_cast<const f32x4 *>(lg + (m * ST::G_PER + j / 2) * PF_ROWS + 16 * g);
                            sg[m][4 * g] = v.x;
                            sg[m][4 * g + 1] = v.y;
                            sg[m][4 * g + 2] = v.z;
                            sg[m][4 * g + 3] = v.w;
                        }
                }
            }
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const i32x4 c =
                        mfma_i8_16x16x32(narrow_w<BITS>(lw + (m * PF_ROWS + 16 * g) * ST::WS, j, q), b);
                    const int32_t cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[m][4 * g + i] = __builtin_fmaf(GROUPED ? d * sg[m][4 * g + i] : d,
                                                           (float)(FOLD ? cv[i] : cv[i] >> SH), acc[m][4 * g + i]);
                }
        }
    }
}

// pf_run for a tile of at most 16 pairs.
template <int BITS, int NM, bool FOLD, bool GROUPED = false>
__device__ __forceinline__ void pf_run_narrow(float (&acc)[NM][8], uint8_t *lds, const PfSrc<NM> &src,
                                              const uint32_t *col_voff, const uint32_t *col_doff, bool active,
                                              int *refold = nullptr) {
    using ST = PfStage<BITS, NM>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q = lane >> 4, c = lane & 15;
    const int n_stages = (src.nb + ST::C - 1) / ST::C;
    PfRegs<BITS, NM> R;
    pf_load<BITS, NM, GROUPED>(R, src, col_voff, col_doff, 0);
    const uint8_t *la = lds + ST::W_BYTES + ST::AS * c;
    const float *ld = reinterpret_cast<const float *>(lds + ST::W_BYTES + ST::A_BYTES) + c;
    const uint8_t *lw = lds + ST::WS * (32 * wave + c);
    const float *lg = reinterpret_cast<const float *>(lds + ST::LDS) + 32 * wave + 4 * q;
    for (int s = 0; s < n_stages; ++s) {
        if (s > 0) __syncthreads();  // every wave is done with the previous stage
        pf_store<BITS, NM, FOLD, GROUPED>(R, lds, refold);
        __syncthreads();
        if (s + 1 < n_stages) pf_load<BITS, NM, GROUPED>(R, src, col_voff, col_doff, s + 1);
        const int nblk = min(ST::C, src.nb - ST::C * s);
        if (active) {
            if (nblk == ST::C)
                pf_blocks_narrow<BITS, NM, FOLD, ST::C, true, GROUPED>(acc, lw, la, ld, q, nblk, lg);
            else
                pf_blocks_narrow<BITS, NM, FOLD, ST::C, false, GROUPED>(acc, lw, la, ld, q, nblk, lg);
        }
    }
}

// pf_run_narrow with the folded or the shifting chain; group-scaled: a tile
// whose group scales fail the fold check is recomputed with the shifting
// chain (as pf_dispatch_grouped).
template <int BITS, int NM, bool GROUPED>
__device__ __forceinline__ void pf_dispatch_narrow(bool fold, float (&acc)[NM][8], uint8_t *lds,
                                                   const PfSrc<NM> &src, const uint32_t *col_voff,
                                                   const uint32_t *col_doff, bool active, int *refold) {
    if (fold) {
        pf_run_narrow<BITS, NM, true, GROUPED>(acc, lds, src, col_voff, col_doff, active, refold);
        if (!GROUPED) return;
        __syncthreads();
        if (!*refold) return;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[m][r] = 0.0f;
    }
    pf_run_narrow<BITS, NM, false, GROUPED>(acc, lds, src, col_voff, col_doff, active, refold);
}

// Columns of the tile: the slot of pair n (the tile's first pair past its
// end) and that slot's token.
struct PfCols {
    int slot, tok;
    bool live;
};
__device__ __forceinline__ PfCols pf_col(const int32_t *pairs, const Tile &tl, int n, int P, int K) {
    PfCols c;
    c.live = n < tl.n;
    c.slot = pairs[tl.p_first + (c.live ? n : 0)];
    c.tok = slot_token(c.slot, P, K);
    return c;
}

// ---- gate/up ------------------------------------------------------------
// Grid (ceil(I / PF_ROWS), tile bound).  Epilogue: row scales, SwiGLU and
// Q8_0 over each wave's 32 rows (one block of h) for every live column.
// GROUPED: int4 with one scale per 64 codes of a row (no row scale).
template <int BITS, bool GROUPED>
__global__ __launch_bounds__(PF_T) __attribute__((amdgpu_waves_per_eu(GROUPED ? 2 : 3))) void k_pf_gateup(const FwdArgs a, const int32_t *__restrict__ tiles) {
    using ST = PfStage<BITS, 2>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[ST::LDS + (GROUPED ? ST::GS_BYTES : 0)];
    __shared__ uint32_t col_voff[32], col_doff[32];
    __shared__ int refold;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int H = a.H, I = a.I, P = a.S * a.K, nb = H / 32;
    if ((int)blockIdx.y >= tiles[0]) return;
    const i32x4 td = reinterpret_cast<const i32x4 *>(tiles + 4)[blockIdx.y];
    const Tile tl{td.x, td.y, td.z};
    const UnitTable U = unit_table(a.S, a.K, a.E);
    const int32_t *tab = reinterpret_cast<const int32_t *>(a.units);
    const int e = tab[U.uexp + tl.u];
    const uint8_t *blob = e < 0 ? a.shared : a.blobs[e];
    if (!blob) {
        if (threadIdx.x == 0 && blockIdx.x == 0) raise_status(a.status, ST_NOTRESIDENT);
        return;
    }
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED ? 64 : 0);
    const PfCols col = pf_col(tab + U.pairs, tl, n, P, a.K);
    if (threadIdx.x < 32) {
        col_voff[n] = (uint32_t)col.tok * (uint32_t)H;
        col_doff[n] = (uint32_t)col.tok * (uint32_t)nb * 4u;
    }
    if (threadIdx.x == 0) refold = 0;
    PfSrc<2> src;
    src.rw = make_rsrc(blob, (uint32_t)BL.total);
    src.ra = make_rsrc(a.qx, (uint32_t)a.S * (uint32_t)H);
    src.rd = make_rsrc(a.dx, (uint32_t)a.S * (uint32_t)nb * 4u);
    src.mat[0] = (uint32_t)BL.gate;
    src.mat[1] = (uint32_t)BL.up;
    src.rb = (uint32_t)H * BITS / 8;
    src.row0 = blockIdx.x * PF_ROWS;
    src.n_rows = I;
    src.nb = nb;
    src.smat[0] = (uint32_t)BL.s_gate;
    src.smat[1] = (uint32_t)BL.s_up;
    src.srow = (uint32_t)(4 * (H / 64));
    __syncthreads();
    const int i0 = src.row0 + 32 * wave;
    const bool active = i0 < I;
    // every wave has the same 32 columns, hence the same choice
    const bool fold = scales_fold<ST::SHIFT, GROUPED>(a.dx + (size_t)col.tok * nb, nb);
    if constexpr (BITS == 4 || (BITS == 8 && !GROUPED)) {
        if (tl.n <= 16) {
            float an[2][8];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 8; ++r) an[m][r] = 0.0f;
            pf_dispatch_narrow<BITS, 2, GROUPED>(fold, an, lds, src, col_voff, col_doff, active, &refold);
            if (!active) return;
            // lane (column c, quarter q) holds rows 16 g + 4 q + i
            const int c = lane & 15, qq = lane >> 4;
            const PfCols cc = pf_col(tab + U.pairs, tl, c, P, a.K);
            const float *sg = reinterpret_cast<const float *>(blob + BL.s_gate) + i0;
            const float *su = reinterpret_cast<const float *>(blob + BL.s_up) + i0;
            float hv[8], amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int row = 16 * (r / 4) + 4 * qq + r % 4;
                hv[r] = GROUPED ? swiglu_f32(an[0][r], an[1][r]) : swiglu_f32(an[0][r] * sg[row], an[1][r] * su[row]);
                amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[r]));
            }
            // Q8_0 over the 32 rows of the column, held by its four lanes
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16, 64));
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
            if (!cc.live) return;
            const float dq = amax / 127.0f;
            int8_t *qrow = a.qh + (size_t)cc.slot * I + i0;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                uint32_t word = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = 0.0f;
                    if (dq != 0.0f) {
                        v = __builtin_roundf(hv[4 * g + i] / dq);
                        v = __builtin_fminf(__builtin_fmaxf(v, -127.0f), 127.0f);
                    }
                    word |= (uint32_t)(uint8_t)(int8_t)(int)v << (8 * i);
                }
                *reinterpret_cast<uint32_t *>(qrow + 16 * g + 4 * qq) = word;
            }
            if (qq == 0) a.dh[(size_t)cc.slot * (I / 32) + i0 / 32] = dq;
            return;
        }
    }
    float acc[2][16];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
    if constexpr (GROUPED) {
        if (nb % ST::C != 0)
            pf_dispatch_grouped<BITS, 2, true>(fold, acc, lds, src, col_voff, col_doff, active, &refold);
        else
            pf_dispatch_grouped<BITS, 2, false>(fold, acc, lds, src, col_voff, col_doff, active, &refold);
    } else {
        if (nb % ST::C != 0)
            pf_dispatch<BITS, 2, true>(fold, acc, lds, src, col_voff, col_doff, active);
        else
            pf_dispatch<BITS, 2, false>(fold, acc, lds, src, col_voff, col_doff, active);
    }
    if (!active || !col.live) return;
    const float *sg = reinterpret_cast<const float *>(blob + BL.s_gate) + i0;
    const float *su = reinterpret_cast<const float *>(blob + BL.s_up) + i0;
    float hv[16], amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = mfma_c_row(lane, r);
        hv[r] = GROUPED ? swiglu_f32(acc[0][r], acc[1][r]) : swiglu_f32(acc[0][r] * sg[row], acc[1][r] * su[row]);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[r]));
    }
    // Q8_0 over the 32 rows of the column, held by lanes n and n + 32
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
    const float dq = amax / 127.0f;
    int8_t *qrow = a.qh + (size_t)col.slot * I + i0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float c = 0.0f;
            if (dq != 0.0f) {
                c = __builtin_roundf(hv[4 * g + q] / dq);
                c = __builtin_fminf(__builtin_fmaxf(c, -127.0f), 127.0f);
            }
            word |= (uint32_t)(uint8_t)(int8_t)(int)c << (8 * q);
        }
        *reinterpret_cast<uint32_t *>(qrow + 8 * g + 4 * h) = word;
    }
    if (h == 0) a.dh[(size_t)col.slot * (I / 32) + i0 / 32] = dq;
}

// ---- down ---------------------------------------------------------------
// Grid (ceil(H / PF_ROWS), tile bound): Y[slot][row] = s_d[row] * chain over
// the I / 32 blocks of Q8_0(h) of the slot.
template <int BITS, bool GROUPED>
__global__ __launch_bounds__(PF_T, 4) void k_pf_down(const FwdArgs a, const int32_t *__restrict__ tiles) {
    using ST = PfStage<BITS, 1>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[ST::LDS + (GROUPED ? ST::GS_BYTES : 0)];
    __shared__ uint32_t col_voff[32], col_doff[32];
    __shared__ int refold;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int H = a.H, I = a.I, P = a.S * a.K, nb = I / 32;
    if ((int)blockIdx.y >= tiles[0]) return;
    const i32x4 td = reinterpret_cast<const i32x4 *>(tiles + 4)[blockIdx.y];
    const Tile tl{td.x, td.y, td.z};
    const UnitTable U = unit_table(a.S, a.K, a.E);
    const int32_t *tab = reinterpret_cast<const int32_t *>(a.units);
    const int e = tab[U.uexp + tl.u];
    const uint8_t *blob = e < 0 ? a.shared : a.blobs[e];
    if (!blob) return;  // reported by the gate/up kernel
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED ? 64 : 0);
    const PfCols col = pf_col(tab + U.pairs, tl, n, P, a.K);
    if (threadIdx.x < 32) {
        col_voff[n] = (uint32_t)col.slot * (uint32_t)I;
        col_doff[n] = (uint32_t)col.slot * (uint32_t)nb * 4u;
    }
    if (threadIdx.x == 0) refold = 0;
    const uint32_t slots = (uint32_t)a.S * (uint32_t)(a.K + 1);
    PfSrc<1> src;
    src.rw = make_rsrc(blob, (uint32_t)BL.total);
    src.ra = make_rsrc(a.qh, slots * (uint32_t)I);
    src.rd = make_rsrc(a.dh, slots * (uint32_t)nb * 4u);
    src.mat[0] = (uint32_t)BL.down;
    src.rb = (uint32_t)I * BITS / 8;
    src.row0 = blockIdx.x * PF_ROWS;
    src.n_rows = H;
    src.nb = nb;
    src.smat[0] = (uint32_t)BL.s_down;
    src.srow = (uint32_t)(4 * (I / 64));
    __syncthreads();
    const int r0 = src.row0 + 32 * wave;
    const bool active = r0 < H;
    const bool fold = scales_fold<ST::SHIFT, GROUPED>(a.dh + (size_t)col.slot * nb, nb);
    if constexpr (BITS == 4 || (BITS == 8 && !GROUPED)) {
        if (tl.n <= 16) {
            float an[1][8];
#pragma unroll
            for (int r = 0; r < 8; ++r) an[0][r] = 0.0f;
            pf_dispatch_narrow<BITS, 1, GROUPED>(fold, an, lds, src, col_voff, col_doff, active, &refold);
            const int c = lane & 15, qq = lane >> 4;
            const PfCols cc = pf_col(tab + U.pairs, tl, c, P, a.K);
            if (!active || !cc.live) return;
            const float *sd = reinterpret_cast<const float *>(blob + BL.s_down) + r0;
            float *yrow = a.Y + (size_t)cc.slot * H + r0;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int rr = 16 * g + 4 * qq;
                f32x4 v;
                v.x = GROUPED ? an[0][4 * g + 0] : an[0][4 * g + 0] * sd[rr + 0];
                v.y = GROUPED ? an[0][4 * g + 1] : an[0][4 * g + 1] * sd[rr + 1];
                v.z = GROUPED ? an[0][4 * g + 2] : an[0][4 * g + 2] * sd[rr + 2];
                v.w = GROUPED ? an[0][4 * g + 3] : an[0][4 * g + 3] * sd[rr + 3];
                *reinterpret_cast<f32x4 *>(yrow + rr) = v;
            }
            return;
        }
    }
    float acc[1][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] = 0.0f;
    if constexpr (GROUPED) {
        if (nb % ST::C != 0)
            pf_dispatch_grouped<BITS, 1, true>(fold, acc, lds, src, col_voff, col_doff, active, &refold);
        else
            pf_dispatch_grouped<BITS, 1, false>(fold, acc, lds, src, col_voff, col_doff, active, &refold);
    } else {
        if (nb % ST::C != 0)
            pf_dispatch<BITS, 1, true>(fold, acc, lds, src, col_voff, col_doff, active);
        else
            pf_dispatch<BITS, 1, false>(fold, acc, lds, src, col_voff, col_doff, active);
    }
    if (!active || !col.live) return;
    const float *sd = reinterpret_cast<const float *>(blob + BL.s_down) + r0;
    float *yrow = a.Y + (size_t)col.slot * H + r0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rr = 8 * g + 4 * h;
        f32x4 v;
        v.x = GROUPED ? acc[0][4 * g + 0] : acc[0][4 * g + 0] * sd[rr + 0];
        v.y = GROUPED ? acc[0][4 * g + 1] : acc[0][4 * g + 1] * sd[rr + 1];
        v.z = GROUPED ? acc[0][4 * g + 2] : acc[0][4 * g + 2] * sd[rr + 2];
        v.w = GROUPED ? acc[0][4 * g + 3] : acc[0][4 * g + 3] * sd[rr + 3];
        *reinterpret_cast<f32x4 *>(yrow + rr) = v;
    }
}

// ---- launchers -----------------------------------------------------------
size_t pf_group_smem(int S, int K, int E) { return smem_plan(S, K, E, 0, 0).total; }

hipError_t launch_logits_tiled(const float *x, const float *W, float *logits, uint32_t *status, int S, int H, int E,
                               hipStream_t st) {
    return launch(k_logits_tiled, dim3((E + 31) / 32, (S + LG_TT - 1) / LG_TT), dim3(PF_T), 0, st, x, W, logits,
                  status, S, H, E);
}

hipError_t launch_group(const int32_t *idx, int S, int K, int E, int n_shared, uint8_t *units, int32_t *tiles,
                        uint32_t *status, hipStream_t st) {
    const size_t smem = pf_group_smem(S, K, E);
    const hipError_t e = ensure_dyn_smem(reinterpret_cast<const void *>(k_group), smem);
    if (e != hipSuccess) return e;
    return launch(k_group, dim3(1), dim3(1024), smem, st, idx, S, K, E, n_shared, units, tiles, status);
}

template <int BITS, bool GROUPED = false>
static hipError_t pf_gateup_bits(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const dim3 grid((a.I + PF_ROWS - 1) / PF_ROWS, pf_tile_bound(a.S, a.K, a.E, a.n_shared));
    return launch(k_pf_gateup<BITS, GROUPED>, grid, dim3(PF_T), 0, st, a, tiles);
}

template <int BITS, bool GROUPED = false>
static hipError_t pf_down_bits(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const dim3 grid((a.H + PF_ROWS - 1) / PF_ROWS, pf_tile_bound(a.S, a.K, a.E, a.n_shared));
    return launch(k_pf_down<BITS, GROUPED>, grid, dim3(PF_T), 0, st, a, tiles);
}

// Group-scaled weights: int4 with groups of 64 (the API routes other group
// sizes to the decode kernels); MXFP4 weights: prefill_mx.hip.
hipError_t launch_pf_gateup(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st) {
    if (a.mx) return launch_pf_gateup_mx(a, tiles, st);
    if (a.group) return pf_gateup_bits<4, true>(a, tiles, st);
    if (bits == 8) return pf_gateup_bits<8>(a, tiles, st);
    if (bits == 4) return pf_gateup_bits<4>(a, tiles, st);
    return pf_gateup_bits<2>(a, tiles, st);
}

hipError_t launch_pf_down(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st) {
    if (a.mx) return launch_pf_down_mx(a, tiles, st);
    if (a.group) return pf_down_bits<4, true>(a, tiles, st);
    if (bits == 8) return pf_down_bits<8>(a, tiles, st);
    if (bits == 4) return pf_down_bits<4>(a, tiles, st);
    return pf_down_bits<2>(a, tiles, st);
}

}  // namespace coli
