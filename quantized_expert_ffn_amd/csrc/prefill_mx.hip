// Batch-union kernels for MXFP4 experts on the FP4 matrix cores of gfx950
// (JustVugg/colibri README v1.12, "Other supported models": routed experts
// kept in their native FP4 format; colibrì README v1.0, "What's
// implemented": batch-union MoE, each unique expert read once and applied
// to every token routed to it).
//
// The work split is the int kernels' (prefill.hip): a workgroup takes 128
// rows (32 per wave) of one unit's matrices and one tile of up to 32 of its
// pairs, K in stages of 8 blocks.  Per 32-code block of a row, one
// v_mfma_scale_f32_32x32x64_f8f6f4 takes the row's E2M1 codes straight from
// the blob (FP4 A, the same 16 bytes in both 32-deep scale blocks, scaled by
// the row's E8M0 byte x) and the column's Q8_0 codes split as
// q = 16 hi + lo (FP8 B, split_e4m3: hi in the first scale block, scaled by
// 2^4, lo in the second), so its binary32 result is
// S_b = 2^(x - 128) * sum_j t_j q_j exactly, t_j twice the E2M1 value (the
// test of the debug hook coli_moe_debug_mfma_f8f6f4 pins this).  The chain
// then costs one fmaf per element and block: acc = fmaf(d_b, S_b, acc),
// which rounds exactly as the layer's acc = fmaf(d_b * 2^(x - 128), isum_b,
// acc) whenever the multiplier d_b * 2^(x - 128) is a normal binary32
// number and S_b is exact.  The kernels check this for every scale a tile
// uses (x in 64 .. 192, d_b zero or in 2^-62 .. 2^47, which keeps both in
// range); a tile with any other scale is recomputed with unscaled products
// (sum_j v_j q_j, exact) and the multiplier d_b * 2^(x - 128) formed per
// element, exact for every input including the E8M0 NaN.
#include "device_common.h"
#include "kernels.h"
#include "mfma.h"
#include "stream.h"

namespace coli {

constexpr int MX_T = 256;      // threads per workgroup (4 waves)
constexpr int MX_ROWS = 128;   // rows per workgroup (32 per wave)
constexpr int MX_C = 8;        // blocks per stage
// stages of loads in flight (two measured no faster than one: the kernels
// are bound by LDS reads, not by the loads)
template <int NM>
constexpr int MX_DEPTH = 1;

// Fast-path scale bounds (see above): x_lo <= x <= x_hi and d = 0 or
// d_lo <= d <= d_hi give 2^-126 <= d * 2^(x - 128) and
// d * 2^(x - 128) * 2^16 < 2^127 for every pair, and S_b normal.
constexpr uint32_t MX_X_LO = 64, MX_X_HI = 192;
constexpr float MX_D_LO = 0x1p-62f, MX_D_HI = 0x1p47f;

// LDS of one stage: the rows' codes (8 blocks of 16 bytes, padded), the
// rows' E8M0 bytes (8), the columns' split codes (8 blocks of 64 bytes,
// padded) and block scales (block-major, one word per column).
template <int NM>
struct MxStage {
    static constexpr int WS = 16 * MX_C + 16;
    static constexpr int AS = 64 * MX_C + 16;
    static constexpr int W_CHUNKS = NM * MX_ROWS * MX_C / MX_T;    // 16-byte code pieces per thread
    static constexpr int X_WORDS = NM * MX_ROWS * 2 / MX_T;        // scale words per thread
    static constexpr int A_CHUNKS = 32 * 4 * MX_C / MX_T;          // 16-byte split pieces per thread
    static constexpr int D_WORDS = 32 * MX_C / MX_T;               // block scales per thread
    static constexpr int W_BYTES = NM * MX_ROWS * WS;
    static constexpr int X_BYTES = NM * MX_ROWS * 8;
    static constexpr int A_BYTES = 32 * AS;
    static constexpr int D_BYTES = 32 * MX_C * 4;
    static constexpr int LDS = W_BYTES + X_BYTES + A_BYTES + D_BYTES;
    static_assert(W_CHUNKS * MX_T == NM * MX_ROWS * MX_C && X_WORDS * MX_T == NM * MX_ROWS * 2, "whole pieces");
    static_assert(A_CHUNKS * MX_T == 32 * 4 * MX_C && D_WORDS * MX_T == 32 * MX_C, "whole pieces");
};

// Operands of a tile: NM matrices (codes at byte offset mat[m], E8M0 bytes
// at smat[m], rb / sb bytes of each per row) of the blob, the columns'
// split codes (ra, col_aoff) and block scales (rd, col_doff).
template <int NM>
struct MxSrc {
    __amdgpu_buffer_rsrc_t rw, ra, rd;
    uint32_t mat[NM], smat[NM];
    uint32_t rb, sb;
    int row0, n_rows, nb;
};

template <int NM>
struct MxRegs {
    u32x4 w[MxStage<NM>::W_CHUNKS];
    uint32_t x[MxStage<NM>::X_WORDS];
    u32x4 a[MxStage<NM>::A_CHUNKS];
    uint32_t d[MxStage<NM>::D_WORDS];
};

// Loads of stage s.  Past a row's (or column's) last block the pieces read
// the next row's bytes, or zeros past the buffer; they are never used.
template <int NM>
__device__ __forceinline__ void mx_load(MxRegs<NM> &R, const MxSrc<NM> &src, const uint32_t *col_aoff,
                                        const uint32_t *col_doff, int s) {
    using ST = MxStage<NM>;
    const int tid = threadIdx.x;
    // chunk i of the codes belongs to matrix i / (W_CHUNKS / NM), word i of
    // the scales to matrix i (compile-time indices into src)
#pragma unroll
    for (int i = 0; i < ST::W_CHUNKS; ++i) {
        constexpr int PER = ST::W_CHUNKS / NM;
        const int m = i / PER, g = (i % PER) * MX_T + tid, row = g / MX_C, piece = g % MX_C;
        const int r = min(src.row0 + row, src.n_rows - 1);
        R.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               src.rw, src.mat[m] + (uint32_t)r * src.rb + 16u * (MX_C * s + piece), 0, 0));
    }
    static_assert(ST::X_WORDS == NM, "one scale word per thread and matrix");
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int row = tid / 2, k = tid % 2;
        const int r = min(src.row0 + row, src.n_rows - 1);
        R.x[m] = __builtin_amdgcn_raw_buffer_load_b32(src.rw, src.smat[m] + (uint32_t)r * src.sb + MX_C * s + 4u * k,
                                                      0, 0);
    }
#pragma unroll
    for (int i = 0; i < ST::A_CHUNKS; ++i) {
        const int g = i * MX_T + tid, col = g / (4 * MX_C), piece = g % (4 * MX_C);
        R.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               src.ra, col_aoff[col] + 64u * MX_C * s + 16u * piece, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < ST::D_WORDS; ++i) {
        const int g = i * MX_T + tid, col = g / MX_C, c = g % MX_C;
        R.d[i] = __builtin_amdgcn_raw_buffer_load_b32(src.rd, col_doff[col] + 4u * (MX_C * s + c), 0, 0);
    }
}

// Stores of a stage of nblk blocks; scales of those blocks outside the fast
// bounds set *bad.
template <int NM>
__device__ __forceinline__ void mx_store(const MxRegs<NM> &R, uint8_t *lds, int nblk, int *bad) {
    using ST = MxStage<NM>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < ST::W_CHUNKS; ++i) {
        // chunk i is piece g % MX_C of row m * MX_ROWS + g / MX_C, as loaded
        const int g = i * MX_T + tid;
        *reinterpret_cast<u32x4 *>(lds + ST::WS * (g / MX_C) + 16 * (g % MX_C)) = R.w[i];
    }
    uint32_t *lx = reinterpret_cast<uint32_t *>(lds + ST::W_BYTES);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int g = m * MX_T + tid;   // word tid % 2 of row m * MX_ROWS + tid / 2
        lx[g] = R.x[m];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t xb = (R.x[m] >> (8 * k)) & 0xFFu;
            if (4 * (g % 2) + k < nblk && (xb < MX_X_LO || xb > MX_X_HI)) *bad = 1;
        }
    }
    uint8_t *la = lds + ST::W_BYTES + ST::X_BYTES;
#pragma unroll
    for (int i = 0; i < ST::A_CHUNKS; ++i) {
        const int g = i * MX_T + tid;
        *reinterpret_cast<u32x4 *>(la + ST::AS * (g / (4 * MX_C)) + 16 * (g % (4 * MX_C))) = R.a[i];
    }
    float *ld = reinterpret_cast<float *>(lds + ST::W_BYTES + ST::X_BYTES + ST::A_BYTES);
#pragma unroll
    for (int i = 0; i < ST::D_WORDS; ++i) {
        const int g = i * MX_T + tid, col = g / MX_C, c = g % MX_C;
        const float d = __uint_as_float(R.d[i]);
        ld[32 * c + col] = d;
        if (c < nblk && !(d == 0.0f || (d >= MX_D_LO && d <= MX_D_HI))) *bad = 1;
    }
}

// The products and chains of the nblk blocks of a stage in LDS.  FAST: each
// product is scaled by the row's E8M0 byte and the chain is
// fmaf(d_b, S_b, acc); otherwise the product is unscaled (half the block
// sum) and the multiplier d_b * 2^(x - 128) is formed per element.
template <int NM, bool FAST>
__device__ __forceinline__ void mx_blocks(float (&acc)[NM][16], const uint8_t *lds, int nblk) {
    using ST = MxStage<NM>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int row = 32 * wave + n;   // the lane's A row within the workgroup
    const uint8_t *lw = lds + ST::WS * row;
    const uint32_t *lx = reinterpret_cast<const uint32_t *>(lds + ST::W_BYTES);
    const uint8_t *lxb = lds + ST::W_BYTES;
    const uint8_t *la = lds + ST::W_BYTES + ST::X_BYTES + ST::AS * n + 32 * h;
    const float *ld = reinterpret_cast<const float *>(lds + ST::W_BYTES + ST::X_BYTES + ST::A_BYTES) + n;
    const int sb = h ? 127 : 131;   // lo unscaled, hi times 2^4
    uint32_t xw[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        xw[m][0] = lx[2 * (m * MX_ROWS + row)];
        xw[m][1] = lx[2 * (m * MX_ROWS + row) + 1];
    }
#pragma unroll
    for (int j = 0; j < MX_C; ++j) {
        if (j >= nblk) continue;   // (no break: the loop stays unrolled, its register indices constant)
        const u32x4 b0 = *reinterpret_cast<const u32x4 *>(la + 64 * j);
        const u32x4 b1 = *reinterpret_cast<const u32x4 *>(la + 64 * j + 16);
        const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const float d = ld[32 * j];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const u32x4 a4 = *reinterpret_cast<const u32x4 *>(lw + m * MX_ROWS * ST::WS + 16 * j);
            const i32x8 av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
            if constexpr (FAST) {
                const int sa = (int)((xw[m][j >> 2] >> (8 * (j & 3))) & 0xFFu);
                const f32x16 c = mfma_scale_f8f6f4<4, 0>(av, bv, sa, sb);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][r] = __builtin_fmaf(d, c[r], acc[m][r]);
            } else {
                const f32x16 c = mfma_scale_f8f6f4<4, 0>(av, bv, 127, sb);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 32 * wave + mfma_c_row(lane, r);
                    const uint32_t x = lxb[8 * (m * MX_ROWS + rr) + j];
                    acc[m][r] = __builtin_fmaf(d * e8m0_half(x), c[r] + c[r], acc[m][r]);
                }
            }
        }
    }
}

// A full stage on the fast path, in the order that keeps the matrix core
// and the vector ALU busy together: the products of unit u = (block j,
// matrix m) go to buffer u % 2, and unit u's product is issued before unit
// u - 1's chain step reads its buffer.
template <int NM>
__device__ __forceinline__ void mx_blocks_full(float (&acc)[NM][16], const uint8_t *lds) {
    using ST = MxStage<NM>;
    constexpr int U = MX_C * NM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int row = 32 * wave + n;
    const uint8_t *lw = lds + ST::WS * row;
    const uint32_t *lx = reinterpret_cast<const uint32_t *>(lds + ST::W_BYTES);
    const uint8_t *la = lds + ST::W_BYTES + ST::X_BYTES + ST::AS * n + 32 * h;
    const float *ld = reinterpret_cast<const float *>(lds + ST::W_BYTES + ST::X_BYTES + ST::A_BYTES) + n;
    const int sb = h ? 127 : 131;
    uint32_t xw[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        xw[m][0] = lx[2 * (m * MX_ROWS + row)];
        xw[m][1] = lx[2 * (m * MX_ROWS + row) + 1];
    }
    f32x16 P[2];
    i32x8 bv;
#pragma unroll
    for (int u = 0; u <= U; ++u) {
        if (u < U) {
            const int j = u / NM, m = u % NM;
            if (m == 0) {
                const u32x4 b0 = *reinterpret_cast<const u32x4 *>(la + 64 * j);
                const u32x4 b1 = *reinterpret_cast<const u32x4 *>(la + 64 * j + 16);
                bv = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            }
            const u32x4 a4 = *reinterpret_cast<const u32x4 *>(lw + m * MX_ROWS * ST::WS + 16 * j);
            const i32x8 av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
            const int sa = (int)((xw[m][j >> 2] >> (8 * (j & 3))) & 0xFFu);
            P[u & 1] = mfma_scale_f8f6f4<4, 0>(av, bv, sa, sb);
        }
        if (u > 0) {
            const int v = u - 1, j = v / NM, m = v % NM;
            const float d = ld[32 * j];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][r] = __builtin_fmaf(d, P[v & 1][r], acc[m][r]);
        }
    }
}

// Every stage of the tile.  All waves load, store and meet at the barriers;
// `active` waves compute.  The loads run DEPTH stages ahead, rotating over
// DEPTH register sets (the barriers order LDS only, so every set stays in
// flight across them).
template <int NM, bool FAST, int DEPTH>
__device__ __forceinline__ void mx_run(float (&acc)[NM][16], uint8_t *lds, const MxSrc<NM> &src,
                                       const uint32_t *col_aoff, const uint32_t *col_doff, bool active, int *bad) {
    const int n_stages = (src.nb + MX_C - 1) / MX_C;
    MxRegs<NM> R[DEPTH];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
        if (k < n_stages) mx_load<NM>(R[k], src, col_aoff, col_doff, k);
    for (int s0 = 0; s0 < n_stages; s0 += DEPTH) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            const int s = s0 + k;
            if (s < n_stages) {
                const int nblk = min(MX_C, src.nb - MX_C * s);
                if (s > 0) lds_barrier();   // every wave is done with the previous stage
                mx_store<NM>(R[k], lds, nblk, bad);
                lds_barrier();
                if (s + DEPTH < n_stages) mx_load<NM>(R[k], src, col_aoff, col_doff, s + DEPTH);
                if (active) {
                    if (FAST && nblk == MX_C)
                        mx_blocks_full<NM>(acc, lds);
                    else
                        mx_blocks<NM, FAST>(acc, lds, nblk);
                }
            }
        }
    }
}

// The fast chain, or (when a scale of the tile is outside its bounds) the
// general one.
template <int NM>
__device__ __forceinline__ void mx_tile(float (&acc)[NM][16], uint8_t *lds, const MxSrc<NM> &src,
                                        const uint32_t *col_aoff, const uint32_t *col_doff, bool active) {
    int bad = 0;
    mx_run<NM, true, MX_DEPTH<NM>>(acc, lds, src, col_aoff, col_doff, active, &bad);
    if (!__syncthreads_or(bad)) return;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
    mx_run<NM, false, MX_DEPTH<NM>>(acc, lds, src, col_aoff, col_doff, active, &bad);
}

struct MxTile {
    int u, p_first, n;
};

// ---- gate/up ------------------------------------------------------------
// Grid (ceil(I / 128), tile bound).  Epilogue: SwiGLU and Q8_0 over each
// wave's 32 rows (one block of h) for every live column, written as codes
// (qh, dh) and split (qhs) for the down kernel.
__global__ __launch_bounds__(MX_T) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_gateup_mx(
    const FwdArgs a, const int32_t *__restrict__ tiles) {
    using ST = MxStage<2>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[ST::LDS];
    __shared__ uint32_t col_aoff[32], col_doff[32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int H = a.H, I = a.I, P = a.S * a.K, nb = H / 32;
    if ((int)blockIdx.y >= tiles[0]) return;
    const i32x4 td = reinterpret_cast<const i32x4 *>(tiles + 4)[blockIdx.y];
    const MxTile tl{td.x, td.y, td.z};
    const UnitTable U = unit_table(a.S, a.K, a.E);
    const int32_t *tab = reinterpret_cast<const int32_t *>(a.units);
    const int e = tab[U.uexp + tl.u];
    const uint8_t *blob = e < 0 ? a.shared : a.blobs[e];
    if (!blob) {
        if (threadIdx.x == 0 && blockIdx.x == 0) raise_status(a.status, ST_NOTRESIDENT);
        return;
    }
    const BlobLayout BL = blob_layout(H, I, 4, 0, true);
    const bool live = n < tl.n;
    const int slot = tab[U.pairs + tl.p_first + (live ? n : 0)];
    const int tok = slot < P ? slot / a.K : slot - P;
    if (threadIdx.x < 32) {
        col_aoff[n] = (uint32_t)tok * (uint32_t)nb * 64u;
        col_doff[n] = (uint32_t)tok * (uint32_t)nb * 4u;
    }
    MxSrc<2> src;
    src.rw = make_rsrc(blob, (uint32_t)BL.total);
    src.ra = make_rsrc(a.qxs, (uint32_t)a.S * (uint32_t)nb * 64u);
    src.rd = make_rsrc(a.dx, (uint32_t)a.S * (uint32_t)nb * 4u);
    src.mat[0] = (uint32_t)BL.gate;
    src.mat[1] = (uint32_t)BL.up;
    src.smat[0] = (uint32_t)BL.s_gate;
    src.smat[1] = (uint32_t)BL.s_up;
    src.rb = (uint32_t)H / 2;
    src.sb = (uint32_t)nb;
    src.row0 = blockIdx.x * MX_ROWS;
    src.n_rows = I;
    src.nb = nb;
    __syncthreads();
    const int i0 = src.row0 + 32 * wave;
    const bool active = i0 < I;
    float acc[2][16];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
    mx_tile<2>(acc, lds, src, col_aoff, col_doff, active);
    if (!active || !live) return;
    float hv[16], amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        hv[r] = swiglu_f32(acc[0][r], acc[1][r]);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[r]));
    }
    // Q8_0 over the 32 rows of the column, held by lanes n and n + 32
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
    const float dq = amax / 127.0f;
    int8_t *qrow = a.qh + (size_t)slot * I + i0;
    uint8_t *srow = a.qhs + ((size_t)slot * (I / 32) + i0 / 32) * 64;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t word = 0, hw = 0, lw = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float c = 0.0f;
            if (dq != 0.0f) {
                c = __builtin_roundf(hv[4 * g + q] / dq);
                c = __builtin_fminf(__builtin_fmaxf(c, -127.0f), 127.0f);
            }
            const int qi = (int)c;
            word |= (uint32_t)(uint8_t)(int8_t)qi << (8 * q);
            hw |= e4m3_small(qi >> 4) << (8 * q);
            lw |= e4m3_small(qi & 15) << (8 * q);
        }
        // rows 8 g + 4 h .. + 3 of the block: codes, then their split bytes
        // (rows 0-15: hi at bytes 0-15, lo at 16-31; rows 16-31: hi at 32-47,
        // lo at 48-63)
        const int rho = 8 * g + 4 * h;
        *reinterpret_cast<uint32_t *>(qrow + rho) = word;
        const int off = rho < 16 ? rho : 32 + (rho - 16);
        *reinterpret_cast<uint32_t *>(srow + off) = hw;
        *reinterpret_cast<uint32_t *>(srow + off + 16) = lw;
    }
    if (h == 0) a.dh[(size_t)slot * (I / 32) + i0 / 32] = dq;
}

// ---- down ---------------------------------------------------------------
// Grid (ceil(H / 128), tile bound): Y[slot][row] = chain over the I / 32
// blocks of Q8_0(h) of the slot (no row scale: the E8M0 bytes are in the
// chain).
__global__ __launch_bounds__(MX_T) __attribute__((amdgpu_waves_per_eu(3))) void k_pf_down_mx(
    const FwdArgs a, const int32_t *__restrict__ tiles) {
    using ST = MxStage<1>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[ST::LDS];
    __shared__ uint32_t col_aoff[32], col_doff[32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
    const int H = a.H, I = a.I, nb = I / 32;
    if ((int)blockIdx.y >= tiles[0]) return;
    const i32x4 td = reinterpret_cast<const i32x4 *>(tiles + 4)[blockIdx.y];
    const MxTile tl{td.x, td.y, td.z};
    const UnitTable U = unit_table(a.S, a.K, a.E);
    const int32_t *tab = reinterpret_cast<const int32_t *>(a.units);
    const int e = tab[U.uexp + tl.u];
    const uint8_t *blob = e < 0 ? a.shared : a.blobs[e];
    if (!blob) return;  // reported by the gate/up kernel
    const BlobLayout BL = blob_layout(H, I, 4, 0, true);
    const bool live = n < tl.n;
    const int slot = tab[U.pairs + tl.p_first + (live ? n : 0)];
    if (threadIdx.x < 32) {
        col_aoff[n] = (uint32_t)slot * (uint32_t)nb * 64u;
        col_doff[n] = (uint32_t)slot * (uint32_t)nb * 4u;
    }
    const uint32_t slots = (uint32_t)a.S * (uint32_t)(a.K + 1);
    MxSrc<1> src;
    src.rw = make_rsrc(blob, (uint32_t)BL.total);
    src.ra = make_rsrc(a.qhs, slots * (uint32_t)nb * 64u);
    src.rd = make_rsrc(a.dh, slots * (uint32_t)nb * 4u);
    src.mat[0] = (uint32_t)BL.down;
    src.smat[0] = (uint32_t)BL.s_down;
    src.rb = (uint32_t)I / 2;
    src.sb = (uint32_t)nb;
    src.row0 = blockIdx.x * MX_ROWS;
    src.n_rows = H;
    src.nb = nb;
    __syncthreads();
    const int r0 = src.row0 + 32 * wave;
    const bool active = r0 < H;
    float acc[1][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] = 0.0f;
    mx_tile<1>(acc, lds, src, col_aoff, col_doff, active);
    if (!active || !live) return;
    float *yrow = a.Y + (size_t)slot * H + r0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rr = 8 * g + 4 * h;
        *reinterpret_cast<f32x4 *>(yrow + rr) =
            f32x4{acc[0][4 * g + 0], acc[0][4 * g + 1], acc[0][4 * g + 2], acc[0][4 * g + 3]};
    }
}

hipError_t launch_pf_gateup_mx(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const dim3 grid((a.I + MX_ROWS - 1) / MX_ROWS, pf_tile_bound(a.S, a.K, a.E, a.n_shared));
    return launch(k_pf_gateup_mx, grid, dim3(MX_T), 0, st, a, tiles);
}

hipError_t launch_pf_down_mx(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const dim3 grid((a.H + MX_ROWS - 1) / MX_ROWS, pf_tile_bound(a.S, a.K, a.E, a.n_shared));
    return launch(k_pf_down_mx, grid, dim3(MX_T), 0, st, a, tiles);
}

}  // namespace coli
