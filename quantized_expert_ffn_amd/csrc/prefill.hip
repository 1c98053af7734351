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
    bool good = true;
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
#pragma unroll
        for (int i = 0; i < LG_TT; ++i)
            good = good && finite_f32(xv[i].x) && finite_f32(xv[i].y) && finite_f32(xv[i].z) && finite_f32(xv[i].w);
#pragma unroll
        for (int i = 0; i < LG_TE; ++i)
            good = good && finite_f32(wv[i].x) && finite_f32(wv[i].y) && finite_f32(wv[i].z) && finite_f32(wv[i].w);
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
    if (!good) raise_status(status, ST_NONFINITE);
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

// ---- weights and activations as matrix-core operands --------------------
// The product of the 16 codes of a lane's weight operand with its 16
// activation codes sums to 2^SHIFT times the true integer sum: int8 codes
// are used as they are, int4 codes as 16 * code (the nibble masked into the
// top of a byte) and int2 codes as 64 * code.
//
// Inside a block the order of the 32 products is free (the sum is exact), so
// lane half h may take any 16 of the block's codes, with its activation codes
// in the same order:
//   int8: codes 16 h .. 16 h + 15 (bytes 16 h .. of the block);
//   int4: the low, then the high nibbles of bytes 8 h .. 8 h + 7, i.e. codes
//         8 h .. 8 h + 7 then 16 + 8 h .. 16 + 8 h + 7, so that a lane reads
//         only its own 8 bytes of the row;
//   int2: fields 2 h and 2 h + 1 of the 8 bytes, codes 16 h .. 16 h + 15.
// Rows and activations are read through buffer resources: the lane's row
// (or vector) offset is its VGPR offset, the block's offset a scalar.
template <int BITS>
struct Operand {
    static constexpr int SHIFT = BITS == 8 ? 0 : (BITS == 4 ? 4 : 6);
    static constexpr int BLOCK = 4 * BITS;  // bytes of a packed 32-code block
    // byte offset of lane half h inside a block of a packed row
    __device__ static int lane_off(int h) { return BITS == 8 ? 16 * h : (BITS == 4 ? 8 * h : 0); }
};

template <int BITS>
__device__ __forceinline__ i32x4 weight_operand(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b, int h);
template <>
__device__ __forceinline__ i32x4 weight_operand<8>(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b, int) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 32 * b, BUF_NT);
    return i32x4{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
}
template <>
__device__ __forceinline__ i32x4 weight_operand<4>(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b, int) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 16 * b, BUF_NT);
    i32x4 o;
    o.x = (int)((w.x << 4) & 0xF0F0F0F0u);
    o.y = (int)((w.y << 4) & 0xF0F0F0F0u);
    o.z = (int)(w.x & 0xF0F0F0F0u);
    o.w = (int)(w.y & 0xF0F0F0F0u);
    return o;
}
template <>
__device__ __forceinline__ i32x4 weight_operand<2>(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b, int h) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 8 * b, BUF_NT);
    const int s0 = 6 - 4 * h, s1 = 4 - 4 * h;  // fields 2 h and 2 h + 1 to bits 6-7
    i32x4 o;
    o.x = (int)((w.x << s0) & 0xC0C0C0C0u);
    o.y = (int)((w.y << s0) & 0xC0C0C0C0u);
    o.z = (int)((w.x << s1) & 0xC0C0C0C0u);
    o.w = (int)((w.y << s1) & 0xC0C0C0C0u);
    return o;
}

// Activation operand of block b; voff = byte offset of the Q8_0 vector.
template <int BITS>
__device__ __forceinline__ i32x4 act_operand(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b, int h) {
    if (BITS == 4) {
        const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 8 * h, 32 * b, 0);
        const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 16 + 8 * h, 32 * b, 0);
        return i32x4{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    }
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * h, 32 * b, 0);
    return i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}

__device__ __forceinline__ float scale_at(__amdgpu_buffer_rsrc_t r, uint32_t voff, int b) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 4 * b, 0));
}

// The tile of workgroup row blockIdx.y: unit, first pair, pairs.
struct Tile {
    int u, p_first, n;
};

// Slot of column n of the tile (-1 past its pairs).
__device__ __forceinline__ int tile_slot(const int32_t *pairs, const Tile &tl, int n) {
    return n < tl.n ? pairs[tl.p_first + n] : -1;
}
__device__ __forceinline__ int slot_token(int slot, int P, int K) { return slot < P ? slot / K : slot - P; }

// Whether d * 2^-SHIFT is exact for the nb block scales d[0 .. nb) of every
// lane of the wave (true unless some scale lies within 2^SHIFT of the
// denormal range).  Then d * 2^-SHIFT times the 2^SHIFT-scaled sum is the
// same product as d times the true sum, and the chain needs no shift.
template <int SHIFT>
__device__ __forceinline__ bool scales_fold(const float *d, int nb) {
    if (SHIFT == 0) return true;
    bool ok = true;
    for (int b = 0; b < nb; ++b) {
        const float v = d[b];
        ok = ok && (v * (1.0f / (float)(1 << SHIFT))) * (float)(1 << SHIFT) == v;
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Chains one 32 x 32 product into the lane's 16 accumulators: with FOLD the
// scale is pre-multiplied by 2^-SHIFT, otherwise the sums are shifted.
template <int SHIFT, bool FOLD>
__device__ __forceinline__ void chain16(float (&acc)[16], const i32x16 &c, float d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(d, (float)(FOLD ? c[r] : c[r] >> SHIFT), acc[r]);
}

template <int SHIFT, bool FOLD>
__device__ __forceinline__ float chain_scale(float d) {
    return FOLD ? d * (1.0f / (float)(1 << SHIFT)) : d;
}

// Accumulators of NM matrices x RT row tiles over nb blocks for the lane's
// column: acc[m][t][r] = chain over b of d_b * isum_b of row
// r0 + 32 t + mfma_c_row(lane, r) of matrix m (wv[m][t] = the row's offset).
template <int BITS, int NM, int RT, bool FOLD>
__device__ __forceinline__ void pf_chains(float (&acc)[NM][RT][16], __amdgpu_buffer_rsrc_t rw,
                                          const uint32_t (&wv)[NM][RT], __amdgpu_buffer_rsrc_t ra, uint32_t av,
                                          __amdgpu_buffer_rsrc_t rd, uint32_t dv, int nb, int h) {
    constexpr int SH = Operand<BITS>::SHIFT;
    i32x4 wa[NM][RT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t) wa[m][t] = weight_operand<BITS>(rw, wv[m][t], 0, h);
    i32x4 xa = act_operand<BITS>(ra, av, 0, h);
    float d = scale_at(rd, dv, 0);
    for (int b = 0; b < nb; ++b) {
        // block b + 1's operands load while block b computes (the last
        // iteration reloads block b, in range)
        const int bn = b + 1 < nb ? b + 1 : b;
        i32x4 wn[NM][RT];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int t = 0; t < RT; ++t) wn[m][t] = weight_operand<BITS>(rw, wv[m][t], bn, h);
        const i32x4 xn = act_operand<BITS>(ra, av, bn, h);
        const float dn = scale_at(rd, dv, bn);
        const float ds = chain_scale<SH, FOLD>(d);
        // all products of the block first, then their chains
        i32x16 c[NM][RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int m = 0; m < NM; ++m) c[m][t] = mfma_i8_32x32x32(wa[m][t], xa);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int m = 0; m < NM; ++m) chain16<SH, FOLD>(acc[m][t], c[m][t], ds);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int t = 0; t < RT; ++t) wa[m][t] = wn[m][t];
        xa = xn;
        d = dn;
    }
}

// ---- gate/up ------------------------------------------------------------
// Grid (ceil(I / (128 RT)), tile bound); wave w takes rows
// 128 RT x + 32 RT w .. + 32 RT - 1 (RT row tiles of 32) for the tile's
// pairs, lane column n = lane % 32, lane half h = lane / 32.  Columns past
// the tile's pairs compute on a copy of its first pair and store nothing.
template <int BITS, int RT>
__global__ __launch_bounds__(PF_T) void k_pf_gateup(const FwdArgs a, const int32_t *__restrict__ tiles) {
    constexpr int SH = Operand<BITS>::SHIFT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I, P = a.S * a.K, nb = H / 32;
    const int i0 = (blockIdx.x * 4 + wave) * 32 * RT;
    if (i0 >= I || (int)blockIdx.y >= tiles[0]) return;
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
    const BlobLayout BL = blob_layout(H, I, BITS);
    const uint32_t rb = (uint32_t)H * BITS / 8;
    const int h = lane >> 5, n = lane & 31;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t wv[2][RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t row = (uint32_t)(i0 + 32 * t + n) * rb + Operand<BITS>::lane_off(h);
        wv[0][t] = (uint32_t)BL.gate + row;
        wv[1][t] = (uint32_t)BL.up + row;
    }
    const int slot = tile_slot(tab + U.pairs, tl, n);
    const bool live = slot >= 0;
    const int tok = slot_token(live ? slot : tab[U.pairs + tl.p_first], P, a.K);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.qx, (uint32_t)a.S * (uint32_t)H);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dx, (uint32_t)a.S * (uint32_t)nb * 4u);
    float acc[2][RT][16];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][t][r] = 0.0f;
    if (scales_fold<SH>(a.dx + (size_t)tok * nb, nb))
        pf_chains<BITS, 2, RT, true>(acc, rw, wv, ra, (uint32_t)tok * H, rd, (uint32_t)tok * nb * 4u, nb, h);
    else
        pf_chains<BITS, 2, RT, false>(acc, rw, wv, ra, (uint32_t)tok * H, rd, (uint32_t)tok * nb * 4u, nb, h);
    if (!live) return;
    // epilogue per row tile: register r of the lane is row 8 (r / 4) + 4 h + r % 4
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r0 = i0 + 32 * t;
        const float *sg = reinterpret_cast<const float *>(blob + BL.s_gate) + r0;
        const float *su = reinterpret_cast<const float *>(blob + BL.s_up) + r0;
        float hv[16], amax = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = mfma_c_row(lane, r);
            hv[r] = swiglu_f32(acc[0][t][r] * sg[row], acc[1][t][r] * su[row]);
            amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[r]));
        }
        // Q8_0 over the 32 rows of the column, held by lanes n and n + 32
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
        const float dq = amax / 127.0f;
        int8_t *qrow = a.qh + (size_t)slot * I + r0;
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
        if (h == 0) a.dh[(size_t)slot * (I / 32) + r0 / 32] = dq;
    }
}

// ---- down ---------------------------------------------------------------
// Grid (ceil(H / (128 RT)), tile bound): Y[slot][row] = s_d[row] * chain over
// the I / 32 blocks of Q8_0(h) of the slot.
template <int BITS, int RT>
__global__ __launch_bounds__(PF_T) void k_pf_down(const FwdArgs a, const int32_t *__restrict__ tiles) {
    constexpr int SH = Operand<BITS>::SHIFT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I, nb = I / 32;
    const int r0 = (blockIdx.x * 4 + wave) * 32 * RT;
    if (r0 >= H || (int)blockIdx.y >= tiles[0]) return;
    const i32x4 td = reinterpret_cast<const i32x4 *>(tiles + 4)[blockIdx.y];
    const Tile tl{td.x, td.y, td.z};
    const UnitTable U = unit_table(a.S, a.K, a.E);
    const int32_t *tab = reinterpret_cast<const int32_t *>(a.units);
    const int e = tab[U.uexp + tl.u];
    const uint8_t *blob = e < 0 ? a.shared : a.blobs[e];
    if (!blob) return;  // reported by the gate/up kernel
    const BlobLayout BL = blob_layout(H, I, BITS);
    const uint32_t rb = (uint32_t)I * BITS / 8;
    const int h = lane >> 5, n = lane & 31;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t wv[1][RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        wv[0][t] = (uint32_t)BL.down + (uint32_t)(r0 + 32 * t + n) * rb + Operand<BITS>::lane_off(h);
    const int slot = tile_slot(tab + U.pairs, tl, n);
    const bool live = slot >= 0;
    const int src = live ? slot : tab[U.pairs + tl.p_first];
    const uint32_t slots = (uint32_t)a.S * (uint32_t)(a.K + 1);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.qh, slots * (uint32_t)I);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dh, slots * (uint32_t)nb * 4u);
    float acc[1][RT][16];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][t][r] = 0.0f;
    if (scales_fold<SH>(a.dh + (size_t)src * nb, nb))
        pf_chains<BITS, 1, RT, true>(acc, rw, wv, ra, (uint32_t)src * I, rd, (uint32_t)src * nb * 4u, nb, h);
    else
        pf_chains<BITS, 1, RT, false>(acc, rw, wv, ra, (uint32_t)src * I, rd, (uint32_t)src * nb * 4u, nb, h);
    if (!live) return;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int rt0 = r0 + 32 * t;
        const float *sd = reinterpret_cast<const float *>(blob + BL.s_down) + rt0;
        float *yrow = a.Y + (size_t)slot * H + rt0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int rr = 8 * g + 4 * h;
            f32x4 v;
            v.x = acc[0][t][4 * g + 0] * sd[rr + 0];
            v.y = acc[0][t][4 * g + 1] * sd[rr + 1];
            v.z = acc[0][t][4 * g + 2] * sd[rr + 2];
            v.w = acc[0][t][4 * g + 3] * sd[rr + 3];
            *reinterpret_cast<f32x4 *>(yrow + rr) = v;
        }
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

template <int BITS>
static hipError_t pf_gateup_bits(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const int ty = pf_tile_bound(a.S, a.K, a.E, a.n_shared);
    if (a.I % 64 == 0)
        return launch(k_pf_gateup<BITS, 2>, dim3((a.I + 255) / 256, ty), dim3(PF_T), 0, st, a, tiles);
    return launch(k_pf_gateup<BITS, 1>, dim3((a.I + 127) / 128, ty), dim3(PF_T), 0, st, a, tiles);
}

template <int BITS>
static hipError_t pf_down_bits(const FwdArgs &a, const int32_t *tiles, hipStream_t st) {
    const int ty = pf_tile_bound(a.S, a.K, a.E, a.n_shared);
    if (a.H % 64 == 0)
        return launch(k_pf_down<BITS, 2>, dim3((a.H + 255) / 256, ty), dim3(PF_T), 0, st, a, tiles);
    return launch(k_pf_down<BITS, 1>, dim3((a.H + 127) / 128, ty), dim3(PF_T), 0, st, a, tiles);
}

hipError_t launch_pf_gateup(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st) {
    if (bits == 8) return pf_gateup_bits<8>(a, tiles, st);
    if (bits == 4) return pf_gateup_bits<4>(a, tiles, st);
    return pf_gateup_bits<2>(a, tiles, st);
}

hipError_t launch_pf_down(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st) {
    if (bits == 8) return pf_down_bits<8>(a, tiles, st);
    if (bits == 4) return pf_down_bits<4>(a, tiles, st);
    return pf_down_bits<2>(a, tiles, st);
}

}  // namespace coli
