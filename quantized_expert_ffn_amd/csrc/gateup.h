// Gate/up of one 32-row tile of one unit (colibrì README v1.0, "What's
// implemented": SwiGLU experts over packed per-row-scaled weights with
// integer dots over Q8_0 activations).  Used by the gate/up kernel for every
// unit, and by the router launch of a layer call, whose extra workgroups run
// the shared expert's tiles while the routing is being decided (the shared
// expert's pairs do not depend on it).
#pragma once

#include "device_common.h"
#include "stream.h"

namespace coli {

// Rows i0 .. i0+31 of the gate and up matrices of `blob` for the np pair
// slots slots[0 .. np): waves 0-1 stream 16 gate rows each, waves 2-3 the
// matching up rows.  Vectors go NT at a time: stage(g0, ng) puts the Q8_0
// codes and block scales of slots g0 .. g0+ng-1 into vq (H codes per
// vector) and vd (vd_stride(H / 32) scales per vector) and ends with a
// workgroup barrier; it runs while the first weights are in flight.  Then
// SwiGLU of each row pair and Q8_0(h) of the 32 values (one block), written
// to qh / dh at the slot.  256 threads.  GROUPED: the blob has one scale per
// `group` codes of a row, staged through the groups_lds_bytes(group, 4)
// bytes of LDS at smem + gs_off.
// MX: the blob is MXFP4 (4-bit E2M1 codes, one E8M0 byte per block; group
// is then 32).
template <int BITS, int NT, bool GROUPED, bool MX = false, typename Stage>
__device__ __forceinline__ void gateup_unit(const uint8_t *blob, int H, int I, int group, int i0, const int *slots,
                                            int np, uint8_t *smem, const SmemPlan &L, size_t gs_off,
                                            int8_t *__restrict__ qh, float *__restrict__ dh, Stage stage) {
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * ROWS_PER_WAVE * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED && !MX ? group : 0, MX);
    const size_t row_bytes = (size_t)H * BITS / 8;
    const int half = wave & 1;            // rows 0-15 or 16-31 of the tile
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[ROWS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < ROWS_PER_WAVE; ++j)
        rowoff[j] = (uint32_t)(mat + (size_t)(i0 + 16 * half + j) * row_bytes);
    const size_t ssec = wave < 2 ? BL.s_gate : BL.s_up;
    const float *scale = reinterpret_cast<const float *>(blob + ssec);
    RowGroups G;
    G.lgb = GROUPED ? group_lgb(group) : -1;
    if (GROUPED) {
        G.rsrc = rsrc;
        G.row_stride = MX ? (uint32_t)(H / 32) : (uint32_t)(4 * (H / group));
        G.base = (uint32_t)(ssec + (size_t)(i0 + 16 * half) * G.row_stride);
        G.lds = reinterpret_cast<float *>(smem + gs_off) + wave * ROWS_PER_WAVE * (64 >> G.lgb);
    }
    const int nb = H / 32;
    const int crow = lane & 15, cvec = lane >> 4;
    for (int g0 = 0; g0 < np; g0 += NT) {
        const int ng = min(NT, np - g0);
        BlockBits<BITS> cur[ROWS_PER_WAVE];
        prime_rows<BITS, ROWS_PER_WAVE>(rsrc, rowoff, nb, cur);
        const float acc = stream_rows<BITS, NT, ROWS_PER_WAVE, GROUPED, MX>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, H,
                                                                       [&]() { stage(g0, ng); }, cur, G);
        if (cvec < ng)
            gu[cvec * 64 + wave * ROWS_PER_WAVE + crow] = GROUPED ? acc : acc * scale[i0 + 16 * half + crow];
        __syncthreads();
        // SwiGLU and Q8_0(h): half-wave (tid >> 5) handles one vector's 32 rows.
        const int vv = tid >> 5, i = tid & 31;
        if (vv < ng) {
            const float h = swiglu_f32(gu[vv * 64 + i], gu[vv * 64 + 32 + i]);
            float d;
            const int8_t q = q8_0_lane(h, &d);
            const int slot = slots[g0 + vv];
            qh[(size_t)slot * I + i0 + i] = q;
            if (i == 0) dh[(size_t)slot * (I / 32) + i0 / 32] = d;
        }
        __syncthreads();
    }
}

// Chunk c (blocks 64 c .. 64 c + 63) of this wave's RPW rows: RPW buffer
// loads, issued whatever the lane (a block past the row's end reads the next
// row, or zeros past the blob; its dot is not used), so that the count of
// memory operations in flight is known to the waits.
template <int BITS, int RPW>
__device__ __forceinline__ void issue_chunk(__amdgpu_buffer_rsrc_t rsrc, const uint32_t (&rowoff)[RPW], int c,
                                            BlockBits<BITS> (&X)[RPW]) {
    const int b = c * 64 + (int)(threadIdx.x & 63);
#pragma unroll
    for (int j = 0; j < RPW; ++j) X[j] = load_block<BITS>(rsrc, rowoff[j], b);
}

// Block dots of chunk c (in X) against the np staged vectors, then the
// chain lanes' binary32 chain over the chunk's blocks in ascending order.
// GROUPED: gs is the chain lane's row of scales in LDS (every chunk's: f32
// group scales, one per 1 << lgb blocks, or with MX the row's E8M0 bytes),
// and the chain takes them (no row scale follows).
template <int BITS, int NT, int RPW, bool GROUPED = false, bool MX = false>
__device__ __forceinline__ float reduce_chunk(const BlockBits<BITS> (&X)[RPW], int c, int nb, int np,
                                              const int8_t *vq, const float *vd, int vds, int vlen,
                                              int32_t *isum_wave, float acc, const uint8_t *gs = nullptr,
                                              int lgb = 0) {
    const int lane = threadIdx.x & 63, crow = lane % RPW, cvec = lane / RPW;
    const int b = c * 64 + lane;
    const bool act = b < nb;
#pragma unroll
    for (int it = 0; it < NT; ++it) {
        if (it < np) {
            int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (act) load_act(vq + (size_t)it * vlen, b, av);
            int32_t *dst = isum_wave + it * RPW * ISUM_PITCH + lane;
            if constexpr (MX) {
                // exact block sums in binary32 (see block_dot_mx_f16)
                f16x2 h[16];
                mx_act_f16(av, h);
#pragma unroll
                for (int j = 0; j < RPW; ++j)
                    dst[j * ISUM_PITCH] = act ? __float_as_int(block_dot_mx_f16(X[j].w, h)) : 0;
            } else {
#pragma unroll
                for (int j = 0; j < RPW; ++j) dst[j * ISUM_PITCH] = act ? block_dot(X[j], av) : 0;
            }
        }
    }
    wave_lds_sync();
    if (cvec < np) {
        const int32_t *is = isum_wave + (cvec * RPW + crow) * ISUM_PITCH;
        const float *dv = vd + cvec * vds + c * 64;
        const int nbc = min(64, nb - c * 64);
        if constexpr (MX)
            acc = chain_chunk_mx_bytes(acc, is, dv, gs + 64 * c, nbc);
        else if constexpr (GROUPED)
            acc = chain_chunk_g(acc, is, dv, reinterpret_cast<const float *>(gs) + (c * 64 >> lgb), lgb, nbc);
        else
            acc = chain_chunk(acc, is, dv, nbc);
    }
    wave_lds_sync();
    return acc;
}

// Bytes of scales per row that the primed tile stages whole (every chunk's
// at once): binary32 group scales of a group-scaled row, or the E8M0 bytes
// of an MXFP4 row; 0 for per-row scales.  The tile takes such rows when a
// wave's 16 rows of them fit PRIMED_GW 16-byte words per lane.
constexpr int PRIMED_GW = 6;
__host__ __device__ inline int primed_scale_row_bytes(int H, int group, bool mx) {
    return mx ? H / 32 : (group ? 4 * (H / group) : 0);
}
__host__ __device__ inline bool primed_scales_fit(int H, int group, bool mx) {
    const int rb = primed_scale_row_bytes(H, group, mx);
    return rb > 0 && rb % 16 == 0 && rb <= 4 * PRIMED_GW * 16;
}
// LDS of the staged scales of a workgroup (4 waves x 16 rows).
__host__ __device__ inline size_t primed_scales_lds_bytes(int H, int group, bool mx) {
    return primed_scales_fit(H, group, mx) ? (size_t)64 * primed_scale_row_bytes(H, group, mx) : 0;
}

// gateup_unit for a unit whose pairs fit one pass (np <= NT), with packed
// codes (BITS 4 or 2), per-row scales and rows of NCH = (H / 32 + 63) / 64
// chunks (at least two; H at most 8192).  The order of the memory
// operations is the point: the activations (Q8_0(x) of the vectors' tokens,
// token tok(v) for vector v) are loaded first, into registers, then each
// lane's row scale, then chunks 0 and 1 of the wave's rows; storing the
// activations to LDS then waits for none of the weights, the workgroup
// barrier orders LDS only, and from there on two chunks are in flight
// (chunk c + 2 is issued once chunk c has been reduced).  The chunks are
// unrolled so that the waits the compiler places for each chunk's
// registers leave the next chunk in flight.  Results as gateup_unit.
//
// GROUPED (group-scaled int4, or MXFP4 with MX), when primed_scales_fit():
// the scales of the wave's 16 rows for every chunk (16 x
// primed_scale_row_bytes, contiguous in the blob) are loaded right after
// the activations, into registers, and stored to LDS at gs_off with them;
// the chain then takes them and no row scale follows.
template <int BITS, int NT, int NCH, typename Tok, bool GROUPED = false, bool MX = false>
__device__ __forceinline__ void gateup_unit_primed(const uint8_t *blob, int H, int I, int i0, const int *slots,
                                                   int np, uint8_t *smem, const SmemPlan &L,
                                                   const int8_t *__restrict__ qx, const float *__restrict__ dx, Tok tok,
                                                   int8_t *__restrict__ qh, float *__restrict__ dh, int group = 0,
                                                   size_t gs_off = 0) {
    static_assert(BITS == 4 || BITS == 2, "one buffer load per block");
    static_assert(!MX || (BITS == 4 && GROUPED), "MXFP4 rows are 4-bit codes with a scale per block");
    constexpr int RPW = ROWS_PER_WAVE;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * RPW * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED && !MX ? group : 0, MX);
    const size_t row_bytes = (size_t)H * BITS / 8;
    const int half = wave & 1;
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) rowoff[j] = (uint32_t)(mat + (size_t)(i0 + 16 * half + j) * row_bytes);
    const int nb = H / 32, vds = vd_stride(nb), w16 = H / 16;
    const uint32_t mw = fast_div_magic(w16), mb = fast_div_magic(nb);
    const int crow = lane % RPW, cvec = lane / RPW;
    // 1. activations (np * H / 16 code words, np * H / 32 scales: at most
    //    2 NT and NT per thread for H <= 8192)
    i32x4 xq[2 * NT];
    float xd[NT];
    stage_fetch(xq, 0, np * w16, [&](int i) {
        const int it = fast_div(i, mw);
        return *reinterpret_cast<const i32x4 *>(qx + (size_t)tok(it) * H + 16 * (i - it * w16));
    });
    stage_fetch(xd, 0, np * nb, [&](int i) {
        const int it = fast_div(i, mb);
        return dx[(size_t)tok(it) * nb + (i - it * nb)];
    });
    // 2. the wave's rows' scales: the row scale of this lane's chain row, or
    //    (GROUPED) every scale of the wave's 16 rows, PRIMED_GW words per
    //    lane, all issued (words past the rows read bytes that are not used),
    //    3. chunk 0, and chunk 1 with per-row scales (grouped and MXFP4 rows,
    //    whose block sums take longer, request chunk 1 once chunk 0 is
    //    reduced: fewer loads out at once)
    const size_t ssec = wave < 2 ? BL.s_gate : BL.s_up;
    const int rb = GROUPED ? primed_scale_row_bytes(H, group, MX) : 0;
    __builtin_amdgcn_sched_barrier(0);
    float rs = 1.0f;
    i32x4 gsw[GROUPED ? PRIMED_GW : 1];
    if constexpr (GROUPED) {
        const uint32_t gbase = (uint32_t)(ssec + (size_t)(i0 + 16 * half) * rb);
#pragma unroll
        for (int k = 0; k < PRIMED_GW; ++k)
            gsw[k] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, gbase + 16u * (uint32_t)(lane + 64 * k), 0, 0));
    } else {
        const uint32_t soff = (uint32_t)(ssec + 4 * (size_t)(i0 + 16 * half + crow));
        rs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, soff, 0, 0));
    }
    BlockBits<BITS> A[RPW], B[RPW];
    issue_chunk<BITS, RPW>(rsrc, rowoff, 0, A);
    __builtin_amdgcn_sched_barrier(0);   // chunk 0's loads ahead of chunk 1's
    if constexpr (!GROUPED) issue_chunk<BITS, RPW>(rsrc, rowoff, 1, B);
    __builtin_amdgcn_sched_barrier(0);
    stage_store(xq, 0, np * w16, [&](int i) {
        const int it = fast_div(i, mw);
        return reinterpret_cast<i32x4 *>(vq + (size_t)it * H) + (i - it * w16);
    });
    stage_store(xd, 0, np * nb, [&](int i) {
        const int it = fast_div(i, mb);
        return vd + it * vds + (i - it * nb);
    });
    uint8_t *gsl = smem + gs_off + (size_t)wave * RPW * rb;   // this wave's rows' scales
    if constexpr (GROUPED) {
#pragma unroll
        for (int k = 0; k < PRIMED_GW; ++k) {
            const int w = lane + 64 * k;
            if (w < rb) reinterpret_cast<i32x4 *>(gsl)[w] = gsw[k];   // RPW x rb / 16 = rb words
        }
    }
    lds_barrier();
    const uint8_t *gs = gsl + (size_t)crow * rb;   // the chain lane's row
    const int lgb = GROUPED && !MX ? group_lgb(group) : 0;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
        acc = reduce_chunk<BITS, NT, RPW, GROUPED, MX>(A, c, nb, np, vq, vd, vds, H, isum_wave, acc, gs, lgb);
        __builtin_amdgcn_sched_barrier(0);
        if (GROUPED && c == 0 && NCH > 1) issue_chunk<BITS, RPW>(rsrc, rowoff, 1, B);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < NCH) issue_chunk<BITS, RPW>(rsrc, rowoff, c + 2, A);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < NCH) {
            acc = reduce_chunk<BITS, NT, RPW, GROUPED, MX>(B, c + 1, nb, np, vq, vd, vds, H, isum_wave, acc, gs, lgb);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 3 < NCH) issue_chunk<BITS, RPW>(rsrc, rowoff, c + 3, B);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (cvec < np) gu[cvec * 64 + wave * RPW + crow] = GROUPED ? acc : acc * rs;
    __syncthreads();
    const int vv = tid >> 5, i = tid & 31;
    if (vv < np) {
        const float h = swiglu_f32(gu[vv * 64 + i], gu[vv * 64 + 32 + i]);
        float d;
        const int8_t q = q8_0_lane(h, &d);
        const int slot = slots[vv];
        qh[(size_t)slot * I + i0 + i] = q;
        if (i == 0) dh[(size_t)slot * (I / 32) + i0 / 32] = d;
    }
}

// gateup_half_f32 with packed codes (BITS 4 or 2), per-row scales and rows
// of NCH = (H / 32 + 63) / 64 <= 4 chunks, for np <= NT vectors x[v * H ..]
// (binary32, not yet quantised).  The memory operations go out in this
// order: each thread's 32-value blocks of x (block j = tid + 256 k of the
// np * H / 32, at most NT per thread), the row scale, then the first chunk
// of the wave's 8 rows.  Q8_0 of the blocks (q8_0_words_of, as the
// quantisation of x everywhere else) then waits for x alone and goes to LDS
// behind a barrier that orders LDS only, and the chunks are reduced in
// order, each one's successor requested as soon as it is reduced: one chunk
// in flight per wave keeps these tiles' loads from crowding out the router
// rows that run beside them.  Results as gateup_half_f32.
template <int BITS, int NT, int NCH>
__device__ __forceinline__ void gateup_half_primed(const uint8_t *blob, int H, int I, int i0, int np, uint8_t *smem,
                                                   const SmemPlan &L, const float *__restrict__ x,
                                                   float *__restrict__ hs) {
    static_assert(BITS == 4 || BITS == 2, "one buffer load per block");
    constexpr int RPW = 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * RPW * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const BlobLayout BL = blob_layout(H, I, BITS, 0, false);
    const size_t row_bytes = (size_t)H * BITS / 8;
    const int r0 = i0 + RPW * (wave & 1);
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) rowoff[j] = (uint32_t)(mat + (size_t)(r0 + j) * row_bytes);
    const int nb = H / 32, vds = vd_stride(nb), nblk = np * nb;
    const int crow = lane % RPW, cvec = lane / RPW;
    // 1. x: block tid + 256 k of the np vectors (a clamped index past the
    //    end, so that every thread issues the same loads)
    f32x4 xr[NT][8];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        if (256 * k < nblk) {
            const int j = min(tid + 256 * k, nblk - 1), it = j / nb, b = j - it * nb;
            const f32x4 *src = reinterpret_cast<const f32x4 *>(x + (size_t)it * H + 32 * b);
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[k][i] = src[i];
        }
    }
    // 2. the row scale, 3. the first chunk
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t soff = (uint32_t)((wave < 2 ? BL.s_gate : BL.s_up) + 4 * (size_t)(r0 + crow));
    const float rs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, soff, 0, 0));
    BlockBits<BITS> X[NCH][RPW];
    issue_chunk<BITS, RPW>(rsrc, rowoff, 0, X[0]);
    __builtin_amdgcn_sched_barrier(0);
    // 4. Q8_0(x) into LDS
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int j = tid + 256 * k;
        if (j < nblk) {
            const int it = j / nb, b = j - it * nb;
            uint32_t w[8];
            bool ok;   // a non-finite x is reported by the quantisation of x
            vd[it * vds + b] = q8_0_words_of(xr[k], w, &ok);
            u32x4 *qv = reinterpret_cast<u32x4 *>(vq + (size_t)it * H + 32 * b);
            qv[0] = u32x4{w[0], w[1], w[2], w[3]};
            qv[1] = u32x4{w[4], w[5], w[6], w[7]};
        }
    }
    lds_barrier();
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        acc = reduce_chunk<BITS, NT, RPW>(X[c], c, nb, np, vq, vd, vds, H, isum_wave, acc);
        if (c + 1 < NCH) {
            __builtin_amdgcn_sched_barrier(0);
            issue_chunk<BITS, RPW>(rsrc, rowoff, c + 1, X[c + 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // gu[v * 32 + k]: gate rows (k < 16) then up rows of vector v
    if (cvec < np) gu[cvec * 32 + wave * RPW + crow] = acc * rs;
    __syncthreads();
    if (tid < np * 16) {
        const int v = tid >> 4, i = tid & 15;
        hs[(size_t)v * I + i0 + i] = swiglu_f32(gu[v * 32 + i], gu[v * 32 + 16 + i]);
    }
}

// Gate/up of rows i0 .. i0+15 of one unit for the np <= NT pair slots
// slots[0 .. np), with SwiGLU: h (binary32, not quantised) of slot v's row
// i0 + i goes to hs[v * I + i0 + i].  Waves 0-1 stream 8 gate rows each,
// waves 2-3 the matching up rows; otherwise as gateup_unit (the staging,
// the block chains and the scales are the same).  Half a Q8_0 block of h:
// whoever joins two such halves quantises them.  256 threads.
template <int BITS, int NT, bool GROUPED, bool MX = false, typename Stage>
__device__ __forceinline__ void gateup_half_f32(const uint8_t *blob, int H, int I, int group, int i0,
                                                int np, uint8_t *smem, const SmemPlan &L, size_t gs_off,
                                                float *__restrict__ hs, Stage stage) {
    constexpr int RPW = 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * RPW * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const BlobLayout BL = blob_layout(H, I, BITS, GROUPED && !MX ? group : 0, MX);
    const size_t row_bytes = (size_t)H * BITS / 8;
    const int r0 = i0 + RPW * (wave & 1);   // this wave's first row
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) rowoff[j] = (uint32_t)(mat + (size_t)(r0 + j) * row_bytes);
    const size_t ssec = wave < 2 ? BL.s_gate : BL.s_up;
    const float *scale = reinterpret_cast<const float *>(blob + ssec);
    RowGroups G;
    G.lgb = GROUPED ? group_lgb(group) : -1;
    if (GROUPED) {
        G.rsrc = rsrc;
        G.row_stride = MX ? (uint32_t)(H / 32) : (uint32_t)(4 * (H / group));
        G.base = (uint32_t)(ssec + (size_t)r0 * G.row_stride);
        G.lds = reinterpret_cast<float *>(smem + gs_off) + wave * RPW * (64 >> G.lgb);
    }
    const int nb = H / 32;
    const int crow = lane % RPW, cvec = lane / RPW;
    const int ng = np;
    BlockBits<BITS> cur[RPW];
    prime_rows<BITS, RPW>(rsrc, rowoff, nb, cur);
    const float acc = stream_rows<BITS, NT, RPW, GROUPED, MX>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, H,
                                                         [&]() { stage(0, ng); }, cur, G);
    // gu[v * 32 + k]: gate rows (k < 16) then up rows of vector v
    if (cvec < ng) gu[cvec * 32 + wave * RPW + crow] = GROUPED ? acc : acc * scale[r0 + crow];
    __syncthreads();
    if (tid < ng * 16) {
        const int v = tid >> 4, i = tid & 15;
        hs[(size_t)v * I + i0 + i] = swiglu_f32(gu[v * 32 + i], gu[v * 32 + 16 + i]);
    }
}

}  // namespace coli
