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
