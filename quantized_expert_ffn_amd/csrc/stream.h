// Streaming machinery shared by the decode kernels: the unit table of a
// batch-union call, and a wave's pass over 16 packed weight rows that yields
// the binary32 block chain fmaf(d_b, isum_b, acc) per (row, vector).
#pragma once

#include "device_common.h"

namespace coli {

constexpr int ROWS_PER_WAVE = 16;
constexpr int ISUM_PITCH = 68;  // padded row of block dots: 16-byte aligned, few bank conflicts

struct SmemPlan {
    size_t cnt, ustart, fill, uexp, uoff, pairs, misc, vq, vd, isum, gu, total;
};

__host__ __device__ inline size_t a16(size_t v) { return (v + 15) & ~(size_t)15; }

// Values read from LDS that are the same in every lane: moving them to a
// scalar register lets the compiler address weights with scalar bases.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// A load through the scalar cache of a value that no wave writes during the
// launch (an earlier launch wrote it): the address must be the same in
// every lane.  Scalar loads count on their own counter, so waiting for one
// does not wait for the vector loads issued before it.
template <typename T>
__device__ __forceinline__ T ld_scalar(const void *p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) T *>(reinterpret_cast<uintptr_t>(p));
}

// Per-vector stride of the staged block scales (a multiple of 4 so every
// chunk of 64 scales starts 16-byte aligned).
__host__ __device__ inline int vd_stride(int nb) { return (nb + 3) & ~3; }

__host__ __device__ inline SmemPlan smem_plan(int S, int K, int E, int NT, int vlen) {
    SmemPlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    p.cnt = 0;
    p.ustart = a16(p.cnt + 4 * (size_t)E);
    p.fill = a16(p.ustart + 4 * (size_t)E);
    p.uexp = a16(p.fill + 4 * (size_t)E);
    p.uoff = a16(p.uexp + 4 * (size_t)umax);
    p.pairs = a16(p.uoff + 4 * (size_t)(umax + 1));
    p.misc = a16(p.pairs + 4 * (size_t)(P + S));
    p.vq = a16(p.misc + 16);
    p.vd = a16(p.vq + (size_t)NT * vlen);
    p.isum = a16(p.vd + 4 * (size_t)NT * vd_stride(vlen / 32));
    p.gu = a16(p.isum + 4 * (size_t)NT * 64 * ISUM_PITCH);
    p.total = a16(p.gu + 4 * (size_t)NT * 64);
    return p;
}

// Builds the unit table in LDS.  Pair p = t*K + k is routed pair (t, k); the
// shared expert's entry for token t is P + t.  Units: experts present in
// topk_idx in ascending id, then the shared expert.  The order of pairs
// inside a unit does not affect any value (every pair has its own output
// slot and its own chain).  With `validate`, out-of-range and repeated
// indices are flagged in the status word.  A thread takes whole tokens and
// loads their indices BU_KC at a time, all in flight together (one memory
// round trip per group, not one per pair), before counting and checking
// them in registers.
constexpr int BU_KC = 8;
__device__ inline void build_units(const int32_t *__restrict__ idx, int S, int K, int E, int n_shared,
                            uint8_t *smem, const SmemPlan &L, uint32_t *status, bool validate) {
    int *cnt = reinterpret_cast<int *>(smem + L.cnt);
    int *ustart = reinterpret_cast<int *>(smem + L.ustart);
    int *fill = reinterpret_cast<int *>(smem + L.fill);
    int *uexp = reinterpret_cast<int *>(smem + L.uexp);
    int *uoff = reinterpret_cast<int *>(smem + L.uoff);
    int *pairs = reinterpret_cast<int *>(smem + L.pairs);
    int *misc = reinterpret_cast<int *>(smem + L.misc);
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int P = S * K;
    for (int e = tid; e < E; e += nthr) {
        cnt[e] = 0;
        fill[e] = 0;
    }
    __syncthreads();
    // indices k0 .. k0 + BU_KC - 1 of token t (-1 past K)
    auto load_group = [&](int t, int k0, int (&v)[BU_KC]) {
#pragma unroll
        for (int j = 0; j < BU_KC; ++j) v[j] = k0 + j < K ? idx[(size_t)t * K + k0 + j] : -1;
    };
    for (int t = tid; t < S; t += nthr) {
        for (int k0 = 0; k0 < K; k0 += BU_KC) {
            int v[BU_KC];
            load_group(t, k0, v);
            bool bad = false;
#pragma unroll
            for (int j = 0; j < BU_KC; ++j) {
                if (k0 + j >= K) break;
                const int e = v[j];
                if (e >= 0 && e < E)
                    atomicAdd(&cnt[e], 1);
                else
                    bad = true;
                if (validate) {
#pragma unroll
                    for (int i = 0; i < j; ++i) bad |= v[i] == e;   // a repeat within the group
                }
            }
            if (validate) {
                // a repeat of an earlier group of the token (top-k above BU_KC)
                for (int q0 = 0; q0 < k0; q0 += BU_KC) {
                    int u[BU_KC];
                    load_group(t, q0, u);
#pragma unroll
                    for (int j = 0; j < BU_KC; ++j)
#pragma unroll
                        for (int i = 0; i < BU_KC; ++i) bad |= k0 + j < K && u[i] == v[j];
                }
                if (bad) raise_status(status, ST_BADINDEX);
            }
        }
    }
    __syncthreads();
    if (tid < 64) {
        const int per = (E + 63) / 64;
        const int e0 = tid * per;
        int sp = 0, su = 0;
        for (int i = 0; i < per; ++i) {
            const int e = e0 + i;
            if (e < E) {
                sp += cnt[e];
                su += cnt[e] > 0 ? 1 : 0;
            }
        }
        int ip = sp, iu = su;
        for (int o = 1; o < 64; o <<= 1) {
            const int a = __shfl_up(ip, o, 64);
            const int b = __shfl_up(iu, o, 64);
            if (tid >= o) {
                ip += a;
                iu += b;
            }
        }
        int xp = ip - sp, xu = iu - su;
        for (int i = 0; i < per; ++i) {
            const int e = e0 + i;
            if (e < E) {
                ustart[e] = xp;
                if (cnt[e] > 0) {
                    uexp[xu] = e;
                    uoff[xu] = xp;
                    ++xu;
                }
                xp += cnt[e];
            }
        }
        if (tid == 63) {
            misc[1] = iu;  // routed units
            misc[2] = ip;  // valid routed pairs
        }
    }
    __syncthreads();
    for (int t = tid; t < S; t += nthr) {
        for (int k0 = 0; k0 < K; k0 += BU_KC) {
            int v[BU_KC];
            load_group(t, k0, v);
#pragma unroll
            for (int j = 0; j < BU_KC; ++j) {
                const int e = v[j];
                if (e >= 0 && e < E) pairs[ustart[e] + atomicAdd(&fill[e], 1)] = t * K + k0 + j;
            }
        }
    }
    const int nr = misc[1], pv = misc[2];
    if (n_shared)
        for (int t = tid; t < S; t += nthr) pairs[pv + t] = P + t;
    if (tid == 0) {
        uoff[nr] = pv;
        if (n_shared) {
            uexp[nr] = -1;
            uoff[nr + 1] = pv + S;
        }
        misc[0] = nr + (n_shared ? 1 : 0);
    }
    __syncthreads();
}

// Staging of device words into LDS in rounds: in round r a thread loads up
// to MW words of an array (word i from src(i), indices clamped into range,
// n >= 1) into registers, and later stores them (to dst(i)).  Callers issue
// the loads of every array of a round before any store, so a round costs a
// single memory latency.
template <int MW, typename T, typename Src>
__device__ __forceinline__ void stage_load(T (&v)[MW], int round, int n, Src src) {
    const int nthr = blockDim.x, base = round * MW * nthr + (int)threadIdx.x;
#pragma unroll
    for (int k = 0; k < MW; ++k) v[k] = *src(min(base + k * nthr, n - 1));
}
template <int MW, typename T, typename Dst>
__device__ __forceinline__ void stage_store(const T (&v)[MW], int round, int n, Dst dst) {
    const int nthr = blockDim.x, base = round * MW * nthr + (int)threadIdx.x;
#pragma unroll
    for (int k = 0; k < MW; ++k)
        if (base + k * nthr < n) *dst(base + k * nthr) = v[k];
}
// As stage_load, with src(i) returning the word itself.
template <int MW, typename T, typename Src>
__device__ __forceinline__ void stage_fetch(T (&v)[MW], int round, int n, Src src) {
    const int nthr = blockDim.x, base = round * MW * nthr + (int)threadIdx.x;
#pragma unroll
    for (int k = 0; k < MW; ++k) v[k] = src(min(base + k * nthr, n - 1));
}
__device__ __forceinline__ int stage_rounds(int n, int per_round) { return (n + per_round - 1) / per_round; }

// Direct global-to-LDS loads (no registers): lane l of the wavefront reads
// 16 (or 4) bytes at its own src and the hardware writes them to
// lds_wave + 16 l (or + 4 l); lds_wave must be the same in every lane.
// Completion is tracked by the vector-memory counter: wait for it, then a
// workgroup barrier, before the LDS data is read.
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_wave) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_wave, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *src, void *lds_wave) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_wave, 4, 0, 0);
}
__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// i / d by a multiply-high for 0 <= i < 2^16, 1 <= d < 2^16: with
// m = floor(2^32 / d) + 1 (2^32 / d when d is a power of two),
// (i * m) >> 32 == floor(i / d); d = 1 is kept as m = 0.
__device__ __forceinline__ uint32_t fast_div_magic(int d) { return d == 1 ? 0u : 0xFFFFFFFFu / (uint32_t)d + 1u; }
__device__ __forceinline__ int fast_div(int i, uint32_t m) { return m ? (int)__umulhi((uint32_t)i, m) : i; }

// Waits until at most N of this thread's vector-memory operations are
// outstanding (they complete in issue order); gfx9 s_waitcnt encoding, with
// expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void drain_vm() { wait_vm<0>(); }

__device__ __forceinline__ void load_act(const int8_t *vq, int b, int32_t a[8]) {
    const i32x4 *p = reinterpret_cast<const i32x4 *>(vq + 32 * b);
    const i32x4 lo = p[0], hi = p[1];
    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
    a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
}

// Makes this wave's LDS writes visible to its own later reads (LDS
// operations of one wave complete in order; the fence orders them for the
// compiler and waits for outstanding LDS traffic).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it (__syncthreads() waits for every one of them).
// Direct global-to-LDS loads are not covered: wait for them (wait_vm) first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Binary32 chain of one chunk for one (row, vector): acc = fmaf(d_b, isum_b,
// acc) for the chunk's blocks in ascending order.  A full chunk is unrolled
// with 16-byte LDS reads so the reads are all in flight before the chain.
__device__ __forceinline__ float chain_chunk(float acc, const int32_t *is, const float *dv, int nbc) {
    if (nbc == 64) {
        // four quarters of 16 blocks; within a quarter all LDS reads are issued first
#pragma unroll 1
        for (int qq = 0; qq < 64; qq += 16) {
            i32x4 iv[4];
            f32x4 dd[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                iv[q4] = *reinterpret_cast<const i32x4 *>(is + qq + 4 * q4);
                dd[q4] = *reinterpret_cast<const f32x4 *>(dv + qq + 4 * q4);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                acc = __builtin_fmaf(dd[q4].x, (float)iv[q4].x, acc);
                acc = __builtin_fmaf(dd[q4].y, (float)iv[q4].y, acc);
                acc = __builtin_fmaf(dd[q4].z, (float)iv[q4].z, acc);
                acc = __builtin_fmaf(dd[q4].w, (float)iv[q4].w, acc);
            }
        }
    } else {
        for (int bb = 0; bb < nbc; ++bb) acc = __builtin_fmaf(dv[bb], (float)is[bb], acc);
    }
    return acc;
}

// The same chain with one scale per group of gb blocks of the row (gs: the
// chunk's group scales of this lane's row): acc = fmaf(dv_b * gs[b / gb],
// isum_b, acc), the multiplier being one binary32 product.  gb = 1 << lgb.
// ISF: the block sums are stored as binary32 bits (exact integers) instead
// of int32.
template <bool ISF = false>
__device__ __forceinline__ float isum_f(int32_t v) {
    return ISF ? __int_as_float(v) : (float)v;
}
template <bool ISF = false>
__device__ __forceinline__ float chain_chunk_g(float acc, const int32_t *is, const float *dv, const float *gs,
                                               int lgb, int nbc) {
    if (nbc == 64) {
#pragma unroll 1
        for (int qq = 0; qq < 64; qq += 16) {
            i32x4 iv[4];
            f32x4 dd[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                iv[q4] = *reinterpret_cast<const i32x4 *>(is + qq + 4 * q4);
                dd[q4] = *reinterpret_cast<const f32x4 *>(dv + qq + 4 * q4);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int b = qq + 4 * q4;
                acc = __builtin_fmaf(dd[q4].x * gs[b >> lgb], isum_f<ISF>(iv[q4].x), acc);
                acc = __builtin_fmaf(dd[q4].y * gs[(b + 1) >> lgb], isum_f<ISF>(iv[q4].y), acc);
                acc = __builtin_fmaf(dd[q4].z * gs[(b + 2) >> lgb], isum_f<ISF>(iv[q4].z), acc);
                acc = __builtin_fmaf(dd[q4].w * gs[(b + 3) >> lgb], isum_f<ISF>(iv[q4].w), acc);
            }
        }
    } else {
        for (int bb = 0; bb < nbc; ++bb) acc = __builtin_fmaf(dv[bb] * gs[bb >> lgb], isum_f<ISF>(is[bb]), acc);
    }
    return acc;
}

// The MXFP4 chain of one chunk with the row's E8M0 bytes xb (one per block,
// raw, in LDS): the same operations as chain_chunk_g<true> with group 32,
// the multiplier 2^(x_b - 128) formed from the byte.
__device__ __forceinline__ float chain_chunk_mx_bytes(float acc, const int32_t *is, const float *dv, const uint8_t *xb,
                                                      int nbc) {
    if (nbc == 64) {
#pragma unroll 1
        for (int qq = 0; qq < 64; qq += 16) {
            i32x4 iv[4];
            f32x4 dd[4];
            const u32x4 xw = *reinterpret_cast<const u32x4 *>(xb + qq);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                iv[q4] = *reinterpret_cast<const i32x4 *>(is + qq + 4 * q4);
                dd[q4] = *reinterpret_cast<const f32x4 *>(dv + qq + 4 * q4);
            }
            const uint32_t xs[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t x = xs[q4];
                acc = __builtin_fmaf(dd[q4].x * e8m0_half(x & 0xFFu), __int_as_float(iv[q4].x), acc);
                acc = __builtin_fmaf(dd[q4].y * e8m0_half((x >> 8) & 0xFFu), __int_as_float(iv[q4].y), acc);
                acc = __builtin_fmaf(dd[q4].z * e8m0_half((x >> 16) & 0xFFu), __int_as_float(iv[q4].z), acc);
                acc = __builtin_fmaf(dd[q4].w * e8m0_half(x >> 24), __int_as_float(iv[q4].w), acc);
            }
        }
    } else {
        for (int bb = 0; bb < nbc; ++bb)
            acc = __builtin_fmaf(dv[bb] * e8m0_half(xb[bb]), __int_as_float(is[bb]), acc);
    }
    return acc;
}

// Group scales of a wave's rows (one f32 per 32 << lgb codes), staged
// through LDS one 64-block chunk at a time: the chunk's RPW x (64 >> lgb)
// scales are 16-byte words w = lane + 64 k, word w holding scales
// 4 p .. 4 p + 3 of the chunk of row w / (16 >> lgb), p = w % (16 >> lgb)
// (lgb <= 4, groups of up to 512 codes, so a row's chunk is whole words).
// A row shorter than a chunk has fewer than 64 >> lgb scales there: its
// words then run on into the next row's scales (or past the blob's end,
// where the buffer resource returns zeros), values that belong to blocks
// past the row's end and are never used.  Loads run through the blob's
// buffer resource.
struct RowGroups {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t base;         // byte offset of the scales of the wave's first row
    uint32_t row_stride;   // bytes of scales per row
    int lgb;               // log2(blocks per group); -1: per-row scales, nothing staged
    float *lds;            // RPW x (64 >> lgb) floats, private to the wave
};

template <int RPW>
__device__ __forceinline__ void groups_load(const RowGroups &G, int c, i32x4 (&gw)[4]) {
    const int lane = threadIdx.x & 63;
    const int wpr = 16 >> G.lgb, words = RPW * wpr;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int w = lane + 64 * k;
        if (w < words) {
            const int row = w / wpr, p = w - row * wpr;
            const uint32_t off = G.base + (uint32_t)row * G.row_stride + (uint32_t)(c * (64 >> G.lgb) + 4 * p) * 4u;
            gw[k] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(G.rsrc, off, 0, 0));
        }
    }
}

template <int RPW>
__device__ __forceinline__ void groups_store(const RowGroups &G, const i32x4 (&gw)[4]) {
    const int lane = threadIdx.x & 63;
    const int wpr = 16 >> G.lgb, words = RPW * wpr;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int w = lane + 64 * k;
        if (w < words) reinterpret_cast<i32x4 *>(G.lds)[w] = gw[k];
    }
}

// MXFP4 rows: one E8M0 byte per block (lgb = 0), row_stride = H / 32 bytes
// (a multiple of 4), staged the same way as floats 2^(x - 128): the chunk's
// 64 bytes of a row are 16 dwords, dword w = lane + 64 k of the wave holding
// bytes 4 p .. 4 p + 3 of row w / 16, p = w % 16, converted on the store.
template <int RPW>
__device__ __forceinline__ void groups_load_mx(const RowGroups &G, int c, uint32_t (&gb)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int w = lane + 64 * k;
        if (w < RPW * 16) {
            const int row = w >> 4, p = w & 15;
            gb[k] = __builtin_amdgcn_raw_buffer_load_b32(G.rsrc, G.base + (uint32_t)row * G.row_stride +
                                                                     (uint32_t)(64 * c + 4 * p), 0, 0);
        }
    }
}

template <int RPW>
__device__ __forceinline__ void groups_store_mx(const RowGroups &G, const uint32_t (&gb)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int w = lane + 64 * k;
        if (w < RPW * 16) {
            const uint32_t v = gb[k];
            reinterpret_cast<f32x4 *>(G.lds)[w] =
                f32x4{e8m0_half(v & 0xFFu), e8m0_half((v >> 8) & 0xFFu), e8m0_half((v >> 16) & 0xFFu),
                      e8m0_half(v >> 24)};
        }
    }
}

// Issues the loads of chunk 0 (blocks 0..63) of this wave's RPW rows.
template <int BITS, int RPW>
__device__ __forceinline__ void prime_rows(__amdgpu_buffer_rsrc_t rsrc, const uint32_t rowoff[RPW],
                                           int nb, BlockBits<BITS> (&cur)[RPW]) {
    const int lane = threadIdx.x & 63;
    if (lane < nb) {
#pragma unroll
        for (int j = 0; j < RPW; ++j) cur[j] = load_block<BITS>(rsrc, rowoff[j], lane);
    }
}

// Streams this wave's RPW rows for the ng staged vectors; `cur` holds chunk 0
// (prime_rows).  Returns, in lane (row = lane % RPW, vector = lane / RPW),
// the chain fmaf(d_b, isum_b, acc) over all blocks of that row in ascending
// order (NT * RPW <= 64).  `stage()` fills the LDS vectors and ends with a
// workgroup barrier; it runs while chunk 0 is in flight.  Each wave then
// works alone on its own LDS region (NT x RPW rows of ISUM_PITCH block
// dots); for int4 / int2 the next chunk's weights are in flight while the
// current chunk is reduced, for int8 each row of the next chunk from the
// moment the current chunk's row has been used.
// With GROUPED (G.lgb >= 0) the chain of chunk c uses the chunk's
// group scales, loaded one chunk ahead with the weights and staged in the
// wave's LDS region G.lds; the row scale is then not applied by the caller.
// MX: the rows are MXFP4 (BITS 4, GROUPED with lgb 0, E8M0 scale bytes).
template <int BITS, int NT, int RPW, bool GROUPED, bool MX = false, typename Stage>
__device__ __forceinline__ float stream_rows(__amdgpu_buffer_rsrc_t rsrc, const uint32_t rowoff[RPW],
                                             int nb, int ng, const int8_t *vq, const float *vd,
                                             int32_t *isum_wave, int vlen, Stage stage,
                                             BlockBits<BITS> (&cur)[RPW], const RowGroups &G) {
    static_assert(NT * RPW <= 64, "one chain per lane");
    static_assert(!MX || (BITS == 4 && GROUPED), "MXFP4 rows are 4-bit codes with a scale per block");
    constexpr bool PREFETCH = BITS < 8;
    const int lane = threadIdx.x & 63;
    const int crow = lane % RPW, cvec = lane / RPW;
    const int vds = vd_stride(nb);
    constexpr bool grouped = GROUPED;
    float acc = 0.0f;
    const int nchunks = (nb + 63) / 64;
    i32x4 gw[4];
    uint32_t gb[4];
    if (MX) groups_load_mx<RPW>(G, 0, gb);
    else if (grouped) groups_load<RPW>(G, 0, gw);
    stage();
    if (MX) groups_store_mx<RPW>(G, gb);
    else if (grouped) groups_store<RPW>(G, gw);
    for (int c = 0; c < nchunks; ++c) {
        const int b = c * 64 + lane;
        const bool act = b < nb;
        BlockBits<BITS> nxt[RPW];
        // the next chunk's group scales are issued before its weights: they
        // are stored at the end of this chunk, and waiting for them must not
        // wait for the weights (loads complete in issue order)
        if (MX && c + 1 < nchunks) groups_load_mx<RPW>(G, c + 1, gb);
        else if (grouped && c + 1 < nchunks) groups_load<RPW>(G, c + 1, gw);
        __builtin_amdgcn_sched_barrier(0);
        if (PREFETCH && b + 64 < nb) {
#pragma unroll
            for (int j = 0; j < RPW; ++j) nxt[j] = load_block<BITS>(rsrc, rowoff[j], b + 64);
        }
        if constexpr (!PREFETCH) {
            // int8: no registers for a second chunk, so row j of the next
            // chunk is requested as soon as row j's block dots are done (the
            // vectors' activations of the block are read first), keeping
            // about one chunk in flight through the reduction
            int32_t av[NT][8];
#pragma unroll
            for (int it = 0; it < NT; ++it) {
#pragma unroll
                for (int k = 0; k < 8; ++k) av[it][k] = 0;
                if (it < ng && act) load_act(vq + (size_t)it * vlen, b, av[it]);
            }
            // every lane issues the refill (after the last chunk through an
            // empty resource, which reads zeros without a memory access), so
            // that the count of loads in flight is the same on every path
            // and the wait for row j + 1 leaves the refills in flight; a
            // lane past the row's end reads bytes it does not use
            const __amdgpu_buffer_rsrc_t rnext = c + 1 < nchunks ? rsrc : make_rsrc(nullptr, 0u);
#pragma unroll
            for (int j = 0; j < RPW; ++j) {
#pragma unroll
                for (int it = 0; it < NT; ++it)
                    if (it < ng) isum_wave[(it * RPW + j) * ISUM_PITCH + lane] = act ? block_dot(cur[j], av[it]) : 0;
                __builtin_amdgcn_sched_barrier(0);
                cur[j] = load_block<BITS>(rnext, rowoff[j], b + 64);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            if (!PREFETCH) break;
            if (it < ng) {
                int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (act) load_act(vq + (size_t)it * vlen, b, av);
                int32_t *dst = isum_wave + it * RPW * ISUM_PITCH + lane;
                if constexpr (MX) {
                    // exact block sums in binary32 (see block_dot_mx_f16)
                    f16x2 h[16];
                    mx_act_f16(av, h);
#pragma unroll
                    for (int j = 0; j < RPW; ++j)
                        dst[j * ISUM_PITCH] = act ? __float_as_int(block_dot_mx_f16(cur[j].w, h)) : 0;
                } else {
#pragma unroll
                    for (int j = 0; j < RPW; ++j) dst[j * ISUM_PITCH] = act ? block_dot(cur[j], av) : 0;
                }
            }
        }
        wave_lds_sync();
        if (cvec < ng) {
            if (grouped)
                acc = chain_chunk_g<MX>(acc, isum_wave + (cvec * RPW + crow) * ISUM_PITCH, vd + cvec * vds + c * 64,
                                        G.lds + crow * (64 >> G.lgb), G.lgb, min(64, nb - c * 64));
            else
                acc = chain_chunk(acc, isum_wave + (cvec * RPW + crow) * ISUM_PITCH, vd + cvec * vds + c * 64,
                                  min(64, nb - c * 64));
        }
        wave_lds_sync();
        if (grouped && c + 1 < nchunks) {
            if (MX)
                groups_store_mx<RPW>(G, gb);
            else
                groups_store<RPW>(G, gw);
            wave_lds_sync();
        }
        if (PREFETCH) {
#pragma unroll
            for (int j = 0; j < RPW; ++j) cur[j] = nxt[j];
        }
    }
    return acc;
}

template <int BITS, int NT, int RPW, typename Stage>
__device__ __forceinline__ float stream_rows(__amdgpu_buffer_rsrc_t rsrc, const uint32_t rowoff[RPW],
                                             int nb, int ng, const int8_t *vq, const float *vd,
                                             int32_t *isum_wave, int vlen, Stage stage,
                                             BlockBits<BITS> (&cur)[RPW]) {
    RowGroups G;
    G.lgb = -1;
    return stream_rows<BITS, NT, RPW, false>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, vlen, stage, cur, G);
}

// LDS bytes of the group-scale staging of a workgroup of `waves` wavefronts
// of 16 rows each (0 for per-row scales).
__host__ __device__ inline size_t groups_lds_bytes(int group, int waves) {
    return group ? (size_t)waves * 16 * (64 / (group / 32)) * 4 : 0;
}
__host__ __device__ inline int group_lgb(int group) {
    int l = -1;
    for (int g = group / 32; g > 0; g >>= 1) ++l;
    return group ? l : -1;
}

}  // namespace coli
