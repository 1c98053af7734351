// Expert FFN kernels of the MoE layer for decode and speculative-verify
// batches (colibrì README v1.0, "What's implemented": SwiGLU experts over
// int8 / packed int4 / packed int2 weights with per-row scales, integer dots
// over Q8_0 activations, batch-union MoE with each unique expert read once).
//
// Work decomposition.  A "unit" is one unique routed expert of the call (in
// ascending id) or the shared expert (last).  Every workgroup rebuilds the
// unit table from topk_idx in LDS (a few hundred integer operations), takes
// unit blockIdx.y and a tile of weight rows blockIdx.x, and streams those
// rows once for all tokens routed to the unit.
//
//   k_gateup: 32 gate rows + the 32 matching up rows (rows i0..i0+31) ->
//             SwiGLU -> one Q8_0 block of h per token, written to the
//             workspace slot of the (token, rank) pair.
//   k_down:   64 down rows -> y per pair slot in the workspace; the last of
//             the units to finish a row tile (integer arrival counter) then
//             combines that tile for every token in rank order.  Each output
//             element has exactly one writer; no floating-point atomics.
//
// Inner loop (both kernels).  Wave w owns 16 rows.  A row is read in chunks
// of 64 Q8_0 blocks: lane l loads block 64c+l of each of its 16 rows
// (contiguous across lanes: 1 KB per row per load for int4), forms the exact
// int32 block dots against the LDS-staged activation codes, and writes them
// to LDS.  Then thread (row, token) runs the binary32 chain
// acc = fmaf(d_b, isum_b, acc) over the chunk's blocks in ascending order —
// the layer's defined order — and finally multiplies by the row scale.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

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
// indices are flagged in the status word.
__device__ void build_units(const int32_t *__restrict__ idx, int S, int K, int E, int n_shared,
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
    for (int p = tid; p < P; p += nthr) {
        const int e = idx[p];
        if (e >= 0 && e < E) {
            atomicAdd(&cnt[e], 1);
            if (validate) {
                const int t0 = (p / K) * K;
                for (int q = t0; q < p; ++q)
                    if (idx[q] == e) raise_status(status, ST_BADINDEX);
            }
        } else if (validate) {
            raise_status(status, ST_BADINDEX);
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
    for (int p = tid; p < P; p += nthr) {
        const int e = idx[p];
        if (e >= 0 && e < E) pairs[ustart[e] + atomicAdd(&fill[e], 1)] = p;
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
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

// Streams this wave's 16 rows for the ng staged vectors.  Returns, in lane
// (row = lane & 15, vector = lane >> 4), the chain fmaf(d_b, isum_b, acc)
// over all blocks of that row in ascending order.  `stage()` fills the LDS
// vectors and ends with a workgroup barrier; it runs after the first chunk's
// weight loads are issued so that their latency overlaps it.  Each wave then
// works alone on its own LDS region; for int4 / int2 the next chunk's
// weights are in flight while the current chunk is reduced.
template <int BITS, int NT, typename Stage>
__device__ __forceinline__ float stream_rows(__amdgpu_buffer_rsrc_t rsrc,
                                             const uint32_t rowoff[ROWS_PER_WAVE], int nb,
                                             int ng, const int8_t *vq, const float *vd,
                                             int32_t *isum_wave, int vlen, Stage stage) {
    constexpr bool PREFETCH = BITS < 8;
    const int lane = threadIdx.x & 63;
    const int crow = lane & 15, cvec = lane >> 4;
    const int vds = vd_stride(nb);
    float acc = 0.0f;
    const int nchunks = (nb + 63) / 64;
    BlockBits<BITS> cur[ROWS_PER_WAVE];
    if (lane < nb) {
#pragma unroll
        for (int j = 0; j < ROWS_PER_WAVE; ++j) cur[j] = load_block<BITS>(rsrc, rowoff[j], lane);
    }
    stage();
    for (int c = 0; c < nchunks; ++c) {
        const int b = c * 64 + lane;
        const bool act = b < nb;
        BlockBits<BITS> nxt[ROWS_PER_WAVE];
        if (PREFETCH && b + 64 < nb) {
#pragma unroll
            for (int j = 0; j < ROWS_PER_WAVE; ++j) nxt[j] = load_block<BITS>(rsrc, rowoff[j], b + 64);
        }
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            if (it < ng) {
                int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (act) load_act(vq + (size_t)it * vlen, b, av);
                int32_t *dst = isum_wave + it * ROWS_PER_WAVE * ISUM_PITCH + lane;
#pragma unroll
                for (int j = 0; j < ROWS_PER_WAVE; ++j)
                    dst[j * ISUM_PITCH] = act ? block_dot(cur[j], av) : 0;
            }
        }
        wave_lds_sync();
        if (cvec < ng)
            acc = chain_chunk(acc, isum_wave + (cvec * ROWS_PER_WAVE + crow) * ISUM_PITCH,
                              vd + cvec * vds + c * 64, min(64, nb - c * 64));
        wave_lds_sync();
        if (PREFETCH) {
#pragma unroll
            for (int j = 0; j < ROWS_PER_WAVE; ++j) cur[j] = nxt[j];
        } else if (c + 1 < nchunks && b + 64 < nb) {
#pragma unroll
            for (int j = 0; j < ROWS_PER_WAVE; ++j) cur[j] = load_block<BITS>(rsrc, rowoff[j], b + 64);
        }
    }
    return acc;
}

template <int BITS, int NT>
__global__ __launch_bounds__(256) void k_gateup(const FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I, P = S * K;
    const SmemPlan L = smem_plan(S, K, E, NT, H);
    build_units(a.idx, S, K, E, a.n_shared, smem, L, a.status,
                blockIdx.x == 0 && blockIdx.y == 0 && a.pend_mode != 2);
    const int *uexp = reinterpret_cast<const int *>(smem + L.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + L.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + L.pairs);
    const int n_units = uniform(reinterpret_cast<const int *>(smem + L.misc)[0]);
    const int u = blockIdx.y;
    if (u >= n_units) return;
    const int e = uniform(uexp[u]);
    if (e >= 0 && a.pend_mode != 0) {
        const bool pend = (a.pend[e >> 5] >> (e & 31)) & 1u;
        if ((a.pend_mode == 1) == pend) return;
    }
    const uint8_t *blob = uniform_ptr(e < 0 ? a.shared : a.blobs[e]);
    if (blob == nullptr) {
        if (tid == 0) raise_status(a.status, ST_NOTRESIDENT);
        return;
    }
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * ROWS_PER_WAVE * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const BlobLayout BL = blob_layout(H, I, BITS);
    const size_t row_bytes = (size_t)H * BITS / 8;
    const int i0 = blockIdx.x * 32;
    const int half = wave & 1;            // rows 0-15 or 16-31 of the tile
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[ROWS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < ROWS_PER_WAVE; ++j)
        rowoff[j] = (uint32_t)(mat + (size_t)(i0 + 16 * half + j) * row_bytes);
    const float *scale = reinterpret_cast<const float *>(blob + (wave < 2 ? BL.s_gate : BL.s_up));
    const int nb = H / 32;
    const int p0 = uniform(uoff[u]), np = uniform(uoff[u + 1]) - p0;
    const bool check_x = blockIdx.x == 0;
    const int crow = lane & 15, cvec = lane >> 4;
    const int vds = vd_stride(nb);
    for (int g0 = 0; g0 < np; g0 += NT) {
        const int ng = min(NT, np - g0);
        // Q8_0 of the hidden states of this group's tokens.  Lanes 0-31 and
        // 32-63 of a wave each hold one 32-element block.
        auto stage = [&]() {
            for (int it = 0; it < ng; ++it) {
                const int v = pairs[p0 + g0 + it];
                const int t = v < P ? v / K : v - P;
                const float *xr = a.x + (size_t)t * H;
                for (int h = tid; h < H; h += 256) {
                    const float xv = xr[h];
                    if (check_x && !finite_f32(xv)) raise_status(a.status, ST_NONFINITE);
                    float d;
                    const int8_t q = q8_0_lane(xv, &d);
                    vq[it * H + h] = q;
                    if ((lane & 31) == 0) vd[it * vds + (h >> 5)] = d;
                }
            }
            __syncthreads();
        };
        const float acc = stream_rows<BITS, NT>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, H, stage);
        if (cvec < ng) gu[cvec * 64 + wave * ROWS_PER_WAVE + crow] = acc * scale[i0 + 16 * half + crow];
        __syncthreads();
        // SwiGLU and Q8_0(h): half-wave (tid >> 5) handles one vector's 32 rows.
        const int vv = tid >> 5, i = tid & 31;
        if (vv < ng) {
            const float h = swiglu_f32(gu[vv * 64 + i], gu[vv * 64 + 32 + i]);
            float d;
            const int8_t q = q8_0_lane(h, &d);
            const int slot = pairs[p0 + g0 + vv];
            a.qh[(size_t)slot * I + i0 + i] = q;
            if (i == 0) a.dh[(size_t)slot * (I / 32) + i0 / 32] = d;
        }
        __syncthreads();
    }
}

// Down projection: 64 rows of one unit per workgroup, y written to the
// pair's slot of the workspace (the combine kernel reads it after this
// kernel has finished, so no cross-workgroup signalling is needed).
template <int BITS, int NT>
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
    const BlobLayout BL = blob_layout(H, I, BITS);
    const size_t row_bytes = (size_t)I * BITS / 8;
    const int rw = r0 + wave * ROWS_PER_WAVE;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
    uint32_t rowoff[ROWS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < ROWS_PER_WAVE; ++j) rowoff[j] = (uint32_t)(BL.down + (size_t)(rw + j) * row_bytes);
    const float *s_down = reinterpret_cast<const float *>(blob + BL.s_down);
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
        const float acc = stream_rows<BITS, NT>(rsrc, rowoff, nb, ng, vq, vd, isum_wave, I, stage);
        if (cvec < ng) {
            const int slot = pairs[p0 + g0 + cvec];
            a.Y[(size_t)slot * H + rw + crow] = acc * s_down[rw + crow];
        }
        __syncthreads();
    }
}

// Combine: out[t, r] = (fmaf chain over k in rank order of w[t,k] * y[t,k][r]
// from 0) + y_shared[t][r].  One thread per output element, one writer.
// Grid (H / 256, S).
__global__ __launch_bounds__(256) void k_combine(const FwdArgs a) {
    const int t = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    const int K = a.K, H = a.H, P = a.S * a.K;
    const float *w = a.w + (size_t)t * K;
    float acc = 0.0f;
    bool ok = true;
    for (int k = 0; k < K; ++k) {
        const float wk = w[k];
        ok = ok && finite_f32(wk);
        acc = __builtin_fmaf(wk, a.Y[(size_t)(t * K + k) * H + r], acc);
    }
    if (a.n_shared) acc = acc + a.Y[(size_t)(P + t) * H + r];
    a.out[(size_t)t * H + r] = acc;
    if (!ok && r == 0) raise_status(a.status, ST_NONFINITE);
}

// ---- launchers -----------------------------------------------------------
static int pick_nt(int S) { return S >= 4 ? 4 : (S >= 2 ? 2 : 1); }

size_t forward_smem_max(int S, int H, int I, int E, int K, int n_shared) {
    (void)n_shared;
    const int nt = pick_nt(S);
    return std::max(smem_plan(S, K, E, nt, H).total, smem_plan(S, K, E, nt, I).total);
}

// Raises a kernel's dynamic-LDS limit once to the largest size it has been
// launched with (so that later launches, including ones under stream capture,
// only enqueue work).  Calls come from one host thread at a time per kernel.
template <typename F>
static hipError_t launch_dyn(F kern, dim3 grid, size_t smem, hipStream_t st, const FwdArgs &a) {
    static size_t raised = 0;
    if (smem > raised) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (err != hipSuccess) return err;
        raised = smem;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), smem, st, a);
    return hipGetLastError();
}

template <int BITS>
static hipError_t gateup_bits(const FwdArgs &a, hipStream_t st) {
    const int P = a.S * a.K;
    const int umax = std::min(P, a.E) + a.n_shared;
    const dim3 grid(a.I / 32, umax);
    const int nt = pick_nt(a.S);
    const size_t smem = smem_plan(a.S, a.K, a.E, nt, a.H).total;
    if (nt == 1) return launch_dyn(k_gateup<BITS, 1>, grid, smem, st, a);
    if (nt == 2) return launch_dyn(k_gateup<BITS, 2>, grid, smem, st, a);
    return launch_dyn(k_gateup<BITS, 4>, grid, smem, st, a);
}

template <int BITS>
static hipError_t down_bits(const FwdArgs &a, hipStream_t st) {
    const int P = a.S * a.K;
    const int umax = std::min(P, a.E) + a.n_shared;
    const dim3 grid(a.H / 64, umax);
    const int nt = pick_nt(a.S);
    const size_t smem = smem_plan(a.S, a.K, a.E, nt, a.I).total;
    if (nt == 1) return launch_dyn(k_down<BITS, 1>, grid, smem, st, a);
    if (nt == 2) return launch_dyn(k_down<BITS, 2>, grid, smem, st, a);
    return launch_dyn(k_down<BITS, 4>, grid, smem, st, a);
}

hipError_t launch_gateup(const FwdArgs &a, int bits, hipStream_t st) {
    if (bits == 8) return gateup_bits<8>(a, st);
    if (bits == 4) return gateup_bits<4>(a, st);
    return gateup_bits<2>(a, st);
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_combine, dim3(a.H / 256, a.S), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_down(const FwdArgs &a, int bits, hipStream_t st) {
    if (bits == 8) return down_bits<8>(a, st);
    if (bits == 4) return down_bits<4>(a, st);
    return down_bits<2>(a, st);
}

}  // namespace coli
