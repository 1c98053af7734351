// Persistent single-launch MoE layer for decode and speculative-verify
// batches (colibrì README v1.0, "What's implemented": DeepSeek-V3-style
// sigmoid router, SwiGLU experts on Q8_0 activations, shared expert,
// batch-union MoE; "Colibri (colibrì): GLM-5.2 local inference on 25 GB of
// RAM", "How it works (validated core mechanics)": the router).
//
// One launch runs the phases of the layer, separated by grid barriers
// instead of kernel boundaries:
//   R  router logits (one wavefront each) and Q8_0(x), one 32-block per half
//      wave; skipped logits when the routing is given;
//   -- barrier --
//      every workgroup selects the top-K of every token itself (same bits
//      everywhere) and builds the unit table of the batch union;
//   1  gate/up items (unit, 32-row tile): 4 waves x 16 rows, SwiGLU and
//      Q8_0(h) in the epilogue;
//   -- barrier --
//   2  down items of 8 output rows (2 per wave) for every unit, then the
//      combine of those rows in the same workgroup (one writer each).
// A workgroup drains its own stores (s_waitcnt) before it issues the next
// phase's weight loads and arrives at the barrier, so the loads are in
// flight during the wait.  Data crossing workgroups (logits, Q8_0(x),
// Q8_0(h)) is written and read with device-scope (sc1) accesses, coherent
// across the L2 slices of the GPU.  Barrier waits are bounded: a grid that
// could not be fully resident ends with a status error, never a hang; the
// host sizes the grid from the kernel's occupancy.
#include <algorithm>
#include <map>
#include <mutex>

#include "device_common.h"
#include "kernels.h"
#include "router.h"
#include "stream.h"

namespace coli {

constexpr uint32_t SPIN_LIMIT = 1u << 22;
constexpr int LT = 256;         // threads per workgroup
constexpr int LW = LT / 64;     // waves per workgroup
constexpr int RW2 = 2;          // down rows per wave
constexpr int ROWS2 = LW * RW2; // down rows per item
constexpr int MAXPB = 32;       // pairs per down batch (chain lanes: RW2 x MAXPB)
constexpr int CPOL_SC1 = 16;    // buffer cache policy: device-scope coherent

__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for every outstanding memory operation of this thread.
__device__ __forceinline__ void drain() { __builtin_amdgcn_s_waitcnt(0); }

// Grid barrier; callers drain() their stores first (loads issued after the
// drain stay in flight).
__device__ __forceinline__ void arrive_wait(uint32_t *ctr, uint32_t nwg, uint32_t *status) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nwg) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins >= SPIN_LIMIT) {
                raise_status(status, ST_TIMEOUT);
                break;
            }
        }
    }
    __syncthreads();
}

// The last workgroup to leave resets the barrier words for the next launch.
__device__ __forceinline__ void grid_exit(uint32_t *sync, int nbar, uint32_t nwg) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&sync[nbar], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == nwg - 1)
            for (int i = 0; i <= nbar; ++i) st_dev(&sync[i], 0u);
    }
}

template <int BITS>
struct DownBatch {
    static constexpr int UB = BITS == 8 ? 4 : 8;  // units per batch
};

struct LayerPlan {
    size_t cnt, ustart, fill, uexp, uoff, pairs, misc;   // unit table
    size_t idx, w, ublob, sig, selsig;                   // routing
    size_t vq, vd, isum, gu;                             // phase 1
    size_t qh, dh, isum2, sdn, y, total;                 // phase 2
};

__host__ __device__ inline LayerPlan layer_plan(int S, int K, int E, int n_shared, int NT, int H, int I) {
    LayerPlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    const int slots = P + S * n_shared;
    const int mpb = slots < MAXPB ? slots : MAXPB;
    p.cnt = 0;
    p.ustart = a16(p.cnt + 4 * (size_t)E);
    p.fill = a16(p.ustart + 4 * (size_t)E);
    p.uexp = a16(p.fill + 4 * (size_t)E);
    p.uoff = a16(p.uexp + 4 * (size_t)umax);
    p.pairs = a16(p.uoff + 4 * (size_t)(umax + 1));
    p.misc = a16(p.pairs + 4 * (size_t)(P + S));
    p.idx = a16(p.misc + 16);
    p.w = a16(p.idx + 4 * (size_t)P);
    p.ublob = a16(p.w + 4 * (size_t)P);
    p.sig = a16(p.ublob + 8 * (size_t)umax);
    p.selsig = a16(p.sig + 4 * (size_t)LW * E);
    const size_t base = a16(p.selsig + 4 * (size_t)LW * 32);
    p.vq = base;
    p.vd = a16(p.vq + (size_t)NT * H);
    p.isum = a16(p.vd + 4 * (size_t)NT * vd_stride(H / 32));
    p.gu = a16(p.isum + 4 * (size_t)LW * NT * ROWS_PER_WAVE * ISUM_PITCH);
    const size_t end1 = a16(p.gu + 4 * (size_t)NT * 64);
    p.qh = base;
    p.dh = a16(p.qh + (size_t)mpb * I);
    p.isum2 = a16(p.dh + 4 * (size_t)mpb * vd_stride(I / 32));
    p.sdn = a16(p.isum2 + 4 * (size_t)LW * RW2 * mpb * ISUM_PITCH);
    p.y = a16(p.sdn + 4 * (size_t)umax * ROWS2);
    const size_t end2 = a16(p.y + 4 * (size_t)slots * ROWS2);
    p.total = end1 > end2 ? end1 : end2;
    return p;
}

template <int BITS, int NT, bool ROUTE, int MAXJ>
__global__ __launch_bounds__(LT) void k_layer(const FwdArgs a, const LayerArgs l) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I, P = S * K;
    const int G = gridDim.x;
    const LayerPlan L = layer_plan(S, K, E, a.n_shared, NT, H, I);
    SmemPlan T;
    T.cnt = L.cnt; T.ustart = L.ustart; T.fill = L.fill; T.uexp = L.uexp;
    T.uoff = L.uoff; T.pairs = L.pairs; T.misc = L.misc;
    int32_t *idx_l = reinterpret_cast<int32_t *>(smem + L.idx);
    float *w_l = reinterpret_cast<float *>(smem + L.w);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(smem + L.ublob);
    const int *uexp = reinterpret_cast<const int *>(smem + L.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + L.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + L.pairs);
    const int nbx = H / 32;
    const BlobLayout BL = blob_layout(H, I, BITS);

    // ---- phase R: router logits and Q8_0(x)
    if (ROUTE) {
        for (int it = blockIdx.x * LW + wave; it < S * E; it += G * LW) {
            const int t = it / E, e = it - t * E;
            bool ok;
            const float p = logit_wave<MAXJ>(a.x + (size_t)t * H, l.router_w + (size_t)e * H, H, &ok);
            if (!ok) raise_status(a.status, ST_NONFINITE);
            if (lane == 0) st_dev(&l.logits[it], p);
        }
    }
    for (int j = blockIdx.x * (LT / 32) + (tid >> 5); j < S * nbx; j += G * (LT / 32)) {
        const int t = j / nbx, b = j - t * nbx;
        const int h = 32 * b + (tid & 31);
        const float v = a.x[(size_t)t * H + h];
        if (!finite_f32(v)) raise_status(a.status, ST_NONFINITE);
        float dd;
        const uint32_t c = (uint8_t)q8_0_lane(v, &dd);
        const uint32_t c1 = __shfl_down(c, 1, 64), c2 = __shfl_down(c, 2, 64), c3 = __shfl_down(c, 3, 64);
        if ((tid & 3) == 0)
            st_dev(reinterpret_cast<uint32_t *>(l.qx + (size_t)t * H + h), c | (c1 << 8) | (c2 << 16) | (c3 << 24));
        if ((tid & 31) == 0) st_dev(l.dx + (size_t)t * nbx + b, dd);
    }

    // ---- routing: the unit table (given routing: before the barrier)
    auto make_units = [&](const int32_t *idx, bool validate) {
        build_units(idx, S, K, E, a.n_shared, smem, T, a.status, validate);
        const int nu = reinterpret_cast<const int *>(smem + L.misc)[0];
        for (int u = tid; u < nu; u += LT) {
            const int e = uexp[u];
            ublob[u] = e < 0 ? a.shared : a.blobs[e];
        }
        __syncthreads();
    };
    if (!ROUTE) make_units(a.idx, blockIdx.x == 0);

    // first gate/up item of this workgroup: rows and their first chunk
    const int ntile = I / 32;
    const size_t hrow = (size_t)H * BITS / 8;
    const int half = wave & 1;
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    BlockBits<BITS> cur[ROWS_PER_WAVE];
    bool primed = false;
    auto rows1 = [&](int it, uint32_t rowoff[ROWS_PER_WAVE]) {
        const int i0 = (it % ntile) * 32;
#pragma unroll
        for (int j = 0; j < ROWS_PER_WAVE; ++j)
            rowoff[j] = (uint32_t)(mat + (size_t)(i0 + 16 * half + j) * hrow);
    };
    auto prime1 = [&](int n_units) {
        if ((int)blockIdx.x < n_units * ntile) {
            const uint8_t *blob = uniform_ptr(ublob[uniform(blockIdx.x / ntile)]);
            if (blob) {
                uint32_t rowoff[ROWS_PER_WAVE];
                rows1(blockIdx.x, rowoff);
                prime_rows<BITS, ROWS_PER_WAVE>(make_rsrc(blob, (uint32_t)BL.total), rowoff, nbx, cur);
                primed = true;
            }
        }
    };
    drain();
    if (!ROUTE) prime1(uniform(reinterpret_cast<const int *>(smem + L.misc)[0]));
    arrive_wait(&l.sync[0], G, a.status);   // logits and Q8_0(x) complete

    if (ROUTE) {
        float *sig_s = reinterpret_cast<float *>(smem + L.sig) + wave * E;
        float *selsig = reinterpret_cast<float *>(smem + L.selsig) + wave * 32;
        bool ok = true;
        for (int t = wave; t < S; t += LW) {
            float *lg = l.logits + (size_t)t * E;
            auto ld = [&](int e) { return ld_dev(lg + e); };
            ok = (E <= 256 ? select_wave<4>(ld, l.bias, E, K, l.rsf, l.norm, idx_l + t * K, w_l + t * K, sig_s, selsig)
                           : select_wave<16>(ld, l.bias, E, K, l.rsf, l.norm, idx_l + t * K, w_l + t * K, sig_s,
                                             selsig)) && ok;
        }
        if (!ok && lane == 0 && blockIdx.x == 0) raise_status(a.status, ST_NONFINITE);
        __syncthreads();
        if (blockIdx.x == 0)
            for (int q = tid; q < P; q += LT) {
                l.idx_out[q] = idx_l[q];
                l.w_out[q] = w_l[q];
            }
        make_units(idx_l, false);
        prime1(uniform(reinterpret_cast<const int *>(smem + L.misc)[0]));
    }
    const int n_units = uniform(reinterpret_cast<const int *>(smem + L.misc)[0]);
    const float *wts = ROUTE ? w_l : a.w;

    // ---- phase 1: gate/up items (unit, 32-row tile)
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * ROWS_PER_WAVE * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const int n_it1 = n_units * ntile;
    const int vds = vd_stride(nbx);
    const int crow = lane & 15, cvec = lane >> 4;
    const __amdgpu_buffer_rsrc_t qx_rs = make_rsrc(l.qx, (uint32_t)((size_t)S * H));
    for (int it = blockIdx.x; it < n_it1; it += G) {
        const int u = uniform(it / ntile);
        const uint8_t *blob = uniform_ptr(ublob[u]);
        if (!blob) {
            if (tid == 0) raise_status(a.status, ST_NOTRESIDENT);
            primed = false;
            continue;
        }
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
        uint32_t rowoff[ROWS_PER_WAVE];
        rows1(it, rowoff);
        const float *scale = reinterpret_cast<const float *>(blob + (wave < 2 ? BL.s_gate : BL.s_up));
        const int i0 = (it % ntile) * 32;
        const int p0 = uniform(uoff[u]), np = uniform(uoff[u + 1]) - p0;
        for (int g0 = 0; g0 < np; g0 += NT) {
            const int ng = min(NT, np - g0);
            if (!primed) prime_rows<BITS, ROWS_PER_WAVE>(rsrc, rowoff, nbx, cur);
            primed = false;
            auto stage = [&]() {
                for (int itk = 0; itk < ng; ++itk) {
                    const int v = pairs[p0 + g0 + itk];
                    const int t = v < P ? v / K : v - P;
                    u32x4 *dst = reinterpret_cast<u32x4 *>(vq + (size_t)itk * H);
                    for (int q = tid; q < H / 16; q += LT)
                        dst[q] = __builtin_amdgcn_raw_buffer_load_b128(qx_rs, (t * H) + 16 * q, 0, CPOL_SC1);
                    for (int q = tid; q < nbx; q += LT) vd[itk * vds + q] = ld_dev(l.dx + (size_t)t * nbx + q);
                }
                __syncthreads();
            };
            const float acc = stream_rows<BITS, NT, ROWS_PER_WAVE>(rsrc, rowoff, nbx, ng, vq, vd, isum_wave, H, stage, cur);
            if (cvec < ng) gu[cvec * 64 + wave * ROWS_PER_WAVE + crow] = acc * scale[i0 + 16 * half + crow];
            __syncthreads();
            // SwiGLU and Q8_0(h): half wave (tid >> 5) handles one vector's 32 rows.
            const int vv = tid >> 5, i = tid & 31;
            if (vv < ng) {
                const float h = swiglu_f32(gu[vv * 64 + i], gu[vv * 64 + 32 + i]);
                float d;
                const uint32_t c = (uint8_t)q8_0_lane(h, &d);
                const uint32_t c1 = __shfl_down(c, 1, 64), c2 = __shfl_down(c, 2, 64),
                               c3 = __shfl_down(c, 3, 64);
                const int slot = pairs[p0 + g0 + vv];
                if ((i & 3) == 0)
                    st_dev(reinterpret_cast<uint32_t *>(a.qh + (size_t)slot * I + i0 + i),
                           c | (c1 << 8) | (c2 << 16) | (c3 << 24));
                if (i == 0) st_dev(a.dh + (size_t)slot * ntile + i0 / 32, d);
            }
            __syncthreads();
        }
    }

    // ---- phase 2: two down rows per wave for every unit, then the combine
    constexpr int UB = DownBatch<BITS>::UB;
    const int nbi = I / 32;
    const int nch2 = (nbi + 63) / 64;
    const int vds2 = vd_stride(nbi);
    const size_t irow = (size_t)I * BITS / 8;
    const int slots = P + S * a.n_shared;
    const int mpb = slots < MAXPB ? slots : MAXPB;
    const int n_it2 = H / ROWS2;
    int8_t *qh_l = reinterpret_cast<int8_t *>(smem + L.qh);
    float *dh_l = reinterpret_cast<float *>(smem + L.dh);
    int32_t *isum2 = reinterpret_cast<int32_t *>(smem + L.isum2) + wave * RW2 * mpb * ISUM_PITCH;
    float *sdn = reinterpret_cast<float *>(smem + L.sdn);
    float *y_l = reinterpret_cast<float *>(smem + L.y);
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
    BlockBits<BITS> wv[UB][RW2];
    auto load_batch = [&](int rt, int u0, int u1, int c) {
        const int b = c * 64 + lane;
        const size_t ro = BL.down + (size_t)(rt * ROWS2 + wave * RW2) * irow;
#pragma unroll
        for (int ui = 0; ui < UB; ++ui) {
            if (u0 + ui < u1) {
                const uint8_t *blob = uniform_ptr(ublob[u0 + ui]);
                if (blob && b < nbi) {
#pragma unroll
                    for (int r = 0; r < RW2; ++r) wv[ui][r] = load_block_ptr<BITS>(blob + ro + r * irow, b);
                }
            }
        }
    };
    // down scales of this item's rows for every unit (LDS)
    auto load_scales = [&](int rt) {
        for (int q = tid; q < n_units * ROWS2; q += LT) {
            const int u = q / ROWS2, r = q - u * ROWS2;
            const uint8_t *blob = ublob[u];
            sdn[q] = blob ? reinterpret_cast<const float *>(blob + BL.s_down)[rt * ROWS2 + r] : 0.0f;
        }
    };
    drain();
    bool primed2 = false;
    if ((int)blockIdx.x < n_it2 && n_units > 0) {
        load_batch(blockIdx.x, 0, batch_end(0), 0);
        primed2 = true;
    }
    arrive_wait(&l.sync[1], G, a.status);   // Q8_0(h) complete
    const __amdgpu_buffer_rsrc_t qh_rs = make_rsrc(a.qh, (uint32_t)((size_t)slots * I));
    auto stage_pairs = [&](int pbase, int npb) {
        for (int pb = 0; pb < npb; ++pb) {
            const int sl = pairs[pbase + pb];
            u32x4 *dst = reinterpret_cast<u32x4 *>(qh_l + (size_t)pb * I);
            for (int q = tid; q < I / 16; q += LT)
                dst[q] = __builtin_amdgcn_raw_buffer_load_b128(qh_rs, sl * I + 16 * q, 0, CPOL_SC1);
            for (int q = tid; q < nbi; q += LT) dh_l[pb * vds2 + q] = ld_dev(a.dh + (size_t)sl * nbi + q);
        }
    };
    const bool one_batch = batch_end(0) == n_units;
    if (one_batch && (int)blockIdx.x < n_it2) stage_pairs(0, uniform(uoff[n_units]));
    for (int rt = blockIdx.x; rt < n_it2; rt += G) {
        const int r0 = rt * ROWS2;
        load_scales(rt);
        __syncthreads();
        for (int u0 = 0; u0 < n_units;) {
            const int u1 = batch_end(u0);
            const int pbase = uniform(uoff[u0]);
            const int npb = uniform(uoff[u1]) - pbase;
            if (!one_batch) {
                __syncthreads();
                stage_pairs(pbase, npb);
                __syncthreads();
            }
            const int cr = lane >> 5, cp = lane & 31;   // chain lane: (row, pair)
            float acc = 0.0f;
            for (int c = 0; c < nch2; ++c) {
                if (!primed2) load_batch(rt, u0, u1, c);
                primed2 = false;
                const int b = c * 64 + lane;
                const bool act = b < nbi;
#pragma unroll
                for (int ui = 0; ui < UB; ++ui) {
                    if (u0 + ui < u1) {
                        const bool live = ublob[u0 + ui] != nullptr;
                        const int q0 = uniform(uoff[u0 + ui]), q1 = uniform(uoff[u0 + ui + 1]);
                        for (int q = q0; q < q1; ++q) {
                            int32_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                            if (act) load_act(qh_l + (size_t)(q - pbase) * I, b, av);
#pragma unroll
                            for (int r = 0; r < RW2; ++r)
                                isum2[(r * mpb + (q - pbase)) * ISUM_PITCH + lane] =
                                    (act && live) ? block_dot(wv[ui][r], av) : 0;
                        }
                    }
                }
                wave_lds_sync();
                if (cp < npb)
                    acc = chain_chunk(acc, isum2 + (cr * mpb + cp) * ISUM_PITCH, dh_l + cp * vds2 + c * 64,
                                      min(64, nbi - c * 64));
                wave_lds_sync();
            }
            if (cp < npb) {
                int ub = u0;   // the pair's unit: the last one whose first pair is at or before it
                while (ub + 1 < u1 && uoff[ub + 1] <= pbase + cp) ++ub;
                const int slot = pairs[pbase + cp];
                const int rl = wave * RW2 + cr;
                y_l[slot * ROWS2 + rl] = ublob[ub] ? acc * sdn[ub * ROWS2 + rl] : 0.0f;
            }
            u0 = u1;
        }
        __syncthreads();
        for (int q = tid; q < S * ROWS2; q += LT) {
            const int t = q / ROWS2, rl = q - t * ROWS2;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const float wk = wts[t * K + k];
                if (!ROUTE && rt == 0 && rl == 0 && !finite_f32(wk)) raise_status(a.status, ST_NONFINITE);
                acc = __builtin_fmaf(wk, y_l[(t * K + k) * ROWS2 + rl], acc);
            }
            if (a.n_shared) acc = acc + y_l[(P + t) * ROWS2 + rl];
            a.out[(size_t)t * H + r0 + rl] = acc;
        }
        __syncthreads();
    }
    grid_exit(l.sync, 2, G);
}

// ---- launchers ----------------------------------------------------------
static int cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            cus = prop.multiProcessorCount;
        if (cus <= 0) cus = 1;
    }
    return cus;
}

// Workgroups of `kern` that fit on the GPU at once with `smem` bytes of LDS
// (cached per kernel and size).
static hipError_t resident_blocks(const void *kern, size_t smem, int *out) {
    static std::mutex mu;
    static std::map<std::pair<const void *, size_t>, int> cache;
    hipError_t e = ensure_dyn_smem(kern, smem);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({kern, smem});
    if (it != cache.end()) {
        *out = it->second;
        return hipSuccess;
    }
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, LT, smem);
    if (e != hipSuccess) return e;
    *out = per_cu * cu_count();
    cache[{kern, smem}] = *out;
    return hipSuccess;
}

static int pick_nt_layer(int S) { return S >= 4 ? 4 : (S >= 2 ? 2 : 1); }

size_t layer_smem(int S, int H, int I, int E, int K, int n_shared) {
    return layer_plan(S, K, E, n_shared, pick_nt_layer(S), H, I).total;
}

template <int BITS, int NT, bool ROUTE, int MAXJ>
static hipError_t layer_launch(const FwdArgs &a, const LayerArgs &l, hipStream_t st) {
    const size_t smem = layer_plan(a.S, a.K, a.E, a.n_shared, NT, a.H, a.I).total;
    int cap = 0;
    hipError_t e = resident_blocks(reinterpret_cast<const void *>(k_layer<BITS, NT, ROUTE, MAXJ>), smem, &cap);
    if (e != hipSuccess) return e;
    const int umax = std::min(a.S * a.K, a.E) + a.n_shared;
    const int want = std::max(umax * (a.I / 32), a.H / ROWS2);
    const int G = std::max(1, std::min(want, cap));
    return launch(k_layer<BITS, NT, ROUTE, MAXJ>, dim3(G), dim3(LT), smem, st, a, l);
}

template <int BITS, bool ROUTE>
static hipError_t layer_bits(const FwdArgs &a, const LayerArgs &l, hipStream_t st) {
    const bool short_rows = a.H <= 24 * 256;
    switch (pick_nt_layer(a.S)) {
        case 4: return short_rows ? layer_launch<BITS, 4, ROUTE, 24>(a, l, st) : layer_launch<BITS, 4, ROUTE, 16>(a, l, st);
        case 2: return short_rows ? layer_launch<BITS, 2, ROUTE, 24>(a, l, st) : layer_launch<BITS, 2, ROUTE, 16>(a, l, st);
        default: return short_rows ? layer_launch<BITS, 1, ROUTE, 24>(a, l, st) : layer_launch<BITS, 1, ROUTE, 16>(a, l, st);
    }
}

hipError_t launch_layer(const FwdArgs &a, const LayerArgs &l, bool route, int bits, hipStream_t st) {
    if (route) {
        if (bits == 8) return layer_bits<8, true>(a, l, st);
        if (bits == 4) return layer_bits<4, true>(a, l, st);
        return layer_bits<2, true>(a, l, st);
    }
    if (bits == 8) return layer_bits<8, false>(a, l, st);
    if (bits == 4) return layer_bits<4, false>(a, l, st);
    return layer_bits<2, false>(a, l, st);
}

}  // namespace coli
