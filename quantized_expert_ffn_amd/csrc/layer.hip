// Persistent single-launch MoE layer for decode and speculative-verify
// batches (colibrì README v1.0, "What's implemented": DeepSeek-V3-style
// sigmoid router, SwiGLU experts on Q8_0 activations, shared expert,
// batch-union MoE; "Colibri (colibrì): GLM-5.2 local inference on 25 GB of
// RAM", "How it works (validated core mechanics)": the router).
//
// One launch runs the layer's phases; grid barriers replace kernel
// boundaries, and every workgroup's work is laid out so that each phase's
// memory traffic starts as early as its inputs allow:
//   R  router logits, one wavefront each, on the highest-numbered
//      workgroups (those with no gate/up item), published with device-scope
//      stores; every workgroup with a possible gate/up item quantises x
//      (Q8_0) into its own LDS;
//   -- barrier A: the logits --
//      routing: every workgroup selects the top-K of every token itself (the
//      same bits everywhere, at raised wave priority) and builds the unit
//      table of the batch union;
//   1  gate/up items (unit, 32-row tile), shared expert first: its
//      workgroups stream before barrier A, since its pairs do not depend on
//      the routing; 4 waves x 16 rows, SwiGLU and Q8_0(h) in the epilogue,
//      published with device-scope stores;
//      each workgroup then issues the weight loads of its down tile;
//   -- barrier B: Q8_0(h) --
//   2  down tiles of 8 output rows for every unit, combined in the
//      workgroup (one writer per output element).
// A workgroup drains its stores (s_waitcnt) before it arrives at a barrier;
// arrivals are agent-scope releases and the waits end in agent-scope acquires.
// Barrier waits are bounded: a grid that could not be fully resident ends
// with a status error, never a hang; the host sizes the grid from the
// kernel's occupancy.
#include <algorithm>
#include <map>
#include <mutex>

#include "device_common.h"
#include "down_rows.h"
#include "kernels.h"
#include "router.h"
#include "stream.h"

namespace coli {

constexpr uint32_t SPIN_LIMIT = 1u << 22;
constexpr int LT = 256;         // threads per workgroup
constexpr int LW = LT / 64;     // waves per workgroup
constexpr int LMAXJ = 12;       // router row steps loaded per round

// Barriers: an arrival counter per barrier, and a release flag per
// workgroup that the last arrival sets.  Each waiting workgroup polls its
// own word: when hundreds of workgroups poll one word, the requests queue at
// that word's memory channel and slow every other access to the channel.
__device__ __forceinline__ uint32_t *flag_word(uint8_t *flags, int k, int copy) {
    return reinterpret_cast<uint32_t *>(flags + ((size_t)k * FLAG_COPIES + copy) * FLAG_STRIDE);
}

// Releases flag k of every workgroup (all lanes of the calling wave, which
// has acquired every arrival).
__device__ __forceinline__ void release(uint8_t *flags, int k) {
    const int lane = threadIdx.x & 63;
    fence_release_agent();
    for (int c = lane; c < (int)gridDim.x; c += 64) st_dev(flag_word(flags, k, c), 1u);
}

// Counts one arrival of the calling wave at counter k (a release of its
// workgroup's drained stores); the arrival that completes `target`
// acquires the others and releases flag k.
__device__ __forceinline__ void signal(uint32_t *sync, uint8_t *flags, int k, uint32_t target) {
    uint32_t prev = 0;
    fence_release_agent();
    if ((threadIdx.x & 63) == 0)
        prev = __hip_atomic_fetch_add(&sync[k], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(prev) == target - 1) {
        fence_acquire_agent();
        release(flags, k);
    }
}

// Workgroup arrival at barrier k (callers drain() their stores first).
__device__ __forceinline__ void arrive(uint32_t *sync, uint8_t *flags, int k, uint32_t nwg) {
    __syncthreads();
    if (threadIdx.x < 64) signal(sync, flags, k, nwg);
}

// Waits (bounded) until this workgroup's flag k is released.
__device__ __forceinline__ void wait_flag(uint8_t *flags, int k, uint32_t *status) {
    if (threadIdx.x == 0) {
        uint32_t *f = flag_word(flags, k, blockIdx.x);
        uint32_t spins = 0;
        while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins >= SPIN_LIMIT) {
                raise_status(status, ST_TIMEOUT);
                break;
            }
        }
        fence_acquire_agent();
    }
    __syncthreads();
}

// The last workgroup to leave resets the counters and flags for the next
// launch (counter `nbar` counts the departures).
__device__ __forceinline__ void grid_exit(uint32_t *sync, uint8_t *flags, int nbar, uint32_t nwg) {
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        fence_release_agent();
        last = __hip_atomic_fetch_add(&sync[nbar], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nwg - 1;
        if (last) fence_acquire_agent();
    }
    __syncthreads();
    if (last) {
        for (int c = threadIdx.x; c < N_FLAGS * (int)nwg; c += blockDim.x)
            st_dev(flag_word(flags, c / (int)nwg, c % (int)nwg), 0u);
        if ((int)threadIdx.x <= nbar) st_dev(&sync[threadIdx.x], 0u);
    }
}

struct LayerPlan {
    SmemPlan T;                   // unit table
    size_t idx, w, ublob;         // routing [P], weights [P], unit blob pointers [umax]
    size_t xq, xd;                // Q8_0(x) of every token: codes [S][H], scales [S][vds]
    size_t vq, vd;                // group staging when NT > 1
    size_t isum, gu;              // block dots per wave, gate/up results
    DownTilePlan tile;            // phase 2 (over the phase-1 region)
    size_t total;
};

__host__ __device__ inline LayerPlan layer_plan(int S, int K, int E, int n_shared, int NT, int H, int I) {
    LayerPlan p;
    const int P = S * K;
    const int umax = (P < E ? P : E) + 1;
    const int vds = vd_stride(H / 32);
    p.T = smem_plan(S, K, E, 0, 0);
    p.idx = a16(p.T.total);
    p.w = a16(p.idx + 4 * (size_t)P);
    p.ublob = a16(p.w + 4 * (size_t)P);
    const size_t base = a16(p.ublob + 8 * (size_t)umax);
    p.xq = base;
    p.xd = a16(p.xq + (size_t)S * H);
    p.vq = a16(p.xd + 4 * (size_t)S * vds);
    p.vd = a16(p.vq + (NT > 1 ? (size_t)NT * H : 0));
    p.isum = a16(p.vd + (NT > 1 ? 4 * (size_t)NT * vds : 0));
    p.gu = a16(p.isum + 4 * (size_t)LW * NT * ROWS_PER_WAVE * ISUM_PITCH);
    const size_t end1 = a16(p.gu + 4 * (size_t)NT * 64);
    p.tile = down_tile_plan(base, S, K, E, n_shared, I);
    p.total = end1 > p.tile.end ? end1 : p.tile.end;
    return p;
}

// ONE_PASS: the grid has a workgroup for every gate/up item and every down
// tile, so each workgroup takes at most one of each (straight-line code,
// which keeps the register count low enough for 3 workgroups per CU).
// FAST: one token, and the grid has a workgroup for every gate/up item and
// every down tile, with the tile's units in a single batch (the host checks
// the worst case): straight-line code with only the decode path in it, so
// that the kernel's code stays small in the instruction cache and its
// register count allows 3 workgroups per CU.  MAXM: router selection width
// (E <= 64 * MAXM).
template <int BITS, int NT, bool ROUTE, bool FAST, int MAXM>
__global__ __launch_bounds__(LT) void k_layer(const FwdArgs a, const LayerArgs l) {
    static_assert(!FAST || NT == 1, "FAST is the one-token path");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.S, K = a.K, E = a.E, H = a.H, I = a.I, P = S * K;
    const int G = gridDim.x, wg = blockIdx.x;
    const LayerPlan L = layer_plan(S, K, E, a.n_shared, NT, H, I);
    const int nbx = H / 32, vds = vd_stride(nbx), ntile = I / 32;
    const int umax = min(P, E) + a.n_shared;
    const int n_it1_max = umax * ntile;
    const int n_q8 = (S * nbx + 63) / 64;   // Q8_0(x) wavefront items
    int32_t *idx_l = reinterpret_cast<int32_t *>(smem + L.idx);
    float *w_l = reinterpret_cast<float *>(smem + L.w);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(smem + L.ublob);
    const int *uexp = reinterpret_cast<const int *>(smem + L.T.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + L.T.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + L.T.pairs);
    const int *misc = reinterpret_cast<const int *>(smem + L.T.misc);
    int8_t *xq = reinterpret_cast<int8_t *>(smem + L.xq);
    float *xd = reinterpret_cast<float *>(smem + L.xd);

    // ---- phase R, on wavefronts counted from the last workgroup down: the
    // router logits (with routing computed here), then Q8_0(x) in items of
    // 64 blocks (one per lane), published with device-scope stores and
    // counted in sync[2]
    {
        const int n_lg = ROUTE ? S * E : 0;
        for (int i = (G - 1 - wg) * LW + wave; i < n_lg + n_q8; i += G * LW) {
            if (i < n_lg) {
                const int t = i / E, e = i - t * E;
                bool ok;
                const float p = logit_wave<LMAXJ>(a.x + (size_t)t * H, l.router_w + (size_t)e * H, H, &ok);
                if (!ok) raise_status(a.status, ST_NONFINITE);
                if (lane == 0) st_dev(&l.logits[i], p);
            } else {
                const int j = (i - n_lg) * 64 + lane;
                if (j < S * nbx) {
                    const int t = j / nbx, b = j - t * nbx;
                    bool ok;
                    uint32_t w[8];
                    const float d = q8_0_block_words(a.x + (size_t)t * H + 32 * b, w, &ok);
                    if (!ok) raise_status(a.status, ST_NONFINITE);
                    uint32_t *q = reinterpret_cast<uint32_t *>(l.qx + (size_t)t * H + 32 * b);
#pragma unroll
                    for (int k = 0; k < 8; ++k) st_dev(q + k, w[k]);
                    st_dev(l.dx + (size_t)t * nbx + b, d);
                }
                drain();
                signal(l.sync, l.flags, 2, (uint32_t)n_q8);
            }
        }
    }
    // unit blob pointers; with given routing, the unit table now
    auto fill_blobs = [&]() {
        const int nu = misc[0];
        for (int u = tid; u < nu; u += LT) {
            const int e = uexp[u];
            ublob[u] = e < 0 ? a.shared : a.blobs[e];
        }
        __syncthreads();
    };
    if (!ROUTE) {
        build_units(a.idx, S, K, E, a.n_shared, smem, L.T, a.status, wg == 0);
        fill_blobs();
    }
    drain();
    if (ROUTE) arrive(l.sync, l.flags, 0, G);

    // Q8_0(x) of every token into LDS, once it is published (device-scope
    // loads; the codes come in 16-byte pieces)
    auto load_x = [&]() {
        wait_flag(l.flags, 2, a.status);   // Q8_0(x) published
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(l.qx, (uint32_t)((size_t)S * H));
        for (int q = tid; q < S * H / 16; q += LT)
            reinterpret_cast<u32x4 *>(xq)[q] = __builtin_amdgcn_raw_buffer_load_b128(qrs, 16 * q, 0, CPOL_SC1);
        for (int j = tid; j < S * nbx; j += LT) {
            const int t = j / nbx, b = j - t * nbx;
            xd[t * vds + b] = ld_dev(l.dx + j);
        }
        __syncthreads();
    };
    auto route = [&]() {
        wait_flag(l.flags, 0, a.status);   // every logit published
        __builtin_amdgcn_s_setprio(2);
        bool ok = true;
        for (int t = wave; t < S; t += LW) {
            const float *lg = l.logits + (size_t)t * E;
            auto ld = [&](int e) { return ld_dev(lg + e); };
            int32_t si;
            float sw;
            ok = select_wave<MAXM>(ld, l.bias, E, K, l.rsf, l.norm, &si, &sw) && ok;
            if (lane < K) {
                idx_l[t * K + lane] = si;
                w_l[t * K + lane] = sw;
            }
        }
        if (!ok && lane == 0 && wg == 0) raise_status(a.status, ST_NONFINITE);
        __syncthreads();
        if (wg == 0)
            for (int q = tid; q < P; q += LT) {
                l.idx_out[q] = idx_l[q];
                l.w_out[q] = w_l[q];
            }
        build_units(idx_l, S, K, E, a.n_shared, smem, L.T, a.status, false);
        fill_blobs();
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- phase 1: gate/up items (unit, 32-row tile); item order puts the
    // shared expert first, then the routed units in table order
    const size_t hrow = (size_t)H * BITS / 8;
    const int half = wave & 1;
    const BlobLayout BL = blob_layout(H, I, BITS);
    const size_t mat = wave < 2 ? BL.gate : BL.up;
    int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
    float *vd = reinterpret_cast<float *>(smem + L.vd);
    int32_t *isum_wave = reinterpret_cast<int32_t *>(smem + L.isum) + wave * NT * ROWS_PER_WAVE * ISUM_PITCH;
    float *gu = reinterpret_cast<float *>(smem + L.gu);
    const int crow = lane & 15, cvec = lane >> 4;
    auto item = [&](int it, bool shared_item) {
        const int uo = it / ntile, i0 = (it - uo * ntile) * 32;
        const int ut = shared_item ? -1 : uo - a.n_shared;   // routed unit (table order)
        const uint8_t *blob = uniform_ptr(shared_item ? a.shared : ublob[ut]);
        if (!blob) {
            // a call with a non-resident expert fails as a whole (status word)
            if (tid == 0) raise_status(a.status, ST_NOTRESIDENT);
            return false;
        }
        const int p0 = shared_item ? 0 : uniform(uoff[ut]);
        const int np = shared_item ? S : uniform(uoff[ut + 1]) - p0;
        auto pair_at = [&](int i) { return shared_item ? P + i : pairs[p0 + i]; };
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, (uint32_t)BL.total);
        uint32_t rowoff[ROWS_PER_WAVE];
#pragma unroll
        for (int j = 0; j < ROWS_PER_WAVE; ++j) rowoff[j] = (uint32_t)(mat + (size_t)(i0 + 16 * half + j) * hrow);
        const float *scale = reinterpret_cast<const float *>(blob + (wave < 2 ? BL.s_gate : BL.s_up));
        for (int g0 = 0; g0 < np; g0 += NT) {
            const int ng = min(NT, np - g0);
            const int8_t *gq = vq;
            const float *gd = vd;
            if (NT == 1) {
                const int v = pair_at(g0);
                const int t = v < P ? v / K : v - P;
                gq = xq + (size_t)t * H;
                gd = xd + t * vds;
            }
            auto stage = [&]() {
                if (NT > 1) {
                    // this group's tokens, copied from the per-token Q8_0(x) in LDS
                    for (int itk = 0; itk < ng; ++itk) {
                        const int v = pair_at(g0 + itk);
                        const int t = v < P ? v / K : v - P;
                        const i32x4 *src = reinterpret_cast<const i32x4 *>(xq + (size_t)t * H);
                        i32x4 *dst = reinterpret_cast<i32x4 *>(vq + (size_t)itk * H);
                        for (int q = tid; q < H / 16; q += LT) dst[q] = src[q];
                        for (int q = tid; q < nbx; q += LT) vd[itk * vds + q] = xd[t * vds + q];
                    }
                    __syncthreads();
                }
            };
            BlockBits<BITS> cur[ROWS_PER_WAVE];
            prime_rows<BITS, ROWS_PER_WAVE>(rsrc, rowoff, nbx, cur);
            const float acc = stream_rows<BITS, NT, ROWS_PER_WAVE>(rsrc, rowoff, nbx, ng, gq, gd, isum_wave, H, stage, cur);
            if (cvec < ng) gu[cvec * 64 + wave * ROWS_PER_WAVE + crow] = acc * scale[i0 + 16 * half + crow];
            __syncthreads();
            // SwiGLU and Q8_0(h): half wave (tid >> 5) handles one vector's 32 rows
            const int vv = tid >> 5, i = tid & 31;
            if (vv < ng) {
                const float h = swiglu_f32(gu[vv * 64 + i], gu[vv * 64 + 32 + i]);
                float d;
                const uint32_t c = (uint8_t)q8_0_lane(h, &d);
                const uint32_t c1 = __shfl_down(c, 1, 64), c2 = __shfl_down(c, 2, 64), c3 = __shfl_down(c, 3, 64);
                const int slot = pair_at(g0 + vv);
                if ((i & 3) == 0)
                    st_dev(reinterpret_cast<uint32_t *>(a.qh + (size_t)slot * I + i0 + i),
                           c | (c1 << 8) | (c2 << 16) | (c3 << 24));
                if (i == 0) st_dev(a.dh + (size_t)slot * ntile + i0 / 32, d);
            }
            __syncthreads();
        }
        return true;
    };

    const bool first_shared = a.n_shared && wg < ntile;   // this workgroup's first item is the shared expert's
    if (FAST) {
        // at most one item per workgroup; the shared expert's workgroups
        // stream it before routing, the others route first (one call site
        // for the item keeps the code small)
        if (ROUTE && !first_shared) route();
        if (first_shared || (wg < n_it1_max && wg < uniform(misc[0]) * ntile)) {
            load_x();
            item(wg, first_shared);
        }
        if (ROUTE && first_shared) route();
    } else {
        bool routed = !ROUTE, have_x = false;
        for (int it = wg; it < n_it1_max; it += G) {
            const bool shared_item = a.n_shared && it < ntile;
            if (!shared_item && !routed) {
                route();
                routed = true;
            }
            if (routed && it >= uniform(misc[0]) * ntile) break;
            if (!have_x) {
                load_x();
                have_x = true;
            }
            if (!item(it, shared_item)) break;
        }
        if (!routed) route();
    }

    // ---- phase 2: down tiles
    drain();
    const int n_units = uniform(misc[0]);
    const int n_tiles = H / DR_ROWS;
    const float *wts = ROUTE ? w_l : a.w;
    if (FAST) {
        // the tile's weights are issued before the barrier
        DownTile<BITS, true, true> tile(a, smem, L.tile, uoff, pairs, ublob, wts, n_units, wg);
        if (wg < n_tiles) tile.issue(0, n_units, 0);
        arrive(l.sync, l.flags, 1, G);
        wait_flag(l.flags, 1, a.status);   // every Q8_0(h) published
        if (wg < n_tiles) tile.run(true);
    } else {
        arrive(l.sync, l.flags, 1, G);
        wait_flag(l.flags, 1, a.status);
        for (int rt = wg; rt < n_tiles; rt += G) {
            DownTile<BITS, NT == 1, true> tile(a, smem, L.tile, uoff, pairs, ublob, wts, n_units, rt);
            tile.run(false);
        }
    }
    grid_exit(l.sync, l.flags, 3, G);
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

// Whether the one-token fast instantiation covers a call: every gate/up item
// and down tile gets its own workgroup, and the down tile's units fit one
// batch in the worst case.
static bool layer_fast(const FwdArgs &a, int cap) {
    const int umax = std::min(a.S * a.K, a.E) + a.n_shared;
    const int slots = a.S * a.K + a.S * a.n_shared;
    const int want = std::max(umax * (a.I / 32), a.H / DR_ROWS);
    return a.S == 1 && want <= cap && a.I <= 2048 && slots <= DR_MAXPB &&
           slots * (a.I / 16) <= DR_MQ * DR_T && slots * (a.I / 32) <= DR_MD * DR_T;
}

template <int BITS, int NT, bool ROUTE, bool FAST, int MAXM>
static hipError_t layer_go(const FwdArgs &a, const LayerArgs &l, size_t smem, int G, hipStream_t st) {
    const void *kern = reinterpret_cast<const void *>(k_layer<BITS, NT, ROUTE, FAST, MAXM>);
    const hipError_t e = ensure_dyn_smem(kern, smem);
    if (e != hipSuccess) return e;
    return launch(k_layer<BITS, NT, ROUTE, FAST, MAXM>, dim3(G), dim3(LT), smem, st, a, l);
}

template <int BITS, int NT, bool ROUTE>
static hipError_t layer_launch(const FwdArgs &a, const LayerArgs &l, hipStream_t st) {
    const size_t smem = layer_plan(a.S, a.K, a.E, a.n_shared, NT, a.H, a.I).total;
    const int umax = std::min(a.S * a.K, a.E) + a.n_shared;
    const int want = std::max(umax * (a.I / 32), a.H / DR_ROWS);
    int cap = 0;
    const auto fits = [](int c) { return std::min(c, FLAG_COPIES); };   // one release flag per workgroup
    if (NT == 1) {
        hipError_t e = resident_blocks(reinterpret_cast<const void *>(k_layer<BITS, 1, ROUTE, true, 4>), smem, &cap);
        if (e != hipSuccess) return e;
        cap = fits(cap);
        if (DownRowsBatch<BITS>::UB >= umax && layer_fast(a, cap)) {
            if (a.E <= 256) return layer_go<BITS, 1, ROUTE, true, 4>(a, l, smem, want, st);
            return layer_go<BITS, 1, ROUTE, true, 16>(a, l, smem, want, st);
        }
    }
    hipError_t e = resident_blocks(reinterpret_cast<const void *>(k_layer<BITS, NT, ROUTE, false, 16>), smem, &cap);
    if (e != hipSuccess) return e;
    cap = fits(cap);
    return layer_go<BITS, NT, ROUTE, false, 16>(a, l, smem, std::max(1, std::min(want, cap)), st);
}

template <int BITS, bool ROUTE>
static hipError_t layer_bits(const FwdArgs &a, const LayerArgs &l, hipStream_t st) {
    switch (pick_nt_layer(a.S)) {
        case 4: return layer_launch<BITS, 4, ROUTE>(a, l, st);
        case 2: return layer_launch<BITS, 2, ROUTE>(a, l, st);
        default: return layer_launch<BITS, 1, ROUTE>(a, l, st);
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
