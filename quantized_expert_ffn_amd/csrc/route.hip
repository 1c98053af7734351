// Router kernels: logits and selection as two launches (coli_moe_route), or
// one launch that also selects and builds the unit table of the call
// (coli_moe_layer, up to ROUTE_FUSE_MAX tokens).  The device routines are
// in router.h.
#include <type_traits>

#include "device_common.h"
#include "gateup.h"
#include "kernels.h"
#include "router.h"
#include "stream.h"

namespace coli {

// Q8_0 of the hidden states, one 32-value block per lane (blocks
// 64 * qblk + lane of token t).
__device__ __forceinline__ void quant_x_wave(const float *__restrict__ x, int8_t *__restrict__ qx,
                                             float *__restrict__ dx, uint32_t *__restrict__ status,
                                             int H, int t, int qblk) {
    const int nbx = H / 32;
    const int b = qblk * 64 + (int)(threadIdx.x & 63);
    if (b < nbx) {
        bool ok;
        const float d = q8_0_block_lane(x + (size_t)t * H + 32 * b, qx + (size_t)t * H + 32 * b, &ok);
        dx[(size_t)t * nbx + b] = d;
        if (!ok && status) raise_status(status, ST_NONFINITE);
    }
}

// One wavefront per (token, expert); with qx, the workgroups past the E
// experts quantise the token's hidden state (64 blocks each).
// Grid: (E + ceil(H / 2048) if qx else E, S), 64 threads.
template <int MAXJ>
__global__ __launch_bounds__(64) void k_router_logits(const float *__restrict__ x,
                                                      const float *__restrict__ W,
                                                      float *__restrict__ logits,
                                                      uint32_t *__restrict__ status, int H,
                                                      int E, int8_t *__restrict__ qx,
                                                      float *__restrict__ dx) {
    const int e = blockIdx.x;
    const int t = blockIdx.y;
    if (e >= E) {
        quant_x_wave(x, qx, dx, status, H, t, e - E);
        return;
    }
    bool ok;
    const float p = logit_wave<MAXJ>(x + (size_t)t * H, W + (size_t)e * H, H, &ok);
    if (status && !ok) raise_status(status, ST_NONFINITE);
    if (threadIdx.x == 0) logits[(size_t)t * E + e] = p;
}

// One wavefront per token.
template <int MAXM>
__global__ __launch_bounds__(64) void k_router_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias,
                                                      int32_t *__restrict__ idx_out,
                                                      float *__restrict__ w_out,
                                                      uint32_t *__restrict__ status, int E, int K,
                                                      float rsf, int norm) {
    const int t = blockIdx.x, lane = threadIdx.x;
    const float *lg = logits + (size_t)t * E;
    int32_t si;
    float sw;
    const bool ok = select_wave<MAXM>([&](int e) { return lg[e]; }, bias, E, K, rsf, norm, &si, &sw);
    if (lane < K) {
        idx_out[(size_t)t * K + lane] = si;
        w_out[(size_t)t * K + lane] = sw;
    }
    if (!ok && lane == 0) raise_status(status, ST_NONFINITE);
}

// The fused router launch.  Grid (ceil(E / L) [+ ceil(ceil(H / 2048) / RF_W)
// with qx], S), RF_W wavefronts per workgroup, L = rf_lpw(S) logits per
// workgroup.  Wave w < L of workgroup (x < ceil(E / L), t) computes logit
// (t, L x + w).  Up to four tokens with at most 256 experts (route_one,
// route_few), each logit is published as a tagged 64-bit slot and one
// workgroup, which waits (bounded) for every slot, selects and writes the
// unit table.  Otherwise each logit goes out with a device-scope store and,
// once all of its waves have drained their stores, the workgroup counts
// itself in the token's arrival counter (one atomic per workgroup); in the
// workgroup that arrives last, wave 0 selects the token's top-K from the
// published logits (device-scope loads), the token counts itself done and
// the last token's workgroup builds the unit table of the batch in LDS.
// Each counter is reset by its last arriver, so the next launch starts from
// zero.  Workgroups past the logits quantise x (one 2048-element slice per
// wave).
//
// With sg, the first I / 16 workgroups of grid row 0 (ahead of the logits,
// being the longest) run the shared expert's gate/up for all S tokens in
// half tiles of 16 rows — its pairs do not depend on the routing —
// quantising x into their own LDS with the same Q8_0 as the workspace copy,
// and write h unquantised to hs; the gate/up launch quantises it and skips
// the shared expert.
constexpr int RF_W = 4;
// logits per workgroup: one per wave, at every batch size
__host__ __device__ inline int rf_lpw(int) { return RF_W; }

// Shared expert, gate/up rows 16 half .. 16 half + 15, every token; h to hs.
template <int BITS, int NT, bool GROUPED, bool MX = false>
__device__ __forceinline__ void shared_gateup_half(const RouteArgs &r, uint8_t *smem, int half) {
    const int tid = threadIdx.x, S = r.S, H = r.H;
    const SmemPlan L = smem_plan(S, r.K, r.E, NT, H);
    const int nb = H / 32, vds = vd_stride(nb);
    auto stage = [&](int g0, int ng) {
        int8_t *vq = reinterpret_cast<int8_t *>(smem + L.vq);
        float *vd = reinterpret_cast<float *>(smem + L.vd);
        for (int j = tid; j < ng * nb; j += blockDim.x) {
            const int it = j / nb, b = j - it * nb;
            bool ok;
            vd[it * vds + b] = q8_0_block_lane(r.x + (size_t)(g0 + it) * H + 32 * b, vq + (size_t)it * H + 32 * b, &ok);
        }
        __syncthreads();
    };
    if constexpr ((BITS == 4 || BITS == 2) && !GROUPED && !MX) {
        const int nch = (nb + 63) / 64;
        if (S <= NT && nch <= 4) {
            auto go = [&](auto nch_c) {
                gateup_half_primed<BITS, NT, decltype(nch_c)::value>(uniform_ptr(r.shared), H, r.I, 16 * half, S,
                                                                     smem, L, r.x, r.hs);
            };
            if (nch == 1)
                go(std::integral_constant<int, 1>());
            else if (nch == 2)
                go(std::integral_constant<int, 2>());
            else if (nch == 3)
                go(std::integral_constant<int, 3>());
            else
                go(std::integral_constant<int, 4>());
            return;
        }
    }
    gateup_half_f32<BITS, NT, GROUPED, MX>(uniform_ptr(r.shared), H, r.I, r.group, 16 * half, S, smem, L, L.total, r.hs,
                                       stage);
}

// The logit workgroups of a one-token launch with at most 256 experts
// ("Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM", "How it
// works (validated core mechanics)": sigmoid scores, the bias ranks only,
// lower id wins a tie, the weights are the unbiased sigmoids renormalised).
// Wave w < lpw of logit workgroup bx computes logit lpw bx + w and publishes
// it as one 64-bit word (tag << 32) | bits, the tag being the workspace's
// epoch + 1, so that no arrival counter is needed.  Logit workgroup 0 then
// selects.  Thread e waits (bounded) until slot e carries the tag and forms
// expert e's sort key (order-preserving key of its score) << 32 | ~e, which
// orders the experts as the selection does (score desc, id asc) with no two
// equal.  The top-K come from ranks: each thread counts the keys of its own
// wavefront above its own (the wavefront's K best are candidates, 4 K in
// all), then each candidate counts the candidates above it; the K
// candidates of rank < K are the selection, in rank order.  It writes idx /
// w (weights: (sig_k / ((sig_0 + sig_1) + ...)) * rsf, or sig_k * rsf), the
// unit table (unit j: the selected expert of the j-th smallest id, its pair
// slot its rank; then the shared expert) and the next epoch.  On a
// non-finite input or weight sum, or a wait that gave up, the table holds
// the shared expert alone.
template <int MAXJ>
__device__ __forceinline__ void route_one(const RouteArgs &r, int bx, int lpw) {
    __shared__ __attribute__((aligned(16))) uint64_t s_key[256];
    __shared__ __attribute__((aligned(16))) uint64_t s_ck[4 * 32];
    __shared__ int32_t s_cid[4 * 32];
    __shared__ float s_sig[256];
    __shared__ int32_t s_sel[32];
    __shared__ const uint8_t *s_blob[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = r.E, K = r.K, H = r.H;
    const uint32_t tag = ld_dev(r.epoch) + 1u;
    const bool selector = bx == 0;
    // the selector's inputs besides the logits, fetched ahead of them
    float my_bias = 0.0f;
    const uint8_t *my_blob = nullptr;
    if (selector && tid < E) {
        if (r.bias) my_bias = r.bias[tid];
        my_blob = r.blobs[tid];
    }
    const int e = bx * lpw + wave;
    if (wave < lpw && e < E) {
        bool ok;
        const float p = logit_wave<MAXJ>(r.x, r.W + (size_t)e * H, H, &ok);
        if (!ok) raise_status(r.status, ST_NONFINITE);
        if (lane == 0) st_dev64(&r.slots[e], ((uint64_t)tag << 32) | __float_as_uint(p));
    }
    if (!selector) return;
    bool late = false;
    float lg = 0.0f;
    const bool valid = tid < E;
    if (valid) {
        const uint32_t want = tag + r.tag_skew;
        uint32_t spins = 0;
        uint64_t v = ld_dev64(&r.slots[tid]);
        while ((uint32_t)(v >> 32) != want) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins >= r.spin_limit) {
                late = true;
                break;
            }
            v = ld_dev64(&r.slots[tid]);
        }
        lg = __uint_as_float((uint32_t)v);
    }
    const float sig = sigmoid_f32(lg);
    const float score = sig + my_bias;
    const bool finite_in = !valid || (finite_f32(lg) && finite_f32(my_bias));
    // the score part is 0 for a missing expert and for a score not above
    // -inf (NaN included); the id part keeps every key distinct and puts the
    // missing experts (ids E and up) last
    const uint32_t sk = valid && score > -__builtin_inff() ? f32_key(score) : 0u;
    const uint64_t key = ((uint64_t)sk << 32) | (uint32_t)~(uint32_t)tid;
    s_key[tid] = key;
    s_sig[tid] = sig;
    s_blob[tid] = my_blob;
    const int bad_in = __syncthreads_or(!finite_in);
    const int timed_out = __syncthreads_or(late);
    // rank within the wavefront: the wavefront's 64 keys read two per LDS
    // access, every read of a half issued before its compares (the ranking
    // is a chain of LDS latencies otherwise)
    auto key_lo = [](u32x4 v) { return ((uint64_t)v.y << 32) | v.x; };
    auto key_hi = [](u32x4 v) { return ((uint64_t)v.w << 32) | v.z; };
    int c1 = 0;
    const u32x4 *wk = reinterpret_cast<const u32x4 *>(s_key + wave * 64);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u32x4 kv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) kv[j] = wk[16 * h + j];
#pragma unroll
        for (int j = 0; j < 16; ++j) c1 += (key_lo(kv[j]) > key ? 1 : 0) + (key_hi(kv[j]) > key ? 1 : 0);
    }
    if (c1 < K) {
        s_ck[wave * K + c1] = key;
        s_cid[wave * K + c1] = tid;
    }
    __syncthreads();
    // each of the 4 K candidates against the others, two per LDS access
    if (tid < 4 * K) {
        int c2 = 0;
        const uint64_t ck = s_ck[tid];
        const u32x4 *cv = reinterpret_cast<const u32x4 *>(s_ck);
#pragma unroll 8
        for (int j = 0; j < 2 * K; ++j) {
            const u32x4 v = cv[j];
            c2 += (key_lo(v) > ck ? 1 : 0) + (key_hi(v) > ck ? 1 : 0);
        }
        if (c2 < K) s_sel[c2] = s_cid[tid];
    }
    __syncthreads();
    if (wave != 0) return;
    const int32_t si = lane < K ? s_sel[lane] : 0;
    const float ssig = lane < K ? s_sig[si] : 0.0f;
    float denom = 1.0f;
    bool wok = true;
    if (r.norm) {
        denom = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssig), 0));
        for (int k = 1; k < K; ++k) denom = denom + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssig), k));
        wok = denom > 0.0f && finite_f32(denom);
    }
    const float sw = r.norm ? (ssig / denom) * r.rsf : ssig * r.rsf;
    const UnitTable U = unit_table(1, K, E);
    int32_t *tab = reinterpret_cast<int32_t *>(r.units);
    const uint8_t **ublob = reinterpret_cast<const uint8_t **>(r.units + U.ublob);
    if (lane < K) {
        r.idx_out[lane] = si;
        r.w_out[lane] = sw;
    }
    const bool good = !bad_in && !timed_out && wok;
    int u = 0;   // position of si among the selected ids, ascending
    for (int j = 0; j < K; ++j) u += __builtin_amdgcn_readlane(si, j) < si ? 1 : 0;
    if (good && lane < K) {
        tab[U.uexp + u] = si;
        tab[U.uoff + u] = u;
        tab[U.pairs + u] = lane;
        ublob[u] = s_blob[si];
    }
    if (lane == 0) {
        const int ns = r.n_shared;
        if (!good) raise_status(r.status, timed_out ? ST_TIMEOUT : ST_NONFINITE);
        const int nr = good ? K : 0;   // routed units
        tab[0] = nr + ns;
        tab[1] = nr;
        tab[2] = nr;
        tab[3] = 0;
        if (ns) {
            tab[U.uexp + nr] = -1;
            tab[U.uoff + nr] = nr;
            tab[U.pairs + nr] = K;
            ublob[nr] = r.shared;
        }
        tab[U.uoff + nr + ns] = nr + ns;
        st_dev(r.epoch, tag);
    }
}

// The unit table of a batch from its selections (idx_l: S x K ids in LDS,
// btab: the first 256 experts' blob pointers in LDS): build_units in LDS,
// then the table's words and blob pointers to the workspace.  Every thread
// of the workgroup.
__device__ __forceinline__ void write_unit_table(const RouteArgs &r, uint8_t *smem, const SmemPlan &T,
                                                 const int32_t *idx_l, const uint8_t *const *btab) {
    const int tid = threadIdx.x, S = r.S, K = r.K, E = r.E, P = S * K;
    build_units(idx_l, S, K, E, r.n_shared, smem, T, r.status, false);
    const UnitTable U = unit_table(S, K, E);
    int32_t *tab = reinterpret_cast<int32_t *>(r.units);
    const int *misc = reinterpret_cast<const int *>(smem + T.misc);
    const int *uexp = reinterpret_cast<const int *>(smem + T.uexp);
    const int *uoff = reinterpret_cast<const int *>(smem + T.uoff);
    const int *pairs = reinterpret_cast<const int *>(smem + T.pairs);
    const int n_units = misc[0];
    if (tid < 4) tab[tid] = tid < 3 ? misc[tid] : 0;
    for (int q = tid; q < n_units; q += blockDim.x) {
        const int ex = uexp[q];
        tab[U.uexp + q] = ex;
        reinterpret_cast<const uint8_t **>(r.units + U.ublob)[q] =
            ex < 0 ? r.shared : (ex < 256 ? btab[ex] : r.blobs[ex]);
    }
    for (int q = tid; q <= n_units; q += blockDim.x) tab[U.uoff + q] = uoff[q];
    for (int q = tid; q < P + S * r.n_shared; q += blockDim.x) tab[U.pairs + q] = pairs[q];
}

// The logit and selecting workgroups of a launch of 2 .. 4 tokens with at
// most 256 experts (the same selection rule as route_one): wave w of logit
// workgroup bx of token t computes logit (t, lpw bx + w) and publishes it as
// a tagged 64-bit slot (slot t E + e).  Workgroup 0 of token 0 then waits
// (bounded) for all S x E slots, wavefront w selects token w with
// select_wave_b from the logits in LDS, and the workgroup builds the unit
// table: one workgroup, no arrival counters and no round trip of the
// selections through memory.  A wait that gave up leaves the shared expert
// alone in the table (status timed-out).
template <int MAXJ>
__device__ __forceinline__ void route_few(const RouteArgs &r, uint8_t *smem, int bx, int lpw, int t) {
    __shared__ float s_lg[4][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = r.E, K = r.K, S = r.S, H = r.H, P = S * K;
    const uint32_t tag = ld_dev(r.epoch) + 1u;
    const bool selector = bx == 0 && t == 0;
    // the selector's inputs besides the logits, fetched ahead of them: the
    // bias (every wave selects) and the blob pointers
    float bpre[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t *bl[4] = {nullptr, nullptr, nullptr, nullptr};
    if (selector) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int ee = min(lane + 64 * m, E - 1);
            if (r.bias) bpre[m] = r.bias[ee];
            if (wave == 0) bl[m] = r.blobs[ee];
        }
    }
    const int e = bx * lpw + wave;
    if (wave < lpw && e < E) {
        bool ok;
        const float p = logit_wave<MAXJ>(r.x + (size_t)t * H, r.W + (size_t)e * H, H, &ok);
        if (!ok) raise_status(r.status, ST_NONFINITE);
        if (lane == 0) st_dev64(&r.slots[(size_t)t * E + e], ((uint64_t)tag << 32) | __float_as_uint(p));
    }
    if (!selector) return;
    bool late = false;
    if (tid < E) {
        const uint32_t want = tag + r.tag_skew;
        uint64_t v[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            if (tt < S) v[tt] = ld_dev64(&r.slots[(size_t)tt * E + tid]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            if (tt < S) {
                uint32_t spins = 0;
                while (!late && (uint32_t)(v[tt] >> 32) != want) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins >= r.spin_limit) late = true;
                    else v[tt] = ld_dev64(&r.slots[(size_t)tt * E + tid]);
                }
                s_lg[tt][tid] = __uint_as_float((uint32_t)v[tt]);
            }
        }
    }
    const SmemPlan T = smem_plan(S, K, E, 0, 0);
    int32_t *idx_l = reinterpret_cast<int32_t *>(smem + T.total);
    const uint8_t **btab = reinterpret_cast<const uint8_t **>(smem + a16(T.total + 4 * (size_t)P));
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (lane + 64 * m < E) btab[lane + 64 * m] = bl[m];
    }
    const int timed_out = __syncthreads_or(late);
    if (timed_out) {
        // the logits are not all in: no routed unit, the shared expert alone
        // (every routing weight 0, so the combine adds no routed term)
        for (int q = tid; q < P; q += blockDim.x) {
            r.idx_out[q] = 0;
            r.w_out[q] = 0.0f;
        }
        if (tid == 0) {
            raise_status(r.status, ST_TIMEOUT);
            const UnitTable U = unit_table(S, K, E);
            int32_t *tab = reinterpret_cast<int32_t *>(r.units);
            const int ns = r.n_shared;
            tab[0] = ns;
            tab[1] = 0;
            tab[2] = 0;
            tab[3] = 0;
            for (int q = 0; q < ns * S; ++q) tab[U.pairs + q] = P + q;
            if (ns) {
                tab[U.uexp] = -1;
                reinterpret_cast<const uint8_t **>(r.units + U.ublob)[0] = r.shared;
            }
            tab[U.uoff] = 0;
            tab[U.uoff + ns] = ns * S;
            st_dev(r.epoch, tag);
        }
        return;
    }
    if (wave < S) {
        int32_t si = 0;
        float sw = 0.0f;
        const bool sok = select_wave_b<4>([&](int q) { return s_lg[wave][q]; }, [&](int m, int) { return bpre[m]; },
                                          E, K, r.rsf, r.norm, &si, &sw);
        if (!sok && lane == 0) raise_status(r.status, ST_NONFINITE);
        if (lane < K) {
            r.idx_out[(size_t)wave * K + lane] = si;
            r.w_out[(size_t)wave * K + lane] = sw;
            idx_l[wave * K + lane] = si;
        }
    }
    __syncthreads();
    write_unit_table(r, smem, T, idx_l, btab);
    if (tid == 0) st_dev(r.epoch, tag);
}

template <int MAXJ, int BITS, int NT, bool GROUPED, bool MX = false>
__global__ __launch_bounds__(64 * RF_W) void k_route_fused(const RouteArgs r) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, t = blockIdx.y;
    const int E = r.E, K = r.K, S = r.S, H = r.H;
    const int n_sg = r.sg ? r.I / 16 : 0;
    if ((int)blockIdx.x < n_sg) {
        if (t == 0) shared_gateup_half<BITS, NT, GROUPED, MX>(r, smem, blockIdx.x);
        return;
    }
    const int bx = (int)blockIdx.x - n_sg;
    const int lpw = rf_lpw(S), n_lw = (E + lpw - 1) / lpw;
    if (bx >= n_lw) {
        quant_x_wave(r.x, r.qx, r.dx, r.status, H, t, (bx - n_lw) * RF_W + wave);
        return;
    }
    if (S == 1 && E <= 256) {
        route_one<MAXJ>(r, bx, lpw);
        return;
    }
    if (S <= 4 && E <= 256) {
        route_few<MAXJ>(r, smem, bx, lpw, t);
        return;
    }
    // wave 0 fetches what the selection needs besides the logits (the bias
    // and the first 256 blob pointers, for the unit table) now, so that the
    // workgroup arriving last waits only for the logits
    float bpre[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t *bl[4] = {nullptr, nullptr, nullptr, nullptr};
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int ee = min(lane + 64 * m, E - 1);
            if (r.bias) bpre[m] = r.bias[ee];
            bl[m] = r.blobs[ee];
        }
    }
    const int e = bx * lpw + wave;
    if (wave < lpw && e < E) {
        bool ok;
        const float p = logit_wave<MAXJ>(r.x + (size_t)t * H, r.W + (size_t)e * H, H, &ok);
        if (!ok) raise_status(r.status, ST_NONFINITE);
        if (lane == 0) st_dev(&r.logits[(size_t)t * E + e], p);
    }
    drain();
    __syncthreads();
    if (tid == 0) {
        fence_release_agent();
        const uint32_t prev = __hip_atomic_fetch_add(&r.sync[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(n_lw - 1);
        if (s_last) {
            fence_acquire_agent();
            st_dev(&r.sync[t], 0u);
        }
    }
    __syncthreads();
    if (!s_last) return;

    // last workgroup of token t: wave 0 selects
    const int P = S * K;
    const SmemPlan T = smem_plan(S, K, E, 0, 0);
    int32_t *idx_l = reinterpret_cast<int32_t *>(smem + T.total);
    const uint8_t **btab = reinterpret_cast<const uint8_t **>(smem + a16(T.total + 4 * (size_t)P));
    int32_t si = 0;
    float sw = 0.0f;
    bool sok = true;
    if (wave == 0) {
        const float *lg = r.logits + (size_t)t * E;
        auto ld = [&](int q) { return ld_dev(lg + q); };
        sok = E <= 256 ? select_wave_b<4>(ld, [&](int m, int) { return bpre[m]; }, E, K, r.rsf, r.norm, &si, &sw)
                       : select_wave<16>(ld, r.bias, E, K, r.rsf, r.norm, &si, &sw);
        if (!sok && lane == 0) raise_status(r.status, ST_NONFINITE);
    }
    if (S == 1) {
        if (wave != 0) return;
        // One token: its selection is the whole routing.  The unit table is
        // written straight from the selection: unit j is the selected expert
        // of rank j in ascending id (its one pair is slot k, the lane that
        // selected it), then the shared expert with slot K.
        const UnitTable U = unit_table(1, K, E);
        int32_t *tab = reinterpret_cast<int32_t *>(r.units);
        const uint8_t **ublob = reinterpret_cast<const uint8_t **>(r.units + U.ublob);
        if (!sok) {
            // Non-finite scores (reported above): the picks may repeat an
            // expert, so no routed unit is listed; the table holds the shared
            // expert alone and the expert kernels read no routed blob.
            if (lane < K) {
                r.idx_out[lane] = si;
                r.w_out[lane] = sw;
            }
            if (lane == 0) {
                const int ns = r.n_shared;
                tab[0] = ns;
                tab[1] = 0;
                tab[2] = 0;
                tab[3] = 0;
                if (ns) {
                    tab[U.uexp] = -1;
                    tab[U.pairs] = K;
                    ublob[0] = r.shared;
                }
                tab[U.uoff] = 0;
                tab[U.uoff + ns] = ns;
            }
            return;
        }
        int rank = 0;
        for (int j = 0; j < K; ++j) rank += __builtin_amdgcn_readlane(si, j) < si ? 1 : 0;
        // blob pointer of expert si: prefetched by lane si % 64 in bl[si / 64]
        const uint8_t *mine = nullptr;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint8_t *v = reinterpret_cast<const uint8_t *>(
                __shfl(reinterpret_cast<uintptr_t>(bl[m]), si & 63, 64));
            if ((si >> 6) == m) mine = v;
        }
        if (lane < K) {
            r.idx_out[lane] = si;
            r.w_out[lane] = sw;
            tab[U.uexp + rank] = si;
            tab[U.uoff + rank] = rank;
            tab[U.pairs + rank] = lane;
            ublob[rank] = si < 256 ? mine : r.blobs[si];
        }
        if (lane == 0) {
            const int ns = r.n_shared;
            tab[0] = K + ns;
            tab[1] = K;
            tab[2] = K;
            tab[3] = 0;
            if (ns) {
                tab[U.uexp + K] = -1;
                tab[U.uoff + K] = K;
                tab[U.pairs + K] = K;
                ublob[K] = r.shared;
            }
            tab[U.uoff + K + ns] = K + ns;
        }
        return;
    }
    if (wave == 0 && lane < K) {
        st_dev(&r.idx_out[(size_t)t * K + lane], si);
        st_dev(&r.w_out[(size_t)t * K + lane], sw);
    }
    drain();
    __syncthreads();
    if (tid == 0) {
        fence_release_agent();
        const uint32_t prev =
            __hip_atomic_fetch_add(&r.sync[ROUTE_FUSE_MAX], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(S - 1);
        if (s_last) {
            fence_acquire_agent();
            st_dev(&r.sync[ROUTE_FUSE_MAX], 0u);
        }
    }
    __syncthreads();
    if (!s_last) return;
    // last token selected: the unit table of the batch
    for (int q = tid; q < P; q += blockDim.x) idx_l[q] = ld_dev(r.idx_out + q);
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (lane + 64 * m < E) btab[lane + 64 * m] = bl[m];
    }
    __syncthreads();
    write_unit_table(r, smem, T, idx_l, btab);
}

size_t route_fused_smem(int S, int K, int E) {
    return a16(a16(smem_plan(S, K, E, 0, 0).total + 4 * (size_t)S * K) + 8 * (size_t)(E < 256 ? E : 256));
}

// Vectors per pass of the shared tiles: two at most, so that their LDS fits
// beside the router's for the decode shapes (later passes re-read the
// tile's rows from L2).
static int route_nt(int S) { return S >= 2 ? 2 : 1; }

size_t route_fused_lds(const RouteArgs &r) {
    const size_t sel = route_fused_smem(r.S, r.K, r.E);
    if (!r.sg) return sel;
    const size_t tile = smem_plan(r.S, r.K, r.E, route_nt(r.S), r.H).total + groups_lds_bytes(r.group, 4);
    return sel > tile ? sel : tile;
}

template <int MAXJ, int BITS, bool GROUPED = false, bool MX = false>
static hipError_t route_fused_bits(const RouteArgs &r, dim3 grid, size_t smem, hipStream_t st) {
    auto go = [&](auto kern) {
        const hipError_t e = ensure_dyn_smem(reinterpret_cast<const void *>(kern), smem);
        if (e != hipSuccess) return e;
        return launch(kern, grid, dim3(64 * RF_W), smem, st, r);
    };
    if (route_nt(r.S) == 1) return go(k_route_fused<MAXJ, BITS, 1, GROUPED, MX>);
    return go(k_route_fused<MAXJ, BITS, 2, GROUPED, MX>);
}

// Group-scaled and MXFP4 weights are 4-bit codes only (the dims check
// refuses the others).
template <int MAXJ>
static hipError_t route_fused_maxj(const RouteArgs &r, dim3 grid, size_t smem, hipStream_t st) {
    if (r.mx) return route_fused_bits<MAXJ, 4, true, true>(r, grid, smem, st);
    if (r.group) return route_fused_bits<MAXJ, 4, true>(r, grid, smem, st);
    if (r.bits == 8) return route_fused_bits<MAXJ, 8>(r, grid, smem, st);
    if (r.bits == 2) return route_fused_bits<MAXJ, 2>(r, grid, smem, st);
    return route_fused_bits<MAXJ, 4>(r, grid, smem, st);
}

hipError_t launch_route_fused(const RouteArgs &r, hipStream_t st) {
    const int lpw = rf_lpw(r.S), n_lw = (r.E + lpw - 1) / lpw, n_q = ((r.H / 32 + 63) / 64 + RF_W - 1) / RF_W;
    const int n_sg = r.sg ? r.I / 16 : 0;
    const dim3 grid(n_sg + n_lw + (r.qx ? n_q : 0), r.S);
    const size_t smem = route_fused_lds(r);
    if (r.H <= 24 * 256) return route_fused_maxj<24>(r, grid, smem, st);
    return route_fused_maxj<16>(r, grid, smem, st);
}

// Q8_0 of the hidden states alone, and with qxs also their split codes
// (split_e4m3) for the MXFP4 grouped kernels.  Grid: (ceil(H / 2048), S),
// 64 threads.
__global__ __launch_bounds__(64) void k_quant_x(const float *__restrict__ x, int8_t *__restrict__ qx,
                                                float *__restrict__ dx, uint8_t *__restrict__ qxs,
                                                uint32_t *__restrict__ status, int H) {
    const int t = blockIdx.y, nbx = H / 32;
    const int b = (int)blockIdx.x * 64 + (int)(threadIdx.x & 63);
    if (b >= nbx) return;
    bool ok;
    uint32_t w[8];
    const float d = q8_0_block_words(x + (size_t)t * H + 32 * b, w, &ok);
    u32x4 *qv = reinterpret_cast<u32x4 *>(qx + (size_t)t * H + 32 * b);
    qv[0] = u32x4{w[0], w[1], w[2], w[3]};
    qv[1] = u32x4{w[4], w[5], w[6], w[7]};
    dx[(size_t)t * nbx + b] = d;
    if (!ok) raise_status(status, ST_NONFINITE);
    if (qxs) {
        u32x4 sp[4];
        split_e4m3(w, sp);
        u32x4 *dst = reinterpret_cast<u32x4 *>(qxs + ((size_t)t * nbx + b) * 64);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = sp[k];
    }
}

hipError_t launch_quant_x(const float *x, int8_t *qx, float *dx, uint8_t *qxs, uint32_t *status, int S, int H,
                          hipStream_t st) {
    return launch(k_quant_x, dim3((H / 32 + 63) / 64, S), dim3(64), 0, st, x, qx, dx, qxs, status, H);
}

hipError_t launch_router_logits(const float *x, const float *W, float *logits, uint32_t *status,
                                int S, int H, int E, int8_t *qx, float *dx, hipStream_t st) {
    const int gx = E + (qx ? (H / 32 + 63) / 64 : 0);
    if (H <= 24 * 256) return launch(k_router_logits<24>, dim3(gx, S), dim3(64), 0, st, x, W, logits, status, H, E, qx, dx);
    return launch(k_router_logits<16>, dim3(gx, S), dim3(64), 0, st, x, W, logits, status, H, E, qx, dx);
}

hipError_t launch_router_select(const float *logits, const float *bias, int32_t *idx, float *w,
                                uint32_t *status, int S, int E, int K, float rsf, int norm,
                                hipStream_t st) {
    if (E <= 256)
        return launch(k_router_select<4>, dim3(S), dim3(64), 0, st, logits, bias, idx, w, status, E, K, rsf, norm);
    return launch(k_router_select<16>, dim3(S), dim3(64), 0, st, logits, bias, idx, w, status, E, K, rsf, norm);
}

}  // namespace coli
