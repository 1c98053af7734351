// C-ABI entry points (include/coli_moe.h): argument checks, workspace
// carve-up, kernel launches, staging copies, status and timing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "coli_moe.h"
#include "device_common.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(COLI_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// The kernels are compiled for gfx950 only; refuse any other device.
int check_device() {
    static std::mutex mu;
    static std::vector<int> ok;  // per device: 0 unknown, 1 ok, -1 refused
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(mu);
    if ((int)ok.size() <= dev) ok.resize(dev + 1, 0);
    if (ok[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (ok[dev] < 0) return fail(COLI_EHIP, "device %d is not gfx950; this library has no other code path", dev);
    return COLI_OK;
}

int check_dims(const coli_moe_dims *d) {
    if (!d) return fail(COLI_EINVAL, "dims is NULL");
    if (d->hidden <= 0 || d->hidden % 256 != 0 || d->hidden > 16384)
        return fail(COLI_EINVAL, "hidden=%d: must be a positive multiple of 256, at most 16384", d->hidden);
    if (d->inter <= 0 || d->inter % 32 != 0 || d->inter > 16384)
        return fail(COLI_EINVAL, "inter=%d: must be a positive multiple of 32, at most 16384", d->inter);
    if (d->n_experts < 1 || d->n_experts > 1024)
        return fail(COLI_EINVAL, "n_experts=%d: must be in 1..1024", d->n_experts);
    if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 32)
        return fail(COLI_EINVAL, "top_k=%d: must be in 1..min(n_experts, 32)", d->top_k);
    if (d->n_shared != 0 && d->n_shared != 1)
        return fail(COLI_EINVAL, "n_shared=%d: must be 0 or 1", d->n_shared);
    if (d->wbits != 8 && d->wbits != 4 && d->wbits != 2)
        return fail(COLI_EINVAL, "wbits=%d: must be 8, 4 or 2", d->wbits);
    const int g = d->group_size;
    if (g != 0 && (g < 32 || g > 512 || (g & (g - 1)) != 0 || d->hidden % g != 0 || d->inter % g != 0))
        return fail(COLI_EINVAL, "group_size=%d: must be 0 or a power of two in 32..512 dividing hidden and inter", g);
    if (g != 0 && d->wbits != 4) return fail(COLI_EINVAL, "group_size=%d needs wbits=4 (group-scaled int4)", g);
    if (d->wformat != COLI_WFMT_INT && d->wformat != COLI_WFMT_MXFP4)
        return fail(COLI_EINVAL, "wformat=%d: must be COLI_WFMT_INT (0) or COLI_WFMT_MXFP4 (1)", d->wformat);
    if (d->wformat == COLI_WFMT_MXFP4 && (d->wbits != 4 || g != 0 || d->inter % 128 != 0))
        return fail(COLI_EINVAL, "MXFP4 experts need wbits=4, group_size=0 and inter a multiple of 128 "
                                 "(wbits=%d, group_size=%d, inter=%d)", d->wbits, g, d->inter);
    return COLI_OK;
}

bool is_mx(const coli_moe_dims *d) { return d->wformat == COLI_WFMT_MXFP4; }

// Hidden states, router gate, outputs and blobs are read and written with
// 16-byte vector accesses.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ---- kernel timing ------------------------------------------------------
struct Timing {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> free_events;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> done[coli::KK_COUNT];
} g_timing;

hipEvent_t take_event() {
    if (!g_timing.free_events.empty()) {
        hipEvent_t e = g_timing.free_events.back();
        g_timing.free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// 0: automatic, 1: multi-launch decode kernels at any batch size,
// 2: persistent kernels only, 3: grouped (matrix-core) kernels at any batch
// size.
int g_force_path = 0;
// coli_moe_debug_route_wait: polls of the one-token selection's wait (0:
// ROUTE_SPIN_LIMIT) and whether it waits for a tag no workgroup writes
uint32_t g_route_spins = 0;
uint32_t g_route_skew = 0;

// Batches of more than GROUPED_MIN_S - 1 tokens take the grouped kernels.
constexpr int GROUPED_MIN_S = 9;

// The grouped kernels take integer codes with per-row scales or groups of
// 64, and MXFP4 codes; other group sizes run the multi-launch kernels at
// every batch size.
bool use_grouped(int S, int group, bool mx) {
    return (mx || group == 0 || group == 64) && (g_force_path == 3 || (g_force_path == 0 && S >= GROUPED_MIN_S));
}

// The group size the kernels see: MXFP4 has one (E8M0) scale per 32 codes.
int kernel_group(const coli_moe_dims *d) { return is_mx(d) ? 32 : d->group_size; }

// LDS of the kernels a forward of S tokens launches.
size_t forward_lds(const coli_moe_dims *d, int S) {
    if (use_grouped(S, d->group_size, is_mx(d))) return coli::pf_group_smem(S, d->top_k, d->n_experts);
    return coli::forward_smem_max(S, d->hidden, d->inter, d->n_experts, d->top_k, d->n_shared, kernel_group(d));
}

// A forced kernel family that does not take the call's weights.
int forced_path_refused(const coli_moe_dims *d) {
    if ((d->group_size || is_mx(d)) && g_force_path == 2)
        return fail(COLI_EINVAL, "the persistent kernel takes integer codes with per-row scales only");
    if (d->group_size && d->group_size != 64 && g_force_path == 3)
        return fail(COLI_EINVAL, "the grouped kernels take per-row scales or groups of 64 (group_size=%d)",
                    d->group_size);
    return COLI_OK;
}

// The persistent kernel takes small batches whose experts are all resident.
bool persistent_fits(const coli_moe_dims *d, int S, bool pending) {
    if (pending || S > 8 || d->group_size || is_mx(d)) return false;
    return coli::layer_smem(S, d->hidden, d->inter, d->n_experts, d->top_k, d->n_shared) <= 160 * 1024;
}

// The automatic choice is the multi-launch kernel set (the faster one on
// MI355X for the shapes measured); the persistent kernel runs when forced.
bool use_persistent(const coli_moe_dims *d, int S, bool pending) {
    return g_force_path == 2 && persistent_fits(d, S, pending);
}

}  // namespace

namespace coli {

// The kind of the launches the calling thread is making (-1: none).
thread_local int tl_kind = -1;

void timing_before(int kind, hipStream_t) { tl_kind = kind; }

void timing_after(int, hipStream_t) { tl_kind = -1; }

bool timing_pair(hipEvent_t *start, hipEvent_t *stop) {
    if (tl_kind < 0) return false;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on) return false;
    hipEvent_t e0 = take_event(), e1 = take_event();
    if (!e0 || !e1) return false;
    g_timing.done[tl_kind].emplace_back(e0, e1);
    *start = e0;
    *stop = e1;
    return true;
}

hipError_t ensure_dyn_smem(const void *kern, size_t smem) {
    static std::mutex mu;
    static std::map<const void *, size_t> raised;
    std::lock_guard<std::mutex> lk(mu);
    size_t &have = raised[kern];
    if (smem <= have) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess) have = smem;
    return e;
}

}  // namespace coli

using namespace coli;

namespace {

FwdArgs fwd_args(const coli_moe_dims *d, int S, const float *x, const int32_t *idx, const float *w,
                 const void *const *expert_blobs, const void *shared_blob, float *out, uint8_t *w8,
                 const WsLayout &L) {
    FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.idx = idx;
    a.w = w;
    a.blobs = reinterpret_cast<const uint8_t *const *>(expert_blobs);
    a.shared = static_cast<const uint8_t *>(shared_blob);
    a.qx = reinterpret_cast<const int8_t *>(w8 + L.qx);
    a.dx = reinterpret_cast<const float *>(w8 + L.dx);
    a.qh = reinterpret_cast<int8_t *>(w8 + L.qh);
    a.dh = reinterpret_cast<float *>(w8 + L.dh);
    a.Y = reinterpret_cast<float *>(w8 + L.Y);
    a.tiles = reinterpret_cast<int32_t *>(w8 + L.tiles);
    a.out = out;
    a.status = reinterpret_cast<uint32_t *>(w8 + L.status);
    a.S = S;
    a.H = d->hidden;
    a.I = d->inter;
    a.E = d->n_experts;
    a.K = d->top_k;
    a.n_shared = d->n_shared;
    a.group = kernel_group(d);
    a.mx = is_mx(d) ? 1 : 0;
    a.qxs = is_mx(d) ? w8 + L.qxs : nullptr;
    a.qhs = is_mx(d) ? w8 + L.qhs : nullptr;
    return a;
}

// Router logits (with Q8_0(x) into the workspace when quant_x) and, with
// select, the top-K selection.
int route_launches(const coli_moe_dims *d, int S, const float *x, const float *router_w,
                   const float *router_bias, int32_t *topk_idx, float *topk_w, uint8_t *w8,
                   const WsLayout &L, bool quant_x, bool select, hipStream_t st) {
    uint32_t *status = reinterpret_cast<uint32_t *>(w8 + L.status);
    float *logits = reinterpret_cast<float *>(w8 + L.logits);
    hipError_t e;
    if (S > ROUTE_FUSE_MAX) {
        // many tokens: a wavefront per 8 tokens x 8 experts, Q8_0(x) apart
        timing_before(KK_ROUTER_LOGITS, st);
        e = launch_logits_tiled(x, router_w, logits, status, S, d->hidden, d->n_experts, st);
        timing_after(KK_ROUTER_LOGITS, st);
        if (e != hipSuccess) return hip_fail(e, "router logits launch");
        if (quant_x) {
            timing_before(KK_QUANT_X, st);
            e = launch_quant_x(x, reinterpret_cast<int8_t *>(w8 + L.qx), reinterpret_cast<float *>(w8 + L.dx),
                               is_mx(d) ? w8 + L.qxs : nullptr, status, S, d->hidden, st);
            timing_after(KK_QUANT_X, st);
            if (e != hipSuccess) return hip_fail(e, "Q8_0(x) launch");
        }
    } else {
        // (MXFP4 experts also need the split codes of Q8_0(x): k_quant_x)
        const bool fused_qx = quant_x && !is_mx(d);
        timing_before(KK_ROUTER_LOGITS, st);
        e = launch_router_logits(x, router_w, logits, status, S, d->hidden, d->n_experts,
                                 fused_qx ? reinterpret_cast<int8_t *>(w8 + L.qx) : nullptr,
                                 fused_qx ? reinterpret_cast<float *>(w8 + L.dx) : nullptr, st);
        timing_after(KK_ROUTER_LOGITS, st);
        if (e != hipSuccess) return hip_fail(e, "router logits launch");
        if (quant_x && !fused_qx) {
            timing_before(KK_QUANT_X, st);
            e = launch_quant_x(x, reinterpret_cast<int8_t *>(w8 + L.qx), reinterpret_cast<float *>(w8 + L.dx),
                               w8 + L.qxs, status, S, d->hidden, st);
            timing_after(KK_QUANT_X, st);
            if (e != hipSuccess) return hip_fail(e, "Q8_0(x) launch");
        }
    }
    if (!select) return COLI_OK;
    timing_before(KK_ROUTER_SELECT, st);
    e = launch_router_select(logits, router_bias, topk_idx, topk_w, status, S, d->n_experts, d->top_k,
                             d->routed_scaling_factor, d->norm_topk_prob, st);
    timing_after(KK_ROUTER_SELECT, st);
    if (e != hipSuccess) return hip_fail(e, "router select launch");
    return COLI_OK;
}

// The multi-launch forward: [Q8_0(x)], gate/up (resident experts first when
// some are pending, then the pending ones after pending_ready), down, combine.
int forward_launches(FwdArgs &a, int bits, bool any_pending, void *pending_ready, bool qx_ready,
                     uint8_t *units_ws, hipStream_t st) {
    hipError_t e;
    if (!qx_ready) {
        timing_before(KK_QUANT_X, st);
        e = launch_quant_x(a.x, const_cast<int8_t *>(a.qx), const_cast<float *>(a.dx), a.qxs, a.status, a.S, a.H, st);
        timing_after(KK_QUANT_X, st);
        if (e != hipSuccess) return hip_fail(e, "Q8_0(x) launch");
    }
    if (use_grouped(a.S, a.group, a.mx != 0)) {
        // grouped kernels: the unit table and tiles, then gate/up and down as
        // int8 matrix-core products per (rows, tile), then the combine.  They
        // do not split resident from pending experts: all wait for the copies.
        if (any_pending && pending_ready) {
            e = hipStreamWaitEvent(st, static_cast<hipEvent_t>(pending_ready), 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        }
        a.units = units_ws;
        timing_before(KK_GROUP, st);
        e = launch_group(a.idx, a.S, a.K, a.E, a.n_shared, units_ws, a.tiles, a.status, st);
        timing_after(KK_GROUP, st);
        if (e != hipSuccess) return hip_fail(e, "grouping launch");
        timing_before(KK_GATEUP, st);
        e = launch_pf_gateup(a, a.tiles, bits, st);
        timing_after(KK_GATEUP, st);
        if (e != hipSuccess) return hip_fail(e, "gate/up launch");
        timing_before(KK_DOWN, st);
        e = launch_pf_down(a, a.tiles, bits, st);
        timing_after(KK_DOWN, st);
        if (e != hipSuccess) return hip_fail(e, "down launch");
        timing_before(KK_COMBINE, st);
        e = launch_combine(a, st);
        timing_after(KK_COMBINE, st);
        if (e != hipSuccess) return hip_fail(e, "combine launch");
        return COLI_OK;
    }
    if (any_pending) {
        a.pend_mode = 1;  // resident experts first
        timing_before(KK_GATEUP, st);
        e = launch_gateup(a, bits, st);
        timing_after(KK_GATEUP, st);
        if (e != hipSuccess) return hip_fail(e, "gate/up launch");
        if (pending_ready) {
            e = hipStreamWaitEvent(st, static_cast<hipEvent_t>(pending_ready), 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        }
        a.pend_mode = 2;  // then the experts that were being staged
    }
    timing_before(KK_GATEUP, st);
    e = launch_gateup(a, bits, st);
    timing_after(KK_GATEUP, st);
    if (e != hipSuccess) return hip_fail(e, "gate/up launch");
    // down + combine by output rows up to 8 tokens while two workgroups fit a
    // CU (the 4-token int8 verify step needs 76 KiB: 76 us against 91 us for
    // the per-unit down and the combine)
    if (a.S <= 8 && down_rows_smem(a.S, a.I, a.E, a.K, a.n_shared, a.group, bits) <= 80 * 1024) {
        timing_before(KK_DOWN, st);
        e = launch_down_rows(a, bits, st);
        timing_after(KK_DOWN, st);
        if (e != hipSuccess) return hip_fail(e, "down+combine launch");
        return COLI_OK;
    }
    timing_before(KK_DOWN, st);
    e = launch_down(a, bits, st);
    timing_after(KK_DOWN, st);
    if (e != hipSuccess) return hip_fail(e, "down launch");
    timing_before(KK_COMBINE, st);
    e = launch_combine(a, st);
    timing_after(KK_COMBINE, st);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return COLI_OK;
}

}  // namespace

extern "C" {

size_t coli_moe_expert_bytes(const coli_moe_dims *d) {
    if (check_dims(d) != COLI_OK) return 0;
    return blob_layout(d->hidden, d->inter, d->wbits, d->group_size, is_mx(d)).total;
}

size_t coli_moe_workspace_bytes(const coli_moe_dims *d, int32_t max_tokens) {
    if (check_dims(d) != COLI_OK || max_tokens < 0 || max_tokens > COLI_MAX_TOKENS) return 0;
    return ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, max_tokens, is_mx(d)).total;
}

const char *coli_moe_last_error(void) { return g_err.c_str(); }

int coli_moe_route(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                   const float *router_bias, int32_t *topk_idx, float *topk_w, void *ws,
                   size_t ws_bytes, void *stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (S < 0 || S > COLI_MAX_TOKENS) return fail(COLI_EINVAL, "n_tokens=%d: must be in 0..%d", S, COLI_MAX_TOKENS);
    if (S == 0) return COLI_OK;
    if (!x || !router_w || !topk_idx || !topk_w || !ws)
        return fail(COLI_EINVAL, "coli_moe_route: NULL pointer argument");
    if (!aligned16(x) || !aligned16(router_w))
        return fail(COLI_EINVAL, "coli_moe_route: x and router_w must be 16-byte aligned");
    const WsLayout L = ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, S, is_mx(d));
    if (ws_bytes < L.total)
        return fail(COLI_EWORKSPACE, "workspace %zu bytes < %zu needed for %d tokens", ws_bytes, L.total, S);
    if ((rc = check_device())) return rc;
    return route_launches(d, S, x, router_w, router_bias, topk_idx, topk_w, static_cast<uint8_t *>(ws), L,
                          false, true, static_cast<hipStream_t>(stream));
}

int coli_moe_forward(const coli_moe_dims *d, int32_t S, const float *x, const int32_t *topk_idx,
                     const float *topk_w, const void *const *expert_blobs, const void *shared_blob,
                     const uint8_t *pending_mask, void *pending_ready, float *out, void *ws,
                     size_t ws_bytes, void *stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (S < 0 || S > COLI_MAX_TOKENS) return fail(COLI_EINVAL, "n_tokens=%d: must be in 0..%d", S, COLI_MAX_TOKENS);
    if (S == 0) return COLI_OK;
    if (!x || !topk_idx || !topk_w || !expert_blobs || !out || !ws)
        return fail(COLI_EINVAL, "coli_moe_forward: NULL pointer argument");
    if (!aligned16(x) || !aligned16(out) || !aligned16(shared_blob))
        return fail(COLI_EINVAL, "coli_moe_forward: x, out and shared_blob must be 16-byte aligned");
    if (d->n_shared && !shared_blob)
        return fail(COLI_ENOTRESIDENT, "n_shared=1 but shared_blob is NULL");
    const WsLayout L = ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, S, is_mx(d));
    if (ws_bytes < L.total)
        return fail(COLI_EWORKSPACE, "workspace %zu bytes < %zu needed for %d tokens", ws_bytes, L.total, S);
    if ((rc = forced_path_refused(d))) return rc;
    const size_t smem = forward_lds(d, S);
    if (smem > 160 * 1024)
        return fail(COLI_EINVAL, "shape needs %zu bytes of LDS per workgroup (> 160 KiB)", smem);
    if ((rc = check_device())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    FwdArgs a = fwd_args(d, S, x, topk_idx, topk_w, expert_blobs, shared_blob, out, w8, L);
    bool any_pending = false;
    if (pending_mask) {
        for (int e = 0; e < d->n_experts; ++e)
            if (pending_mask[e]) {
                a.pend[e >> 5] |= 1u << (e & 31);
                any_pending = true;
            }
    }
    hipError_t e;
    if (g_force_path == 2 && !persistent_fits(d, S, any_pending))
        return fail(COLI_EINVAL, "persistent kernel forced but the call has pending experts, more than 8 tokens "
                                 "or a shape beyond its LDS budget");
    if (use_persistent(d, S, any_pending)) {
        LayerArgs l;
        std::memset(&l, 0, sizeof l);
        l.qx = reinterpret_cast<int8_t *>(w8 + L.qx);
        l.dx = reinterpret_cast<float *>(w8 + L.dx);
        l.sync = reinterpret_cast<uint32_t *>(w8) + WS_SYNC_LAYER;
        l.flags = w8 + L.flags;
        timing_before(KK_FORWARD_PERSISTENT, st);
        e = launch_layer(a, l, false, d->wbits, st);
        timing_after(KK_FORWARD_PERSISTENT, st);
        if (e != hipSuccess) return hip_fail(e, "forward launch");
        return COLI_OK;
    }
    return forward_launches(a, d->wbits, any_pending, pending_ready, false, w8 + L.units, st);
}

}  // extern "C"

namespace {

// Argument checks of a layer call that need no device (dims, pointers,
// alignment); 0 or the failure code.
int layer_args_ok(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                  const void *const *expert_blobs, const void *shared_blob, const int32_t *topk_idx,
                  const float *topk_w, const float *out, const char *who) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (S < 0 || S > COLI_MAX_TOKENS) return fail(COLI_EINVAL, "n_tokens=%d: must be in 0..%d", S, COLI_MAX_TOKENS);
    if (S == 0) return COLI_OK;
    if (!x || !router_w || !expert_blobs || !topk_idx || !topk_w || !out)
        return fail(COLI_EINVAL, "%s: NULL pointer argument", who);
    if (!aligned16(x) || !aligned16(router_w) || !aligned16(out) || !aligned16(shared_blob))
        return fail(COLI_EINVAL, "%s: x, router_w, out and shared_blob must be 16-byte aligned", who);
    if (d->n_shared && !shared_blob) return fail(COLI_ENOTRESIDENT, "n_shared=1 but shared_blob is NULL");
    return COLI_OK;
}

// The launches of a layer call on a workspace of at least
// ws_layout(...).total bytes (arguments already checked).
int layer_launches(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                   const float *router_bias, const void *const *expert_blobs, const void *shared_blob,
                   int32_t *topk_idx, float *topk_w, float *out, void *ws, hipStream_t st) {
    int rc;
    const WsLayout L = ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, S, is_mx(d));
    if ((rc = forced_path_refused(d))) return rc;
    if (g_force_path == 2 && !persistent_fits(d, S, false))
        return fail(COLI_EINVAL, "persistent kernel forced but the call has more than 8 tokens or a shape beyond "
                                 "its LDS budget");
    if ((rc = check_device())) return rc;
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    FwdArgs a = fwd_args(d, S, x, topk_idx, topk_w, expert_blobs, shared_blob, out, w8, L);
    if (!use_persistent(d, S, false)) {
        const size_t smem = forward_lds(d, S);
        if (smem > 160 * 1024)
            return fail(COLI_EINVAL, "shape needs %zu bytes of LDS per workgroup (> 160 KiB)", smem);
        // up to ROUTE_FUSE_MAX tokens: one router launch also selects the
        // routing and writes the call's unit table, which the expert kernels read
        if (S <= ROUTE_FUSE_MAX && !use_grouped(S, d->group_size, is_mx(d))) {
            RouteArgs r;
            std::memset(&r, 0, sizeof r);
            r.x = x;
            r.W = router_w;
            r.bias = router_bias;
            r.logits = reinterpret_cast<float *>(w8 + L.logits);
            r.status = reinterpret_cast<uint32_t *>(w8 + L.status);
            r.qx = reinterpret_cast<int8_t *>(w8 + L.qx);
            r.dx = reinterpret_cast<float *>(w8 + L.dx);
            r.idx_out = topk_idx;
            r.w_out = topk_w;
            r.blobs = reinterpret_cast<const uint8_t *const *>(expert_blobs);
            r.shared = static_cast<const uint8_t *>(shared_blob);
            r.units = w8 + L.units;
            r.sync = reinterpret_cast<uint32_t *>(w8) + WS_SYNC_ROUTE;
            r.S = S;
            r.H = d->hidden;
            r.E = d->n_experts;
            r.K = d->top_k;
            r.n_shared = d->n_shared;
            r.norm = d->norm_topk_prob;
            r.rsf = d->routed_scaling_factor;
            r.hs = reinterpret_cast<float *>(w8 + L.hs);
            r.slots = reinterpret_cast<uint64_t *>(w8 + L.slots);
            r.epoch = reinterpret_cast<uint32_t *>(w8) + WS_EPOCH;
            r.spin_limit = g_route_spins ? g_route_spins : ROUTE_SPIN_LIMIT;
            r.tag_skew = g_route_skew;
            r.I = d->inter;
            r.bits = d->wbits;
            r.group = kernel_group(d);
            r.mx = is_mx(d) ? 1 : 0;
            // the shared expert's gate/up half tiles run in the router launch
            // when they are short enough to finish beside it (one pass over at
            // most 128 KiB of rows per workgroup) and their LDS fits there
            r.sg = d->n_shared && route_shared_fits(S, d->hidden, d->wbits) ? 1 : 0;
            if (route_fused_lds(r) > 64 * 1024) r.sg = 0;
            if (route_fused_lds(r) <= 64 * 1024) {
                timing_before(KK_ROUTER_LOGITS, st);
                const hipError_t e = launch_route_fused(r, st);
                timing_after(KK_ROUTER_LOGITS, st);
                if (e != hipSuccess) return hip_fail(e, "router launch");
                a.units = w8 + L.units;
                a.shared_done = r.sg;
                a.hs = r.hs;
                return forward_launches(a, d->wbits, false, nullptr, true, w8 + L.units, st);
            }
        }
        rc = route_launches(d, S, x, router_w, router_bias, topk_idx, topk_w, w8, L, true, true, st);
        if (rc) return rc;
        return forward_launches(a, d->wbits, false, nullptr, true, w8 + L.units, st);
    }
    LayerArgs l;
    std::memset(&l, 0, sizeof l);
    l.router_w = router_w;
    l.bias = router_bias;
    l.idx_out = topk_idx;
    l.w_out = topk_w;
    l.logits = reinterpret_cast<float *>(w8 + L.logits);
    l.rsf = d->routed_scaling_factor;
    l.norm = d->norm_topk_prob;
    l.qx = reinterpret_cast<int8_t *>(w8 + L.qx);
    l.dx = reinterpret_cast<float *>(w8 + L.dx);
    l.sync = reinterpret_cast<uint32_t *>(w8) + WS_SYNC_LAYER;
    l.flags = w8 + L.flags;
    timing_before(KK_LAYER, st);
    hipError_t e = launch_layer(a, l, true, d->wbits, st);
    timing_after(KK_LAYER, st);
    if (e != hipSuccess) return hip_fail(e, "layer launch");
    return COLI_OK;
}

}  // namespace

extern "C" {

int coli_moe_layer(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                   const float *router_bias, const void *const *expert_blobs, const void *shared_blob,
                   int32_t *topk_idx, float *topk_w, float *out, void *ws, size_t ws_bytes, void *stream) {
    int rc = layer_args_ok(d, S, x, router_w, expert_blobs, shared_blob, topk_idx, topk_w, out, "coli_moe_layer");
    if (rc || S == 0) return rc;
    if (!ws) return fail(COLI_EINVAL, "coli_moe_layer: NULL pointer argument");
    const WsLayout L = ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, S, is_mx(d));
    if (ws_bytes < L.total)
        return fail(COLI_EWORKSPACE, "workspace %zu bytes < %zu needed for %d tokens", ws_bytes, L.total, S);
    return layer_launches(d, S, x, router_w, router_bias, expert_blobs, shared_blob, topk_idx, topk_w, out, ws,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- the layer without a caller workspace -------------------------------
// A file-scope device array serves as the workspace of
// coli_moe_layer_noalloc.  Each GPU the library runs on holds its own copy
// (zero at load, as a workspace must start) until the process ends; its
// address on a device comes from hipGetSymbolAddress, taken once per device
// with that device current.  In host code the array's name is not a device
// address: only the pointer looked up here is ever handed to kernels.
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

// Device address of this device's scratch array (looked up on first use).
int scratch_ptr(uint8_t **out) {
    static std::mutex mu;
    static std::vector<uint8_t *> ptrs;  // per device; null until looked up
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(mu);
    if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(COLI_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        ptrs[dev] = static_cast<uint8_t *>(p);
    }
    *out = ptrs[dev];
    return COLI_OK;
}

// Moves the scratch's status word to the caller's word (when given) and
// clears it, with vector stores (one thread).
__global__ void k_take_status(uint32_t *ws_status, uint32_t *status_out) {
    const uint32_t s = __hip_atomic_load(ws_status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (status_out) *status_out = s;
    __hip_atomic_store(ws_status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

extern "C" {

int coli_moe_layer_noalloc(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                           const float *router_bias, const void *const *expert_blobs, const void *shared_blob,
                           int32_t *topk_idx, float *topk_w, float *out, uint32_t *status_out, void *stream) {
    int rc = layer_args_ok(d, S, x, router_w, expert_blobs, shared_blob, topk_idx, topk_w, out,
                           "coli_moe_layer_noalloc");
    if (rc || S == 0) return rc;
    const WsLayout L = ws_layout(d->hidden, d->inter, d->n_experts, d->top_k, S, is_mx(d));
    if (L.total > NOALLOC_SCRATCH_BYTES)
        return fail(COLI_EWORKSPACE,
                    "coli_moe_layer_noalloc: %d tokens need %zu bytes of scratch, more than its %zu; "
                    "use coli_moe_layer with a workspace",
                    S, L.total, NOALLOC_SCRATCH_BYTES);
    if ((rc = check_device())) return rc;
    uint8_t *ws = nullptr;
    if ((rc = scratch_ptr(&ws))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = layer_launches(d, S, x, router_w, router_bias, expert_blobs, shared_blob, topk_idx, topk_w, out, ws, st);
    if (rc) return rc;
    hipLaunchKernelGGL(k_take_status, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t *>(ws + L.status),
                       status_out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? COLI_OK : hip_fail(e, "status launch");
}

int coli_moe_stage_experts(int32_t n, const void *const *host_src, void *const *dev_dst,
                           size_t bytes_each, void *copy_stream, void *done_event) {
    if (n < 0) return fail(COLI_EINVAL, "n=%d < 0", n);
    if (n > 0 && (!host_src || !dev_dst)) return fail(COLI_EINVAL, "NULL pointer array");
    for (int i = 0; i < n; ++i)
        if (!host_src[i] || !dev_dst[i]) return fail(COLI_EINVAL, "NULL source or destination %d", i);
    hipStream_t st = static_cast<hipStream_t>(copy_stream);
    for (int i = 0; i < n; ++i) {
        hipError_t e = hipMemcpyAsync(dev_dst[i], host_src[i], bytes_each, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    }
    if (done_event) {
        hipError_t e = hipEventRecord(static_cast<hipEvent_t>(done_event), st);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    return COLI_OK;
}

int coli_moe_status(void *ws, void *stream) {
    if (!ws) return fail(COLI_EINVAL, "workspace is NULL");
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t s = 0;
    e = hipMemcpy(&s, ws, sizeof s, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "status read");
    if (s == 0) return COLI_OK;
    e = hipMemset(ws, 0, sizeof s);
    if (e != hipSuccess) return hip_fail(e, "status clear");
    if (s & ST_TIMEOUT)
        return fail(COLI_EHIP, "a kernel's wait for the other workgroups of its launch timed out: not all of them "
                               "were resident (status 0x%x)", s);
    if (s & ST_BADINDEX) return fail(COLI_EINVAL, "expert index out of range or repeated within a token (status 0x%x)", s);
    if (s & ST_NONFINITE) return fail(COLI_ENONFINITE, "non-finite input or undefined gate weights (status 0x%x)", s);
    return fail(COLI_ENOTRESIDENT, "a routed expert blob was NULL (status 0x%x)", s);
}

int coli_moe_timing_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = enable != 0;
    return COLI_OK;
}

int coli_moe_timing_read(int32_t kind, double *total_ms, int64_t *launches) {
    if (kind < 0 || kind >= KK_COUNT || !total_ms || !launches)
        return fail(COLI_EINVAL, "bad timing query");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double tot = 0.0;
    int64_t n = 0;
    for (auto &pr : g_timing.done[kind]) {
        hipError_t e = hipEventSynchronize(pr.second);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, pr.first, pr.second);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        tot += ms;
        ++n;
        g_timing.free_events.push_back(pr.first);
        g_timing.free_events.push_back(pr.second);
    }
    g_timing.done[kind].clear();
    *total_ms = tot;
    *launches = n;
    return COLI_OK;
}

int coli_moe_debug_force_path(int32_t path) {
    if (path < 0 || path > 3) return fail(COLI_EINVAL, "path must be 0, 1, 2 or 3");
    g_force_path = path;
    return COLI_OK;
}

int coli_moe_debug_route_wait(uint32_t spins, int32_t unreachable) {
    if (unreachable != 0 && unreachable != 1) return fail(COLI_EINVAL, "unreachable must be 0 or 1");
    if (unreachable && spins == 0) return fail(COLI_EINVAL, "an unreachable wait needs a spin bound");
    g_route_spins = spins;
    g_route_skew = (uint32_t)unreachable;
    return COLI_OK;
}

int coli_moe_debug_unpack(int32_t bits, int32_t n_rows, int32_t cols, const void *src, int8_t *out,
                          void *stream) {
    if ((bits != 8 && bits != 4 && bits != 2 && bits != COLI_MXFP4) || n_rows < 0 || cols <= 0 || cols % 32 || !src || !out ||
        (uint64_t)n_rows * (uint64_t)cols * (uint64_t)(bits == COLI_MXFP4 ? 4 : bits) / 8 >= (1ull << 31))
        return fail(COLI_EINVAL, "debug_unpack: bad arguments");
    if (n_rows == 0) return COLI_OK;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_unpack(bits, n_rows, cols, src, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_unpack launch");
}

int coli_moe_debug_block_dots(int32_t bits, int32_t n_rows, int32_t cols, const void *src,
                              const int8_t *q, int32_t *out, void *stream) {
    if ((bits != 8 && bits != 4 && bits != 2 && bits != COLI_MXFP4) || n_rows < 0 || cols <= 0 || cols % 32 || !src || !q || !out ||
        (uint64_t)n_rows * (uint64_t)cols * (uint64_t)(bits == COLI_MXFP4 ? 4 : bits) / 8 >= (1ull << 31))
        return fail(COLI_EINVAL, "debug_block_dots: bad arguments");
    if (n_rows == 0) return COLI_OK;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_block_dots(bits, n_rows, cols, src, q, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_block_dots launch");
}

int coli_moe_debug_logits(const coli_moe_dims *d, int32_t S, const float *x, const float *router_w,
                          float *logits, void *stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (S < 0 || S > COLI_MAX_TOKENS || !x || !router_w || !logits) return fail(COLI_EINVAL, "debug_logits: bad arguments");
    if (S == 0) return COLI_OK;
    if ((rc = check_device())) return rc;
    // no workspace here: the kernel skips its status report when given none
    hipError_t e = launch_router_logits(x, router_w, logits, nullptr, S, d->hidden, d->n_experts, nullptr,
                                        nullptr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_logits launch");
}

int coli_moe_debug_expf(int64_t n, const float *x, float *y, void *stream) {
    if (n < 0 || !x || !y) return fail(COLI_EINVAL, "debug_expf: bad arguments");
    if (n == 0) return COLI_OK;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_expf(n, x, y, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_expf launch");
}

int coli_moe_debug_q8_0(int32_t n_rows, int32_t cols, const float *v, int8_t *q, float *d, void *stream) {
    if (n_rows < 0 || cols <= 0 || cols % 32 || !v || !q || !d) return fail(COLI_EINVAL, "debug_q8_0: bad arguments");
    if (n_rows == 0) return COLI_OK;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_q8_0(n_rows, cols, v, q, d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_q8_0 launch");
}

int coli_moe_debug_mfma_i8(const int8_t *a, const int8_t *b, int32_t *c, void *stream) {
    if (!a || !b || !c) return fail(COLI_EINVAL, "debug_mfma_i8: NULL pointer argument");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_mfma_i8(a, b, c, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_mfma_i8 launch");
}

int coli_moe_debug_mfma_i8_16(const int8_t *a, const int8_t *b, int32_t *c, void *stream) {
    if (!a || !b || !c) return fail(COLI_EINVAL, "debug_mfma_i8_16: NULL pointer argument");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_mfma_i8_16(a, b, c, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_mfma_i8_16 launch");
}

int coli_moe_debug_mfma_f8f6f4(int32_t fmt_a, int32_t fmt_b, const uint8_t *a, const uint8_t *b, const uint8_t *sa,
                               const uint8_t *sb, float *c, void *stream) {
    if (!a || !b || !sa || !sb || !c) return fail(COLI_EINVAL, "debug_mfma_f8f6f4: NULL pointer argument");
    if (!((fmt_a == 0 || fmt_a == 4) && fmt_b == 0))
        return fail(COLI_EINVAL, "debug_mfma_f8f6f4: formats (A, B) must be (0, 0) or (4, 0)");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_debug_mfma_f8f6f4(fmt_a, fmt_b, a, b, sa, sb, c, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "debug_mfma_f8f6f4 launch");
}

size_t coli_moe_roof_sink_words(void) { return (size_t)ROOF_GRID * 256; }

int coli_moe_roof_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink || bytes % 16) return fail(COLI_EINVAL, "roof_stream_read: bad arguments");
    if (bytes == 0) return COLI_OK;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_roof_stream(src, bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "roof_stream_read launch");
}

int coli_moe_roof_mfma_i8(int32_t iters, int32_t *sink, void *stream) {
    if (iters < 1 || !sink) return fail(COLI_EINVAL, "roof_mfma_i8: bad arguments");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_roof_mfma(iters, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? COLI_OK : hip_fail(e, "roof_mfma_i8 launch");
}

}  // extern "C"
