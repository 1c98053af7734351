// Private interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace coli {

// Workspace carve-up for a call with S tokens.  The status word sits at a
// fixed offset (it persists between calls); the rest is per call.
struct WsLayout {
    size_t status, flags, logits, units, tiles, qx, dx, qh, dh, Y, hs, slots, qxs, qhs, total;
};

// Tiles of the batch-union kernels for large batches: up to PF_TOK pairs of
// one unit.  A unit of n pairs makes ceil(n / PF_TOK) tiles, so a call makes
// at most floor(pairs / PF_TOK) + units of them.
constexpr int PF_TOK = 32;
__host__ __device__ inline int pf_tile_bound(int S, int K, int E, int n_shared) {
    const int P = S * K;
    const int umax = (P < E ? P : E) + n_shared;
    return (P + S * n_shared) / PF_TOK + umax;
}

// Release flags of the persistent kernel's barriers: one per workgroup
// (FLAG_COPIES of them, FLAG_STRIDE bytes apart), so that every waiting
// workgroup polls a word of its own.
constexpr int FLAG_COPIES = 2048;
constexpr int FLAG_STRIDE = 64;
constexpr int N_FLAGS = 3;   // barrier A, Q8_0(x) published, barrier B

// Word index, inside the first 256 bytes of the workspace, of the four
// barrier words of the persistent layer kernel.
constexpr int WS_SYNC_LAYER = 32;
// Word index of the router launch's arrival counters: one per token (up to
// ROUTE_FUSE_MAX tokens), then one for the tokens whose selection is done.
constexpr int WS_SYNC_ROUTE = 48;
constexpr int ROUTE_FUSE_MAX = 8;
// Word index of the one-token router's epoch: the number of one-token router
// launches on this workspace so far (mod 2^32); a launch tags its published
// logits with epoch + 1 and its selecting workgroup stores epoch + 1.
constexpr int WS_EPOCH = 60;
// Polls before the one-token selection's bounded wait for the published
// logits gives up (a test hook can lower it).
constexpr uint32_t ROUTE_SPIN_LIMIT = 1u << 22;

inline size_t al256h(size_t v) { return (v + 255) & ~(size_t)255; }

// Unit table of a call, as int32 words: [0] units, [1] routed units,
// [2] valid routed pairs, [3] 0, then uexp[umax] (expert id, -1 = shared),
// uoff[umax + 1] (first pair of each unit), pairs[P + S] (pair slots grouped
// by unit); then, 16-byte aligned, ublob[umax] (blob pointers).
struct UnitTable {
    int umax, words;      // units at most; int32 words before ublob
    int uexp, uoff, pairs;
    size_t ublob, total;  // byte offsets
};
__host__ __device__ inline UnitTable unit_table(int S, int K, int E) {
    UnitTable u;
    const int P = S * K;
    u.umax = (P < E ? P : E) + 1;
    u.uexp = 4;
    u.uoff = u.uexp + u.umax;
    u.pairs = u.uoff + u.umax + 1;
    u.words = u.pairs + P + S;
    u.ublob = ((size_t)4 * u.words + 15) & ~(size_t)15;
    u.total = u.ublob + (size_t)8 * u.umax;
    return u;
}

// mx: MXFP4 experts, whose grouped kernels also take the Q8_0 codes of x
// and of h split for the matrix cores (split_e4m3: 64 bytes per block).
inline WsLayout ws_layout(int H, int I, int E, int K, int S, bool mx = false) {
    WsLayout L;
    const size_t slots = (size_t)S * (size_t)(K + 1);
    L.status = 0;
    L.flags = 256;
    L.logits = L.flags + (size_t)N_FLAGS * FLAG_COPIES * FLAG_STRIDE;
    L.units = al256h(L.logits + 4 * (size_t)S * (size_t)E);
    L.tiles = al256h(L.units + unit_table(S, K, E).total);
    L.qx = al256h(L.tiles + 16 * (size_t)(1 + pf_tile_bound(S, K, E, 1)));
    L.dx = al256h(L.qx + (size_t)S * (size_t)H);
    L.qh = al256h(L.dx + 4 * (size_t)S * (size_t)(H / 32));
    L.dh = al256h(L.qh + slots * (size_t)I);
    L.Y = al256h(L.dh + 4 * slots * (size_t)(I / 32));
    L.hs = al256h(L.Y + 4 * slots * (size_t)H);
    L.slots = al256h(L.hs + 4 * (size_t)(S < 2 ? S : 2) * (size_t)I);
    L.qxs = al256h(L.slots + 8 * (size_t)E * (size_t)(S < 4 ? S : 4));   // tagged logits of up to 4 tokens
    L.qhs = al256h(L.qxs + (mx ? 2 * (size_t)S * (size_t)H : 0));
    L.total = al256h(L.qhs + (mx ? 2 * slots * (size_t)I : 0));
    return L;
}

// Arguments of the forward kernels (passed by value).
struct FwdArgs {
    const float *x;                // [S, H]
    const int32_t *idx;            // [S, K]
    const float *w;                // [S, K]
    const uint8_t *const *blobs;   // device array [E]
    const uint8_t *shared;         // shared expert blob or null
    const int8_t *qx;              // [S, H]   Q8_0(x) codes
    const float *dx;               // [S, H/32]
    const uint8_t *units;          // unit table of the call (workspace), or null: built per workgroup
    int8_t *qh;                    // [S*(K+1), I]   Q8_0(h) codes per pair slot
    float *dh;                     // [S*(K+1), I/32]
    float *Y;                      // [S*(K+1), H]   expert outputs per pair slot
    int32_t *tiles;                // tile list of the grouped kernels (workspace)
    float *out;                    // [S, H]
    uint32_t *status;
    int S, H, I, E, K, n_shared;
    int pend_mode;                 // 0: all units, 1: skip pending experts, 2: only pending
    int shared_done;               // 1: the router launch wrote the shared expert's h to hs
    const float *hs;               // [S, I]  the shared expert's h, binary32 (with shared_done)
    int group;                     // 0: per-row scales; else one scale per `group` codes of a row
    int mx;                        // 1: MXFP4 codes and E8M0 scales (group is then 32)
    uint8_t *qxs;                  // MXFP4 grouped kernels: Q8_0(x) split [S][H / 32][64] (split_e4m3)
    uint8_t *qhs;                  // and Q8_0(h) split [S*(K+1)][I / 32][64]
    uint32_t pend[32];             // bit e: expert e pending
};

// Router launch of coli_moe_layer for up to ROUTE_FUSE_MAX tokens: logits,
// Q8_0(x), the top-K of each token (by the last workgroup to finish its
// logits) and the unit table (by the last token to be selected).
struct RouteArgs {
    const float *x, *W, *bias;
    float *logits;
    uint32_t *status;
    int8_t *qx;
    float *dx;
    int32_t *idx_out;
    float *w_out;
    const uint8_t *const *blobs;
    const uint8_t *shared;
    uint8_t *units;
    uint32_t *sync;
    float *hs;                     // with sg: the shared expert's h [S, I], binary32
    uint64_t *slots;               // up to 4 tokens: [S][E] published logits, (tag << 32) | binary32 bits
    uint32_t *epoch;               // one token: the workspace's router epoch (WS_EPOCH)
    uint32_t spin_limit;           // one token: polls before the selection's wait gives up
    uint32_t tag_skew;             // one token: 0, or (test hook) 1 to wait for a tag no one writes
    int S, H, E, K, n_shared, norm;
    int I, bits, group, mx;        // expert shape, code width, scale group, MXFP4 (for sg)
    int sg;                        // 1: the launch also runs the shared expert's gate/up tiles
    float rsf;
};
hipError_t launch_route_fused(const RouteArgs &r, hipStream_t st);
size_t route_fused_lds(const RouteArgs &r);
// Shared-expert half tiles in the router launch: up to two tokens (one pass
// over the half tile's 32 rows) and at most 128 KiB of those rows per
// workgroup.
inline bool route_shared_fits(int S, int H, int bits) {
    return S <= 2 && (size_t)32 * H * bits / 8 <= 128 * 1024;
}

// Router logits; with qx non-null the same launch writes Q8_0(x) to qx / dx.
hipError_t launch_router_logits(const float *x, const float *W, float *logits, uint32_t *status,
                                int S, int H, int E, int8_t *qx, float *dx, hipStream_t st);
hipError_t launch_quant_x(const float *x, int8_t *qx, float *dx, uint8_t *qxs, uint32_t *status, int S, int H,
                          hipStream_t st);
hipError_t launch_router_select(const float *logits, const float *bias, int32_t *idx, float *w,
                                uint32_t *status, int S, int E, int K, float rsf, int norm,
                                hipStream_t st);

// Kernel kinds for timing.
enum KernelKind {
    KK_ROUTER_LOGITS = 0,
    KK_ROUTER_SELECT = 1,
    KK_GATEUP = 2,
    KK_DOWN = 3,
    KK_COMBINE = 4,
    KK_LAYER = 5,
    KK_FORWARD_PERSISTENT = 6,
    KK_QUANT_X = 7,
    KK_GROUP = 8,
    KK_COUNT = 9
};

// Timing hooks implemented by the API layer.
// While kernel timing is on and a timed kind is open on this thread, hands
// out a start / stop event pair for the next launch (recorded by the
// runtime at the kernel's own start and end) and files it under that kind.
bool timing_pair(hipEvent_t *start, hipEvent_t *stop);

// Every kernel of the library is launched through here.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t smem, hipStream_t st,
                         Args &&...args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timing_pair(&e0, &e1))
        hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)smem, st, e0, e1, 0, std::forward<Args>(args)...);
    else
        hipLaunchKernelGGL(kern, grid, block, smem, st, std::forward<Args>(args)...);
    return hipGetLastError();
}

// Raises `kern`'s dynamic-LDS limit to at least `smem` bytes (once per
// kernel and size, so launches under stream capture only enqueue work).
hipError_t ensure_dyn_smem(const void *kern, size_t smem);
void timing_before(int kind, hipStream_t st);
void timing_after(int kind, hipStream_t st);

// Extra arguments of the persistent layer kernel.
struct LayerArgs {
    const float *router_w;   // [E, H]   (routing computed in the kernel)
    const float *bias;       // [E] or null
    int32_t *idx_out;        // [S, K]   routing written by the kernel
    float *w_out;            // [S, K]
    float *logits;           // [S, E]   workspace
    float rsf;
    int norm;
    int8_t *qx;              // [S, H]   workspace: Q8_0(x)
    float *dx;               // [S, H/32]
    uint32_t *sync;          // 4 barrier words in the workspace
    uint8_t *flags;          // release flags (N_FLAGS x FLAG_COPIES, FLAG_STRIDE apart)
};

// The persistent layer kernel: route = true computes the routing itself
// (coli_moe_layer); route = false takes it from the arguments (coli_moe_forward).
size_t route_fused_smem(int S, int K, int E);
// Down projection + combine by output-row tiles (up to 8 tokens).
hipError_t launch_down_rows(const FwdArgs &a, int bits, hipStream_t st);
size_t down_rows_smem(int S, int I, int E, int K, int n_shared, int group, int bits);
hipError_t launch_layer(const FwdArgs &a, const LayerArgs &l, bool route, int bits, hipStream_t st);
size_t layer_smem(int S, int H, int I, int E, int K, int n_shared);

hipError_t launch_gateup(const FwdArgs &a, int bits, hipStream_t st);
hipError_t launch_down(const FwdArgs &a, int bits, hipStream_t st);
hipError_t launch_combine(const FwdArgs &a, hipStream_t st);
hipError_t launch_logits_tiled(const float *x, const float *W, float *logits, uint32_t *status, int S, int H, int E,
                               hipStream_t st);
hipError_t launch_group(const int32_t *idx, int S, int K, int E, int n_shared, uint8_t *units, int32_t *tiles,
                        uint32_t *status, hipStream_t st);
size_t pf_group_smem(int S, int K, int E);
hipError_t launch_pf_gateup(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st);
hipError_t launch_pf_down(const FwdArgs &a, const int32_t *tiles, int bits, hipStream_t st);
hipError_t launch_pf_gateup_mx(const FwdArgs &a, const int32_t *tiles, hipStream_t st);
hipError_t launch_pf_down_mx(const FwdArgs &a, const int32_t *tiles, hipStream_t st);
size_t forward_smem_max(int S, int H, int I, int E, int K, int n_shared, int group);

hipError_t launch_debug_unpack(int bits, int rows, int cols, const void *src, int8_t *out,
                               hipStream_t st);
hipError_t launch_debug_block_dots(int bits, int rows, int cols, const void *src, const int8_t *q,
                                   int32_t *out, hipStream_t st);
hipError_t launch_debug_expf(int64_t n, const float *x, float *y, hipStream_t st);
hipError_t launch_debug_mfma_i8(const int8_t *a, const int8_t *b, int32_t *c, hipStream_t st);
hipError_t launch_debug_mfma_i8_16(const int8_t *a, const int8_t *b, int32_t *c, hipStream_t st);
hipError_t launch_debug_mfma_f8f6f4(int fa, int fb, const uint8_t *a, const uint8_t *b, const uint8_t *sa,
                                    const uint8_t *sb, float *c, hipStream_t st);
// Measured roofs: ROOF_GRID workgroups of 256 threads, one sink word per thread.
constexpr int ROOF_GRID = 2048;
hipError_t launch_roof_stream(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_roof_mfma(int iters, int32_t *sink, hipStream_t st);
hipError_t launch_debug_q8_0(int rows, int cols, const float *v, int8_t *q, float *d,
                             hipStream_t st);

}  // namespace coli
