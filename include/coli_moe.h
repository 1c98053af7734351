/*
 * coli_moe.h — C ABI of the routed-expert MoE layer on MI355X (gfx950).
 *
 * The layer (colibrì README v1.0, "What's implemented": DeepSeek-V3-style
 * sigmoid router with routed_scaling_factor and a shared expert; integer-dot
 * kernels over Q8_0-style int8 activations; int8 / packed int4 / packed int2
 * weights with per-row scales; batch-union MoE):
 *
 *   logits = W_r x                      (binary32, fixed reduction order)
 *   sel    = top-K of sigmoid(logits) + bias, ties to the lower expert id
 *   w_k    = sigmoid_k / sum(sigmoid_sel) * routed_scaling_factor
 *   out    = sum_k w_k * FFN_{sel_k}(x) + FFN_shared(x)
 *   FFN(x) = W_d Q8_0( silu(W_g Q8_0(x)) * (W_u Q8_0(x)) )
 *
 * Every binary32 operation happens in one defined order, so the results are
 * bitwise reproducible and independent of the batch size.
 *
 * Conventions for every call:
 *  - Pointers documented "device" are HIP device (or managed) memory; "host"
 *    pointers are read before the call returns.  The library allocates no
 *    device memory: scratch space is the caller's workspace.
 *  - stream / event arguments are hipStream_t / hipEvent_t passed as void*;
 *    NULL means the default stream.  Calls enqueue work and return without
 *    synchronising, except coli_moe_status.
 *  - Return value 0 on success or a negative COLI_E* code; the message of the
 *    last failure on this thread is available from coli_moe_last_error().
 *  - Conditions only the device can see (non-finite values, an out-of-range
 *    or repeated expert index, a routed expert that is not resident) set bits
 *    of a status word inside the workspace; they are sticky until
 *    coli_moe_status() reads and clears them.  When the status is non-zero
 *    the outputs of the calls since the last read are unspecified.
 *  - There is no CPU fallback: without a usable gfx950 device every compute
 *    call fails with COLI_EHIP (colibrì README v1.0, "Experimental resident
 *    CUDA backend": a requested GPU backend that cannot run fails at startup
 *    instead of silently falling back to the CPU).
 *  - Hidden states, router gate, outputs and expert blobs are accessed with
 *    16-byte vector loads and stores: x, router_w, out and shared_blob must
 *    be 16-byte aligned (COLI_EINVAL otherwise), and so must every pointer of
 *    the expert blob table (not checked: the table lives on the device).
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_OK 0
#define COLI_EINVAL (-1)        /* bad dimension, pointer, index or size */
#define COLI_ENONFINITE (-2)    /* NaN/Inf in an input, or undefined gate weights */
#define COLI_EHIP (-3)          /* a HIP runtime call failed */
#define COLI_ENOTRESIDENT (-4)  /* a routed expert's blob pointer is NULL */
#define COLI_EWORKSPACE (-5)    /* workspace too small for this call */

/* coli_moe_dims.wformat */
#define COLI_WFMT_INT 0         /* integer codes of wbits bits, per-row or group f32 scales */
#define COLI_WFMT_MXFP4 1       /* MXFP4: E2M1 codes, one E8M0 scale per 32 codes of a row */
/* the debug hooks' `bits` value selecting MXFP4 codes */
#define COLI_MXFP4 (-4)

/* Most tokens one call takes (n_tokens, max_tokens): the workspace's int32
 * pair and unit counts stay far from overflow below it.  Larger batches are
 * split by the caller; COLI_EINVAL (0 from coli_moe_workspace_bytes)
 * beyond it. */
#define COLI_MAX_TOKENS 65536

/* Layer shape.  All fields are preconditions checked on every call. */
typedef struct coli_moe_dims {
    int32_t hidden;               /* H: multiple of 256 (router order) */
    int32_t inter;                /* I: expert intermediate size, multiple of 32 */
    int32_t n_experts;            /* E: routed experts, 1..1024 */
    int32_t top_k;                /* K: 1..min(E, 32) */
    int32_t n_shared;             /* 0 or 1 shared expert */
    int32_t wbits;                /* 8, 4 or 2: weight code width */
    float routed_scaling_factor;  /* multiplies the gate weights */
    int32_t norm_topk_prob;       /* 1: weights renormalised over the K selected */
    int32_t group_size;           /* 0: one f32 scale per weight row; with wbits = 4, a power of two in 32..512
                                     dividing H and I: one f32 scale per group_size consecutive codes
                                     of a row (JustVugg/colibri, "Get started" / "Other supported
                                     models": the group-scaled "int4-g64" containers) */
    int32_t wformat;              /* COLI_WFMT_INT, or COLI_WFMT_MXFP4 (JustVugg/colibri, "Other supported
                                     models": routed experts streamed in their checkpoints' native MXFP4,
                                     without conversion), which needs wbits = 4, group_size = 0 and I a
                                     multiple of 128 */
} coli_moe_dims;

/*
 * Size in bytes of one expert blob.  Layout (row-major, reduction dimension
 * contiguous, each section starting on a 256-byte boundary):
 *   [gate codes: I rows x H*bits/8][up codes: I rows x H*bits/8]
 *   [down codes: H rows x I*bits/8][gate scales: I f32][up scales: I f32]
 *   [down scales: H f32]
 * Codes per 32-element block: int8 as bytes; int4 16 bytes, byte j = code j
 * (bits 0-3) | code j+16 (bits 4-7); int2 8 bytes, byte j = code j+8i in bits
 * 2i..2i+1.  Two's complement.  (README v1.0 "The idea": about 19 MB per
 * expert at int4; GLM-5.2 shape gives 18 915 328 bytes.)  With group_size
 * G > 0 the three scale sections hold one f32 per G codes of a row,
 * row-major: gate and up [I][H/G], down [H][I/G] (21 233 664 bytes at the
 * GLM-5.2 shape with G = 64, int4).  A row's dot product is then
 * acc = fmaf(d_b * s[row][32 b / G], isum_b, acc) over blocks b ascending
 * (d_b the activation block scale), with no scale after the chain.
 * With wformat = COLI_WFMT_MXFP4 (OCP Microscaling FP4) the code sections
 * hold 4-bit E2M1 codes, byte j of a row = element 2j (bits 0-3) | element
 * 2j + 1 (bits 4-7), and the three scale sections one E8M0 byte per 32
 * codes of a row, row-major: gate and up [I][H/32], down [H][I/32]
 * (20 054 016 bytes at the GLM-5.2 shape).  With t_j = 2 v_j (an integer in
 * [-12, 12]) and x_b the block's scale byte, a row's dot product is
 * acc = fmaf(d_b * 2^(x_b - 128), sum_j t_j q_j, acc) over blocks b ascending,
 * the multiplier one binary32 product, no scale after the chain.
 * Returns 0 when dims are invalid.
 */
size_t coli_moe_expert_bytes(const coli_moe_dims *dims);

/* Workspace bytes needed for calls with up to max_tokens tokens.  The pages
 * define no scratch memory: the workspace is this library's way of keeping
 * every device allocation with the caller (colibrì README v1.0,
 * "Experimental resident CUDA backend": resident tensors are uploaded once
 * and reused, and the runtime keeps a fixed per-device reserve).  It holds
 * the status word, the router's logits, the call's unit table, Q8_0(x),
 * Q8_0(h) and the per-pair expert outputs.  It must be zero-filled once
 * before its first use (the status word lives in it); afterwards the
 * library keeps it consistent.  Returns 0 if dims are invalid or
 * max_tokens is outside 0..COLI_MAX_TOKENS. */
size_t coli_moe_workspace_bytes(const coli_moe_dims *dims, int32_t max_tokens);

/*
 * Router: logits, bias-corrected top-K and gate weights for n_tokens tokens
 * ("Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM", "How it
 * works (validated core mechanics)": the bias ranks only, weights are the
 * unbiased sigmoids renormalised, lower id wins a tie; non-finite input is
 * rejected).
 *   x           device f32 [n_tokens, H]
 *   router_w    device f32 [E, H]  (nn.Linear layout)
 *   router_bias device f32 [E] or NULL (zeros)
 *   topk_idx    device int32 [n_tokens, K] out, rank order
 *   topk_w      device f32  [n_tokens, K] out, same order
 * n_tokens == 0 is a no-op.  Non-finite x / W_r / bias / logits set
 * COLI_ENONFINITE in the status word.
 */
int coli_moe_route(const coli_moe_dims *dims, int32_t n_tokens, const float *x,
                   const float *router_w, const float *router_bias, int32_t *topk_idx,
                   float *topk_w, void *ws, size_t ws_bytes, void *stream);

/*
 * Expert FFNs and combine for n_tokens tokens with given routing (README
 * v1.0 "What's implemented": SwiGLU experts on Q8_0 activations, shared
 * expert, batch-union: each unique expert of the call is read once and
 * applied to every token routed to it).
 *   x            device f32 [n_tokens, H]
 *   topk_idx     device int32 [n_tokens, K], topk_w device f32 [n_tokens, K]
 *   expert_blobs device array [E] of device blob pointers; NULL = not resident
 *   shared_blob  device blob, or NULL when n_shared == 0
 *   pending_mask host uint8 [E] or NULL: experts whose blobs are still being
 *                staged; they run after the stream waits for pending_ready
 *                (a hipEvent_t, may be NULL), all others run before it;
 *                batches of 9 or more tokens wait for the event first
 *   out          device f32 [n_tokens, H]; each element written once
 * Batches of up to 8 tokens run the decode kernels (GEMV-shaped, bound by
 * HBM bandwidth; down and combine in one launch by output rows while its
 * LDS stays within 80 KiB).  Larger batches run the grouped kernels (per-row
 * scales or groups of 64; other group sizes keep the decode kernels): one
 * launch builds
 * the unit table and its tiles of up to 32 (token, expert) pairs of one
 * expert, then gate/up and down are int8 matrix-core products per (32-row
 * tile, pair tile) with the exact per-block f32 chains, then the combine.
 * Their grouping launch holds the pair list in LDS, which limits n_tokens to
 * about 4400 at top_k = 8 (COLI_EINVAL beyond 160 KiB).
 */
int coli_moe_forward(const coli_moe_dims *dims, int32_t n_tokens, const float *x,
                     const int32_t *topk_idx, const float *topk_w,
                     const void *const *expert_blobs, const void *shared_blob,
                     const uint8_t *pending_mask, void *pending_ready, float *out, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * The whole layer in one call: the result of coli_moe_route followed by
 * coli_moe_forward (same bits), with the routing also written to topk_idx /
 * topk_w.  By default it runs the multi-launch kernels of those two calls,
 * with Q8_0(x) produced once by the router-logit launch; up to 8 tokens that
 * launch also selects the routing and writes the call's unit table, and up
 * to 2 tokens (when the shared expert's 16-row gate/up half tiles hold at
 * most 128 KiB of codes) it also runs the shared expert's gate/up, whose
 * pairs do not depend on the routing, leaving its h in the workspace for the
 * gate/up launch to quantise.  A persistent
 * single-launch kernel (router, gate/up and down+combine phases separated
 * by grid barriers) serves up to 8 tokens when selected with
 * coli_moe_debug_force_path.  Arguments as for coli_moe_route and
 * coli_moe_forward.
 */
int coli_moe_layer(const coli_moe_dims *dims, int32_t n_tokens, const float *x,
                   const float *router_w, const float *router_bias,
                   const void *const *expert_blobs, const void *shared_blob, int32_t *topk_idx,
                   float *topk_w, float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * coli_moe_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it): the same launches and
 * the same bits as coli_moe_layer, with a library-owned scratch array of
 * 32 MiB per GPU (a static device array, kept until the process ends) as
 * the workspace.  The call allocates nothing.
 *   n_tokens     at most what fits 32 MiB of workspace
 *                (coli_moe_workspace_bytes <= 32 MiB: 132 tokens at the
 *                GLM-5.2 shape); beyond it COLI_EWORKSPACE, nothing launched
 *   status_out   device uint32 or NULL: after the layer's kernels, one more
 *                launch moves the scratch's status word there and clears it:
 *                0, or bit 0 (1) non-finite input or gate weights, bit 1 (2)
 *                an expert index out of range or repeated in a token, bit 2
 *                (4) a routed expert's blob pointer is NULL, bit 3 (8) a
 *                kernel's bounded wait for the other workgroups of its launch
 *                gave up; with NULL the bits are cleared unread
 * Other arguments as for coli_moe_layer.  Every call on one GPU shares
 * that GPU's scratch, so calls that overlap on one GPU (several streams or
 * threads at once) race and give unspecified results; calls on one stream
 * are safe.
 */
int coli_moe_layer_noalloc(const coli_moe_dims *dims, int32_t n_tokens, const float *x,
                           const float *router_w, const float *router_bias,
                           const void *const *expert_blobs, const void *shared_blob,
                           int32_t *topk_idx, float *topk_w, float *out, uint32_t *status_out,
                           void *stream);

/*
 * Expert staging (README v1.0 "What's implemented": async expert readahead —
 * the next experts are fetched while the current ones are multiplied).
 * Enqueues n host-to-device copies of bytes_each bytes, host_src[i] (pinned
 * host memory) to dev_dst[i] (device), on copy_stream, then records
 * done_event (may be NULL).  host_src / dev_dst are host arrays of pointers,
 * read before return; the source memory must stay valid until the event
 * completes.
 */
int coli_moe_stage_experts(int32_t n, const void *const *host_src, void *const *dev_dst,
                           size_t bytes_each, void *copy_stream, void *done_event);

/* Synchronises `stream`, returns the status recorded in the workspace since
 * the last read (0 or the most severe COLI_E* code) and clears it.  This is
 * how conditions only the kernels see reach the caller: non-finite input is
 * rejected ("Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM",
 * "How it works (validated core mechanics)": the router's self-test refuses
 * NaN), and a failure is reported, never hidden behind a fallback (colibrì
 * README v1.0, "Experimental resident CUDA backend").  COLI_EINVAL when ws
 * is NULL, COLI_EHIP when the synchronisation or the read fails. */
int coli_moe_status(void *ws, void *stream);

/* Message of the last failure on the calling thread ("" if none): the text
 * behind a non-zero return, so that a refused call says why (colibrì README
 * v1.0, "Experimental resident CUDA backend": failures are reported rather
 * than silently worked around).  The pointer stays valid until the thread's
 * next failing call. */
const char *coli_moe_last_error(void);

/*
 * Kernel timing.  While enabled, every kernel launched by the library
 * carries a pair of HIP events that the runtime records at the kernel's own
 * start and end (hipExtLaunchKernel); coli_moe_timing_read() synchronises the
 * recorded events and returns the accumulated milliseconds and launch count
 * of one kernel kind (0 router logits, 1 router select, 2 gate/up, 3 down,
 * 4 combine, 5 persistent layer, 6 persistent forward, 7 Q8_0 of the
 * hidden states, 8 grouping of the grouped kernels), then resets that kind.
 * For measurement only.
 */
int coli_moe_timing_enable(int32_t enable);
int coli_moe_timing_read(int32_t kind, double *total_ms, int64_t *launches);

/* ---- test hooks: the same device functions as the production kernels ---- */

/* Kernel family for subsequent calls in this process: 0 automatic (default:
 * the multi-launch decode kernels up to 8 tokens, the grouped kernels
 * beyond), 1 multi-launch decode kernels at any batch size, 2 persistent
 * (single-launch) kernels — a forced persistent kernel fails with
 * COLI_EINVAL where it does not apply (pending experts, more than 8 tokens,
 * a shape beyond 160 KiB of LDS) — 3 grouped kernels at any batch size. */
int coli_moe_debug_force_path(int32_t path);

/* Failure-path hook for later calls in this process (not for concurrent
 * calls).  The router launch of one to four tokens (at most 256 experts)
 * selects in one workgroup that waits, bounded, for every logit of the
 * launch; the wait
 * gives up after `spins` polls (0: the default bound, 2^22).  With
 * unreachable = 1 (spins must then be nonzero) it waits for a tag that no
 * workgroup writes, so it always gives up: coli_moe_status then reports
 * COLI_EHIP (a timed-out wait), the router writes a unit table holding the
 * shared expert alone (with several tokens, every routing weight 0), and
 * every launch still ends normally, so `out` is the shared expert's output.
 * unreachable = 0 restores the normal wait.
 * Returns COLI_EINVAL
 * for unreachable outside {0, 1} or an unreachable wait without a bound. */
int coli_moe_debug_route_wait(uint32_t spins, int32_t unreachable);

/* Unpacks n_rows packed rows of `cols` codes (device src, row stride
 * cols*bits/8 bytes) into device int8 out [n_rows, cols].  bits = COLI_MXFP4
 * reads MXFP4 rows (4 bits a code) and gives twice each E2M1 value; the
 * block dots then use those doubled values. */
int coli_moe_debug_unpack(int32_t bits, int32_t n_rows, int32_t cols, const void *src,
                          int8_t *out, void *stream);

/* Exact int32 block dot products isum[r, b] = sum_{j<32} w[r, 32b+j] * q[32b+j]
 * of n_rows packed rows (device src) with a device int8 vector q [cols];
 * out device int32 [n_rows, cols/32]. */
int coli_moe_debug_block_dots(int32_t bits, int32_t n_rows, int32_t cols, const void *src,
                              const int8_t *q, int32_t *out, void *stream);

/* Router logits only: device f32 logits [n_tokens, E]. */
int coli_moe_debug_logits(const coli_moe_dims *dims, int32_t n_tokens, const float *x,
                          const float *router_w, float *logits, void *stream);

/* The device exponential used by the router and SwiGLU, element-wise on
 * device f32 arrays of n elements. */
int coli_moe_debug_expf(int64_t n, const float *x, float *y, void *stream);

/* One v_mfma_i32_32x32x32_i8 on raw lane registers: lane l (of 64) takes
 * its A and B registers from bytes 16 l .. 16 l + 15 of device a and b and
 * writes its 16 int32 result registers to device c[16 l .. 16 l + 15] (the
 * lane layout of the prefill kernels is checked against a host matmul). */
int coli_moe_debug_mfma_i8(const int8_t *a, const int8_t *b, int32_t *c, void *stream);

/* One v_mfma_i32_16x16x32_i8 on raw lane registers: lane l (of 64) takes
 * its A and B registers from bytes 8 l .. 8 l + 7 of device a and b and
 * writes its 4 int32 result registers to device c[4 l .. 4 l + 3] (the lane
 * layout of the prefill kernels' tiles of at most 16 pairs is checked
 * against a host matmul). */
int coli_moe_debug_mfma_i8_16(const int8_t *a, const int8_t *b, int32_t *c, void *stream);

/* One v_mfma_scale_f32_32x32x64_f8f6f4 on raw lane registers: lane l (of
 * 64) takes its A and B registers from bytes 32 l .. 32 l + 31 of device a
 * and b and its E8M0 scales from byte l of device sa and sb, and writes its
 * 16 binary32 results to device c[16 l .. 16 l + 15].  fmt_a / fmt_b: 0 FP8
 * E4M3, 4 FP4 E2M1 (A only); COLI_EINVAL for other pairs.  The lane layout
 * and scaling the MXFP4 prefill kernels assume are checked against a host
 * model through it. */
int coli_moe_debug_mfma_f8f6f4(int32_t fmt_a, int32_t fmt_b, const uint8_t *a, const uint8_t *b,
                               const uint8_t *sa, const uint8_t *sb, float *c, void *stream);

/* Q8_0 of device f32 v [n_rows, cols] into device int8 q and f32 d
 * [n_rows, cols/32], with the device quantiser the kernels use. */
int coli_moe_debug_q8_0(int32_t n_rows, int32_t cols, const float *v, int8_t *q, float *d,
                        void *stream);

/* ---- measured roofs (benchmarking) ----------------------------------
 * Reference kernels for the ceilings the layer's kernels are compared
 * with: a plain streaming read of HBM and the int8 matrix cores alone.
 * Both run 2048 workgroups of 256 threads and write one 32-bit word per
 * thread to a device `sink` of coli_moe_roof_sink_words() words (the
 * values are meaningless; they keep the work alive).  Enqueued on
 * `stream`; time them with events around the call. */
size_t coli_moe_roof_sink_words(void);

/* Reads `bytes` (a multiple of 16) of device memory at `src` once, with
 * 16-byte non-temporal loads, eight per thread in flight.  COLI_EINVAL on
 * NULL pointers or a size that is not a multiple of 16. */
int coli_moe_roof_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Every wavefront runs `iters` (>= 1) rounds of four independent
 * v_mfma_i32_32x32x32_i8 accumulations on register operands:
 * 2048 * 4 * iters * 4 * 65536 integer operations (multiply and add
 * counted apart).  COLI_EINVAL on iters < 1 or a NULL sink. */
int coli_moe_roof_mfma_i8(int32_t iters, int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* COLI_MOE_H */
