/*
 * CPU oracle of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never links, imports or calls it, and
 * this file shares no code, header or table with that path.
 *
 * Plain C11, built with -O2 -ffp-contract=off and without -ffast-math:
 * every floating-point operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even, and every fused multiply-add is an explicit
 * fmaf().  Each token's arithmetic is single-threaded and sequential.  The
 * same source is also built with OpenMP: then the loops over tokens, which
 * share no data, run their iterations on several threads, and nothing else
 * changes, so both builds give the same bits (a CPU test checks this).  Where the pages leave an operation order or a rounding
 * rule open, the reading taken is stated at the function; the layer's output
 * is then one exactly defined binary32 value per element.
 *
 * Sources, by page title and section:
 *  [README]  colibrì README v1.0 (aihot.virxact.com mirror),
 *            "What's implemented" and "The idea".
 *  [ROUTER]  "Colibri (colibrì): GLM-5.2 local inference on 25 GB of RAM"
 *            (ai-infrastructure.net), "How it works (validated core
 *            mechanics)": the sigmoid noaux_tc router and its self-test.
 *  [LAYOUT]  JustVugg/colibri (topgit.dev), the repository layout: the shared
 *            routed-expert FFN kernel header (SwiGLU experts).
 *  [GS64]    JustVugg/colibri (topgit.dev), "Get started" and "Other
 *            supported models": the group-scaled int4 containers (one scale
 *            per 64 weights of a row, "int4-g64"), preferred to per-row int4.
 *  [MXFP4]   JustVugg/colibri (topgit.dev), "Other supported models": models
 *            whose routed experts are streamed in their checkpoints' native
 *            4-bit floating-point format, MXFP4, without conversion.  The
 *            format itself is the OCP Microscaling (MX) specification's:
 *            E2M1 elements, one E8M0 power-of-two scale per 32 elements.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OQ_OK 0
#define OQ_EINVAL (-1)
#define OQ_ENONFINITE (-2)
#define OQ_ENOTRESIDENT (-4)
#define OQ_ENOMEM (-6)

/* ------------------------------------------------------------------------
 * Exponential.  The pages do not say how exp is evaluated.  Reading: a
 * Cody-Waite range reduction (Cody & Waite, "Software Manual for the
 * Elementary Functions", 1980) and the degree-7 Taylor polynomial of e^r in
 * Horner form, every step an explicit binary32 operation, so that any
 * implementation following the same steps gets the same bits.
 *   n = rint(x * log2(e));  r = x - n*ln2_hi (exact, one fma);  r -= n*ln2_lo
 *   p = sum_{k=0..7} r^k / k!  (Horner, fmaf);  result = p * 2^n
 * Constants come from the mathematics: ln2_hi = RN32(ln 2),
 * ln2_lo = RN32(ln 2 - ln2_hi), log2e = RN32(1/ln 2), c_k = RN32(1/k!).
 * Range: e^x rounds to +inf above x = 0x1.62e42ep+6 and to 0 below
 * x = -0x1.9fe368p+6 (e^x < 2^-150 there).
 * ---------------------------------------------------------------------- */
static float pow2i(int n) { /* 2^n for -126 <= n <= 127 */
    uint32_t bits = (uint32_t)(n + 127) << 23;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

float oq_expf(float x) {
    if (isnan(x)) return x;
    if (x > 0x1.62e42ep+6f) return INFINITY;
    if (x < -0x1.9fe368p+6f) return 0.0f;
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e430p-1f;
    const float ln2_lo = -0x1.05c610p-29f;
    const float c2 = (float)(1.0 / 2.0), c3 = (float)(1.0 / 6.0), c4 = (float)(1.0 / 24.0);
    const float c5 = (float)(1.0 / 120.0), c6 = (float)(1.0 / 720.0), c7 = (float)(1.0 / 5040.0);
    float t = x * log2e;
    float fn = rintf(t);
    float r = fmaf(-fn, ln2_hi, x);
    r = fmaf(-fn, ln2_lo, r);
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int n = (int)fn;
    if (n > 127) return (p * pow2i(127)) * pow2i(n - 127);
    if (n < -126) return (p * pow2i(n + 64)) * pow2i(-64);
    return p * pow2i(n);
}

/* Logistic function sigma(v) = 1 / (1 + e^-v), one correctly rounded division. */
float oq_sigmoid(float v) { return 1.0f / (1.0f + oq_expf(-v)); }

/* SwiGLU gate: silu(g) * u with silu(g) = g / (1 + e^-g)  [LAYOUT: SwiGLU experts].
 * Reading: the division produces silu(g), which is then multiplied by u. */
float oq_swiglu(float g, float u) { return (g / (1.0f + oq_expf(-g))) * u; }

/* ------------------------------------------------------------------------
 * Q8_0 activation quantisation  [README "What's implemented": integer-dot
 * kernels over Q8_0-style int8 activations].  Blocks of 32 values, one
 * binary32 scale per block.  The pages name the scheme only; reading (the
 * usual Q8_0 block rule):
 *   amax = max_j |v_j|;  d = amax / 127;
 *   q_j = clamp(round_half_away_from_zero(v_j / d), -127, 127), q = 0 when d == 0.
 * n must be a multiple of 32.
 * ---------------------------------------------------------------------- */
void oq_q8_0(const float *v, int n, int8_t *q, float *d) {
    for (int b = 0; b < n / 32; ++b) {
        const float *vb = v + 32 * b;
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(vb[j]));
        float db = amax / 127.0f;
        d[b] = db;
        for (int j = 0; j < 32; ++j) {
            float c = 0.0f;
            if (db != 0.0f) {
                c = roundf(vb[j] / db);
                if (c > 127.0f) c = 127.0f;
                if (c < -127.0f) c = -127.0f;
            }
            q[32 * b + j] = (int8_t)c;
        }
    }
}

/* ------------------------------------------------------------------------
 * Packed weight codes  [README "What's implemented": int8, packed int4 and
 * packed int2 weights with per-row scales, dequantised on use, the packing
 * identical to the int8 container].  Byte layout per 32-element block:
 *   int8: 32 bytes, byte j = code j.
 *   int4: 16 bytes, byte j = code j (bits 0-3) | code j+16 (bits 4-7).
 *   int2:  8 bytes, byte j = code j+8i in bits 2i..2i+1, i = 0..3.
 * Codes are two's complement: int4 in [-8, 7], int2 in [-2, 1].
 * ---------------------------------------------------------------------- */
void oq_unpack(const uint8_t *src, int n, int bits, int8_t *out) {
    for (int b = 0; b < n / 32; ++b) {
        for (int j = 0; j < 32; ++j) {
            int v;
            if (bits == 8) {
                v = (int8_t)src[32 * b + j];
            } else if (bits == 4) {
                int byte = src[16 * b + (j % 16)];
                int nib = (j < 16) ? (byte & 0xF) : (byte >> 4);
                v = (nib >= 8) ? nib - 16 : nib;
            } else {
                int byte = src[8 * b + (j % 8)];
                int f = (byte >> (2 * (j / 8))) & 3;
                v = (f >= 2) ? f - 4 : f;
            }
            out[32 * b + j] = (int8_t)v;
        }
    }
}

/* Byte offsets of an expert blob: [gate codes][up codes][down codes]
 * [gate scales][up scales][down scales], each section 256-byte aligned. */
static uint64_t al256(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

void oq_blob_layout(int H, int I, int bits, uint64_t off[7]) {
    uint64_t gate = (uint64_t)I * (uint64_t)H * (uint64_t)bits / 8u;
    uint64_t down = (uint64_t)H * (uint64_t)I * (uint64_t)bits / 8u;
    off[0] = 0;
    off[1] = al256(off[0] + gate);
    off[2] = al256(off[1] + gate);
    off[3] = al256(off[2] + down);
    off[4] = al256(off[3] + 4u * (uint64_t)I);
    off[5] = al256(off[4] + 4u * (uint64_t)I);
    off[6] = al256(off[5] + 4u * (uint64_t)H);
}

/* Group-scaled blobs [GS64]: the same code sections, then one f32 scale per
 * `group` consecutive codes of each row, row-major: gate and up scales
 * [I][H / group], down scales [H][I / group].  group = 0 is the per-row
 * layout above.  Reading: the group scale replaces the per-row scale (the
 * pages compare the two as alternatives), and groups start at column 0. */
void oq_blob_layout_g(int H, int I, int bits, int group, uint64_t off[7]) {
    if (group == 0) {
        oq_blob_layout(H, I, bits, off);
        return;
    }
    uint64_t gate = (uint64_t)I * (uint64_t)H * (uint64_t)bits / 8u;
    uint64_t down = (uint64_t)H * (uint64_t)I * (uint64_t)bits / 8u;
    uint64_t sgu = 4u * (uint64_t)I * (uint64_t)(H / group), sd = 4u * (uint64_t)H * (uint64_t)(I / group);
    off[0] = 0;
    off[1] = al256(off[0] + gate);
    off[2] = al256(off[1] + gate);
    off[3] = al256(off[2] + down);
    off[4] = al256(off[3] + sgu);
    off[5] = al256(off[4] + sgu);
    off[6] = al256(off[5] + sd);
}

/* ------------------------------------------------------------------------
 * Row dot product of an integer weight row with a Q8_0 vector.
 * isum_b = sum_{j<32} w_{32b+j} * q_{32b+j} exactly in int32 (|isum| <=
 * 32*128*127).  Reading for the floating-point part (the pages leave it
 * open): acc = 0; for b ascending: acc = fmaf(d_b, (float)isum_b, acc);
 * result = acc * row_scale.
 * ---------------------------------------------------------------------- */
int32_t oq_block_isum(const int8_t *w, const int8_t *q) {
    int32_t s = 0;
    for (int j = 0; j < 32; ++j) s += (int32_t)w[j] * (int32_t)q[j];
    return s;
}

float oq_row_dot(const int8_t *w, const int8_t *q, const float *d, int n, float row_scale) {
    float acc = 0.0f;
    for (int b = 0; b < n / 32; ++b)
        acc = fmaf(d[b], (float)oq_block_isum(w + 32 * b, q + 32 * b), acc);
    return acc * row_scale;
}

/* Row dot with group scales [GS64]: gs[g] scales codes g*group ..
 * (g+1)*group - 1 of the row (group a multiple of 32).  The weight of code j
 * is gs[j / group] * w_j, so block b contributes d_b * gs[g(b)] * isum_b.
 * Reading for the order: the same chain over blocks, the block's
 * multiplier being the binary32 product d_b * gs[g(b)]:
 *   acc = 0; for b ascending: acc = fmaf(d_b * gs[32 b / group], isum_b, acc)
 * and no scale after the chain. */
float oq_row_dot_g(const int8_t *w, const int8_t *q, const float *d, int n, const float *gs, int group) {
    float acc = 0.0f;
    for (int b = 0; b < n / 32; ++b) {
        float m = d[b] * gs[(32 * b) / group];
        acc = fmaf(m, (float)oq_block_isum(w + 32 * b, q + 32 * b), acc);
    }
    return acc;
}

/* MXFP4 blobs [MXFP4]: code sections of 4 bits per weight, then one E8M0
 * byte per 32 codes of a row, row-major: gate and up [I][H / 32], down
 * [H][I / 32]; each section 256-byte aligned. */
void oq_blob_layout_mx(int H, int I, uint64_t off[7]) {
    uint64_t gate = (uint64_t)I * (uint64_t)H / 2u;
    uint64_t down = (uint64_t)H * (uint64_t)I / 2u;
    uint64_t sgu = (uint64_t)I * (uint64_t)(H / 32), sd = (uint64_t)H * (uint64_t)(I / 32);
    off[0] = 0;
    off[1] = al256(off[0] + gate);
    off[2] = al256(off[1] + gate);
    off[3] = al256(off[2] + down);
    off[4] = al256(off[3] + sgu);
    off[5] = al256(off[4] + sgu);
    off[6] = al256(off[5] + sd);
}

/* ------------------------------------------------------------------------
 * MXFP4 elements [MXFP4].  An E2M1 code c (4 bits) has sign s = bit 3,
 * exponent field e = bits 2-1 and mantissa bit m = bit 0; its value is
 * (-1)^s * (m / 2) when e == 0 (zero or the subnormal 0.5) and
 * (-1)^s * (1 + m / 2) * 2^(e - 1) otherwise: magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6.  An E8M0 byte x scales by 2^(x - 127); x = 255 is NaN.
 * Twice an E2M1 value is an integer in [-12, 12]; the unpacking below
 * returns that integer so that block sums stay exact integers.
 * Row layout (reading: the element order of checkpoints that store MXFP4
 * two codes per byte): byte j of a row holds element 2j in bits 0-3 and
 * element 2j + 1 in bits 4-7.
 * ---------------------------------------------------------------------- */
float oq_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * ldexpf(1.0f, e - 1);
    return s ? -mag : mag;
}

float oq_e8m0(int x) {
    if (x == 255) return NAN;
    return ldexpf(1.0f, x - 127);
}

void oq_unpack_mx(const uint8_t *src, int n, int8_t *out) {
    /* the 16 values 2 * e2m1(code), taken from oq_e2m1 once per call */
    int8_t twice[16];
    for (int code = 0; code < 16; ++code) twice[code] = (int8_t)(2.0f * oq_e2m1(code));
    for (int j = 0; j < n; ++j) {
        int byte = src[j / 2];
        int code = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        out[j] = twice[code];
    }
}

/* Row dot of an MXFP4 row (t = twice the element values, from
 * oq_unpack_mx) with a Q8_0 vector.  Block b's weights are
 * 2^(x_b - 127) * t_j / 2, so its term is d_b * 2^(x_b - 128) * isum_b with
 * isum_b = sum_j t_j q_j exact.  Reading for the order (that of the
 * group-scaled rows): the block's multiplier is the binary32 product
 * d_b * (e8m0(x_b) / 2) (the halving exact), then
 *   acc = 0; for b ascending: acc = fmaf(multiplier_b, isum_b, acc)
 * and no scale after the chain. */
float oq_row_dot_mx(const int8_t *t, const int8_t *q, const float *d, int n, const uint8_t *x) {
    float acc = 0.0f;
    for (int b = 0; b < n / 32; ++b) {
        float m = d[b] * (oq_e8m0(x[b]) * 0.5f);
        acc = fmaf(m, (float)oq_block_isum(t + 32 * b, q + 32 * b), acc);
    }
    return acc;
}

/* ------------------------------------------------------------------------
 * Router logit  [README "What's implemented" and [ROUTER]: logits of the
 * hidden state against the router gate].  logit = sum_h x_h * w_h in
 * binary32.  Reading for the order (the pages leave it open): 64 partial
 * sums; partial l owns the elements h = 256j + 4l + c (j ascending, then
 * c = 0..3) and accumulates them with fmaf from 0; then six rounds
 * p_l <- p_l + p_{l xor o} for o = 32, 16, 8, 4, 2, 1; the logit is p_0.
 * H must be a multiple of 256.
 * ---------------------------------------------------------------------- */
float oq_router_logit(const float *x, const float *w, int H) {
    float p[64], t[64];
    for (int l = 0; l < 64; ++l) {
        float a = 0.0f;
        for (int j = 0; j < H / 256; ++j)
            for (int c = 0; c < 4; ++c) {
                int h = 256 * j + 4 * l + c;
                a = fmaf(x[h], w[h], a);
            }
        p[l] = a;
    }
    for (int o = 32; o >= 1; o >>= 1) {
        for (int l = 0; l < 64; ++l) t[l] = p[l] + p[l ^ o];
        memcpy(p, t, sizeof p);
    }
    return p[0];
}

/* ------------------------------------------------------------------------
 * Selection and gate weights  [ROUTER]: the selection score is
 * sigmoid(logit) + bias, the bias ranks experts only; the top K are ordered
 * by (score descending, expert id ascending), so the lower id wins a tie;
 * the combination weights are the unbiased sigmoids of the selected experts
 * divided by their sum; routed_scaling_factor multiplies them afterwards
 * ([README]: DeepSeek-V3-style sigmoid router with routed_scaling_factor).
 * Readings: the sum runs over the K selected in rank order starting from
 * the first; no epsilon is added; w_k = (sig_k / sum) * rsf; with
 * norm == 0, w_k = sig_k * rsf.  Non-finite input is rejected [ROUTER].
 * ---------------------------------------------------------------------- */
int oq_select(const float *logit, const float *bias, int E, int K, float rsf, int norm,
              int32_t *idx, float *w, float *sig_out) {
    if (E <= 0 || K < 1 || K > E) return OQ_EINVAL;
    float *sig = (float *)malloc(sizeof(float) * (size_t)E);
    float *score = (float *)malloc(sizeof(float) * (size_t)E);
    char *taken = (char *)calloc((size_t)E, 1);
    if (!sig || !score || !taken) { free(sig); free(score); free(taken); return OQ_ENOMEM; }
    int rc = OQ_OK;
    for (int e = 0; e < E; ++e) {
        float b = bias ? bias[e] : 0.0f;
        if (!isfinite(logit[e]) || !isfinite(b)) rc = OQ_ENONFINITE;
        sig[e] = oq_sigmoid(logit[e]);
        score[e] = sig[e] + b;
        if (sig_out) sig_out[e] = sig[e];
    }
    if (rc == OQ_OK) {
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || score[e] > score[best]) best = e;
            }
            taken[best] = 1;
            idx[k] = best;
        }
        if (norm) {
            float denom = sig[idx[0]];
            for (int k = 1; k < K; ++k) denom = denom + sig[idx[k]];
            if (!(denom > 0.0f)) rc = OQ_ENONFINITE;
            for (int k = 0; k < K; ++k) w[k] = (sig[idx[k]] / denom) * rsf;
        } else {
            for (int k = 0; k < K; ++k) w[k] = sig[idx[k]] * rsf;
        }
    }
    free(sig);
    free(score);
    free(taken);
    return rc;
}

/* ------------------------------------------------------------------------
 * One SwiGLU expert on one token  [LAYOUT: routed-expert SwiGLU FFN;
 * README: integer dots over Q8_0 activations, per-row scales].
 *   g_i = row_dot(gate_i, qx, dx) , u_i = row_dot(up_i, qx, dx)   (i < I)
 *   h_i = swiglu(g_i, u_i);  (qh, dh) = Q8_0(h)
 *   y_r = row_dot(down_r, qh, dh)                                  (r < H)
 * Reading: the down projection consumes Q8_0(h) like every other integer
 * dot in the layer.  Optional debug outputs may be NULL.
 * ---------------------------------------------------------------------- */
/* fmt = 0: integer codes of `bits` bits with per-row (group = 0) or
 * group scales; fmt = 1: MXFP4 (bits 4, group 0: one E8M0 scale per 32
 * codes is part of the format). */
int oq_expert_f(const uint8_t *blob, int H, int I, int bits, int group, int fmt, const int8_t *qx,
                const float *dx, float *y, float *g_out, float *u_out, float *h_out, int8_t *qh_out,
                float *dh_out) {
    if (group != 0 && (group % 32 != 0 || H % group != 0 || I % group != 0)) return OQ_EINVAL;
    if (fmt != 0 && (fmt != 1 || bits != 4 || group != 0)) return OQ_EINVAL;
    uint64_t off[7];
    if (fmt == 1)
        oq_blob_layout_mx(H, I, off);
    else
        oq_blob_layout_g(H, I, bits, group, off);
    int n = H > I ? H : I;
    int8_t *row = (int8_t *)malloc((size_t)n);
    float *g = (float *)malloc(sizeof(float) * (size_t)I);
    float *u = (float *)malloc(sizeof(float) * (size_t)I);
    float *h = (float *)malloc(sizeof(float) * (size_t)I);
    int8_t *qh = (int8_t *)malloc((size_t)I);
    float *dh = (float *)malloc(sizeof(float) * (size_t)(I / 32));
    if (!row || !g || !u || !h || !qh || !dh) {
        free(row); free(g); free(u); free(h); free(qh); free(dh);
        return OQ_ENOMEM;
    }
    uint64_t hrow = (uint64_t)H * (uint64_t)bits / 8u, irow = (uint64_t)I * (uint64_t)bits / 8u;
    if (fmt == 1) {
        const uint8_t *x_g = blob + off[3], *x_u = blob + off[4], *x_d = blob + off[5];
        for (int i = 0; i < I; ++i) {
            oq_unpack_mx(blob + off[0] + (uint64_t)i * hrow, H, row);
            g[i] = oq_row_dot_mx(row, qx, dx, H, x_g + (size_t)i * (H / 32));
            oq_unpack_mx(blob + off[1] + (uint64_t)i * hrow, H, row);
            u[i] = oq_row_dot_mx(row, qx, dx, H, x_u + (size_t)i * (H / 32));
            h[i] = oq_swiglu(g[i], u[i]);
        }
        oq_q8_0(h, I, qh, dh);
        for (int r = 0; r < H; ++r) {
            oq_unpack_mx(blob + off[2] + (uint64_t)r * irow, I, row);
            y[r] = oq_row_dot_mx(row, qh, dh, I, x_d + (size_t)r * (I / 32));
        }
    } else {
        const float *s_g = (const float *)(blob + off[3]);
        const float *s_u = (const float *)(blob + off[4]);
        const float *s_d = (const float *)(blob + off[5]);
        int hg = group ? H / group : 0, ig = group ? I / group : 0;
        for (int i = 0; i < I; ++i) {
            oq_unpack(blob + off[0] + (uint64_t)i * hrow, H, bits, row);
            g[i] = group ? oq_row_dot_g(row, qx, dx, H, s_g + (size_t)i * hg, group)
                         : oq_row_dot(row, qx, dx, H, s_g[i]);
            oq_unpack(blob + off[1] + (uint64_t)i * hrow, H, bits, row);
            u[i] = group ? oq_row_dot_g(row, qx, dx, H, s_u + (size_t)i * hg, group)
                         : oq_row_dot(row, qx, dx, H, s_u[i]);
            h[i] = oq_swiglu(g[i], u[i]);
        }
        oq_q8_0(h, I, qh, dh);
        for (int r = 0; r < H; ++r) {
            oq_unpack(blob + off[2] + (uint64_t)r * irow, I, bits, row);
            y[r] = group ? oq_row_dot_g(row, qh, dh, I, s_d + (size_t)r * ig, group)
                         : oq_row_dot(row, qh, dh, I, s_d[r]);
        }
    }
    if (g_out) memcpy(g_out, g, sizeof(float) * (size_t)I);
    if (u_out) memcpy(u_out, u, sizeof(float) * (size_t)I);
    if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
    if (qh_out) memcpy(qh_out, qh, (size_t)I);
    if (dh_out) memcpy(dh_out, dh, sizeof(float) * (size_t)(I / 32));
    free(row); free(g); free(u); free(h); free(qh); free(dh);
    return OQ_OK;
}

int oq_expert_g(const uint8_t *blob, int H, int I, int bits, int group, const int8_t *qx, const float *dx,
                float *y, float *g_out, float *u_out, float *h_out, int8_t *qh_out, float *dh_out) {
    return oq_expert_f(blob, H, I, bits, group, 0, qx, dx, y, g_out, u_out, h_out, qh_out, dh_out);
}

int oq_expert(const uint8_t *blob, int H, int I, int bits, const int8_t *qx, const float *dx,
              float *y, float *g_out, float *u_out, float *h_out, int8_t *qh_out, float *dh_out) {
    return oq_expert_g(blob, H, I, bits, 0, qx, dx, y, g_out, u_out, h_out, qh_out, dh_out);
}

static int dims_ok(int H, int I, int E, int K, int n_shared, int bits) {
    if (H <= 0 || I <= 0 || H % 256 != 0 || I % 32 != 0) return 0;
    if (E <= 0 || K < 1 || K > E) return 0;
    if (n_shared != 0 && n_shared != 1) return 0;
    if (bits != 8 && bits != 4 && bits != 2) return 0;
    return 1;
}

static int all_finite(const float *v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

/* ------------------------------------------------------------------------
 * Routing of S tokens: logits, selection and weights (see above).
 * logits_out / sig_out ([S,E]) may be NULL.
 * ---------------------------------------------------------------------- */
int oq_moe_route(int H, int E, int K, float rsf, int norm, int S, const float *x,
                 const float *router_w, const float *bias, int32_t *idx, float *w,
                 float *logits_out, float *sig_out) {
    if (H <= 0 || H % 256 != 0 || E <= 0 || K < 1 || K > E || S < 0) return OQ_EINVAL;
    if (!all_finite(x, (size_t)S * (size_t)H) || !all_finite(router_w, (size_t)E * (size_t)H) ||
        (bias && !all_finite(bias, (size_t)E)))
        return OQ_ENONFINITE;
    int rc = OQ_OK;
    /* tokens are independent: each iteration reads its own x row and writes
     * its own rows of the outputs */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int t = 0; t < S; ++t) {
        float *lg = (float *)malloc(sizeof(float) * (size_t)E);
        int r = lg ? OQ_OK : OQ_ENOMEM;
        if (r == OQ_OK) {
            for (int e = 0; e < E; ++e)
                lg[e] = oq_router_logit(x + (size_t)t * H, router_w + (size_t)e * H, H);
            if (logits_out) memcpy(logits_out + (size_t)t * E, lg, sizeof(float) * (size_t)E);
            r = oq_select(lg, bias, E, K, rsf, norm, idx + (size_t)t * K, w + (size_t)t * K,
                          sig_out ? sig_out + (size_t)t * E : NULL);
        }
        free(lg);
        if (r != OQ_OK) {
#ifdef _OPENMP
#pragma omp critical(oq_rc)
#endif
            if (rc == OQ_OK) rc = r;
        }
    }
    return rc;
}

/* ------------------------------------------------------------------------
 * Expert FFNs and combine for S tokens with given routing.
 *   out[t,r] = (fmaf chain over k in rank order of w[t,k] * y_{idx[t,k]}[r],
 *               starting from 0) + y_shared[r]
 * [README "What's implemented": DeepSeek-V3-style router with a shared
 * expert; [ROUTER]: gate-weighted sum over the selected experts].  Readings:
 * the shared expert has the routed experts' format and weight 1 and is added
 * after the routed sum; without a shared expert out is the routed sum.
 * blobs[e] == NULL marks expert e as not resident.
 * ---------------------------------------------------------------------- */
/* One token of oq_moe_forward_g: out_t[r] for r < H (inputs validated). */
static int forward_token(int H, int I, int K, int n_shared, int bits, int group, int fmt, const float *x_t,
                         const int32_t *idx_t, const float *w_t, const uint8_t *const *blobs,
                         const uint8_t *shared_blob, float *out_t) {
    int8_t *qx = (int8_t *)malloc((size_t)H);
    float *dx = (float *)malloc(sizeof(float) * (size_t)(H / 32));
    float *y = (float *)malloc(sizeof(float) * (size_t)H * (size_t)K);
    float *ysh = (float *)malloc(sizeof(float) * (size_t)H);
    int rc = (qx && dx && y && ysh) ? OQ_OK : OQ_ENOMEM;
    if (rc == OQ_OK) oq_q8_0(x_t, H, qx, dx);
    for (int k = 0; k < K && rc == OQ_OK; ++k)
        rc = oq_expert_f(blobs[idx_t[k]], H, I, bits, group, fmt, qx, dx, y + (size_t)k * H, NULL, NULL, NULL,
                         NULL, NULL);
    if (rc == OQ_OK && n_shared)
        rc = oq_expert_f(shared_blob, H, I, bits, group, fmt, qx, dx, ysh, NULL, NULL, NULL, NULL, NULL);
    for (int r = 0; r < H && rc == OQ_OK; ++r) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) acc = fmaf(w_t[k], y[(size_t)k * H + r], acc);
        out_t[r] = n_shared ? acc + ysh[r] : acc;
    }
    free(qx); free(dx); free(y); free(ysh);
    return rc;
}

int oq_moe_forward_f(int H, int I, int E, int K, int n_shared, int bits, int group, int fmt, int S,
                     const float *x, const int32_t *idx, const float *w, const uint8_t *const *blobs,
                     const uint8_t *shared_blob, float *out) {
    if (!dims_ok(H, I, E, K, n_shared, bits) || S < 0) return OQ_EINVAL;
    if (group != 0 && (group % 32 != 0 || H % group != 0 || I % group != 0)) return OQ_EINVAL;
    if (fmt != 0 && (fmt != 1 || bits != 4 || group != 0)) return OQ_EINVAL;
    if (n_shared && !shared_blob) return OQ_ENOTRESIDENT;
    if (!all_finite(x, (size_t)S * (size_t)H) || !all_finite(w, (size_t)S * (size_t)K))
        return OQ_ENONFINITE;
    for (int t = 0; t < S; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t e = idx[(size_t)t * K + k];
            if (e < 0 || e >= E) return OQ_EINVAL;
            for (int k2 = 0; k2 < k; ++k2)
                if (idx[(size_t)t * K + k2] == e) return OQ_EINVAL;
            if (!blobs[e]) return OQ_ENOTRESIDENT;
        }
    int rc = OQ_OK;
    /* tokens are independent: each iteration reads its own x, idx and w rows
     * and writes its own out row */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int t = 0; t < S; ++t) {
        int r = forward_token(H, I, K, n_shared, bits, group, fmt, x + (size_t)t * H, idx + (size_t)t * K,
                              w + (size_t)t * K, blobs, shared_blob, out + (size_t)t * H);
        if (r != OQ_OK) {
#ifdef _OPENMP
#pragma omp critical(oq_rc)
#endif
            if (rc == OQ_OK) rc = r;
        }
    }
    return rc;
}

int oq_moe_forward_g(int H, int I, int E, int K, int n_shared, int bits, int group, int S, const float *x,
                     const int32_t *idx, const float *w, const uint8_t *const *blobs,
                     const uint8_t *shared_blob, float *out) {
    return oq_moe_forward_f(H, I, E, K, n_shared, bits, group, 0, S, x, idx, w, blobs, shared_blob, out);
}

int oq_moe_forward(int H, int I, int E, int K, int n_shared, int bits, int S, const float *x,
                   const int32_t *idx, const float *w, const uint8_t *const *blobs,
                   const uint8_t *shared_blob, float *out) {
    return oq_moe_forward_g(H, I, E, K, n_shared, bits, 0, S, x, idx, w, blobs, shared_blob, out);
}

/* Whole layer: routing then forward. */
int oq_moe_layer(int H, int I, int E, int K, int n_shared, int bits, float rsf, int norm, int S,
                 const float *x, const float *router_w, const float *bias,
                 const uint8_t *const *blobs, const uint8_t *shared_blob, float *out,
                 int32_t *idx, float *w) {
    if (!dims_ok(H, I, E, K, n_shared, bits)) return OQ_EINVAL;
    int rc = oq_moe_route(H, E, K, rsf, norm, S, x, router_w, bias, idx, w, NULL, NULL);
    if (rc != OQ_OK) return rc;
    return oq_moe_forward(H, I, E, K, n_shared, bits, S, x, idx, w, blobs, shared_blob, out);
}

/* Element-wise batch forms of the scalar functions above (for sweeps). */
void oq_expf_n(const float *x, float *y, uint64_t n) {
    for (uint64_t i = 0; i < n; ++i) y[i] = oq_expf(x[i]);
}

void oq_sigmoid_n(const float *x, float *y, uint64_t n) {
    for (uint64_t i = 0; i < n; ++i) y[i] = oq_sigmoid(x[i]);
}

void oq_swiglu_n(const float *g, const float *u, float *h, uint64_t n) {
    for (uint64_t i = 0; i < n; ++i) h[i] = oq_swiglu(g[i], u[i]);
}

/* Threads of the token loops: n > 0 sets them (OpenMP build); returns the
 * number the loops will use (1 in the single-threaded build). */
int oq_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
