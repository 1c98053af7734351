/*
 * Sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle entry point on small seeded inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer, including the error paths (NULL blob,
 * repeated index, non-finite input).  The values are not checked here (the
 * Python pins do that); a sanitizer report or an unexpected return code
 * fails the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oq_expf(float x);
void oq_q8_0(const float *v, int n, int8_t *q, float *d);
void oq_unpack(const uint8_t *src, int n, int bits, int8_t *out);
void oq_unpack_mx(const uint8_t *src, int n, int8_t *out);
void oq_blob_layout_g(int H, int I, int bits, int group, uint64_t off[7]);
void oq_blob_layout_mx(int H, int I, uint64_t off[7]);
int oq_select(const float *logit, const float *bias, int E, int K, float rsf, int norm, int32_t *idx, float *w,
              float *sig_out);
int oq_moe_route(int H, int E, int K, float rsf, int norm, int S, const float *x, const float *router_w,
                 const float *bias, int32_t *idx, float *w, float *logits_out, float *sig_out);
int oq_moe_forward_f(int H, int I, int E, int K, int n_shared, int bits, int group, int fmt, int S, const float *x,
                     const int32_t *idx, const float *w, const uint8_t *const *blobs, const uint8_t *shared_blob,
                     float *out);
int oq_threads(int n);

static uint64_t rs = 0x9E3779B97F4A7C15ULL;
static uint32_t rnd(void) {
    rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
    return (uint32_t)(rs >> 16);
}
static float frnd(void) { return ((float)(rnd() % 20001) - 10000.0f) / 5000.0f; }

static int fail(const char *what, int rc) {
    fprintf(stderr, "unexpected result in %s: %d\n", what, rc);
    return 1;
}

static int layer(int H, int I, int E, int K, int bits, int group, int fmt, int S) {
    uint64_t off[7];
    if (fmt)
        oq_blob_layout_mx(H, I, off);
    else
        oq_blob_layout_g(H, I, bits, group, off);
    size_t bb = (size_t)off[6];
    uint8_t **blobs = calloc((size_t)E, sizeof *blobs);
    uint8_t *shared = malloc(bb);
    float *x = malloc(sizeof(float) * (size_t)S * H), *W = malloc(sizeof(float) * (size_t)E * H);
    float *bias = malloc(sizeof(float) * (size_t)E), *w = malloc(sizeof(float) * (size_t)S * K);
    float *out = malloc(sizeof(float) * (size_t)S * H);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)S * K);
    for (int e = 0; e < E; ++e) {
        blobs[e] = malloc(bb);
        for (size_t i = 0; i < bb; ++i) blobs[e][i] = (uint8_t)rnd();
    }
    for (size_t i = 0; i < bb; ++i) shared[i] = (uint8_t)rnd();
    /* finite scales: overwrite the scale sections with small positive values */
    for (int e = 0; e <= E; ++e) {
        uint8_t *b = e < E ? blobs[e] : shared;
        if (fmt) {
            for (size_t i = off[3]; i < off[6]; ++i) b[i] = (uint8_t)(110 + rnd() % 20);
        } else {
            for (size_t i = off[3]; i + 4 <= off[6]; i += 4) {
                float v = 0.001f + (float)(rnd() % 1000) * 1e-5f;
                memcpy(b + i, &v, 4);
            }
        }
    }
    for (int i = 0; i < S * H; ++i) x[i] = frnd();
    for (int i = 0; i < E * H; ++i) W[i] = frnd() * 0.05f;
    for (int i = 0; i < E; ++i) bias[i] = frnd() * 0.01f;
    int rc = oq_moe_route(H, E, K, 2.5f, 1, S, x, W, bias, idx, w, NULL, NULL);
    if (rc) return fail("route", rc);
    rc = oq_moe_forward_f(H, I, E, K, 1, bits, group, fmt, S, x, idx, w, (const uint8_t *const *)blobs, shared, out);
    if (rc) return fail("forward", rc);
    /* error paths */
    uint8_t *keep = blobs[idx[0]];
    blobs[idx[0]] = NULL;
    rc = oq_moe_forward_f(H, I, E, K, 1, bits, group, fmt, S, x, idx, w, (const uint8_t *const *)blobs, shared, out);
    if (rc != -4) return fail("not resident", rc);
    blobs[idx[0]] = keep;
    if (K > 1) {
        int32_t t = idx[1];
        idx[1] = idx[0];
        rc = oq_moe_forward_f(H, I, E, K, 1, bits, group, fmt, S, x, idx, w, (const uint8_t *const *)blobs, shared,
                              out);
        if (rc != -1) return fail("repeated index", rc);
        idx[1] = t;
    }
    x[3] = NAN;
    rc = oq_moe_route(H, E, K, 2.5f, 1, S, x, W, bias, idx, w, NULL, NULL);
    if (rc != -2) return fail("non-finite", rc);
    for (int e = 0; e < E; ++e) free(blobs[e]);
    free(blobs); free(shared); free(x); free(W); free(bias); free(w); free(out); free(idx);
    return 0;
}

int main(void) {
    oq_threads(3);
    int8_t q[256], u[256];
    float d[8], v[256];
    uint8_t raw[256];
    for (int i = 0; i < 256; ++i) { v[i] = frnd(); raw[i] = (uint8_t)rnd(); }
    oq_q8_0(v, 256, q, d);
    for (int bits = 2; bits <= 8; bits *= 2) oq_unpack(raw, 256, bits, u);
    oq_unpack_mx(raw, 256, u);
    float xs[] = {0.0f, -0.0f, 88.7f, 89.0f, -104.0f, -87.0f, NAN, INFINITY, -INFINITY, 1e-40f};
    for (unsigned i = 0; i < sizeof xs / sizeof xs[0]; ++i) (void)oq_expf(xs[i]);
    float lg[16], bias[16], w[16];
    int32_t idx[16];
    for (int i = 0; i < 16; ++i) { lg[i] = frnd(); bias[i] = 0.0f; }
    if (oq_select(lg, bias, 16, 16, 1.0f, 1, idx, w, NULL)) return fail("select", -99);
    int rc = 0;
    rc |= layer(256, 128, 16, 2, 4, 0, 0, 5);
    rc |= layer(256, 128, 16, 3, 8, 0, 0, 3);
    rc |= layer(256, 128, 12, 2, 2, 0, 0, 2);
    rc |= layer(512, 256, 9, 4, 4, 64, 0, 3);
    rc |= layer(256, 128, 16, 2, 4, 0, 1, 4);
    if (rc) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
