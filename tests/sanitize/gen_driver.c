/*
 * Sanitizer driver for the input generator's C helper (test
 * infrastructure): fills small and odd-shaped blobs of every recipe under
 * AddressSanitizer and UndefinedBehaviorSanitizer, into buffers of exactly
 * the returned size, and checks the refused shapes return 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint64_t synth_fill_blob_cdf_g(const uint64_t *keys, int hidden, int inter, int bits, int group,
                               const int8_t *table, float scale_nominal, float scale_jitter, uint8_t *out,
                               int nthreads);
uint64_t synth_fill_blob_mx(const uint64_t *keys, int hidden, int inter, const uint8_t *table, int scale_lo,
                            int scale_span, uint8_t *out, int nthreads);

static uint64_t al(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

static uint64_t blob_bytes(int H, int I, int bits, int group, int mx) {
    uint64_t g = (uint64_t)I * H * (mx ? 4 : bits) / 8, dn = (uint64_t)H * I * (mx ? 4 : bits) / 8;
    uint64_t sgu = mx ? (uint64_t)I * (H / 32) : 4ull * I * (group ? H / group : 1);
    uint64_t sd = mx ? (uint64_t)H * (I / 32) : 4ull * H * (group ? I / group : 1);
    uint64_t o = al(g);
    o = al(o + g);
    o = al(o + dn);
    o = al(o + sgu);
    o = al(o + sgu);
    return al(o + sd);
}

int main(void) {
    uint64_t keys[6] = {1, 2, 3, 4, 5, 6};
    int8_t table[65536];
    uint8_t mtab[65536];
    for (int i = 0; i < 65536; ++i) { table[i] = (int8_t)((i % 15) - 7); mtab[i] = (uint8_t)(i % 16); }
    const int shapes[][4] = {{256, 128, 4, 0}, {256, 32, 8, 0}, {512, 96, 2, 0}, {256, 128, 4, 64}, {768, 256, 4, 128}};
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        int H = shapes[s][0], I = shapes[s][1], b = shapes[s][2], g = shapes[s][3];
        uint64_t n = blob_bytes(H, I, b, g, 0);
        uint8_t *out = malloc(n);
        uint64_t got = synth_fill_blob_cdf_g(keys, H, I, b, g, table, 0.01f, 0.1f, out, 2);
        free(out);
        if (got != n) { fprintf(stderr, "cdf size %llu != %llu\n", (unsigned long long)got, (unsigned long long)n); return 1; }
    }
    const int mx[][2] = {{256, 128}, {512, 256}, {256, 32}};
    for (unsigned s = 0; s < sizeof mx / sizeof mx[0]; ++s) {
        uint64_t n = blob_bytes(mx[s][0], mx[s][1], 4, 0, 1);
        uint8_t *out = malloc(n);
        uint64_t got = synth_fill_blob_mx(keys, mx[s][0], mx[s][1], mtab, 119, 3, out, 2);
        free(out);
        if (got != n) { fprintf(stderr, "mx size mismatch\n"); return 1; }
    }
    if (synth_fill_blob_cdf_g(keys, 250, 128, 4, 0, table, 0.01f, 0.1f, NULL, 1) != 0) return 1;
    if (synth_fill_blob_mx(keys, 256, 128, mtab, 250, 10, NULL, 1) != 0) return 1;
    printf("generator sanitizer run ok\n");
    return 0;
}
