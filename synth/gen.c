/*
 * Fast seeded generator for large synthetic expert blobs.
 *
 * Input-generation helper only: it writes packed weight codes and per-row
 * scales in the expert-blob byte layout, and nothing else.  It contains no
 * arithmetic of the MoE layer itself (no activation quantisation, routing,
 * dot products or combine).  The CPU oracle and the HIP library both read
 * the bytes it writes; neither links this file.
 *
 * Random numbers: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: value i of stream `key` is mix(key + (i + 1) * GAMMA).
 *
 * Codes are drawn i.i.d. from a caller-supplied 65536-entry table that maps a
 * 16-bit uniform to a signed code (the caller builds it from the CDF of a
 * quantised Gaussian).  Row (or row-group) scales are
 * nominal * (1 + jitter * (u - 0.5)).
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GAMMA);
}

static uint64_t align256(uint64_t n) { return (n + 255u) & ~(uint64_t)255u; }

/* Packs one row of codes (ncols, multiple of 32) into `dst`. */
static void pack_row(const int8_t *q, int ncols, int bits, uint8_t *dst) {
    int nb = ncols / 32;
    for (int b = 0; b < nb; ++b) {
        const int8_t *c = q + 32 * b;
        if (bits == 8) {
            memcpy(dst + 32 * b, c, 32);
        } else if (bits == 4) {
            uint8_t *o = dst + 16 * b;
            for (int j = 0; j < 16; ++j)
                o[j] = (uint8_t)(((uint8_t)c[j] & 0x0Fu) | (((uint8_t)c[j + 16] & 0x0Fu) << 4));
        } else { /* bits == 2 */
            uint8_t *o = dst + 8 * b;
            for (int j = 0; j < 8; ++j) {
                unsigned v = 0;
                for (int i = 0; i < 4; ++i) v |= ((unsigned)(uint8_t)c[j + 8 * i] & 3u) << (2 * i);
                o[j] = (uint8_t)v;
            }
        }
    }
}

/*
 * Fills one matrix section (rows x cols codes) and its scale section: one
 * scale per row, or with group > 0 one per `group` codes of a row (row-major
 * [rows][cols / group]).  key_codes / key_scales select the two random streams.
 */
static void fill_matrix(uint64_t key_codes, uint64_t key_scales, int rows, int cols, int bits, int group,
                        const int8_t *table, float scale_nominal, float scale_jitter,
                        uint8_t *codes_out, float *scales_out, int nthreads) {
    int row_bytes = cols * bits / 8;
    int ns = group ? cols / group : 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int r = 0; r < rows; ++r) {
        int8_t q[32768];
        uint64_t base = (uint64_t)r * (uint64_t)(cols / 4);
        for (int g = 0; g < cols / 4; ++g) {
            uint64_t u = stream_at(key_codes, base + (uint64_t)g);
            q[4 * g + 0] = table[(u >> 0) & 0xFFFF];
            q[4 * g + 1] = table[(u >> 16) & 0xFFFF];
            q[4 * g + 2] = table[(u >> 32) & 0xFFFF];
            q[4 * g + 3] = table[(u >> 48) & 0xFFFF];
        }
        pack_row(q, cols, bits, codes_out + (uint64_t)r * (uint64_t)row_bytes);
        for (int g = 0; g < ns; ++g) {
            uint64_t us = stream_at(key_scales, (uint64_t)r * (uint64_t)ns + (uint64_t)g);
            double uu = (double)(us >> 11) * (1.0 / 9007199254740992.0);
            scales_out[(uint64_t)r * (uint64_t)ns + (uint64_t)g] =
                (float)((double)scale_nominal * (1.0 + (double)scale_jitter * (uu - 0.5)));
        }
    }
}

/*
 * Writes one expert blob: [gate codes][up codes][down codes][s_gate][s_up][s_down],
 * each section starting on a 256-byte boundary.  `keys` holds six stream keys:
 * codes and scales for gate, up and down.  Returns the number of bytes written.
 */
uint64_t synth_fill_blob_cdf_g(const uint64_t *keys, int hidden, int inter, int bits, int group,
                               const int8_t *table, float scale_nominal, float scale_jitter,
                               uint8_t *out, int nthreads) {
    if (hidden <= 0 || inter <= 0 || hidden % 32 || inter % 32 || hidden > 32768 || inter > 32768)
        return 0;
    if (bits != 8 && bits != 4 && bits != 2) return 0;
    if (group != 0 && (group % 32 || hidden % group || inter % group)) return 0;
    uint64_t gate_bytes = (uint64_t)inter * (uint64_t)(hidden * bits / 8);
    uint64_t down_bytes = (uint64_t)hidden * (uint64_t)(inter * bits / 8);
    uint64_t sgu = 4ull * (uint64_t)inter * (uint64_t)(group ? hidden / group : 1);
    uint64_t sd = 4ull * (uint64_t)hidden * (uint64_t)(group ? inter / group : 1);
    uint64_t off_g = 0;
    uint64_t off_u = align256(off_g + gate_bytes);
    uint64_t off_d = align256(off_u + gate_bytes);
    uint64_t off_sg = align256(off_d + down_bytes);
    uint64_t off_su = align256(off_sg + sgu);
    uint64_t off_sd = align256(off_su + sgu);
    uint64_t total = align256(off_sd + sd);
    memset(out, 0, total);
    fill_matrix(keys[0], keys[1], inter, hidden, bits, group, table, scale_nominal, scale_jitter,
                out + off_g, (float *)(out + off_sg), nthreads);
    fill_matrix(keys[2], keys[3], inter, hidden, bits, group, table, scale_nominal, scale_jitter,
                out + off_u, (float *)(out + off_su), nthreads);
    fill_matrix(keys[4], keys[5], hidden, inter, bits, group, table, scale_nominal, scale_jitter,
                out + off_d, (float *)(out + off_sd), nthreads);
    return total;
}

uint64_t synth_fill_blob_cdf(const uint64_t *keys, int hidden, int inter, int bits,
                             const int8_t *table, float scale_nominal, float scale_jitter,
                             uint8_t *out, int nthreads) {
    return synth_fill_blob_cdf_g(keys, hidden, inter, bits, 0, table, scale_nominal, scale_jitter, out,
                                 nthreads);
}

/*
 * MXFP4 blob (OCP Microscaling FP4): [gate codes][up codes][down codes]
 * [gate scales][up scales][down scales], each section 256-byte aligned.
 * Codes are 4-bit E2M1 codes drawn i.i.d. from a 65536-entry table (16-bit
 * uniform -> code), two per byte (element 2j in bits 0-3, 2j+1 in bits 4-7);
 * scales are one E8M0 byte per 32 codes of a row, uniform over
 * scale_lo .. scale_lo + scale_span - 1.  Returns the bytes written.
 */
static void fill_matrix_mx(uint64_t key_codes, uint64_t key_scales, int rows, int cols, const uint8_t *table,
                           int scale_lo, int scale_span, uint8_t *codes_out, uint8_t *scales_out, int nthreads) {
    int row_bytes = cols / 2, nb = cols / 32;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int r = 0; r < rows; ++r) {
        uint8_t *o = codes_out + (uint64_t)r * (uint64_t)row_bytes;
        uint64_t base = (uint64_t)r * (uint64_t)(cols / 4);
        for (int g = 0; g < cols / 4; ++g) {
            uint64_t u = stream_at(key_codes, base + (uint64_t)g);
            uint8_t c0 = table[(u >> 0) & 0xFFFF], c1 = table[(u >> 16) & 0xFFFF];
            uint8_t c2 = table[(u >> 32) & 0xFFFF], c3 = table[(u >> 48) & 0xFFFF];
            o[2 * g] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
            o[2 * g + 1] = (uint8_t)((c2 & 0xF) | ((c3 & 0xF) << 4));
        }
        for (int b = 0; b < nb; ++b) {
            uint64_t us = stream_at(key_scales, (uint64_t)r * (uint64_t)nb + (uint64_t)b);
            scales_out[(uint64_t)r * (uint64_t)nb + (uint64_t)b] = (uint8_t)(scale_lo + (int)(us % (uint64_t)scale_span));
        }
    }
}

uint64_t synth_fill_blob_mx(const uint64_t *keys, int hidden, int inter, const uint8_t *table, int scale_lo,
                            int scale_span, uint8_t *out, int nthreads) {
    if (hidden <= 0 || inter <= 0 || hidden % 32 || inter % 32 || hidden > 32768 || inter > 32768) return 0;
    if (scale_lo < 0 || scale_span < 1 || scale_lo + scale_span > 255) return 0;
    uint64_t gate_bytes = (uint64_t)inter * (uint64_t)(hidden / 2);
    uint64_t down_bytes = (uint64_t)hidden * (uint64_t)(inter / 2);
    uint64_t sgu = (uint64_t)inter * (uint64_t)(hidden / 32), sd = (uint64_t)hidden * (uint64_t)(inter / 32);
    uint64_t off_g = 0;
    uint64_t off_u = align256(off_g + gate_bytes);
    uint64_t off_d = align256(off_u + gate_bytes);
    uint64_t off_sg = align256(off_d + down_bytes);
    uint64_t off_su = align256(off_sg + sgu);
    uint64_t off_sd = align256(off_su + sgu);
    uint64_t total = align256(off_sd + sd);
    memset(out, 0, total);
    fill_matrix_mx(keys[0], keys[1], inter, hidden, table, scale_lo, scale_span, out + off_g, out + off_sg, nthreads);
    fill_matrix_mx(keys[2], keys[3], inter, hidden, table, scale_lo, scale_span, out + off_u, out + off_su, nthreads);
    fill_matrix_mx(keys[4], keys[5], hidden, inter, table, scale_lo, scale_span, out + off_d, out + off_sd, nthreads);
    return total;
}
