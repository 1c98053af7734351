// Device building blocks shared by the MoE kernels and their test hooks.
//
// Floating point: this library is compiled with -ffp-contract=off and
// correctly rounded binary32 division, so each expression below is exactly
// the binary32 operation it spells, and every fused multiply-add is an
// explicit __builtin_fmaf.  The operation orders are the layer's defined
// orders (see the notes at each function); the integer parts are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "coli_moe.h"

namespace coli {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- status word bits (first word of the workspace) ------------------------
enum : uint32_t {
    ST_NONFINITE = 1u,     // NaN/Inf in x, W_r, bias, logits or gate weights
    ST_BADINDEX = 2u,      // expert index out of range or repeated in a token
    ST_NOTRESIDENT = 4u,   // routed expert blob pointer is NULL
    ST_TIMEOUT = 8u,       // a wait for other workgroups of the launch gave up (bounded spin)
};

// Device-scope (all L2 slices) relaxed accesses, for data exchanged between
// workgroups inside one launch; a writer drains its stores (drain()) before
// it signals through an atomic.
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for every outstanding memory operation of this thread.
__device__ __forceinline__ void drain() { __builtin_amdgcn_s_waitcnt(0); }

// Hand-offs between workgroups of one launch follow the release/acquire
// pattern: the producers' stores, a workgroup barrier, an agent-scope
// release fence, then the relaxed arrival atomic; the consumer that sees the
// last arrival (or a released flag) issues an agent-scope acquire fence
// before it reads.  The data itself moves with device-scope accesses
// (st_dev / ld_dev) and each writer drains before the barrier.
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ void raise_status(uint32_t *status, uint32_t bit) {
    // vector-memory atomic; the address is a plain global pointer
    __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool finite_f32(float v) {
    return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u;
}

// ---- exponential -------------------------------------------------------
// e^x by Cody-Waite reduction and the degree-7 Taylor polynomial of e^r
// (Cody & Waite 1980): n = rint(x log2 e); r = x - n ln2_hi (exact under
// fma) - n ln2_lo; p = Horner(1/k!, r); result p * 2^n, scaled in two steps
// at the ends of the range.  Constants are the binary32 roundings of ln 2,
// ln 2 - RN(ln 2), 1/ln 2 and 1/k!.  e^x rounds to +inf above 0x1.62e42ep+6
// and to 0 below -0x1.9fe368p+6.
__device__ __forceinline__ float pow2i(int n) {  // -126 <= n <= 127
    return __uint_as_float((uint32_t)(n + 127) << 23);
}

__device__ __forceinline__ float exp_f32(float x) {
    if (x != x) return x;
    if (x > 0x1.62e42ep+6f) return __builtin_inff();
    if (x < -0x1.9fe368p+6f) return 0.0f;
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e430p-1f;
    const float ln2_lo = -0x1.05c610p-29f;
    const float t = x * log2e;
    const float fn = __builtin_rintf(t);
    float r = __builtin_fmaf(-fn, ln2_hi, x);
    r = __builtin_fmaf(-fn, ln2_lo, r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int n = (int)fn;
    if (n > 127) return (p * pow2i(127)) * pow2i(n - 127);
    if (n < -126) return (p * pow2i(n + 64)) * pow2i(-64);
    return p * pow2i(n);
}

// sigmoid(v) = 1 / (1 + e^-v), one correctly rounded division.
__device__ __forceinline__ float sigmoid_f32(float v) { return 1.0f / (1.0f + exp_f32(-v)); }

// SwiGLU: (g / (1 + e^-g)) * u.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    return (g / (1.0f + exp_f32(-g))) * u;
}

// ---- Q8_0 --------------------------------------------------------------
// One 32-value block held by 32 consecutive lanes (a half wavefront): every
// lane passes its value and gets its code; *d receives the block scale.
// d = amax / 127, q = clamp(round-half-away(v / d), +-127), q = 0 if d == 0.
__device__ __forceinline__ int8_t q8_0_lane(float v, float *d_out) {
    float a = __builtin_fabsf(v);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, o, 64));
    const float d = a / 127.0f;
    *d_out = d;
    float c = 0.0f;
    if (d != 0.0f) {
        c = __builtin_roundf(v / d);
        c = __builtin_fminf(__builtin_fmaxf(c, -127.0f), 127.0f);
    }
    return (int8_t)(int)c;
}

// The same quantisation with one lane holding a whole 32-value block v
// (in registers): returns d and the 32 codes as 8 little-endian words in w.
// *ok is cleared on a non-finite input.
__device__ __forceinline__ float q8_0_words_of(const f32x4 (&xv)[8], uint32_t w[8], bool *ok) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const f32x4 t = xv[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    float a = 0.0f;
    bool good = true;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        good = good && finite_f32(v[i]);
        a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    }
    *ok = good;
    const float d = a / 127.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float c = 0.0f;
            if (d != 0.0f) {
                c = __builtin_roundf(v[4 * i + j] / d);
                c = __builtin_fminf(__builtin_fmaxf(c, -127.0f), 127.0f);
            }
            word |= (uint32_t)(uint8_t)(int8_t)(int)c << (8 * j);
        }
        w[i] = word;
    }
    return d;
}

// q8_0_words_of for the block at x[0..31] (16-byte aligned).
__device__ __forceinline__ float q8_0_block_words(const float *__restrict__ x, uint32_t w[8], bool *ok) {
    f32x4 xv[8];
    const f32x4 *src = reinterpret_cast<const f32x4 *>(x);
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = src[i];
    return q8_0_words_of(xv, w, ok);
}

// E4M3 byte (OCP FP8: 1 sign, 4 exponent bits of bias 7, 3 mantissa bits)
// of an integer v in -15 .. 15, exact: |v| = 1.m * 2^e with e = floor(log2 |v|).
__device__ __forceinline__ uint32_t e4m3_small(int v) {
    const uint32_t u = (uint32_t)(v < 0 ? -v : v);
    if (u == 0) return 0u;
    const int e = 31 - __builtin_clz(u);
    return (v < 0 ? 0x80u : 0u) | ((uint32_t)(e + 7) << 3) | ((u << (3 - e)) & 7u);
}

// The Q8_0 codes of one block (w: 32 int8 codes, four per word) split for
// the FP8 matrix cores: q = 16 hi + lo with hi = q >> 4 in -8 .. 7 and
// lo = q & 15 in 0 .. 15, both exact in E4M3.  64 bytes: the E4M3 of hi for
// codes 0-15, of lo for codes 0-15, of hi for 16-31, of lo for 16-31 — the
// two 32-byte halves are the B operands of lane halves 0 and 1 (bytes 0-15
// in the first scale block, scaled by 2^4, bytes 16-31 in the second).
__device__ __forceinline__ void split_e4m3(const uint32_t w[8], u32x4 out[4]) {
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t h = 0, l = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = (int)(int8_t)(uint8_t)(w[i] >> (8 * j));
            h |= e4m3_small(q >> 4) << (8 * j);
            l |= e4m3_small(q & 15) << (8 * j);
        }
        hw[i] = h;
        lw[i] = l;
    }
    out[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
    out[1] = u32x4{lw[0], lw[1], lw[2], lw[3]};
    out[2] = u32x4{hw[4], hw[5], hw[6], hw[7]};
    out[3] = u32x4{lw[4], lw[5], lw[6], lw[7]};
}

// As q8_0_block_words, storing the codes to q[0..31] (16-byte aligned).
__device__ __forceinline__ float q8_0_block_lane(const float *__restrict__ x, int8_t *__restrict__ q, bool *ok) {
    uint32_t w[8];
    const float d = q8_0_block_words(x, w, ok);
    u32x4 *qv = reinterpret_cast<u32x4 *>(q);
    qv[0] = u32x4{w[0], w[1], w[2], w[3]};
    qv[1] = u32x4{w[4], w[5], w[6], w[7]};
    return d;
}

// ---- packed rows: exact block dot products -----------------------------
// A "block" is 32 consecutive codes of a row: 32 bytes (int8), 16 (int4) or
// 8 (int2).  Activation codes arrive as 8 little-endian int32 words holding
// the block's 32 int8 values in order.
//
// int4: byte j of the block holds code j in bits 0-3 and code j+16 in bits
// 4-7.  Masking a nibble into the top half of its byte gives 16*code as a
// signed byte, so four codes feed one v_dot4 with no sign extension; the sum
// is then exactly divisible by 16.
__device__ __forceinline__ int32_t block_dot_int4(u32x4 w, const int32_t a[8]) {
    int32_t s = 0;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (ws[k] << 4) & 0xF0F0F0F0u;   // codes 4k..4k+3, x16
        const uint32_t hi = ws[k] & 0xF0F0F0F0u;          // codes 16+4k.., x16
        s = __builtin_amdgcn_sdot4((int)lo, a[k], s, false);
        s = __builtin_amdgcn_sdot4((int)hi, a[4 + k], s, false);
    }
    return s >> 4;
}

// int2: byte j (of 8) holds code j+8i in bits 2i..2i+1.  Shifting field i
// into the top two bits of each byte gives 64*code as a signed byte.
// Word m (bytes 4m..4m+3) field i covers codes 8i+4m..8i+4m+3.
__device__ __forceinline__ int32_t block_dot_int2(u32x2 w, const int32_t a[8]) {
    int32_t s = 0;
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t f = (ws[m] << (6 - 2 * i)) & 0xC0C0C0C0u;
            s = __builtin_amdgcn_sdot4((int)f, a[2 * i + m], s, false);
        }
    return s >> 6;
}

// int8: 32 codes in 8 words.
__device__ __forceinline__ int32_t block_dot_int8(u32x4 w0, u32x4 w1, const int32_t a[8]) {
    int32_t s = 0;
    s = __builtin_amdgcn_sdot4((int)w0.x, a[0], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.y, a[1], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.z, a[2], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.w, a[3], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.x, a[4], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.y, a[5], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.z, a[6], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.w, a[7], s, false);
    return s;
}

// MXFP4 (OCP Microscaling FP4): a block's 32 E2M1 codes in 16 bytes, byte j
// = element 2j (bits 0-3) | element 2j + 1 (bits 4-7); code bits: sign (3),
// exponent (2-1), mantissa (0); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
// Twice a value is an integer in [-12, 12], so the block dot
// isum = sum_j 2 v_j q_j is an exact int32 and feeds v_dot4.
//
// Bits 0-3 of each byte of x as four signed bytes 2 v: the magnitude index
// (bits 0-2) looks up 2|v| and -2|v| in two 8-byte tables (v_perm), and a
// third v_perm takes each byte from the table its sign bit names.
__device__ __forceinline__ uint32_t mx_twice(uint32_t x) {
    const uint32_t m = x & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, m);   // 0 1 2 3 | 4 6 8 12
    const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, m);   // -(the same)
    const uint32_t sel = ((x >> 1) & 0x04040404u) | 0x03020100u;               // byte i: i, or 4 + i if negative
    return __builtin_amdgcn_perm(neg, pos, sel);
}

// Activation codes of a block (8 words, elements in order) rearranged to
// pair with the MXFP4 bytes: even[k] holds elements 8k, 8k+2, 8k+4, 8k+6 and
// odd[k] elements 8k+1, 8k+3, 8k+5, 8k+7 (the low and high nibbles of weight
// word k).
__device__ __forceinline__ void mx_split_act(const int32_t a[8], int32_t even[4], int32_t odd[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        even[k] = (int32_t)__builtin_amdgcn_perm((uint32_t)a[2 * k + 1], (uint32_t)a[2 * k], 0x06040200u);
        odd[k] = (int32_t)__builtin_amdgcn_perm((uint32_t)a[2 * k + 1], (uint32_t)a[2 * k], 0x07050301u);
    }
}

// isum = sum_j 2 v_j q_j of one MXFP4 block against activations split by
// mx_split_act.
__device__ __forceinline__ int32_t block_dot_mx(u32x4 w, const int32_t even[4], const int32_t odd[4]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    int32_t s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s = __builtin_amdgcn_sdot4((int)mx_twice(ws[k]), even[k], s, false);
        s = __builtin_amdgcn_sdot4((int)mx_twice(ws[k] >> 4), odd[k], s, false);
    }
    return s;
}

// The same block sum through the hardware FP4 conversion: each byte's two
// codes become two f16 values 2 v (v_cvt_scalef32_pk_f16_fp4 with scale 2,
// exact) and v_dot2 multiplies them with the activation pair in f32.  Every
// product and partial sum is an integer of magnitude below 2^16, so the f32
// result is exactly isum whatever the order of its additions.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 32 activation codes of a block (8 words, in order) as 16 f16 pairs
// (q_2j, q_2j+1), exact: each byte is flipped to offset binary, placed under
// the f16 exponent of 1024 (0x64) and 1024 + 128 is subtracted.
__device__ __forceinline__ void mx_act_f16(const int32_t a[8], f16x2 h[16]) {
    const f16x2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t u = (uint32_t)a[k] ^ 0x80808080u;
        const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);   // bytes u0, 64, u1, 64
        const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u);   // bytes u2, 64, u3, 64
        h[2 * k] = __builtin_bit_cast(f16x2, p0) + off;
        h[2 * k + 1] = __builtin_bit_cast(f16x2, p1) + off;
    }
}

__device__ __forceinline__ float block_dot_mx_f16(u32x4 w, const f16x2 h[16]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[k], 2.0f, 0), h[4 * k], s, false);
        s = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[k], 2.0f, 1), h[4 * k + 1], s, false);
        s = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[k], 2.0f, 2), h[4 * k + 2], s, false);
        s = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[k], 2.0f, 3), h[4 * k + 3], s, false);
    }
    return s;
}

// Half the value of an E8M0 scale byte, 2^(x - 128), as binary32 (exact:
// 2^-128 and 2^-127 are subnormal numbers); x = 255 (NaN in E8M0) gives NaN.
__device__ __forceinline__ float e8m0_half(uint32_t x) {
    const uint32_t bits = x >= 2u ? (x - 1u) << 23 : 0x00200000u << x;
    return __uint_as_float(x == 255u ? 0x7FC00000u : bits);
}

// Raw bytes of one block of a packed row, as loaded by one lane.
template <int BITS>
struct BlockBits;
template <>
struct BlockBits<8> {
    u32x4 w0, w1;
};
template <>
struct BlockBits<4> {
    u32x4 w;
};
template <>
struct BlockBits<2> {
    u32x2 w;
};

// Vector-memory instructions that load one block per lane.
template <int BITS>
struct BlockLoads {
    static constexpr int N = BITS == 8 ? 2 : 1;
};

// Weight rows are read through a buffer resource covering the whole blob:
// the row's byte offset is a scalar, the lane's offset a single VGPR, and
// every access is range-checked by the hardware (reads past num_records
// return zeros).  Loads are marked non-temporal: each weight byte is used
// once per call.
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw (untyped) buffer on gfx9-family GPUs

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)RSRC_WORD3);
}

constexpr int BUF_NT = 2;  // cache-policy bits: non-temporal

template <int BITS>
__device__ __forceinline__ BlockBits<BITS> load_block(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int b);

template <>
__device__ __forceinline__ BlockBits<8> load_block<8>(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int b) {
    BlockBits<8> v;
    v.w0 = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * b, row_off, BUF_NT);
    v.w1 = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * b + 16, row_off, BUF_NT);
    return v;
}
template <>
__device__ __forceinline__ BlockBits<4> load_block<4>(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int b) {
    BlockBits<4> v;
    v.w = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * b, row_off, BUF_NT);
    return v;
}
template <>
__device__ __forceinline__ BlockBits<2> load_block<2>(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int b) {
    BlockBits<2> v;
    v.w = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * b, row_off, BUF_NT);
    return v;
}

// The same blocks read through a plain global pointer (row start + block).
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const u32x2 g_u32x2;

template <int BITS>
__device__ __forceinline__ BlockBits<BITS> load_block_ptr(const uint8_t *row, int b);
template <>
__device__ __forceinline__ BlockBits<8> load_block_ptr<8>(const uint8_t *row, int b) {
    g_u32x4 *p = (g_u32x4 *)(row + 32 * b);
    BlockBits<8> v;
    v.w0 = __builtin_nontemporal_load(p);
    v.w1 = __builtin_nontemporal_load(p + 1);
    return v;
}
template <>
__device__ __forceinline__ BlockBits<4> load_block_ptr<4>(const uint8_t *row, int b) {
    BlockBits<4> v;
    v.w = __builtin_nontemporal_load((g_u32x4 *)(row + 16 * b));
    return v;
}
template <>
__device__ __forceinline__ BlockBits<2> load_block_ptr<2>(const uint8_t *row, int b) {
    BlockBits<2> v;
    v.w = __builtin_nontemporal_load((g_u32x2 *)(row + 8 * b));
    return v;
}

__device__ __forceinline__ int32_t block_dot(const BlockBits<8> &w, const int32_t a[8]) {
    return block_dot_int8(w.w0, w.w1, a);
}
__device__ __forceinline__ int32_t block_dot(const BlockBits<4> &w, const int32_t a[8]) {
    return block_dot_int4(w.w, a);
}
__device__ __forceinline__ int32_t block_dot(const BlockBits<2> &w, const int32_t a[8]) {
    return block_dot_int2(w.w, a);
}

// Codes of one block (test hook for the unpacking): code j of the block.
template <int BITS>
__device__ __forceinline__ int8_t block_code(const BlockBits<BITS> &w, int j);
template <>
__device__ __forceinline__ int8_t block_code<8>(const BlockBits<8> &w, int j) {
    const uint32_t ws[8] = {w.w0.x, w.w0.y, w.w0.z, w.w0.w, w.w1.x, w.w1.y, w.w1.z, w.w1.w};
    return (int8_t)(ws[j >> 2] >> (8 * (j & 3)));
}
template <>
__device__ __forceinline__ int8_t block_code<4>(const BlockBits<4> &w, int j) {
    const uint32_t ws[4] = {w.w.x, w.w.y, w.w.z, w.w.w};
    const int byte = j & 15;
    const uint32_t word = ws[byte >> 2];
    const uint32_t v = (j < 16) ? (word << 4) & 0xF0F0F0F0u : word & 0xF0F0F0F0u;
    return (int8_t)((int8_t)(v >> (8 * (byte & 3))) >> 4);
}
template <>
__device__ __forceinline__ int8_t block_code<2>(const BlockBits<2> &w, int j) {
    const int byte = j & 7, i = j >> 3;
    const uint32_t word = (byte < 4) ? w.w.x : w.w.y;
    const uint32_t f = (word << (6 - 2 * i)) & 0xC0C0C0C0u;
    return (int8_t)((int8_t)(f >> (8 * (byte & 3))) >> 6);
}

// ---- misc --------------------------------------------------------------
__host__ __device__ constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BlobLayout {
    size_t gate, up, down, s_gate, s_up, s_down, total;
};

// Expert blob sections.  group = 0: one f32 scale per row; group > 0: one
// per `group` codes of a row, row-major ([I][H / group] for gate and up,
// [H][I / group] for down).  mx: MXFP4, 4-bit codes and one E8M0 byte per 32
// codes of a row, row-major ([I][H / 32], [I][H / 32], [H][I / 32]).
__host__ __device__ inline BlobLayout blob_layout(int H, int I, int bits, int group = 0, bool mx = false) {
    BlobLayout L;
    const size_t gate = (size_t)I * (size_t)H * (size_t)bits / 8;
    const size_t down = (size_t)H * (size_t)I * (size_t)bits / 8;
    const size_t sgu = mx ? (size_t)I * (size_t)(H / 32) : 4 * (size_t)I * (size_t)(group ? H / group : 1);
    const size_t sd = mx ? (size_t)H * (size_t)(I / 32) : 4 * (size_t)H * (size_t)(group ? I / group : 1);
    L.gate = 0;
    L.up = align256(L.gate + gate);
    L.down = align256(L.up + gate);
    L.s_gate = align256(L.down + down);
    L.s_up = align256(L.s_gate + sgu);
    L.s_down = align256(L.s_up + sgu);
    L.total = align256(L.s_down + sd);
    return L;
}

}  // namespace coli
