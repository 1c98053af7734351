// Test hooks: thin kernels around the same device functions the forward
// kernels use (packed-row unpacking and block dots, the exponential, Q8_0),
// so their exact integer and binary32 results can be compared element by
// element with the CPU oracle.
#include "device_common.h"
#include "mfma.h"
#include "kernels.h"

namespace coli {

template <int BITS>
__global__ __launch_bounds__(64) void k_debug_unpack(const uint8_t *__restrict__ src,
                                                     int8_t *__restrict__ out, int cols) {
    const int r = blockIdx.x;
    const int nb = cols / 32;
    const uint32_t row_bytes = (uint32_t)cols * BITS / 8;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src, row_bytes * gridDim.x);
    for (int b = threadIdx.x; b < nb; b += 64) {
        const BlockBits<BITS> w = load_block<BITS>(rsrc, (uint32_t)r * row_bytes, b);
#pragma unroll
        for (int j = 0; j < 32; ++j) out[(size_t)r * cols + 32 * b + j] = block_code<BITS>(w, j);
    }
}

template <int BITS>
__global__ __launch_bounds__(64) void k_debug_block_dots(const uint8_t *__restrict__ src,
                                                         const int8_t *__restrict__ q,
                                                         int32_t *__restrict__ out, int cols) {
    const int r = blockIdx.x;
    const int nb = cols / 32;
    const uint32_t row_bytes = (uint32_t)cols * BITS / 8;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src, row_bytes * gridDim.x);
    for (int b = threadIdx.x; b < nb; b += 64) {
        const BlockBits<BITS> w = load_block<BITS>(rsrc, (uint32_t)r * row_bytes, b);
        int32_t a[8];
        for (int k = 0; k < 8; ++k) {
            const int8_t *p = q + 32 * b + 4 * k;
            a[k] = (int32_t)((uint32_t)(uint8_t)p[0] | ((uint32_t)(uint8_t)p[1] << 8) |
                             ((uint32_t)(uint8_t)p[2] << 16) | ((uint32_t)(uint8_t)p[3] << 24));
        }
        out[(size_t)r * nb + b] = block_dot(w, a);
    }
}

// MXFP4 rows (16 bytes per block): twice the E2M1 value of each code, and
// the exact block dots, through the forward kernels' decode.
__global__ __launch_bounds__(64) void k_debug_unpack_mx(const uint8_t *__restrict__ src,
                                                        int8_t *__restrict__ out, int cols) {
    const int r = blockIdx.x;
    const int nb = cols / 32;
    const uint32_t row_bytes = (uint32_t)cols / 2;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src, row_bytes * gridDim.x);
    for (int b = threadIdx.x; b < nb; b += 64) {
        const BlockBits<4> w = load_block<4>(rsrc, (uint32_t)r * row_bytes, b);
        const uint32_t ws[4] = {w.w.x, w.w.y, w.w.z, w.w.w};
        int8_t *o = out + (size_t)r * cols + 32 * b;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = mx_twice(ws[k]), hi = mx_twice(ws[k] >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[8 * k + 2 * i] = (int8_t)(lo >> (8 * i));
                o[8 * k + 2 * i + 1] = (int8_t)(hi >> (8 * i));
            }
        }
    }
}

__global__ __launch_bounds__(64) void k_debug_block_dots_mx(const uint8_t *__restrict__ src,
                                                            const int8_t *__restrict__ q,
                                                            int32_t *__restrict__ out, int cols) {
    const int r = blockIdx.x;
    const int nb = cols / 32;
    const uint32_t row_bytes = (uint32_t)cols / 2;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src, row_bytes * gridDim.x);
    for (int b = threadIdx.x; b < nb; b += 64) {
        const BlockBits<4> w = load_block<4>(rsrc, (uint32_t)r * row_bytes, b);
        int32_t a[8], ae[4], ao[4];
        for (int k = 0; k < 8; ++k) {
            const int8_t *p = q + 32 * b + 4 * k;
            a[k] = (int32_t)((uint32_t)(uint8_t)p[0] | ((uint32_t)(uint8_t)p[1] << 8) |
                             ((uint32_t)(uint8_t)p[2] << 16) | ((uint32_t)(uint8_t)p[3] << 24));
        }
        mx_split_act(a, ae, ao);
        // both device sums (int8 lookups and the f16 conversion path) must
        // agree; a disagreement is reported as INT32_MIN
        f16x2 h[16];
        mx_act_f16(a, h);
        const int32_t si = block_dot_mx(w.w, ae, ao);
        const float sf = block_dot_mx_f16(w.w, h);
        out[(size_t)r * nb + b] = (float)si == sf ? si : INT32_MIN;
    }
}

__global__ void k_debug_expf(const float *__restrict__ x, float *__restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = exp_f32(x[i]);
}

// One wavefront per row; each half wave quantises one 32-element block.
__global__ __launch_bounds__(64) void k_debug_q8_0(const float *__restrict__ v,
                                                   int8_t *__restrict__ q, float *__restrict__ d,
                                                   int cols) {
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    for (int h0 = 0; h0 < cols; h0 += 64) {
        const int h = h0 + lane;
        if (h0 + (lane & 32) < cols) {  // whole half wave in or out
            float dd;
            const int8_t c = q8_0_lane(v[(size_t)r * cols + h], &dd);
            q[(size_t)r * cols + h] = c;
            if ((lane & 31) == 0) d[(size_t)r * (cols / 32) + (h >> 5)] = dd;
        }
    }
}

hipError_t launch_debug_unpack(int bits, int rows, int cols, const void *src, int8_t *out,
                               hipStream_t st) {
    const uint8_t *s = static_cast<const uint8_t *>(src);
    if (bits == COLI_MXFP4) hipLaunchKernelGGL(k_debug_unpack_mx, dim3(rows), dim3(64), 0, st, s, out, cols);
    else if (bits == 8) hipLaunchKernelGGL(k_debug_unpack<8>, dim3(rows), dim3(64), 0, st, s, out, cols);
    else if (bits == 4) hipLaunchKernelGGL(k_debug_unpack<4>, dim3(rows), dim3(64), 0, st, s, out, cols);
    else hipLaunchKernelGGL(k_debug_unpack<2>, dim3(rows), dim3(64), 0, st, s, out, cols);
    return hipGetLastError();
}

hipError_t launch_debug_block_dots(int bits, int rows, int cols, const void *src, const int8_t *q,
                                   int32_t *out, hipStream_t st) {
    const uint8_t *s = static_cast<const uint8_t *>(src);
    if (bits == COLI_MXFP4)
        hipLaunchKernelGGL(k_debug_block_dots_mx, dim3(rows), dim3(64), 0, st, s, q, out, cols);
    else if (bits == 8)
        hipLaunchKernelGGL(k_debug_block_dots<8>, dim3(rows), dim3(64), 0, st, s, q, out, cols);
    else if (bits == 4)
        hipLaunchKernelGGL(k_debug_block_dots<4>, dim3(rows), dim3(64), 0, st, s, q, out, cols);
    else
        hipLaunchKernelGGL(k_debug_block_dots<2>, dim3(rows), dim3(64), 0, st, s, q, out, cols);
    return hipGetLastError();
}

hipError_t launch_debug_expf(int64_t n, const float *x, float *y, hipStream_t st) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_debug_expf, dim3((unsigned)blocks), dim3(256), 0, st, x, y, n);
    return hipGetLastError();
}

// One int8 MFMA on raw lane registers: lane l's A and B registers are
// bytes 16 l .. 16 l + 15 of a and b; its 16 result registers go to
// c[16 l .. 16 l + 15].
__global__ __launch_bounds__(64) void k_debug_mfma_i8(const int8_t *__restrict__ a, const int8_t *__restrict__ b,
                                                       int32_t *__restrict__ c) {
    const int l = threadIdx.x;
    const i32x4 av = reinterpret_cast<const i32x4 *>(a)[l];
    const i32x4 bv = reinterpret_cast<const i32x4 *>(b)[l];
    const i32x16 cv = mfma_i8_32x32x32(av, bv);
#pragma unroll
    for (int r = 0; r < 16; ++r) c[16 * l + r] = cv[r];
}

hipError_t launch_debug_mfma_i8(const int8_t *a, const int8_t *b, int32_t *c, hipStream_t st) {
    hipLaunchKernelGGL(k_debug_mfma_i8, dim3(1), dim3(64), 0, st, a, b, c);
    return hipGetLastError();
}

// One v_mfma_i32_16x16x32_i8 on raw lane registers: lane l's A and B
// registers are bytes 8 l .. 8 l + 7 of a and b; its 4 results go to
// c[4 l .. 4 l + 3].
__global__ __launch_bounds__(64) void k_debug_mfma_i8_16(const int8_t *__restrict__ a, const int8_t *__restrict__ b,
                                                          int32_t *__restrict__ c) {
    const int l = threadIdx.x;
    const int64_t av = reinterpret_cast<const int64_t *>(a)[l];
    const int64_t bv = reinterpret_cast<const int64_t *>(b)[l];
    const i32x4 cv = mfma_i8_16x16x32(av, bv);
    reinterpret_cast<i32x4 *>(c)[l] = cv;
}

hipError_t launch_debug_mfma_i8_16(const int8_t *a, const int8_t *b, int32_t *c, hipStream_t st) {
    hipLaunchKernelGGL(k_debug_mfma_i8_16, dim3(1), dim3(64), 0, st, a, b, c);
    return hipGetLastError();
}

// One scaled f8f6f4 MFMA on raw lane registers: lane l's A and B registers
// are bytes 32 l .. 32 l + 31 of a and b, its scales bytes l of sa and sb;
// its 16 results go to c[16 l .. 16 l + 15].  FA / FB: operand formats.
template <int FA, int FB>
__global__ __launch_bounds__(64) void k_debug_mfma_f8f6f4(const uint8_t *__restrict__ a,
                                                          const uint8_t *__restrict__ b,
                                                          const uint8_t *__restrict__ sa,
                                                          const uint8_t *__restrict__ sb, float *__restrict__ c) {
    const int l = threadIdx.x;
    const i32x8 av = reinterpret_cast<const i32x8 *>(a)[l];
    const i32x8 bv = reinterpret_cast<const i32x8 *>(b)[l];
    const f32x16 cv = mfma_scale_f8f6f4<FA, FB>(av, bv, (int)sa[l], (int)sb[l]);
#pragma unroll
    for (int r = 0; r < 16; ++r) c[16 * l + r] = cv[r];
}

hipError_t launch_debug_mfma_f8f6f4(int fa, int fb, const uint8_t *a, const uint8_t *b, const uint8_t *sa,
                                    const uint8_t *sb, float *c, hipStream_t st) {
    if (fa == 0 && fb == 0)
        hipLaunchKernelGGL((k_debug_mfma_f8f6f4<0, 0>), dim3(1), dim3(64), 0, st, a, b, sa, sb, c);
    else if (fa == 4 && fb == 0)
        hipLaunchKernelGGL((k_debug_mfma_f8f6f4<4, 0>), dim3(1), dim3(64), 0, st, a, b, sa, sb, c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---- measured roofs ------------------------------------------------------
// A streaming read of n16 16-byte words (ROOF_SR_UNROLL loads per thread in
// flight, grid-stride), every thread XOR-folding what it read into one sink
// word so that no load is dead.
constexpr int ROOF_SR_UNROLL = 8;
__global__ __launch_bounds__(256) void k_roof_stream(const i32x4 *__restrict__ src, uint64_t n16,
                                                     uint32_t *__restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    i32x4 acc = {0, 0, 0, 0};
    for (; i + (ROOF_SR_UNROLL - 1) * stride < n16; i += ROOF_SR_UNROLL * stride) {
        i32x4 v[ROOF_SR_UNROLL];
#pragma unroll
        for (int k = 0; k < ROOF_SR_UNROLL; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
        for (int k = 0; k < ROOF_SR_UNROLL; ++k) acc ^= v[k];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

// The int8 matrix cores alone: each wavefront runs `iters` rounds of four
// independent v_mfma_i32_32x32x32_i8 accumulations on register operands.
__global__ __launch_bounds__(256) void k_roof_mfma(int iters, int32_t *__restrict__ sink) {
    const int t = (int)threadIdx.x;
    const i32x4 a = {t, t + 1, t + 2, t + 3};
    i32x4 b[4];   // a different B per chain, so that no two chains are the same computation
#pragma unroll
    for (int k = 0; k < 4; ++k) b[k] = i32x4{3 * t + k, 5 * t + k, 7 * t + k, 11 * t + k};
    i32x16 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[k][r] = 0;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[k], c[k], 0, 0, 0);
    }
    int32_t x = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= c[k][r];
    sink[(size_t)blockIdx.x * 256 + t] = x;
}

hipError_t launch_roof_stream(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t st) {
    hipLaunchKernelGGL(k_roof_stream, dim3(ROOF_GRID), dim3(256), 0, st, static_cast<const i32x4 *>(src),
                       bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_roof_mfma(int iters, int32_t *sink, hipStream_t st) {
    hipLaunchKernelGGL(k_roof_mfma, dim3(ROOF_GRID), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

hipError_t launch_debug_q8_0(int rows, int cols, const float *v, int8_t *q, float *d,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_debug_q8_0, dim3(rows), dim3(64), 0, st, v, q, d, cols);
    return hipGetLastError();
}

}  // namespace coli
