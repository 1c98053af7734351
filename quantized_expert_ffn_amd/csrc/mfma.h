// The int8 matrix-core operation of the prefill kernels on gfx950,
// v_mfma_i32_32x32x32_i8: C[32x32] = A[32x32] * B[32x32] over K = 32, one
// Q8_0 block per instruction.  Lane layout (checked by the debug hook
// coli_moe_debug_mfma_i8 against a host matmul):
//   A: lane l holds A[i][k], i = l % 32, k = 16 (l / 32) + j, in byte j of
//      its four registers;
//   B: lane l holds B[k][n], n = l % 32, k = 16 (l / 32) + j, likewise;
//   C: register r of lane l holds C[i][n], n = l % 32,
//      i = 8 (r / 4) + 4 (l / 32) + r % 4.
#pragma once

#include "device_common.h"

namespace coli {

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b) {
    const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
}

__host__ __device__ inline int mfma_c_row(int lane, int r) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

// v_mfma_i32_16x16x32_i8: C[16x16] = A[16x32] * B[32x16], one Q8_0 block
// per instruction over 16 rows and 16 columns.  Lane layout (checked by the
// debug hook coli_moe_debug_mfma_i8_16 against a host matmul):
//   A: lane l holds A[i][k], i = l % 16, k = 8 (l / 16) + j, in byte j of
//      its two registers;
//   B: lane l holds B[k][n], n = l % 16, k = 8 (l / 16) + j, likewise;
//   C: register r of lane l holds C[i][n], n = l % 16, i = 4 (l / 16) + r.
__device__ __forceinline__ i32x4 mfma_i8_16x16x32(int64_t a, int64_t b) {
    const i32x4 zero = {0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, zero, 0, 0, 0);
}

// The scaled low-precision matrix-core operation of gfx950,
// v_mfma_scale_f32_32x32x64_f8f6f4: C[32x32] = sum over K = 64 of A * B, in
// binary32, each 32-deep half of K multiplied by the E8M0 scales of its A
// row and B column (2^(s - 127)).  FA / FB pick the operand formats (0 FP8
// E4M3, 4 FP4 E2M1).  Lane layout (measured on MI355X; checked by the debug
// hook coli_moe_debug_mfma_f8f6f4 against a host model), with K in two
// 32-deep scale blocks kb = 0, 1:
//   FP8 operands: lane l holds row (A) or column (B) l % 32; its bytes 0-15
//      are elements 16 (l / 32) .. 16 (l / 32) + 15 of block 0 and its bytes
//      16-31 the same elements of block 1;
//   FP4 A: lane l holds block l / 32 of row l % 32, element j in nibble j of
//      its first 16 bytes (even j in the low nibble); the last four registers
//      are not read;
//   scales: the E8M0 byte of lane 32 kb + i scales block kb of row (A) or
//      column (B) i;
//   C: as for the int8 operation (mfma_c_row).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_scale_f8f6f4(i32x8 a, i32x8 b, int sa, int sb) {
    const f32x16 zero = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                         0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, zero, FA, FB, 0, sa, 0, sb);
}

}  // namespace coli
