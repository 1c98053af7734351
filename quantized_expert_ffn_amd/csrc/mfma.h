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

}  // namespace coli
