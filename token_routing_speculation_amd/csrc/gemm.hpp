// Internal (not exported) entry to the staged bf16 product of gate.hip, for
// other translation units of the library: C[M][N] = A[M][Kd] . B[N][Kd]^T in
// binary32, A and B bf16 rows (Kd % 8 == 0, 16-byte aligned). Returns a
// ROUTE_* status; enqueues on s.
#pragma once

#include "common.hpp"

namespace route {
int gemm_f32(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N, float* C,
             hipStream_t s);
}  // namespace route
