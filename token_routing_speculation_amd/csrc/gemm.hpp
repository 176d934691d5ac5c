// Internal (not exported) entries to the bf16 products, for the translation
// units of the library: C[M][N] = A[M][Kd] . B[N][Kd]^T in binary32, A and B
// bf16 rows (Kd % 8 == 0, 16-byte aligned), with an optional epilogue per
// element. Each returns a ROUTE_* status and enqueues on s.
#pragma once

#include "common.hpp"

namespace route {

// Epilogues: v = C[i][j] (+ bias[j]); stored as binary32, or as bf16 (nearest
// even) of the exact GELU.
enum GemmEpi { kEpiF32 = 0, kEpiBiasGeluBf16 = 1, kEpiBiasF32 = 2 };

// GELU with the error function (not the tanh approximation):
// GELU(x) = x Phi(x) = (x / 2) erfc(-x / sqrt 2). erfc(z), z >= 0, comes from
// the Chebyshev fit published in Numerical Recipes (2nd ed., section 6.2,
// "erfcc"), t exp(-z^2 + P(t)) with t = 1 / (1 + z / 2): its fractional
// error is below 1.2e-7 for every z (1.04e-7 measured against a float64
// erfc), so GELU keeps that relative accuracy in the negative tail too, and
// the bf16 result is the correctly rounded one except within ~1e-6 of a
// rounding boundary. One exponential and one reciprocal instead of a
// general-purpose erf: the epilogue of the estimator's first product
// (2048 -> 512 per token) was about a quarter of that kernel's time.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float ec = t * __expf(fmaf(-z, z, p));  // erfc(|x| / sqrt 2)
  return 0.5f * x * (x >= 0.f ? 2.0f - ec : ec);
}

// gate.hip: picks the kernel for the shape (the matrix-core kernel of
// mma.hip where it applies) and launches it.
int gemm_f32(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N, float* C,
             hipStream_t s);

// mma.hip: the matrix-core kernels with operands staged straight into LDS
// (32 x 32 x 16 tiles; 64 x 160 tiles of 16 x 16 x 32 for 129..160 columns).
// They take Kd % 128 == 0 and N > 32; mma_launch returns
// ROUTE_ERR_UNSUPPORTED for any other shape.
bool mma_fits(int64_t M, int Kd, int N);
int mma_launch(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N, const float* bias,
               void* C, int epi, hipStream_t s);

}  // namespace route
