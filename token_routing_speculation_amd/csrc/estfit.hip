// Fitting the lightweight estimator's output layer: "Speculating Experts
// Accelerates Inference for Mixture-of-Experts", technical summary item 2.C
// (a shallow network predicts the next layer's router logits from q_l) and
// item 4 (a few million training tokens suffice). The hidden layer
// GELU(q W1^T + b1) stays as drawn (random features, the estimator's own
// bf16 activations); the output layer is the ridge fit
//     (H'^T H' + lambda I) W' = H'^T Y,  H' = [H | 1],
//     lambda = ridge * trace(H'^T H') / (hd + 1),
// solved on the GPU in float64:
//   est_gram_kernel / est_gram_reduce : H'^T [H' | Y] as 64 x 64 tiles over K
//       slices (float64 products of bf16 and binary32 values are exact),
//       slices summed in slice order;
//   chol_diag / chol_panel / chol_update : blocked right-looking Cholesky,
//       64-wide blocks, in place in the lower triangle;
//   tri_solve_fwd / tri_solve_bwd : L Z = R (row dot products) and
//       L^T W = Z (row updates), one workgroup per right-hand side;
//   est_weights_kernel : W2 = W'[:hd]^T rounded once to bf16 (float64 ->
//       bf16 directly, nearest even), b2 = W'[hd].
// Every step has a fixed operation order, so results are reproducible.
#include "common.hpp"

#pragma clang fp contract(off)

namespace route {

constexpr int kFitTile = 64;
constexpr int kFitThreads = 256;
constexpr int kFitKc = 16;        // rows of the K dimension staged per step
constexpr int kFitSlices = 16;    // K slices of the Gram product

// Element (n, c) of [H | 1 | Y] (c < hd: feature; c == hd: the bias column;
// c < hd + 1 + E: target; beyond: zero padding).
__device__ __forceinline__ double fit_col(const uint16_t* __restrict__ h,
                                          const float* __restrict__ y, int64_t n, int c, int hd,
                                          int E) {
  if (c < hd) return static_cast<double>(__uint_as_float(static_cast<uint32_t>(h[n * hd + c]) << 16));
  if (c == hd) return 1.0;
  if (c < hd + 1 + E) return static_cast<double>(y[n * E + (c - hd - 1)]);
  return 0.0;
}

// part[s][i][j] = sum over rows of slice s of H'[n][i] * X[n][j], i < m = hd + 1,
// j < m + E. A 64 x 64 output tile per workgroup, 4 x 4 per thread (rows
// ty + 16 a, columns tx + 16 b), rows staged kFitKc at a time in LDS.
__global__ __launch_bounds__(kFitThreads) void est_gram_kernel(const uint16_t* __restrict__ h,
                                                               const float* __restrict__ y,
                                                               int64_t n, int hd, int E,
                                                               double* __restrict__ part) {
  __shared__ double sa[kFitKc][kFitTile];
  __shared__ double sb[kFitKc][kFitTile];
  const int m = hd + 1, mc = hd + 1 + E;
  const int i0 = blockIdx.x * kFitTile, j0 = blockIdx.y * kFitTile;
  const int s = blockIdx.z;
  const int64_t lo = n * s / kFitSlices, hi = n * (s + 1) / kFitSlices;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t k0 = lo; k0 < hi; k0 += kFitKc) {
    // each thread stages 4 elements of each operand: row r = t / 16 ... ,
    // column (t % 16) + 16 q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = t / 16, c = t % 16 + 16 * q;
      const int64_t nn = k0 + r;
      const bool in = nn < hi;
      sa[r][c] = (in && i0 + c < m) ? fit_col(h, y, nn, i0 + c, hd, E) : 0.0;
      sb[r][c] = (in && j0 + c < mc) ? fit_col(h, y, nn, j0 + c, hd, E) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kFitKc; ++r) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = sa[r][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = sb[r][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = acc[a][b] + av[a] * bv[b];
    }
    __syncthreads();
  }
  double* out = part + static_cast<int64_t>(s) * m * mc;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty + 16 * a;
    if (i >= m) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tx + 16 * b;
      if (j < mc) out[static_cast<int64_t>(i) * mc + j] = acc[a][b];
    }
  }
}

// gram[i][j] (j < m) and rhs[i][j - m] from the slices, summed in slice order.
__global__ __launch_bounds__(kFitThreads) void est_gram_reduce(const double* __restrict__ part,
                                                               int m, int E,
                                                               double* __restrict__ gram,
                                                               double* __restrict__ rhs) {
  const int mc = m + E;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kFitThreads + threadIdx.x;
  if (t >= static_cast<int64_t>(m) * mc) return;
  const int i = static_cast<int>(t / mc), j = static_cast<int>(t - static_cast<int64_t>(i) * mc);
  double acc = 0.0;
  for (int s = 0; s < kFitSlices; ++s) acc = acc + part[static_cast<int64_t>(s) * m * mc + t];
  if (j < m)
    gram[static_cast<int64_t>(i) * m + j] = acc;
  else
    rhs[static_cast<int64_t>(i) * E + (j - m)] = acc;
}

// lambda = ridge * trace / m added to the diagonal (one thread: the trace in
// index order).
__global__ void fit_regularise(double* __restrict__ A, int m, double ridge) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double tr = 0.0;
  for (int i = 0; i < m; ++i) tr = tr + A[static_cast<int64_t>(i) * m + i];
  const double lam = ridge * tr / static_cast<double>(m);
  for (int i = 0; i < m; ++i) A[static_cast<int64_t>(i) * m + i] = A[static_cast<int64_t>(i) * m + i] + lam;
}

// Factor of the diagonal block at k0 (b = min(64, m - k0) rows), in LDS.
__global__ __launch_bounds__(kFitThreads) void chol_diag(double* __restrict__ A, int m, int k0,
                                                         int* __restrict__ info) {
  __shared__ double T[kFitTile][kFitTile + 1];
  const int b = m - k0 < kFitTile ? m - k0 : kFitTile;
  const int t = threadIdx.x;
  for (int e = t; e < b * b; e += kFitThreads) {
    const int r = e / b, c = e - r * b;
    T[r][c] = A[static_cast<int64_t>(k0 + r) * m + k0 + c];
  }
  __syncthreads();
  for (int j = 0; j < b; ++j) {
    if (t == 0) {
      const double d = T[j][j];
      if (!(d > 0.0) && info) atomicOr(info, 1);
      T[j][j] = sqrt(d > 0.0 ? d : 1.0);
    }
    __syncthreads();
    for (int r = j + 1 + t; r < b; r += kFitThreads) T[r][j] = T[r][j] / T[j][j];
    __syncthreads();
    const int w = b - j - 1;  // trailing block (j < c <= r < b), row-major pairs
    for (int e = t; e < w * w; e += kFitThreads) {
      const int r = j + 1 + e / w, c = j + 1 + e % w;
      if (c <= r) T[r][c] = T[r][c] - T[r][j] * T[c][j];
    }
    __syncthreads();
  }
  for (int e = t; e < b * b; e += kFitThreads) {
    const int r = e / b, c = e - r * b;
    if (c <= r) A[static_cast<int64_t>(k0 + r) * m + k0 + c] = T[r][c];
  }
}

// Panel below the diagonal block: rows x of A21 become x L11^{-T} (forward
// substitution along the row). One thread per row of a 64-row block.
__global__ __launch_bounds__(kFitTile) void chol_panel(double* __restrict__ A, int m, int k0) {
  __shared__ double L[kFitTile][kFitTile + 1];
  __shared__ double X[kFitTile][kFitTile + 1];
  const int b = m - k0 < kFitTile ? m - k0 : kFitTile;
  const int t = threadIdx.x;
  for (int e = t; e < b * b; e += kFitTile) {
    const int r = e / b, c = e - r * b;
    L[r][c] = A[static_cast<int64_t>(k0 + r) * m + k0 + c];
  }
  const int row = k0 + b + blockIdx.x * kFitTile + t;
  __syncthreads();
  if (row >= m) return;  // no barrier below
  double* a = A + static_cast<int64_t>(row) * m + k0;
  for (int j = 0; j < b; ++j) {
    double v = a[j];
    for (int l = 0; l < j; ++l) v = v - X[t][l] * L[j][l];
    X[t][j] = v / L[j][j];
  }
  for (int j = 0; j < b; ++j) a[j] = X[t][j];
}

// Trailing update A22 -= L21 L21^T for the 64 x 64 tile (bi, bj), bj <= bi,
// of the blocks after k0 + 64; the panel (64 columns) staged in LDS.
__global__ __launch_bounds__(kFitThreads) void chol_update(double* __restrict__ A, int m, int k0) {
  const int bi = blockIdx.x, bj = blockIdx.y;
  if (bj > bi) return;
  __shared__ double Li[kFitTile][kFitTile + 1];
  __shared__ double Lj[kFitTile][kFitTile + 1];
  const int base = k0 + kFitTile;
  const int r0 = base + bi * kFitTile, c0 = base + bj * kFitTile;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  for (int e = t; e < kFitTile * kFitTile; e += kFitThreads) {
    const int r = e / kFitTile, c = e % kFitTile;
    Li[r][c] = r0 + r < m ? A[static_cast<int64_t>(r0 + r) * m + k0 + c] : 0.0;
    Lj[r][c] = c0 + r < m ? A[static_cast<int64_t>(c0 + r) * m + k0 + c] : 0.0;
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = 0.0;
  for (int l = 0; l < kFitTile; ++l) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[a][q] = acc[a][q] + Li[ty + 16 * a][l] * Lj[tx + 16 * q][l];
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = r0 + ty + 16 * a;
    if (r >= m) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + tx + 16 * q;
      if (c < m && c <= r) {
        double* p = A + static_cast<int64_t>(r) * m + c;
        *p = *p - acc[a][q];
      }
    }
  }
}

// L z = r for right-hand side column e (blockIdx.x): z[i] = (r[i] - sum_{j<i}
// L[i][j] z[j]) / L[i][i]; the dot product reduced wave by wave in a fixed
// tree, the waves' partials in wave order.
__global__ __launch_bounds__(kFitThreads) void tri_solve_fwd(const double* __restrict__ L, int m,
                                                             double* __restrict__ R, int E) {
  extern __shared__ double z[];
  __shared__ double wpart[kFitThreads / kWave];
  const int e = blockIdx.x, t = threadIdx.x, w = wave_id();
  for (int i = 0; i < m; ++i) {
    const double* li = L + static_cast<int64_t>(i) * m;
    double p = 0.0;
    for (int j = t; j < i; j += kFitThreads) p = p + li[j] * z[j];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) p = p + __shfl_xor(p, o, kWave);
    if (lane_id() == 0) wpart[w] = p;
    __syncthreads();
    if (t == 0) {
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kFitThreads / kWave; ++q) s = s + wpart[q];
      z[i] = (R[static_cast<int64_t>(i) * E + e] - s) / li[i];
    }
    __syncthreads();
  }
  for (int i = t; i < m; i += kFitThreads) R[static_cast<int64_t>(i) * E + e] = z[i];
}

// L^T w = z for column e: for i = m-1 .. 0, w[i] = z[i] / L[i][i], then
// z[j] -= L[i][j] w[i] for j < i (row i of L, read contiguously).
__global__ __launch_bounds__(kFitThreads) void tri_solve_bwd(const double* __restrict__ L, int m,
                                                             double* __restrict__ R, int E) {
  extern __shared__ double z[];
  const int e = blockIdx.x, t = threadIdx.x;
  for (int i = t; i < m; i += kFitThreads) z[i] = R[static_cast<int64_t>(i) * E + e];
  __syncthreads();
  for (int i = m - 1; i >= 0; --i) {
    const double* li = L + static_cast<int64_t>(i) * m;
    const double wi = z[i] / li[i];
    for (int j = t; j < i; j += kFitThreads) z[j] = z[j] - li[j] * wi;
    __syncthreads();
    if (t == 0) z[i] = wi;
    __syncthreads();
  }
  for (int i = t; i < m; i += kFitThreads) R[static_cast<int64_t>(i) * E + e] = z[i];
}

// float64 -> bf16 bits, nearest even in one rounding: x scaled by its bf16
// spacing 2^(max(e, -126) - 7) (exact), rounded to an integer, scaled back;
// magnitudes past the largest finite bf16 become infinities, NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x != x) return 0x7FC0u;
  if (x == 0.0) return static_cast<uint16_t>(__double2hiint(x) < 0 ? 0x8000u : 0u);
  int ex;
  frexp(x, &ex);               // |x| in [2^(ex-1), 2^ex)
  int e = ex - 1;
  e = e < -126 ? -126 : e;
  const double r = ldexp(rint(ldexp(x, 7 - e)), e - 7);
  if (fabs(r) > 3.3895313892515355e38) return static_cast<uint16_t>(r < 0 ? 0xFF80u : 0x7F80u);
  return static_cast<uint16_t>(__float_as_uint(static_cast<float>(r)) >> 16);  // exact
}

__global__ __launch_bounds__(kFitThreads) void est_weights_kernel(const double* __restrict__ W,
                                                                  int hd, int E,
                                                                  uint16_t* __restrict__ w2,
                                                                  float* __restrict__ b2) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kFitThreads + threadIdx.x;
  if (t < static_cast<int64_t>(E) * hd) {
    const int e = static_cast<int>(t / hd), k = static_cast<int>(t - static_cast<int64_t>(e) * hd);
    w2[t] = f64_to_bf16(W[static_cast<int64_t>(k) * E + e]);
  }
  if (t < E) b2[t] = static_cast<float>(W[static_cast<int64_t>(hd) * E + t]);
}

}  // namespace route

using namespace route;

ROUTE_API size_t est_fit_gram_workspace_size(int64_t n, int32_t hd, int32_t E) {
  if (n < 0 || hd < 1 || E < 1) return 0;
  return align_up(static_cast<size_t>(kFitSlices) * (hd + 1) * (hd + 1 + E) * sizeof(double), 256);
}

ROUTE_API int est_fit_gram(const uint16_t* h, const float* y, int64_t n, int32_t hd, int32_t E,
                           double* gram, double* rhs, void* ws, size_t ws_bytes, hipStream_t s) {
  if (n < 1 || hd < 1 || E < 1) return ROUTE_ERR_SHAPE;
  if (hd > 4096 || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (!h || !y || !gram || !rhs) return ROUTE_ERR_NULL;
  if (!ws || ws_bytes < est_fit_gram_workspace_size(n, hd, E)) return ROUTE_ERR_WORKSPACE;
  const int m = hd + 1, mc = hd + 1 + E;
  dim3 grid(ceil_div(m, kFitTile), ceil_div(mc, kFitTile), kFitSlices);
  double* part = static_cast<double*>(ws);
  est_gram_kernel<<<grid, kFitThreads, 0, s>>>(h, y, n, hd, E, part);
  est_gram_reduce<<<ceil_div(static_cast<int64_t>(m) * mc, kFitThreads), kFitThreads, 0, s>>>(
      part, m, E, gram, rhs);
  return launch_status();
}

ROUTE_API int est_fit_solve(double* gram, double* rhs, int32_t m, int32_t E, double ridge,
                            int32_t* info, hipStream_t s) {
  if (m < 1 || E < 1 || !(ridge >= 0.0)) return ROUTE_ERR_SHAPE;
  if (m > 4097 || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (!gram || !rhs) return ROUTE_ERR_NULL;
  fit_regularise<<<1, 64, 0, s>>>(gram, m, ridge);
  for (int k0 = 0; k0 < m; k0 += kFitTile) {
    chol_diag<<<1, kFitThreads, 0, s>>>(gram, m, k0, info);
    const int rest = m - k0 - kFitTile;
    if (rest > 0) {
      const unsigned nb = ceil_div(rest, kFitTile);
      chol_panel<<<nb, kFitTile, 0, s>>>(gram, m, k0);
      chol_update<<<dim3(nb, nb), kFitThreads, 0, s>>>(gram, m, k0);
    }
  }
  const size_t zb = static_cast<size_t>(m) * sizeof(double);
  tri_solve_fwd<<<E, kFitThreads, zb, s>>>(gram, m, rhs, E);
  tri_solve_bwd<<<E, kFitThreads, zb, s>>>(gram, m, rhs, E);
  return launch_status();
}

ROUTE_API int est_fit_weights(const double* wsol, int32_t hd, int32_t E, uint16_t* w2, float* b2,
                              hipStream_t s) {
  if (hd < 1 || E < 1) return ROUTE_ERR_SHAPE;
  if (!wsol || !w2 || !b2) return ROUTE_ERR_NULL;
  est_weights_kernel<<<ceil_div(static_cast<int64_t>(E) * hd, kFitThreads), kFitThreads, 0, s>>>(
      wsol, hd, E, w2, b2);
  return launch_status();
}
