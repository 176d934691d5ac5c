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
//       slices, one wave per tile with 8 x 8 accumulators per lane, tiles
//       below the Gram block's diagonal skipped (float64 products of bf16
//       and binary32 values are exact), slices summed in slice order;
//   chol_diag / chol_panel / chol_update : blocked right-looking Cholesky,
//       64-wide blocks, L in place in the lower triangle and L^T written to
//       the strict upper one (so both solves read rows of 64 contiguous
//       values); the diagonal block and the panel rows one wave each, a lane
//       per row, the row in registers;
//   tri_solve : L Z = R, then L^T W = Z, one workgroup per right-hand side,
//       64-row blocks solved by one wave, the rest updated by all;
//   est_weights_kernel : W2 = W'[:hd]^T rounded once to bf16 (float64 ->
//       bf16 directly, nearest even), b2 = W'[hd].
// Every step has a fixed operation order, so results are reproducible. Fused
// multiply-adds are allowed: in the Gram products they change nothing (each
// product is exact in float64), and the factor and solves are accurate to
// float64 rounding either way.
#include "common.hpp"

namespace route {

constexpr int kFitTile = 64;
constexpr int kFitThreads = 256;
constexpr int kFitKc = 8;         // rows of the K dimension staged per step
constexpr int kFitSlices = 32;    // K slices of the Gram product

// Tiles of H'^T [H' | Y] below the diagonal of the Gram block (every column
// j < m, tile column < tile row) are not computed: G is symmetric, and their
// entries equal their mirror images bit for bit (the same exact products
// summed in the same row order), which the mirror tiles write for them.
__host__ __device__ __forceinline__ bool gram_tile_skipped(int bi, int bj, int m) {
  return bj < bi && (bj + 1) * kFitTile <= m;
}

// part[s][i][j] = sum over rows of slice s of H'[n][i] * X[n][j], i < m = hd + 1,
// j < m + E. One wave per 64 x 64 output tile and slice, 8 x 8 accumulators
// per lane (rows ty + 8 a, columns tx + 8 b); rows staged kFitKc at a time in
// LDS as float64, the next chunk's loads issued before this chunk's FMAs.
constexpr int kGramThreads = 64;

__global__ __launch_bounds__(kGramThreads) void est_gram_kernel(const uint16_t* __restrict__ h,
                                                                const float* __restrict__ y,
                                                                int64_t n, int hd, int E,
                                                                double* __restrict__ part) {
  __shared__ double sa[2][kFitKc][kFitTile];
  __shared__ double sb[2][kFitKc][kFitTile];
  const int m = hd + 1, mc = hd + 1 + E;
  const int nbj = (mc + kFitTile - 1) / kFitTile;
  const int bi = blockIdx.x / nbj, bj = blockIdx.x % nbj;
  if (gram_tile_skipped(bi, bj, m)) return;
  const int i0 = bi * kFitTile, j0 = bj * kFitTile;
  const int s = blockIdx.z;
  const int64_t lo = n * s / kFitSlices, hi = n * (s + 1) / kFitSlices;
  const int t = threadIdx.x, tx = t % 8, ty = t / 8;
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  // lane t stages column t of both operands for the chunk's kFitKc rows. The
  // column's kind is fixed per lane (0: feature h, 1: the bias column of
  // ones, 2: target y, 3: padding); the loads keep raw bits so that none
  // waits before the chunk's products, and rows past the slice are zeroed
  // when published (their loads are clamped onto the last row, n >= 1).
  const int ca = i0 + t, cb = j0 + t;
  const int ka = ca < hd ? 0 : (ca == hd ? 1 : 3);
  const int kb = cb < hd ? 0 : (cb == hd ? 1 : (cb < mc ? 2 : 3));
  // every load is unconditional (indices clamped in bounds) so none waits
  // behind a branch; the kind selects among them when publishing
  const int64_t hca = ca < hd ? ca : hd - 1;
  const int64_t hcb = cb < hd ? cb : hd - 1;
  const int64_t ycb = cb - hd - 1 < 0 ? 0 : (cb - hd - 1 < E ? cb - hd - 1 : E - 1);
  uint32_t ra[kFitKc], rbh[kFitKc], rby[kFitKc];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < kFitKc; ++r) {
      const int64_t nn = k0 + r < n ? k0 + r : n - 1;  // n >= 1; rows past the slice zeroed
      ra[r] = h[nn * hd + hca];
      rbh[r] = h[nn * hd + hcb];
      rby[r] = __float_as_uint(y[nn * E + ycb]);
    }
  };
  auto value = [&](int kind, uint32_t hbits, uint32_t ybits, bool in) -> double {
    const float f = kind == 0 ? __uint_as_float(hbits << 16) : __uint_as_float(ybits);
    const double v = kind == 1 ? 1.0 : (kind == 3 ? 0.0 : static_cast<double>(f));
    return in ? v : 0.0;
  };
  auto publish = [&](int buf, int64_t k0) {
#pragma unroll
    for (int r = 0; r < kFitKc; ++r) {
      const bool in = k0 + r < hi;
      sa[buf][r][t] = value(ka, ra[r], 0u, in);
      sb[buf][r][t] = value(kb, rbh[r], rby[r], in);
    }
  };
  int buf = 0;
  fetch(lo);
  publish(0, lo);
  __syncthreads();
  for (int64_t k0 = lo; k0 < hi; k0 += kFitKc) {
    const bool more = k0 + kFitKc < hi;
    if (more) fetch(k0 + kFitKc);
#pragma unroll 2
    for (int r = 0; r < kFitKc; ++r) {
      double av[8], bv[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) av[a] = sa[buf][r][ty + 8 * a];
#pragma unroll
      for (int b = 0; b < 8; ++b) bv[b] = sb[buf][r][tx + 8 * b];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = acc[a][b] + av[a] * bv[b];
    }
    if (more) publish(buf ^ 1, k0 + kFitKc);
    __syncthreads();
    buf ^= 1;
  }
  double* out = part + static_cast<int64_t>(s) * m * mc;
  // a tile whose mirror image is skipped also writes its transpose there
  const bool mirror = gram_tile_skipped(bj, bi, m);
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = i0 + ty + 8 * a;
    if (i >= m) continue;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int j = j0 + tx + 8 * b;
      if (j < mc) out[static_cast<int64_t>(i) * mc + j] = acc[a][b];
      if (mirror && j < m) out[static_cast<int64_t>(j) * mc + i] = acc[a][b];
    }
  }
}

// gram = sum of the slices in slice order (entries of skipped tiles were
// written by their mirror tiles), rhs likewise.
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

// lambda = ridge * trace / m added to the diagonal: the diagonal loaded in
// parallel into LDS, summed by one thread in index order.
__global__ __launch_bounds__(kFitThreads) void fit_regularise(double* __restrict__ A, int m,
                                                              double ridge) {
  extern __shared__ double dg[];
  __shared__ double lam;
  for (int i = threadIdx.x; i < m; i += kFitThreads) dg[i] = A[static_cast<int64_t>(i) * m + i];
  __syncthreads();
  if (threadIdx.x == 0) {
    double tr = 0.0;
    for (int i = 0; i < m; ++i) tr = tr + dg[i];
    lam = ridge * tr / static_cast<double>(m);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += kFitThreads)
    A[static_cast<int64_t>(i) * m + i] = dg[i] + lam;
}

// v of lane `lane` (wave-uniform) to every lane.
__device__ __forceinline__ double lane_bcast(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

// Factor of the diagonal block at k0 (b = min(64, m - k0) rows): one wave,
// lane r holds row r in registers. Step j: L[j][j] = sqrt(a[j][j]),
// L[r][j] = a[r][j] / L[j][j] (r > j), then a[r][c] -= L[r][j] L[c][j] for
// j < c <= r, with column j shared through LDS. Writes L (lower) and L^T
// (strict upper) of the block; info |= 1 where a pivot is not positive.
__global__ __launch_bounds__(kWave) void chol_diag(double* __restrict__ A, int m, int k0,
                                                   int* __restrict__ info) {
  __shared__ double T[kFitTile][kFitTile + 1];
  __shared__ double colv[kFitTile];
  const int b = m - k0 < kFitTile ? m - k0 : kFitTile;
  const int r = threadIdx.x;
  // the block's lower triangle, row i read across the lanes (coalesced), all
  // 64 loads issued before the first is used
  {
    double v[kFitTile];
#pragma unroll
    for (int i = 0; i < kFitTile; ++i)
      v[i] = (i < b && r <= i) ? A[static_cast<int64_t>(k0 + i) * m + k0 + r] : 0.0;
#pragma unroll
    for (int i = 0; i < kFitTile; ++i) T[i][r] = v[i];
  }
  __syncthreads();
  double a[kFitTile];
#pragma unroll
  for (int c = 0; c < kFitTile; ++c) a[c] = r < b ? T[r][c] : 0.0;
#pragma unroll
  for (int j = 0; j < kFitTile; ++j) {
    if (j < b) {
      const double d = lane_bcast(a[j], j);
      if (r == 0 && !(d > 0.0) && info) atomicOr(info, 1);
      const double sd = sqrt(d > 0.0 ? d : 1.0);
      const double l = r > j ? a[j] * (1.0 / sd) : (r == j ? sd : 0.0);
      a[j] = l;
      colv[r] = r > j ? l : 0.0;
      __syncthreads();
#pragma unroll
      for (int c = j + 1; c < kFitTile; ++c) a[c] = a[c] - l * colv[c];
      __syncthreads();
    }
  }
#pragma unroll
  for (int c = 0; c < kFitTile; ++c) T[r][c] = a[c];
  __syncthreads();
  if (r < b)
    for (int i = 0; i < b; ++i)  // row i: L[i][r] for r <= i, L^T[i][r] = L[r][i] for r > i
      A[static_cast<int64_t>(k0 + i) * m + k0 + r] = r <= i ? T[i][r] : T[r][i];
}

// Panel below the diagonal block: each row x of A21 becomes x L11^{-T}:
// x[j] *= 1 / L[j][j], then x[c] -= x[j] L[c][j] for c > j, j ascending
// (forward substitution along the row, by columns). One wave per 64 rows, a
// lane per row held in registers; L11^T (the block's upper triangle) and the
// pivots' reciprocals are read from LDS by broadcast. Launched only while
// rows remain below a full 64-wide diagonal block. Writes the rows (lower)
// and their transpose (upper).
__global__ __launch_bounds__(kWave) void chol_panel(double* __restrict__ A, int m, int k0) {
  __shared__ double U[kFitTile][kFitTile + 1];  // U[j][c] = L[c][j], c >= j
  __shared__ double X[kFitTile][kFitTile + 1];
  __shared__ double rpiv[kFitTile];
  const int lane = threadIdx.x;
  const int row0 = k0 + kFitTile + blockIdx.x * kFitTile;
  const int nr = m - row0 < kFitTile ? m - row0 : kFitTile;
  {
    double v[kFitTile], u[kFitTile];  // all loads in flight together
    const int64_t rl = row0 + (lane < nr ? lane : 0);
#pragma unroll
    for (int j = 0; j < kFitTile; ++j) u[j] = A[static_cast<int64_t>(k0 + j) * m + k0 + lane];
#pragma unroll
    for (int c = 0; c < kFitTile; ++c) v[c] = A[rl * m + k0 + c];
#pragma unroll
    for (int j = 0; j < kFitTile; ++j) U[j][lane] = u[j];
#pragma unroll
    for (int c = 0; c < kFitTile; ++c) X[lane][c] = v[c];
  }
  __syncthreads();
  rpiv[lane] = 1.0 / U[lane][lane];
  __syncthreads();
  double x[kFitTile];
#pragma unroll
  for (int c = 0; c < kFitTile; ++c) x[c] = X[lane][c];
#pragma unroll
  for (int j = 0; j < kFitTile; ++j) {
    x[j] = x[j] * rpiv[j];
#pragma unroll
    for (int c = j + 1; c < kFitTile; ++c) x[c] = x[c] - x[j] * U[j][c];
  }
  if (lane < nr) {
    double* arow = A + static_cast<int64_t>(row0 + lane) * m + k0;
#pragma unroll
    for (int c = 0; c < kFitTile; ++c) {
      arow[c] = x[c];                                              // lower
      A[static_cast<int64_t>(k0 + c) * m + row0 + lane] = x[c];  // upper, coalesced
    }
  }
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
  {
    constexpr int kPer = kFitTile * kFitTile / kFitThreads;
    double vi[kPer], vj[kPer];  // all loads in flight together
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = t + q * kFitThreads, r = e / kFitTile, c = e % kFitTile;
      vi[q] = r0 + r < m ? A[static_cast<int64_t>(r0 + r) * m + k0 + c] : 0.0;
      vj[q] = c0 + r < m ? A[static_cast<int64_t>(c0 + r) * m + k0 + c] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = t + q * kFitThreads, r = e / kFitTile, c = e % kFitTile;
      Li[r][c] = vi[q];
      Lj[r][c] = vj[q];
    }
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

// L Z = R, then L^T W = Z, for right-hand side column e (blockIdx.x); the
// vector sits in LDS and is solved 64 rows at a time. Wave 0 solves the
// block's triangle one row per step (lane = row, the solved value broadcast
// from its lane, each pivot applied as its reciprocal); then all threads
// subtract the block's contribution from the rows still unsolved, a thread
// per row, its 64 values loaded together. Forward: z[r] -= L[r][j] z[j],
// j ascending; backward: w[r] -= L[j][r] w[j], j descending. Row j of the
// factor as stored (L below the diagonal, L^T above) holds L[r][j] (r > j)
// and L[j][r] (r < j) contiguous in r, so every load is coalesced.
constexpr int kFitMaxM = 4097;  // hd <= 4096 features plus the bias column

// One 64-row block of the triangle by wave 0 (lane = row): forward
// z[k0 + i] = acc_i / L_ii, then acc_r -= L[r][i] z_i (r > i), i ascending;
// backward the same with L^T, i descending. FULL: b == 64 (no row guards).
template <bool FULL>
__device__ __forceinline__ void solve_block(const double* __restrict__ A, int m, int k0, int b,
                                            int pass, double* __restrict__ z) {
  const int lane = lane_id();
  const bool live = FULL || lane < b;
  const int64_t cl = k0 + (live ? lane : 0);
  double col[kFitTile];  // col[i] = stored (k0 + i, k0 + lane)
#pragma unroll
  for (int i = 0; i < kFitTile; ++i)
    col[i] = (FULL || i < b) ? A[static_cast<int64_t>(k0 + (FULL || i < b ? i : 0)) * m + cl] : 0.0;
  const double rinv = 1.0 / A[cl * m + cl];
  double acc = live ? z[k0 + lane] : 0.0;
  double mine = 0.0;
  if (pass == 0) {
#pragma unroll
    for (int i = 0; i < kFitTile; ++i) {
      if (FULL || i < b) {
        const double zi = lane_bcast(acc * rinv, i);
        mine = lane == i ? zi : mine;
        acc = acc - col[i] * zi;  // lanes > i: L[lane][i]
      }
    }
  } else {
#pragma unroll
    for (int i = kFitTile - 1; i >= 0; --i) {
      if (FULL || i < b) {
        const double wi = lane_bcast(acc * rinv, i);
        mine = lane == i ? wi : mine;
        acc = acc - col[i] * wi;  // lanes < i: L[i][lane]
      }
    }
  }
  if (live) z[k0 + lane] = mine;
}

// The solved block's contribution to the unsolved rows [lo, hi), a thread
// per row: forward z[r] -= L[r][j] z[j] (j ascending), backward
// w[r] -= L[j][r] w[j] (j descending), j over the block.
template <bool FULL>
__device__ __forceinline__ void update_rows(const double* __restrict__ A, int m, int k0, int b,
                                            int pass, int lo, int hi, double* __restrict__ z) {
  for (int r = lo + static_cast<int>(threadIdx.x); r < hi; r += kFitThreads) {
    double v[kFitTile];
#pragma unroll
    for (int jj = 0; jj < kFitTile; ++jj)
      v[jj] = (FULL || jj < b) ? A[static_cast<int64_t>(k0 + jj) * m + r] : 0.0;
    double acc = z[r];
    if (pass == 0) {
#pragma unroll
      for (int jj = 0; jj < kFitTile; ++jj)
        if (FULL || jj < b) acc = acc - v[jj] * z[k0 + jj];
    } else {
#pragma unroll
      for (int jj = kFitTile - 1; jj >= 0; --jj)
        if (FULL || jj < b) acc = acc - v[jj] * z[k0 + jj];
    }
    z[r] = acc;
  }
}

__global__ __launch_bounds__(kFitThreads) void tri_solve(const double* __restrict__ A, int m,
                                                         double* __restrict__ R, int E) {
  extern __shared__ double z[];
  const int e = blockIdx.x, t = threadIdx.x;
  const bool lead = t < kWave;
  for (int i = t; i < m; i += kFitThreads) z[i] = R[static_cast<int64_t>(i) * E + e];
  __syncthreads();
  const int nblk = (m + kFitTile - 1) / kFitTile;
  for (int pass = 0; pass < 2; ++pass) {
    for (int q = 0; q < nblk; ++q) {
      const int kb = pass == 0 ? q : nblk - 1 - q;
      const int k0 = kb * kFitTile;
      const int b = m - k0 < kFitTile ? m - k0 : kFitTile;
      if (lead) {
        if (b == kFitTile)
          solve_block<true>(A, m, k0, b, pass, z);
        else
          solve_block<false>(A, m, k0, b, pass, z);
      }
      __syncthreads();
      const int lo = pass == 0 ? k0 + b : 0, hi = pass == 0 ? m : k0;
      if (b == kFitTile)
        update_rows<true>(A, m, k0, b, pass, lo, hi, z);
      else
        update_rows<false>(A, m, k0, b, pass, lo, hi, z);
      __syncthreads();
    }
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
  if (hd + 1 > kFitMaxM || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (!h || !y || !gram || !rhs) return ROUTE_ERR_NULL;
  if (!ws || ws_bytes < est_fit_gram_workspace_size(n, hd, E)) return ROUTE_ERR_WORKSPACE;
  const int m = hd + 1, mc = hd + 1 + E;
  dim3 grid(ceil_div(m, kFitTile) * ceil_div(mc, kFitTile), 1, kFitSlices);
  double* part = static_cast<double*>(ws);
  est_gram_kernel<<<grid, kGramThreads, 0, s>>>(h, y, n, hd, E, part);
  est_gram_reduce<<<ceil_div(static_cast<int64_t>(m) * mc, kFitThreads), kFitThreads, 0, s>>>(
      part, m, E, gram, rhs);
  return launch_status();
}

ROUTE_API int est_fit_solve(double* gram, double* rhs, int32_t m, int32_t E, double ridge,
                            int32_t* info, hipStream_t s) {
  if (m < 1 || E < 1 || !(ridge >= 0.0)) return ROUTE_ERR_SHAPE;
  if (m > kFitMaxM || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (!gram || !rhs) return ROUTE_ERR_NULL;
  fit_regularise<<<1, kFitThreads, static_cast<size_t>(m) * sizeof(double), s>>>(gram, m, ridge);
  for (int k0 = 0; k0 < m; k0 += kFitTile) {
    chol_diag<<<1, kWave, 0, s>>>(gram, m, k0, info);
    const int rest = m - k0 - kFitTile;
    if (rest > 0) {
      const unsigned nb = ceil_div(rest, kFitTile);
      chol_panel<<<nb, kWave, 0, s>>>(gram, m, k0);
      chol_update<<<dim3(nb, nb), kFitThreads, 0, s>>>(gram, m, k0);
    }
  }
  tri_solve<<<E, kFitThreads, static_cast<size_t>(m) * sizeof(double), s>>>(gram, m, rhs, E);
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
