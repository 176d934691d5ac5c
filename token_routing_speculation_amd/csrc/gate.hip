// route_gate and route_estimator: skinny "NT" products C = A . B^T with A
// [M][K] and B [N][K] both K-contiguous bf16, on gfx950's bf16 MFMA
// (v_mfma_f32_16x16x32_bf16), binary32 accumulation.
//
// Router shapes have few columns (E = 4..160) and long rows (d = 2K..5K):
// the product is bound by streaming A once from HBM, not by the matrix
// cores. A workgroup owns 16*MT rows x 16*NT columns and its four waves split
// the K dimension (wave w takes the 32-wide K steps w, w+4, ...), so each
// operand byte is fetched by exactly one wave, straight into registers in
// the MFMA operand layout (8 contiguous bf16 per lane and row). The A stream
// (from HBM) is prefetched two steps ahead, the small B (L2-resident) one
// step ahead. Partial tiles are summed through LDS at the end; each wave
// finishes a quarter of the tiles.
//
// Used by the "Federation of Experts (FoE)" article's router scores g[i]
// and by "Speculating Experts Accelerates Inference for Mixture-of-Experts"
// (item 2.A: next gate on q_l; item 2.C: the estimator MLP).
#include "common.hpp"

namespace route {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
enum { EPI_F32 = 0, EPI_BIAS_GELU_BF16 = 1, EPI_BIAS_F32 = 2 };

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

template <int MT, int NT>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_nt(const uint16_t* __restrict__ A,
                                                           int64_t M, int Kd,
                                                           const uint16_t* __restrict__ B,
                                                           int N, const float* __restrict__ bias,
                                                           void* __restrict__ C, int epi) {
  constexpr int TILES = MT * NT;
  __shared__ f32x4 red[TILES * 3 * kWave];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (16 * MT);
  const int col0 = blockIdx.y * (16 * NT);
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;  // this lane's 8 contiguous k inside a 32-wide step

  // Rows past M and columns past N are clamped onto the last valid one: their
  // results are never stored, so their operands need no masking.
  const uint16_t* ap[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t row = row0 + 16 * m + r16;
    ap[m] = A + (row < M ? row : M - 1) * static_cast<int64_t>(Kd) + kq;
  }
  const uint16_t* bp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = col0 + 16 * t + r16;
    bp[t] = B + static_cast<int64_t>(col < N ? col : N - 1) * Kd + kq;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Step s covers k in [32 s, 32 s + 32). Only the last step can run past Kd
  // (Kd % 32 != 0): those lanes read k = 0 of the same row (in bounds, finite)
  // and their A operand is zeroed, so they add nothing. Loads past the last
  // step are clamped onto it (their data is never used): no branches.
  const int nsteps = (Kd + 31) / 32;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto koff = [&](int st) {
    st = st < nsteps ? st : nsteps - 1;
    const int k = 32 * st;
    return k + kq < Kd ? k : 0;
  };
  auto load_a = [&](u32x4 (&a)[MT], int st) {
    const int k = koff(st);
    const bool ok = 32 * st + kq < Kd || st >= nsteps;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 x = ld16_stream(ap[m] + k);
      a[m] = ok ? x : zero;
    }
  };
  auto load_b = [&](u32x4 (&b)[NT], int st) {
    const int k = koff(st);
#pragma unroll
    for (int t = 0; t < NT; ++t) b[t] = ld16(bp[t] + k);
  };

  if (w < nsteps) {
    u32x4 a0[MT], a1[MT], a2[MT], b0[NT], b1[NT];
    load_a(a0, w);
    load_b(b0, w);
    load_a(a1, w + 4);
    for (int st = w; st < nsteps; st += 4) {
      load_a(a2, st + 8);
      load_b(b1, st + 4);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = mfma16x16x32(a0[m], b0[t], acc[m][t]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        a0[m] = a1[m];
        a1[m] = a2[m];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) b0[t] = b1[t];
    }
  }

  // split-K reduction: tile i is finished by wave i % 4; the other three
  // waves park their partial tile in LDS slot (i * 3 + writer rank).
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = m * NT + t;
      const int owner = i & 3;
      if (w != owner) {
        const int rank = w < owner ? w : w - 1;
        red[(i * 3 + rank) * kWave + lane] = acc[m][t];
      }
    }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = m * NT + t;
      if (w != (i & 3)) continue;
      f32x4 v = acc[m][t];
#pragma unroll
      for (int r = 0; r < 3; ++r) v += red[(i * 3 + r) * kWave + lane];
      const int col = col0 + 16 * t + r16;
      if (col >= N) continue;
      const float bcol = epi != EPI_F32 ? bias[col] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = row0 + 16 * m + 4 * (lane >> 4) + j;
        if (row >= M) continue;
        const int64_t o = row * N + col;
        if (epi == EPI_BIAS_GELU_BF16) {
          static_cast<uint16_t*>(C)[o] =
              static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(v[j] + bcol)));
        } else {
          static_cast<float*>(C)[o] = v[j] + bcol;
        }
      }
    }
}

template <int MT>
static void launch_nt(int NT, dim3 grid, hipStream_t s, const uint16_t* A, int64_t M, int Kd,
                      const uint16_t* B, int N, const float* bias, void* C, int epi) {
  switch (NT) {
#define ROUTE_NT_CASE(nt)                                                                  \
  case nt:                                                                                 \
    if constexpr (true)                                                                    \
      gemm_nt<MT, nt><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);         \
    break;
    ROUTE_NT_CASE(1) ROUTE_NT_CASE(2) ROUTE_NT_CASE(3) ROUTE_NT_CASE(4) ROUTE_NT_CASE(5)
    ROUTE_NT_CASE(6) ROUTE_NT_CASE(7) ROUTE_NT_CASE(8) ROUTE_NT_CASE(9) ROUTE_NT_CASE(10)
#undef ROUTE_NT_CASE
    default: break;
  }
}

// Picks the tile shape: all columns in one block when E <= 160 (A streamed
// once), else blocks of 128 columns; rows per block shrink until the grid
// has at least one workgroup per CU, and to 32 when a 64-row tile would not
// fit in registers.
static int gemm_launch(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N,
                       const float* bias, void* C, int epi, hipStream_t s) {
  if (M == 0) return ROUTE_OK;
  const int ntiles = (N + 15) / 16;
  const int NT = ntiles <= 10 ? ntiles : 8;
  const unsigned gy = ceil_div(ntiles, NT);
  // 64-row tiles with more than 7 column tiles exceed the register file
  int MT = 4;
  while (MT > 1 && static_cast<int64_t>(ceil_div(M, 16 * MT)) * gy < 256) MT >>= 1;
  dim3 grid(ceil_div(M, 16 * MT), gy);
  if (MT == 4)
    launch_nt<4>(NT, grid, s, A, M, Kd, B, N, bias, C, epi);
  else if (MT == 2)
    launch_nt<2>(NT, grid, s, A, M, Kd, B, N, bias, C, epi);
  else
    launch_nt<1>(NT, grid, s, A, M, Kd, B, N, bias, C, epi);
  return launch_status();
}

}  // namespace route

using namespace route;

ROUTE_API int route_gate(const uint16_t* x, int64_t n, int32_t d, const uint16_t* w, int32_t E,
                         float* logits, hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || E < 1) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!x || !w || !logits) return ROUTE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  return gemm_launch(x, n, d, w, E, nullptr, logits, EPI_F32, s);
}

ROUTE_API size_t route_estimator_workspace_size(int64_t n, int32_t hd) {
  if (n < 0 || hd < 0) return 0;
  return align_up(static_cast<size_t>(n) * hd * sizeof(uint16_t), 256);
}

ROUTE_API int route_estimator(const uint16_t* q, int64_t n, int32_t d, const uint16_t* w1,
                              const float* b1, int32_t hd, const uint16_t* w2, const float* b2,
                              int32_t E, float* logits, void* ws, size_t ws_bytes,
                              hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || hd < 8 || hd % 8 != 0 || E < 1) return ROUTE_ERR_SHAPE;
  if (hd > 4096 || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!q || !w1 || !b1 || !w2 || !b2 || !logits) return ROUTE_ERR_NULL;
  if (!aligned16(q) || !aligned16(w1) || !aligned16(w2)) return ROUTE_ERR_ALIGN;
  if (!ws || ws_bytes < route_estimator_workspace_size(n, hd)) return ROUTE_ERR_WORKSPACE;
  if (!aligned16(ws)) return ROUTE_ERR_ALIGN;
  uint16_t* h = static_cast<uint16_t*>(ws);
  int st = gemm_launch(q, n, d, w1, hd, b1, h, EPI_BIAS_GELU_BF16, s);
  if (st != ROUTE_OK) return st;
  return gemm_launch(h, n, hd, w2, E, b2, logits, EPI_BIAS_F32, s);
}
