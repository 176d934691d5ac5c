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
// (from HBM) is prefetched kPfa steps ahead, the small B (L2-resident) one
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
constexpr int kPfa = 3;  // A-operand prefetch depth, in K steps
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
  const int w = wave_id();
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
#pragma unroll
    for (int m = 0; m < MT; ++m) a[m] = ld16_stream(ap[m] + k);
  };
  // zero the lanes of a partial last step (applied at use, not at load, so
  // the select never waits for a load still in flight)
  auto mask_tail = [&](u32x4 (&a)[MT], int st) {
    if (32 * st + 32 > Kd) {
      const bool ok = 32 * st + kq < Kd;
#pragma unroll
      for (int m = 0; m < MT; ++m) a[m] = ok ? a[m] : zero;
    }
  };
  auto load_b = [&](u32x4 (&b)[NT], int st) {
    const int k = koff(st);
#pragma unroll
    for (int t = 0; t < NT; ++t) b[t] = ld16(bp[t] + k);
  };

  // Loads retire in issue order (one vmcnt counter), so each step issues the
  // B operand it needs next before the A operand it needs three steps later:
  // waiting for B then never waits for the A loads still in flight. The loop
  // body is written out over the four A buffers and two B buffers so no
  // buffer is ever copied (a copy would wait for its load); scheduling
  // barriers keep the compiler from sinking the prefetch next to its use.
  static_assert(kPfa == 3, "the ring below holds kPfa + 1 = 4 A buffers");
  if (w < nsteps) {
    u32x4 a0[MT], a1[MT], a2[MT], a3[MT], b0[NT], b1[NT];
    load_a(a0, w);
    load_a(a1, w + 4);
    load_a(a2, w + 8);
    load_b(b0, w);
    int st = w;
// one K step: prefetch B for the next step and A for three steps on, then
// multiply the current A and B
#define ROUTE_GATE_STEP(AU, AL, BU, BL)                                              \
  load_b(BL, st + 4);                                                              \
  load_a(AL, st + 12);                                                             \
  __builtin_amdgcn_sched_barrier(0);                                               \
  mask_tail(AU, st);                                                               \
  _Pragma("unroll") for (int m = 0; m < MT; ++m)                                   \
      _Pragma("unroll") for (int t = 0; t < NT; ++t) acc[m][t] =                   \
          mfma16x16x32(AU[m], BU[t], acc[m][t]);                                   \
  __builtin_amdgcn_sched_barrier(0);                                               \
  st += 4;
    // this wave's steps: w, w+4, ... < nsteps; full groups of four, then the rest
    const int mine = (nsteps - w + 3) / 4;
    for (int g = 0; g < mine / 4; ++g) {
      ROUTE_GATE_STEP(a0, a3, b0, b1)
      ROUTE_GATE_STEP(a1, a0, b1, b0)
      ROUTE_GATE_STEP(a2, a1, b0, b1)
      ROUTE_GATE_STEP(a3, a2, b1, b0)
    }
    const int rest = mine % 4;
    if (rest > 0) { ROUTE_GATE_STEP(a0, a3, b0, b1) }
    if (rest > 1) { ROUTE_GATE_STEP(a1, a0, b1, b0) }
    if (rest > 2) { ROUTE_GATE_STEP(a2, a1, b0, b1) }
#undef ROUTE_GATE_STEP
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
    ROUTE_NT_CASE(1) ROUTE_NT_CASE(2)
#undef ROUTE_NT_CASE
    default: break;
  }
}

// ---------------------------------------------------------------------------
// LDS-staged product for wider outputs (E > 32). A workgroup owns a BM x BN
// tile (BM = 16 MTW WR rows, BN = 16 NTW WC columns) and walks K in 64-wide
// steps. Each step's A and B slabs are fetched by all 256 threads as whole
// 128-byte lines (16 bytes per thread and load), kept in a four-deep register
// ring, written to one of two LDS buffers (row stride 144 bytes, so the MFMA
// fragment reads of 16 consecutive rows spread over the banks) and consumed
// by the four waves, laid out WR x WC over the tile, each owning a
// 16 MTW x 16 NTW block of accumulators. The register ring is written out
// over four statically named slots so no slot is ever copied (a copy would
// wait for its load): the loads of step s+3 are in flight while step s runs.
// ---------------------------------------------------------------------------
constexpr int kLdsRowBytes = 144;  // 128 data bytes + 16 pad

template <int BM, int BN>
struct StageRegs {
  static constexpr int A_CH = BM * 8 / kGemmThreads;  // 16-byte chunks per thread
  static constexpr int B_CH = BN * 8 / kGemmThreads;
  u32x4 a[A_CH];
  u32x4 b[B_CH];
};

template <int MTW, int NTW, int WR>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_lds(const uint16_t* __restrict__ A,
                                                            int64_t M, int Kd,
                                                            const uint16_t* __restrict__ B,
                                                            int N, const float* __restrict__ bias,
                                                            void* __restrict__ C, int epi) {
  constexpr int WC = 4 / WR;
  constexpr int BM = 16 * MTW * WR;
  constexpr int BN = 16 * NTW * WC;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "slabs must split evenly over 256 threads");
  using Regs = StageRegs<BM, BN>;
  constexpr int ABYTES = BM * kLdsRowBytes;
  constexpr int BBYTES = BN * kLdsRowBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * (ABYTES + BBYTES)];

  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int wr = w % WR;
  const int wc = w / WR;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int col0 = blockIdx.y * BN;

  // global chunk c of a slab: row c / 8, 16-byte piece c % 8 of its 128 bytes
  const uint16_t* agp[Regs::A_CH];
  int alds[Regs::A_CH];
#pragma unroll
  for (int i = 0; i < Regs::A_CH; ++i) {
    const int c = tid + i * kGemmThreads;
    const int64_t row = row0 + c / 8;
    agp[i] = A + (row < M ? row : M - 1) * static_cast<int64_t>(Kd) + (c % 8) * 8;
    alds[i] = (c / 8) * kLdsRowBytes + (c % 8) * 16;
  }
  const uint16_t* bgp[Regs::B_CH];
  int blds[Regs::B_CH];
#pragma unroll
  for (int i = 0; i < Regs::B_CH; ++i) {
    const int c = tid + i * kGemmThreads;
    const int col = col0 + c / 8;
    bgp[i] = B + static_cast<int64_t>(col < N ? col : N - 1) * Kd + (c % 8) * 8;
    blds[i] = ABYTES + (c / 8) * kLdsRowBytes + (c % 8) * 16;
  }
  const int kpiece = tid % 8 * 8;  // this thread's k offset inside a step (same for all chunks)

  const int nsteps = (Kd + 63) / 64;
  auto load = [&](Regs& r, int st) {
    st = st < nsteps ? st : nsteps - 1;  // past the end: reload the last step (unused)
    const int k = 64 * st;
    const int ko = k + kpiece < Kd ? k : 0;  // a partial last step reads in bounds
#pragma unroll
    for (int i = 0; i < Regs::A_CH; ++i) r.a[i] = ld16_stream(agp[i] + ko);
#pragma unroll
    for (int i = 0; i < Regs::B_CH; ++i) r.b[i] = ld16(bgp[i] + ko);
  };
  auto store = [&](const Regs& r, int st, int buf) {
    char* base = lds + buf * (ABYTES + BBYTES);
#pragma unroll
    for (int i = 0; i < Regs::A_CH; ++i) *reinterpret_cast<u32x4*>(base + alds[i]) = r.a[i];
#pragma unroll
    for (int i = 0; i < Regs::B_CH; ++i) *reinterpret_cast<u32x4*>(base + blds[i]) = r.b[i];
    // a partial last step: the pieces past Kd (read from k = 0) become zeros.
    // Done as a second store behind a branch, so no select on the loaded data
    // can be hoisted ahead of its load.
    if (64 * st + 64 > Kd && 64 * st + kpiece >= Kd) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < Regs::A_CH; ++i) *reinterpret_cast<u32x4*>(base + alds[i]) = zero;
#pragma unroll
      for (int i = 0; i < Regs::B_CH; ++i) *reinterpret_cast<u32x4*>(base + blds[i]) = zero;
    }
  };

  f32x4 acc[MTW][NTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment addresses: A tile m, k half h -> row 16 m + (lane & 15), piece 4 h + lane / 16
  const int afrag = (wr * 16 * MTW + (lane & 15)) * kLdsRowBytes + (lane >> 4) * 16;
  const int bfrag = ABYTES + (wc * 16 * NTW + (lane & 15)) * kLdsRowBytes + (lane >> 4) * 16;
  auto compute = [&](int buf) {
    const char* base = lds + buf * (ABYTES + BBYTES);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 af[MTW], bf[NTW];
#pragma unroll
      for (int m = 0; m < MTW; ++m)
        af[m] = *reinterpret_cast<const u32x4*>(base + afrag + m * 16 * kLdsRowBytes + h * 64);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        bf[t] = *reinterpret_cast<const u32x4*>(base + bfrag + t * 16 * kLdsRowBytes + h * 64);
#pragma unroll
      for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[m][t] = mfma16x16x32(af[m], bf[t], acc[m][t]);
    }
  };

  Regs r0, r1, r2, r3;
  load(r0, 0);
  load(r1, 1);
  load(r2, 2);
  int st = 0;
// one K step: prefetch step st+3, publish step st to LDS, multiply it
#define ROUTE_LDS_STEP(RU, RL, BUF) \
  load(RL, st + 3);                 \
  store(RU, st, BUF);               \
  __syncthreads();                  \
  compute(BUF);                     \
  ++st;
  for (int g = 0; g < nsteps / 4; ++g) {
    ROUTE_LDS_STEP(r0, r3, 0)
    ROUTE_LDS_STEP(r1, r0, 1)
    ROUTE_LDS_STEP(r2, r1, 0)
    ROUTE_LDS_STEP(r3, r2, 1)
  }
  const int rest = nsteps % 4;
  if (rest > 0) { ROUTE_LDS_STEP(r0, r3, 0) }
  if (rest > 1) { ROUTE_LDS_STEP(r1, r0, 1) }
  if (rest > 2) { ROUTE_LDS_STEP(r2, r1, 0) }
#undef ROUTE_LDS_STEP

#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int col = col0 + wc * 16 * NTW + 16 * t + (lane & 15);
      if (col >= N) continue;
      const float bcol = epi != EPI_F32 ? bias[col] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = row0 + wr * 16 * MTW + 16 * m + 4 * (lane >> 4) + j;
        if (row >= M) continue;
        const int64_t o = row * N + col;
        const float v = acc[m][t][j] + bcol;
        if (epi == EPI_BIAS_GELU_BF16)
          static_cast<uint16_t*>(C)[o] = static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(v)));
        else
          static_cast<float*>(C)[o] = v;
      }
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
  if (N > 32) {
    // LDS-staged tiles: 64 x 160 for E <= 160 (one pass over A), else 64 x 128
    // blocks of columns; 32-row tiles when 64-row ones would leave CUs idle
    const bool wide = ntiles > 8;
    const unsigned gy = wide && ntiles > 10 ? ceil_div(ntiles, 8) : 1;
    const int bn = gy > 1 ? 128 : (ntiles <= 4 ? 64 : (ntiles <= 8 ? 128 : 160));
    const bool tall = static_cast<int64_t>(ceil_div(M, 64)) * gy >= 256;
    dim3 grid(ceil_div(M, tall ? 64 : 32), gy);
    if (bn == 160 && tall)
      gemm_lds<2, 5, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    else if (bn == 160)
      gemm_lds<1, 5, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    else if (bn == 128 && tall)
      gemm_lds<2, 4, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    else if (bn == 128)
      gemm_lds<1, 4, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    else if (tall)
      gemm_lds<2, 2, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    else
      gemm_lds<1, 2, 2><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    return launch_status();
  }
  // skinny outputs (E <= 32): split-K register kernel, 16..64-row tiles
  const int NT = ntiles;
  int MT = 4;
  while (MT > 1 && static_cast<int64_t>(ceil_div(M, 16 * MT)) < 256) MT >>= 1;
  dim3 grid(ceil_div(M, 16 * MT), 1);
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
