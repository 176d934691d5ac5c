// route_qhidden: q_l = LN_{l+1}(d_l + r_l), "Speculating Experts Accelerates
// Inference for Mixture-of-Experts", technical summary item 2.A. One wave
// per row: the row (d <= 8192) is held in registers as 16-byte vectors, the
// mean and the centred variance are two wave reductions in binary32, and the
// normalised row is stored as bf16 (nearest even). The block's eight rows
// share d_l, staged once in LDS (read from L2 per row it would be twice the
// row's own bytes); the row loads are unconditional (vectors past the row
// end reload vector 0 and are masked out), so they issue back to back.
#include "common.hpp"
#include "gemm.hpp"
#include "mfma.hpp"
#include "topk.hpp"

#include <type_traits>

namespace route {

constexpr int kLnThreads = 512;
constexpr int kLnMaxD = 8192;

// Wave-wide float sum, every lane gets it: DPP row reductions, then the four
// row sums through scalar reads.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xf, 0xf, true));
  };
  v += dpp(v, std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + e);
}

// q for one row, held by one wave: lane `lane` owns 16-byte vectors
// v = lane + c * 64 (c < CPL, v < nv = d / 8) of r + d_l (d_l staged in LDS
// as sd), normalised with the row's binary32 mean and centred variance,
// scaled and shifted (gamma, beta: nullable), rounded to bf16 (nearest
// even) and packed eight to a vector in q[c]. raw[] holds the row's loads
// (vectors past the row end were loaded from vector 0 and are ignored).
template <int CPL>
__device__ __forceinline__ void ln_row(const u32x4 (&raw)[CPL], const float* __restrict__ sd,
                                       const float* __restrict__ gamma,
                                       const float* __restrict__ beta, int d, float eps,
                                       int lane, u32x4 (&q)[CPL]) {
  const int nv = d >> 3;
  float x[CPL][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    const int vv = v < nv ? v : 0;
    unpack8(raw[c], x[c]);
    const float4 d0 = *reinterpret_cast<const float4*>(sd + 8 * vv);
    const float4 d1 = *reinterpret_cast<const float4*>(sd + 8 * vv + 4);
    x[c][0] += d0.x; x[c][1] += d0.y; x[c][2] += d0.z; x[c][3] += d0.w;
    x[c][4] += d1.x; x[c][5] += d1.y; x[c][6] += d1.z; x[c][7] += d1.w;
    if (v < nv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += x[c][e];
    }
  }
  const float mean = wave_sum_f32(sum) / static_cast<float>(d);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = x[c][e] - mean;
        ss += t * t;
      }
    }
  }
  const float var = wave_sum_f32(ss) / static_cast<float>(d);
  const float inv = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    const int vv = v < nv ? v : 0;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (x[c][e] - mean) * inv;
    if (gamma) {
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * vv);
      const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * vv + 4);
      y[0] *= g0.x; y[1] *= g0.y; y[2] *= g0.z; y[3] *= g0.w;
      y[4] *= g1.x; y[5] *= g1.y; y[6] *= g1.z; y[7] *= g1.w;
    }
    if (beta) {
      const float4 b0 = *reinterpret_cast<const float4*>(beta + 8 * vv);
      const float4 b1 = *reinterpret_cast<const float4*>(beta + 8 * vv + 4);
      y[0] += b0.x; y[1] += b0.y; y[2] += b0.z; y[3] += b0.w;
      y[4] += b1.x; y[5] += b1.y; y[6] += b1.z; y[7] += b1.w;
    }
    q[c] = pack8_cvt(y);
  }
}

template <int CPL>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ row, int nv, int lane,
                                         u32x4 (&raw)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    raw[c] = ld16_stream(row + 8 * (v < nv ? v : 0));
  }
}

template <int CPL>  // 16-byte vectors per lane
__global__ __launch_bounds__(kLnThreads) void qhidden_kernel(
    const uint16_t* __restrict__ r, const float* __restrict__ dvec,
    const float* __restrict__ gamma, const float* __restrict__ beta, int64_t n, int d,
    float eps, uint16_t* __restrict__ q) {
  __shared__ __attribute__((aligned(16))) float sd[kLnMaxD];
  for (int j = threadIdx.x * 4; j < d; j += kLnThreads * 4)
    *reinterpret_cast<float4*>(sd + j) = *reinterpret_cast<const float4*>(dvec + j);
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kLnThreads / kWave) + wave_id();
  if (i >= n) return;
  const int lane = lane_id();
  const int nv = d >> 3;
  u32x4 raw[CPL], y[CPL];
  load_row<CPL>(r + static_cast<size_t>(i) * d, nv, lane, raw);
  ln_row<CPL>(raw, sd, gamma, beta, d, eps, lane, y);
  uint16_t* out = q + static_cast<size_t>(i) * d;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) st16(out + 8 * v, y[c]);
  }
}

// ---------------------------------------------------------------------------
// route_qgate: the next gate applied to q_l without q leaving the chip. A
// workgroup of eight waves owns BM rows: each row's q is computed by
// ln_row (the same arithmetic as route_qhidden, so the bf16 values are the
// same) and kept in LDS as a BM x D bf16 tile (128 KB of the CU's 160 KB);
// then the waves take the 16-column groups of W in turn and multiply the
// resident tile by W's rows, read from L2 as whole lines kQgLead pairs of K
// steps ahead and turned into MFMA fragments through a small per-wave LDS
// buffer. q is neither written nor read back.
// ---------------------------------------------------------------------------
constexpr int kQgThreads = 512;
constexpr int kQgLead = 3;  // W line loads in flight, in pairs of K steps (measured: 3 beats 1, 7 and 15)
// With W packed in fragment order (route_gate_pack), each wave streams its
// column group's fragments straight into registers, this many K steps ahead
// (measured at the Qwen3 shape: 4, 8 and 16 steps 22.4, 22.0 and 22.7 us per
// launch, against 24.9 us for the line loads through LDS; the same bits).
constexpr int kQgPackLead = 8;

// LDS offset of 16-byte piece p of tile row rr. Rows are a multiple of 256
// bytes long, so every row starts at the same bank; gfx950's LDS serves a
// 16-byte read for 16 lanes at a time from a 256-byte window of banks, and
// the piece is XOR-ed with the row's low four bits (within aligned groups of
// sixteen pieces) so the sixteen rows of an MFMA fragment read fall on
// sixteen distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int qg_off(int rr, int p) {
  return rr * D * 2 + ((p ^ (rr & 15)) << 4);
}

// The per-wave W staging rows are 128 bytes: two rows share a 256-byte bank
// window, so the piece is XOR-ed with (row / 2) % 8.
__device__ __forceinline__ int wst_off(int rr, int p) { return rr * 128 + ((p ^ ((rr >> 1) & 7)) << 4); }

// TOPK > 0: also pick each row's top K columns (E <= 128 TOPK, K <= 16), in
// route_topk's order (largest logit first, equal logits to the lower column,
// -0.0 == +0.0), from the logits gathered in LDS; logits may then be NULL.
// TOPK = 0: the product alone. PW: w is in the packed fragment order of
// route_gate_pack instead of rows.
// LN false: the tile is r's rows themselves (dvec, gamma, beta, eps unused),
// for a product whose input is already on hand (the estimator's hidden
// layer). bias (nullable, [E]) is added to every logit before it is stored
// or ranked. hout (TOPK = 0, nullable): instead of the logits, each value
// goes out as bf16(GELU(logit + bias)) into hout [n][E] (the estimator's
// hidden layer, with the arithmetic of the matrix-core kernel's epilogue).
// H2 > 0 (TOPK > 0, PW): the estimator on q_l in one kernel. w (packed) is
// W1 with H2 rows and bias its b1: each value becomes bf16(GELU(. + b1)) as
// above, into the tile (q is done with by then) as an H2-wide bf16 tile; the
// product, top-K and hit count then run on that tile with w2 (packed, E
// rows) and bias2.
template <int BM, int D, int TOPK, bool PW, bool LN = true, int H2 = 0>
__global__ __launch_bounds__(kQgThreads, 1) void qgate_kernel(
    const uint16_t* __restrict__ r, const float* __restrict__ dvec,
    const float* __restrict__ gamma, const float* __restrict__ beta, int64_t n, float eps,
    const uint16_t* __restrict__ w, int E, float* __restrict__ logits, int K,
    int* __restrict__ idx, const int32_t* __restrict__ truth,
    unsigned long long* __restrict__ hits, const float* __restrict__ bias = nullptr,
    uint16_t* __restrict__ hout = nullptr, const uint16_t* __restrict__ w2 = nullptr,
    const float* __restrict__ bias2 = nullptr) {
  static_assert(H2 == 0 || (TOPK > 0 && PW && H2 % 256 == 0 && BM * H2 <= BM * D),
                "the estimator's hidden layer is a packed product into the q tile");
  constexpr int CPL = D / 8 / kWave;
  constexpr int NV = D / 8;
  constexpr int RPW = BM / (kQgThreads / kWave);  // rows per wave
  constexpr int MT = BM / 16;
  constexpr int NPAIRS = D / 64;  // pairs of 32-wide K steps
  static_assert(CPL * 8 * kWave == D && RPW >= 1 && BM % 16 == 0, "tile shape");
  static_assert(NPAIRS % (kQgLead + 1) == 0, "the ring cycles whole");
  __shared__ __attribute__((aligned(16))) float sd[LN ? D : 4];
  __shared__ __attribute__((aligned(16))) char tile[BM * D * 2];
  // the line loads' per-wave staging (16 bytes when W comes packed: the hit
  // count's word only)
  __shared__ __attribute__((aligned(16))) char wstage[PW ? 16 : (kQgThreads / kWave) * 2048];
  const int lane = lane_id(), wv = wave_id();
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  // the top-K epilogue gives row 4 wv + lane / 16 to a 16-lane segment; the
  // true pick this lane compares against is loaded now, so its latency
  // overlaps the rest of the kernel
  int tv = -1;
  if constexpr (TOPK > 0) {
    const int rr = 4 * wv + (lane >> 4);
    if (hits && rr < BM && row0 + rr < n && (lane & 15) < K) tv = truth[(row0 + rr) * K + (lane & 15)];
  }
  if constexpr (LN) {
    for (int j = threadIdx.x * 4; j < D; j += kQgThreads * 4)
      *reinterpret_cast<float4*>(sd + j) = *reinterpret_cast<const float4*>(dvec + j);
    __syncthreads();
  }
  // q rows: wave wv takes tile rows wv, wv + 8, ...; all their loads are
  // issued before the first is normalised. Rows past n repeat row n - 1
  // (their logits are never stored).
  u32x4 raw[RPW][CPL];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int64_t i = row0 + wv + 8 * k;
    load_row<CPL>(r + static_cast<size_t>(i < n ? i : n - 1) * D, NV, lane, raw[k]);
  }
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    u32x4 y[CPL];
    if constexpr (LN) {
      ln_row<CPL>(raw[k], sd, gamma, beta, D, eps, lane, y);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = raw[k][c];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      *reinterpret_cast<u32x4*>(tile + qg_off<D>(wv + 8 * k, lane + c * kWave)) = y[c];
  }
  __syncthreads();
  // W: wave wv takes the 16-column groups wv, wv + 8, ... Each pair of K
  // steps (64 k) of its 16 rows is loaded as whole 128-byte lines (8 lanes
  // per row, two loads), kQgLead pairs ahead, then passed through the wave's
  // own 2 KB of LDS into the fragment layout (LDS operations of one wave
  // complete in order, so no barrier is needed).
  const int r16 = lane & 15, kq = lane >> 4;
  const int ngroups = (E + 15) / 16;
  // packed W: group g, K step st (32 k), lane l's fragment at
  // (g * NSTEPS + st) * 64 + l in 16-byte units; the tile's rows are RL
  // values long (D for q, H2 for the estimator's hidden layer)
  constexpr int NSTEPS = D / 32;
  auto gemm_packed = [&](auto rl, const uint16_t* wsrc, int g, f32x4 (&acc)[MT]) {
    constexpr int RL = decltype(rl)::value;
    constexpr int NS = RL / 32;
    const u32x4* wp = reinterpret_cast<const u32x4*>(wsrc) + static_cast<size_t>(g) * NS * kWave + lane;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_assert(NS % kQgPackLead == 0, "the ring cycles whole");
    u32x4 ring[kQgPackLead];
#pragma unroll
    for (int j = 0; j < kQgPackLead; ++j) ring[j] = wp[j * kWave];
#pragma unroll 1
    for (int st0 = 0; st0 < NS; st0 += kQgPackLead) {
#pragma unroll
      for (int j = 0; j < kQgPackLead; ++j) {
        const int st = st0 + j;
        const u32x4 bf = ring[j];
        // past the last step: reload the last one (in bounds, never used)
        const int nx = st + kQgPackLead < NS ? st + kQgPackLead : NS - 1;
        ring[j] = wp[nx * kWave];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 af =
              *reinterpret_cast<const u32x4*>(tile + qg_off<RL>(16 * m + r16, 4 * st + kq));
          acc[m] = mfma16x16x32(af, bf, acc[m]);
        }
      }
    }
  };
  auto gemm_group_packed = [&](int g, f32x4 (&acc)[MT]) {
    gemm_packed(std::integral_constant<int, D>{}, w, g, acc);
  };
  char* wst = wstage + (PW ? 0 : wv * 2048);
  const int lrow = lane >> 3, lchunk = lane & 7;  // line-load mapping: row, 16-byte chunk
  auto gemm_group_lines = [&](int g, f32x4 (&acc)[MT]) {
    const uint16_t* wq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 16 * g + lrow + 8 * h;
      wq[h] = w + static_cast<int64_t>(c < E ? c : E - 1) * D + 8 * lchunk;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 ring[kQgLead + 1][2];
    auto ldw = [&](u32x4 (&dst)[2], int pp) {
      pp = pp < NPAIRS ? pp : NPAIRS - 1;
#pragma unroll
      for (int h = 0; h < 2; ++h) dst[h] = ld16(wq[h] + 64 * pp);
    };
#pragma unroll
    for (int j = 0; j < kQgLead; ++j) ldw(ring[j], j);
#pragma unroll 1
    for (int p0 = 0; p0 < NPAIRS; p0 += kQgLead + 1) {
#pragma unroll
      for (int j = 0; j <= kQgLead; ++j) {
        const int pp = p0 + j;
        ldw(ring[(j + kQgLead) % (kQgLead + 1)], pp + kQgLead);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = lrow + 8 * h;
          *reinterpret_cast<u32x4*>(wst + wst_off(rr, lchunk)) = ring[j][h];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4 bf = *reinterpret_cast<const u32x4*>(wst + wst_off(r16, kq + 4 * half));
          const int st = 2 * pp + half;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 af =
                *reinterpret_cast<const u32x4*>(tile + qg_off<D>(16 * m + r16, 4 * st + kq));
            acc[m] = mfma16x16x32(af, bf, acc[m]);
          }
        }
      }
    }
  };
  auto gemm_group = [&](int g, f32x4 (&acc)[MT]) {
    if constexpr (PW)
      gemm_group_packed(g, acc);
    else
      gemm_group_lines(g, acc);
  };
  // the bias of the logits the kernel ranks (b2 in the two-layer form)
  const float* const bfin = H2 > 0 ? bias2 : bias;
  auto store_logits = [&](int g, const f32x4 (&acc)[MT]) {
    const int colr = 16 * g + r16;
    if (colr < E) {
      const float b = bfin ? bfin[colr] : 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t row = row0 + 16 * m + 4 * kq + jj;
          if (row < n) logits[row * E + colr] = acc[m][jj] + b;
        }
    }
  };
  auto store_hidden = [&](int g, const f32x4 (&acc)[MT]) {
    const int colr = 16 * g + r16;
    if (colr < E) {
      const float b = bias ? bias[colr] : 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t row = row0 + 16 * m + 4 * kq + jj;
          if (row < n)
            hout[row * E + colr] =
                static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(acc[m][jj] + b)));
        }
    }
  };
  if constexpr (TOPK == 0) {
    for (int g = wv; g < ngroups; g += kQgThreads / kWave) {
      f32x4 acc[MT];
      gemm_group(g, acc);
      if (hout)
        store_hidden(g, acc);
      else
        store_logits(g, acc);
    }
  } else {
    // at most two column groups per wave (E <= 256)
    constexpr int NW = kQgThreads / kWave;
    if constexpr (H2 > 0) {
      // the hidden layer: wave wv takes W1's 16-column groups wv, wv + 8, ...
      // into registers; once every wave is done with q, the tile takes them
      // as bf16(GELU(. + b1)), H2 values a row, laid out as a q tile of
      // that width
      constexpr int GPW = H2 / 16 / NW;
      f32x4 hacc[GPW][MT];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) gemm_group(wv + NW * gi, hacc[gi]);
      __syncthreads();
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int col = 16 * (wv + NW * gi) + r16;
        const float b = bias[col];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<uint16_t*>(tile + qg_off<H2>(16 * m + 4 * kq + jj, col >> 3) +
                                         2 * (col & 7)) =
                static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(hacc[gi][m][jj] + b)));
      }
      __syncthreads();
    }
    f32x4 accs[2][MT];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = wv + NW * gi;
      if (g < ngroups) {
        if constexpr (H2 > 0)
          gemm_packed(std::integral_constant<int, (H2 > 0 ? H2 : D)>{}, w2, g, accs[gi]);
        else
          gemm_group(g, accs[gi]);
        if (logits) store_logits(g, accs[gi]);
      }
    }
    __syncthreads();  // every wave is done with the q tile: it now holds the logits
    float* lt = reinterpret_cast<float*>(tile);  // BM x E
    // this workgroup's hit count, in the W staging area (free from here on)
    unsigned* hit_lds = reinterpret_cast<unsigned*>(wstage);
    if (threadIdx.x == 0) *hit_lds = 0u;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = wv + NW * gi;
      const int col = 16 * g + r16;
      if (g < ngroups && col < E) {
        const float b = bfin ? bfin[col] : 0.f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            lt[(16 * m + 4 * kq + jj) * E + col] = accs[gi][m][jj] + b;
      }
    }
    __syncthreads();
    // a 16-lane segment per row, four rows per wave (rows 4 wv + seg): lane
    // s of a segment holds columns s, s + 16, ... (8 of them for E <= 128);
    // K rounds of a segment max of the keys, equal keys resolved to the
    // lowest column
    constexpr int KPL = 8 * TOPK;  // keys per lane
    const int seg = lane >> 4, sl = lane & 15;
    const int rr = 4 * wv + seg;
    if (4 * wv < BM) {
      const int rrc = rr < BM ? rr : BM - 1;
      uint32_t key[KPL];
#pragma unroll
      for (int v = 0; v < KPL; ++v) {
        const int c = sl + 16 * v;
        key[v] = c < E ? order_key(lt[rrc * E + c]) : 0u;
      }
      int myc = 0;
#pragma unroll
      for (int pick = 0; pick < kMaxK; ++pick) {
        if (pick < K) {
          uint32_t best = 0u;
          int bv = 0;
#pragma unroll
          for (int v = 0; v < KPL; ++v)
            if (key[v] > best) {  // strict: the lowest v on equal keys
              best = key[v];
              bv = v;
            }
          const uint32_t mx = seg_max<16>(best);
          const int col = static_cast<int>(
              seg_min<16>(best == mx ? static_cast<uint32_t>(sl + 16 * bv) : 0xffffffffu));
          const bool mine = sl == (col & 15);
#pragma unroll
          for (int v = 0; v < KPL; ++v) key[v] = (mine && bv == v) ? 0u : key[v];
          if (sl == pick) myc = col;
        }
      }
      const int64_t grow = row0 + rr;
      const bool live = rr < BM && grow < n;
      if (live && sl < K) idx[grow * K + sl] = myc;
      if (hits) {
        // hit count: a pick counts when it is among the row's true experts.
        // The segment ORs its true picks into a bitmask over the columns (a
        // repeated or foreign true pick sets no extra bit) and each lane
        // tests its own pick's bit
        uint32_t mask[KPL / 2];
#pragma unroll
        for (int q = 0; q < KPL / 2; ++q) {
          uint32_t m = (tv >= 32 * q && tv < 32 * q + 32) ? 1u << (tv - 32 * q) : 0u;
          m |= dpp<kDppXor1>(m);
          m |= dpp<kDppXor2>(m);
          m |= dpp<kDppHalfMirror>(m);
          m |= dpp<kDppMirror>(m);
          mask[q] = m;
        }
        uint32_t word = mask[0];
#pragma unroll
        for (int q = 1; q < KPL / 2; ++q) word = (myc >> 5) == q ? mask[q] : word;
        const bool in_truth = (word >> (myc & 31)) & 1u;
        const unsigned long long ball = __ballot(live && sl < K && in_truth);
        if (lane == 0) atomicAdd(hit_lds, static_cast<unsigned>(__popcll(ball)));
      }
    }
    if (hits) {
      __syncthreads();
      if (threadIdx.x == 0 && *hit_lds) atomicAdd(hits, static_cast<unsigned long long>(*hit_lds));
    }
  }
}

// 32 rows per workgroup (16 at d = 4096, where the q tile's rows are twice as long)
template <int TOPK, bool PW = false>
void qgate_launch(int d, int64_t n, hipStream_t s, const uint16_t* r, const float* dvec,
                  const float* gamma, const float* beta, float eps, const uint16_t* w, int E,
                  float* logits, int K, int* idx, const int32_t* truth, unsigned long long* hits) {
  if (d == 1024)
    qgate_kernel<32, 1024, TOPK, PW><<<ceil_div(n, 32), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w, E, logits, K, idx, truth, hits);
  else if (d == 2048)
    qgate_kernel<32, 2048, TOPK, PW><<<ceil_div(n, 32), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w, E, logits, K, idx, truth, hits);
  else
    qgate_kernel<16, 4096, TOPK, PW><<<ceil_div(n, 16), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w, E, logits, K, idx, truth, hits);
}

// route_gate_pack: one thread per 16-byte fragment piece of the packed
// layout (group g of 16 router rows, K step st of 32, lane l); rows past E
// are zeros.
__global__ void gate_pack_kernel(const uint16_t* __restrict__ w, int E, int d,
                                 uint16_t* __restrict__ wp) {
  const int nsteps = d / 32;
  const int64_t total = static_cast<int64_t>((E + 15) / 16) * nsteps * kWave;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= total) return;
  const int l = static_cast<int>(q & (kWave - 1));
  const int64_t gs = q / kWave;
  const int st = static_cast<int>(gs % nsteps);
  const int g = static_cast<int>(gs / nsteps);
  const int row = 16 * g + (l & 15);
  u32x4 v = u32x4{0, 0, 0, 0};
  if (row < E) v = ld16(w + static_cast<size_t>(row) * d + 32 * st + 8 * (l >> 4));
  st16(wp + q * 8, v);
}

}  // namespace route

using namespace route;

ROUTE_API size_t route_gate_packed_size(int32_t E, int32_t d) {
  if (E < 1 || d < 32 || d % 32 != 0) return 0;
  return static_cast<size_t>((E + 15) / 16) * 16 * static_cast<size_t>(d) * sizeof(uint16_t);
}

ROUTE_API int route_gate_pack(const uint16_t* w, int32_t E, int32_t d, uint16_t* wp,
                              hipStream_t s) {
  if (E < 1 || d < 32 || d % 32 != 0) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (!w || !wp) return ROUTE_ERR_NULL;
  if (!aligned16(w) || !aligned16(wp)) return ROUTE_ERR_ALIGN;
  const int64_t total = static_cast<int64_t>((E + 15) / 16) * (d / 32) * kWave;
  gate_pack_kernel<<<ceil_div(total, 256), 256, 0, s>>>(w, E, d, wp);
  return launch_status();
}

ROUTE_API int route_qhidden(const uint16_t* r, const float* dvec, const float* gamma,
                            const float* beta, int64_t n, int32_t d, float eps, uint16_t* q,
                            hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f)) return ROUTE_ERR_SHAPE;
  if (d > 8192) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !q) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(q) || !aligned16(dvec)) return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
  const unsigned grid = ceil_div(n, kLnThreads / kWave);
  const int nv = d / 8;
  if (nv <= 64)
    qhidden_kernel<1><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 128)
    qhidden_kernel<2><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 256)
    qhidden_kernel<4><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 512)
    qhidden_kernel<8><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else
    qhidden_kernel<16><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  return launch_status();
}

ROUTE_API int route_qgate(const uint16_t* r, const float* dvec, const float* gamma,
                          const float* beta, int64_t n, int32_t d, float eps, const uint16_t* w,
                          int32_t E, float* logits, hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f) || E < 1) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || (d != 1024 && d != 2048 && d != 4096)) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !w || !logits) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(dvec) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
  qgate_launch<0>(d, n, s, r, dvec, gamma, beta, eps, w, E, logits, 0, nullptr, nullptr, nullptr);
  return launch_status();
}

// Host checks shared by the two top-K forms.
static int qgate_topk_check(const uint16_t* r, const float* dvec, const float* gamma,
                            const float* beta, int64_t n, int32_t d, float eps, const uint16_t* w,
                            int32_t E, int32_t K, const int32_t* idx, const int32_t* truth,
                            const unsigned long long* hits) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f) || E < 1 || K < 1 || K > E)
    return ROUTE_ERR_SHAPE;
  if (E > 256 || K > kMaxK || (d != 1024 && d != 2048 && d != 4096)) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !w || !idx || (!truth != !hits)) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(dvec) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
  return ROUTE_OK;
}

ROUTE_API int route_qgate_topk(const uint16_t* r, const float* dvec, const float* gamma,
                               const float* beta, int64_t n, int32_t d, float eps,
                               const uint16_t* w, int32_t E, int32_t K, float* logits,
                               int32_t* idx, const int32_t* truth, unsigned long long* hits,
                               hipStream_t s) {
  const int st = qgate_topk_check(r, dvec, gamma, beta, n, d, eps, w, E, K, idx, truth, hits);
  if (st != ROUTE_OK || n == 0) return st;
  if (E <= 128)
    qgate_launch<1>(d, n, s, r, dvec, gamma, beta, eps, w, E, logits, K, idx, truth, hits);
  else
    qgate_launch<2>(d, n, s, r, dvec, gamma, beta, eps, w, E, logits, K, idx, truth, hits);
  return launch_status();
}

ROUTE_API int route_est_out_topk_packed(const uint16_t* h, int64_t n, int32_t hd,
                                        const uint16_t* w2p, const float* b2, int32_t E,
                                        int32_t K, float* logits, int32_t* idx,
                                        const int32_t* truth, unsigned long long* hits,
                                        hipStream_t s) {
  if (n < 0 || hd < 8 || hd % 8 != 0 || E < 1 || K < 1 || K > E) return ROUTE_ERR_SHAPE;
  if (E > 256 || K > kMaxK || (hd != 512 && hd != 1024 && hd != 2048))
    return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!h || !w2p || !idx || (!truth != !hits)) return ROUTE_ERR_NULL;
  if (!aligned16(h) || !aligned16(w2p)) return ROUTE_ERR_ALIGN;
  const unsigned grid = ceil_div(n, 32);
#define ROUTE_EST_OUT(D, T)                                                                   \
  qgate_kernel<32, D, T, true, false><<<grid, kQgThreads, 0, s>>>(                            \
      h, nullptr, nullptr, nullptr, n, 0.f, w2p, E, logits, K, idx, truth, hits, b2)
  if (hd == 512) {
    if (E <= 128) ROUTE_EST_OUT(512, 1); else ROUTE_EST_OUT(512, 2);
  } else if (hd == 1024) {
    if (E <= 128) ROUTE_EST_OUT(1024, 1); else ROUTE_EST_OUT(1024, 2);
  } else {
    if (E <= 128) ROUTE_EST_OUT(2048, 1); else ROUTE_EST_OUT(2048, 2);
  }
#undef ROUTE_EST_OUT
  return launch_status();
}

ROUTE_API int route_qest_hidden_packed(const uint16_t* r, const float* dvec, const float* gamma,
                                       const float* beta, int64_t n, int32_t d, float eps,
                                       const uint16_t* w1p, const float* b1, int32_t hd,
                                       uint16_t* h, hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f) || hd < 8 || hd % 8 != 0)
    return ROUTE_ERR_SHAPE;
  if (hd > kMaxExperts || (d != 1024 && d != 2048 && d != 4096)) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !w1p || !b1 || !h) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(dvec) || !aligned16(w1p)) return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
  if (d == 1024)
    qgate_kernel<32, 1024, 0, true><<<ceil_div(n, 32), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w1p, hd, nullptr, 0, nullptr, nullptr, nullptr, b1, h);
  else if (d == 2048)
    qgate_kernel<32, 2048, 0, true><<<ceil_div(n, 32), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w1p, hd, nullptr, 0, nullptr, nullptr, nullptr, b1, h);
  else
    qgate_kernel<16, 4096, 0, true><<<ceil_div(n, 16), kQgThreads, 0, s>>>(
        r, dvec, gamma, beta, n, eps, w1p, hd, nullptr, 0, nullptr, nullptr, nullptr, b1, h);
  return launch_status();
}

ROUTE_API int route_qest_topk_packed(const uint16_t* r, const float* dvec, const float* gamma,
                                     const float* beta, int64_t n, int32_t d, float eps,
                                     const uint16_t* w1p, const float* b1, int32_t hd,
                                     const uint16_t* w2p, const float* b2, int32_t E, int32_t K,
                                     float* logits, int32_t* idx, const int32_t* truth,
                                     unsigned long long* hits, hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f) || hd < 8 || hd % 8 != 0 || E < 1 ||
      K < 1 || K > E)
    return ROUTE_ERR_SHAPE;
  if ((d != 1024 && d != 2048 && d != 4096) || (hd != 512 && hd != 1024) || hd > d ||
      E > 256 || K > kMaxK)
    return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !w1p || !b1 || !w2p || !idx || (!truth != !hits)) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(dvec) || !aligned16(w1p) || !aligned16(w2p))
    return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
#define ROUTE_QEST(BM, D, T, H)                                                               \
  qgate_kernel<BM, D, T, true, true, H><<<ceil_div(n, BM), kQgThreads, 0, s>>>(              \
      r, dvec, gamma, beta, n, eps, w1p, E, logits, K, idx, truth, hits, b1, nullptr, w2p, b2)
#define ROUTE_QEST_T(BM, D, H)                    \
  do {                                            \
    if (E <= 128) ROUTE_QEST(BM, D, 1, H);        \
    else ROUTE_QEST(BM, D, 2, H);                 \
  } while (0)
  if (hd == 512) {
    if (d == 1024) ROUTE_QEST_T(32, 1024, 512);
    else if (d == 2048) ROUTE_QEST_T(32, 2048, 512);
    else ROUTE_QEST_T(16, 4096, 512);
  } else {
    if (d == 1024) ROUTE_QEST_T(32, 1024, 1024);
    else if (d == 2048) ROUTE_QEST_T(32, 2048, 1024);
    else ROUTE_QEST_T(16, 4096, 1024);
  }
#undef ROUTE_QEST_T
#undef ROUTE_QEST
  return launch_status();
}
ROUTE_API int route_qgate_topk_packed(const uint16_t* r, const float* dvec, const float* gamma,
                                      const float* beta, int64_t n, int32_t d, float eps,
                                      const uint16_t* wp, int32_t E, int32_t K, float* logits,
                                      int32_t* idx, const int32_t* truth,
                                      unsigned long long* hits, hipStream_t s) {
  const int st = qgate_topk_check(r, dvec, gamma, beta, n, d, eps, wp, E, K, idx, truth, hits);
  if (st != ROUTE_OK || n == 0) return st;
  if (E <= 128)
    qgate_launch<1, true>(d, n, s, r, dvec, gamma, beta, eps, wp, E, logits, K, idx, truth, hits);
  else
    qgate_launch<2, true>(d, n, s, r, dvec, gamma, beta, eps, wp, E, logits, K, idx, truth, hits);
  return launch_status();
}
