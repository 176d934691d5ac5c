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
// is prefetched kPfa steps ahead, the small B (L2-resident) one step ahead.
// Partial tiles are summed through LDS at the end; each wave finishes a
// quarter of the tiles.
//
// A is read with plain (not streaming) loads in both kernels: in the routing
// pass the activations were just written by the shuffle and are read again by
// the dispatch, and plain loads leave them resident in MI355X's memory-side
// cache for that second read (about 40 us of HBM reads per DeepSeek-V2-shaped
// pass, measured against streaming loads here).
//
// Used by the "Federation of Experts (FoE)" article's router scores g[i]
// and by "Speculating Experts Accelerates Inference for Mixture-of-Experts"
// (item 2.A: next gate on q_l; item 2.C: the estimator MLP).
//
// gemm_launch picks the kernel per shape: the split-K register kernel for
// E <= 32, the matrix-core kernels of mma.hip when K % 128 == 0 (faster on
// every measured shape), and the staged kernel below otherwise.
#include "common.hpp"
#include "gemm.hpp"
#include "mfma.hpp"
#include <type_traits>

namespace route {

constexpr int kGemmThreads = 256;
constexpr int kPfa = 3;  // A-operand prefetch depth, in K steps

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
    for (int m = 0; m < MT; ++m) a[m] = ld16(ap[m] + k);
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
      const float bcol = epi != kEpiF32 ? bias[col] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = row0 + 16 * m + 4 * (lane >> 4) + j;
        if (row >= M) continue;
        const int64_t o = row * N + col;
        if (epi == kEpiBiasGeluBf16) {
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
// steps. Each step's slabs are fetched as whole 128-byte lines (16 bytes per
// lane and load), written to one of two LDS buffers and consumed by four
// waves laid out WR x WC over the tile, each owning a 16 MTW x 16 NTW block
// of accumulators. Slab rows are 128 bytes with the 16-byte piece index
// XORed with the row's low three bits, so neither the row-wise stores nor
// the MFMA fragment reads (16 consecutive rows, one piece) pile onto a few
// LDS banks; on gfx950 this measured as fast as the best padded stride
// (160 bytes) in less LDS.
//
// Staging is split by operand: waves 0-1 fetch the A slab, waves 2-3 the B
// slab. Loads retire in issue order per wave, so a wave that fetched both
// would wait on its long-latency A stream whenever it needs B; with the
// roles split, A runs further ahead than B (small, L2-resident). Each role's
// register ring is indexed with compile-time slots only, so no slot is ever
// copied (a copy would wait for its load).
// ---------------------------------------------------------------------------
constexpr bool kLdsSwizzle = true;
constexpr int kLdsRowBytes = 160;  // row stride when not swizzled: 128 data bytes + 32 pad

// LDS byte offset of 16-byte piece `piece` (0..7) of slab row rbase + r16,
// where rbase is a multiple of 16. gfx950's LDS serves a 16-byte read for 16
// lanes at a time from a 256-byte window of banks, i.e. two 128-byte rows:
// the piece is XOR-ed with (r16 / 2) % 8, so the 16 rows of a fragment read
// (one piece each) fall on 16 distinct 16-byte bank groups. Swizzling by
// r16 % 8 instead leaves rows r and r + 8 on the same banks (measured: half
// of all LDS cycles were bank conflicts).
__device__ __forceinline__ int lds_off(int rbase, int r16, int piece) {
  if (kLdsSwizzle) return (rbase + r16) * 128 + ((piece ^ ((r16 >> 1) & 7)) << 4);
  return (rbase + r16) * kLdsRowBytes + (piece << 4);
}
constexpr int kLdsRow = kLdsSwizzle ? 128 : kLdsRowBytes;

// Prefetch leads (steps in flight ahead of the one consumed) for KG K groups
// per workgroup: with two groups sharing a CU each needs half the lead, and
// the smaller rings keep both groups' waves within 256 registers.
template <int KG>
struct Leads;
template <>
struct Leads<1> {
  static constexpr int A = 7, B = 3;
};
template <>
struct Leads<2> {
  static constexpr int A = 3, B = 1;
};

// Operand loads of the staged kernel: a wave-uniform base and a 32-bit byte
// offset per lane. POL < 0 is a plain global load; POL >= 0 a buffer load
// whose cache-policy bits are POL (bit 0 sc0, bit 1 nt, bit 4 sc1); buffer
// loads also return zeros for any offset past the descriptor's extent.
constexpr int kLdGlobal = -1;

struct Operand {
  const char* base;  // wave-uniform
  __amdgpu_buffer_rsrc_t rsrc;
};

__device__ __forceinline__ Operand make_operand(const void* base, uint32_t extent_bytes) {
  Operand o;
  o.base = static_cast<const char*>(base);
  // dword 3: the raw (untyped) buffer format of gfx9-family descriptors
  o.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(extent_bytes), 0x00020000);
  return o;
}

template <int POL>
__device__ __forceinline__ u32x4 ld_operand(const Operand& o, uint32_t off) {
  if constexpr (POL < 0) {
    return *reinterpret_cast<const u32x4*>(o.base + off);
  } else {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         o.rsrc, static_cast<int>(off), 0, POL));
  }
}

// One role's K loop over nsteps 64-wide steps starting at k0: NCH 16-byte
// chunks per lane and step (byte offsets off[] from the operand base), a ring
// of LEAD + 1 slots. Each step prefetches step st + LEAD, publishes step st
// to LDS buffer st % 2, waits at the barrier and multiplies that buffer.
// Steps, or pieces of a step, at k >= Kd are published as zeros (their loads
// are redirected in bounds to k = 0).
template <int NCH, int LEAD, int POL, class Compute>
__device__ __forceinline__ void stage_loop(const Operand& op, const uint32_t (&off)[NCH],
                                           const int (&lo)[NCH], char* lds, int buf_bytes, int k0,
                                           int nsteps, int Kd, int kpiece, Compute&& compute) {
  constexpr int NSLOT = LEAD + 1;
  static_assert(8 % NSLOT == 0, "a group of eight steps must cycle the ring whole");
  auto koff = [&](int st) {
    st = st < nsteps ? st : nsteps - 1;
    const int k = k0 + 64 * st;
    return static_cast<uint32_t>(k + kpiece < Kd ? k : 0) * 2u;
  };
  u32x4 r[NSLOT][NCH];
  auto load = [&](u32x4 (&d)[NCH], int st) {
    const uint32_t ko = koff(st);
#pragma unroll
    for (int i = 0; i < NCH; ++i) d[i] = ld_operand<POL>(op, off[i] + ko);
  };
  auto store = [&](const u32x4 (&v)[NCH], int st, int buf) {
    char* base = lds + buf * buf_bytes;
#pragma unroll
    for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(base + lo[i]) = v[i];
    // a second store behind a branch, so no select on the loaded data can be
    // hoisted ahead of its load
    const int k = k0 + 64 * st;
    if (k + 64 > Kd && k + kpiece >= Kd) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < NCH; ++i) *reinterpret_cast<u32x4*>(base + lo[i]) = zero;
    }
  };
  // step st at ring slot j (j = st mod 8, a compile-time constant)
  auto step = [&](auto jc, int st) {
    constexpr int j = decltype(jc)::value;
    load(r[(j + LEAD) % NSLOT], st + LEAD);
    store(r[j % NSLOT], st, j & 1);
    __syncthreads();
    compute(j & 1);
  };
#pragma unroll
  for (int j = 0; j < LEAD; ++j) load(r[j], j);
  int st = 0;
  for (int g = 0; g < nsteps / 8; ++g, st += 8) {
    step(std::integral_constant<int, 0>{}, st);
    step(std::integral_constant<int, 1>{}, st + 1);
    step(std::integral_constant<int, 2>{}, st + 2);
    step(std::integral_constant<int, 3>{}, st + 3);
    step(std::integral_constant<int, 4>{}, st + 4);
    step(std::integral_constant<int, 5>{}, st + 5);
    step(std::integral_constant<int, 6>{}, st + 6);
    step(std::integral_constant<int, 7>{}, st + 7);
  }
  const int rest = nsteps % 8;
  if (rest > 0) step(std::integral_constant<int, 0>{}, st);
  if (rest > 1) step(std::integral_constant<int, 1>{}, st + 1);
  if (rest > 2) step(std::integral_constant<int, 2>{}, st + 2);
  if (rest > 3) step(std::integral_constant<int, 3>{}, st + 3);
  if (rest > 4) step(std::integral_constant<int, 4>{}, st + 4);
  if (rest > 5) step(std::integral_constant<int, 5>{}, st + 5);
  if (rest > 6) step(std::integral_constant<int, 6>{}, st + 6);
}

constexpr int kPolA = kLdGlobal;  // cache policy of the A (activation) slabs
constexpr int kPolB = kLdGlobal;  // and of the B (weight) slabs

// KG groups of four waves per workgroup split K in KG contiguous ranges of
// equal step count (the last padded with zero steps, so every wave meets the
// same barriers); each group stages and multiplies its own range in its own
// pair of LDS buffers, and the groups' partial tiles are summed in group
// order at the end. Two groups on one CU overlap one group's LDS phase with
// the other's matrix-core phase.
template <int MTW, int NTW, int WR, int KG>
__global__ __launch_bounds__(kGemmThreads * KG, 1) void gemm_lds(
    const uint16_t* __restrict__ A, int64_t M, int Kd, const uint16_t* __restrict__ B, int N,
    const float* __restrict__ bias, void* __restrict__ C, int epi) {
  constexpr int WC = 4 / WR;
  constexpr int BM = 16 * MTW * WR;
  constexpr int BN = 16 * NTW * WC;
  static_assert(BM % 16 == 0 && BN % 16 == 0, "slabs must split evenly over two waves");
  constexpr int A_CH = BM * 8 / 128;  // 16-byte chunks per lane and step, A role
  constexpr int B_CH = BN * 8 / 128;
  constexpr int ABYTES = BM * kLdsRow;
  constexpr int BBYTES = BN * kLdsRow;
  constexpr int BUF = ABYTES + BBYTES;
  static_assert(KG == 1 || (KG - 1) * 4 * MTW * NTW * kWave * 16 <= KG * 2 * BUF,
                "partial tiles must fit in the staging buffers");
  __shared__ __attribute__((aligned(16))) char lds[KG * 2 * BUF];

  const int wave = wave_id();
  const int grp = wave / 4;  // K group
  const int w = wave % 4;    // wave inside its group
  const int lane = threadIdx.x & (kWave - 1);
  const int wr = w % WR;
  const int wc = w / WR;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int col0 = blockIdx.y * BN;
  const int sub = (w & 1) * kWave + lane;  // lane index inside its role's two waves
  const int kpiece = lane % 8 * 8;         // k offset of this lane's piece inside a step
  char* glds = lds + grp * 2 * BUF;
  const int per = ((Kd + 63) / 64 + KG - 1) / KG;  // steps per group
  const int k0 = grp * per * 64;

  f32x4 acc[MTW][NTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments: A tile m, k half h -> slab row 16 m + (lane & 15), piece 4 h + lane / 16
  auto compute = [&](int buf) {
    const char* base = glds + buf * BUF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 af[MTW], bf[NTW];
#pragma unroll
      for (int m = 0; m < MTW; ++m)
        af[m] = *reinterpret_cast<const u32x4*>(
            base + lds_off(wr * 16 * MTW + 16 * m, lane & 15, 4 * h + (lane >> 4)));
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        bf[t] = *reinterpret_cast<const u32x4*>(
            base + ABYTES + lds_off(wc * 16 * NTW + 16 * t, lane & 15, 4 * h + (lane >> 4)));
#pragma unroll
      for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[m][t] = mfma16x16x32(af[m], bf[t], acc[m][t]);
    }
  };

  // chunk c of a slab: row c / 8, 16-byte piece c % 8 of the row's 128 bytes.
  // Offsets are in bytes from this tile's first row (first column) and stay
  // below BM * Kd * 2 (BN * Kd * 2); rows past M and columns past N are
  // clamped onto the last valid one (their results are never stored).
  if (w < 2) {
    const int64_t rows = M - row0 < BM ? M - row0 : BM;
    const Operand op = make_operand(A + row0 * Kd, static_cast<uint32_t>(rows * Kd * 2));
    uint32_t off[A_CH];
    int lo[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = sub + i * 128;
      const int r = c / 8 < rows ? c / 8 : static_cast<int>(rows) - 1;
      off[i] = static_cast<uint32_t>(r * Kd + (c % 8) * 8) * 2u;
      lo[i] = lds_off(c / 128 * 16, c / 8 % 16, c % 8);
    }
    stage_loop<A_CH, Leads<KG>::A, kPolA>(op, off, lo, glds, BUF, k0, per, Kd, kpiece, compute);
  } else {
    const int cols = N - col0 < BN ? N - col0 : BN;
    const Operand op = make_operand(B + static_cast<int64_t>(col0) * Kd,
                                    static_cast<uint32_t>(static_cast<int64_t>(cols) * Kd * 2));
    uint32_t off[B_CH];
    int lo[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = sub + i * 128;
      const int r = c / 8 < cols ? c / 8 : cols - 1;
      off[i] = static_cast<uint32_t>(r * Kd + (c % 8) * 8) * 2u;
      lo[i] = ABYTES + lds_off(c / 128 * 16, c / 8 % 16, c % 8);
    }
    stage_loop<B_CH, Leads<KG>::B, kPolB>(op, off, lo, glds, BUF, k0, per, Kd, kpiece, compute);
  }

  if (KG > 1) {
    // groups 1.. park their partial tiles in LDS; group 0 adds them in order
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    __syncthreads();
    if (grp > 0) {
#pragma unroll
      for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          red[(((grp - 1) * 4 + w) * MTW * NTW + m * NTW + t) * kWave + lane] = acc[m][t];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g)
#pragma unroll
      for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[m][t] += red[(((g - 1) * 4 + w) * MTW * NTW + m * NTW + t) * kWave + lane];
  }

#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int col = col0 + wc * 16 * NTW + 16 * t + (lane & 15);
      if (col >= N) continue;
      const float bcol = epi != kEpiF32 ? bias[col] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = row0 + wr * 16 * MTW + 16 * m + 4 * (lane >> 4) + j;
        if (row >= M) continue;
        const int64_t o = row * N + col;
        const float v = acc[m][t][j] + bcol;
        if (epi == kEpiBiasGeluBf16)
          static_cast<uint16_t*>(C)[o] = static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(v)));
        else
          static_cast<float*>(C)[o] = v;
      }
    }
}

template <int MTW, int NTW, int WR>
static void launch_lds(int kg, dim3 grid, hipStream_t s, const uint16_t* A, int64_t M, int Kd,
                       const uint16_t* B, int N, const float* bias, void* C, int epi) {
  if (kg == 2)
    gemm_lds<MTW, NTW, WR, 2><<<grid, kGemmThreads * 2, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
  else
    gemm_lds<MTW, NTW, WR, 1><<<grid, kGemmThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
}

static int gemm_launch(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N,
                       const float* bias, void* C, int epi, hipStream_t s) {
  if (M == 0) return ROUTE_OK;
  // the staged kernel's tile byte offsets are 32-bit; the same limit holds
  // for every E > 32, whichever kernel runs
  if (N > 32 && Kd > (1 << 22)) return ROUTE_ERR_UNSUPPORTED;
  // K a multiple of 128: the matrix-core kernels of mma.hip (faster than the
  // staged kernel below on every measured shape)
  if (mma_fits(M, Kd, N)) return mma_launch(A, M, Kd, B, N, bias, C, epi, s);
  const int ntiles = (N + 15) / 16;
  if (N > 32) {
    // LDS-staged tiles: 64 x 160 for E <= 160 (one pass over A), else 64 x 128
    // blocks of columns; 32-row tiles when 64-row ones would leave CUs idle
    const bool wide = ntiles > 8;
    const unsigned gy = wide && ntiles > 10 ? ceil_div(ntiles, 8) : 1;
    const int bn = gy > 1 ? 128 : (ntiles <= 4 ? 64 : (ntiles <= 8 ? 128 : 160));
    const bool tall = static_cast<int64_t>(ceil_div(M, 64)) * gy >= 256;
    dim3 grid(ceil_div(M, tall ? 64 : 32), gy);
    // two K groups per workgroup when one workgroup per CU is all the grid
    // gives (the groups then share the CU's SIMDs); one group otherwise
    const int kg = static_cast<int64_t>(grid.x) * grid.y <= 256 ? 2 : 1;
    if (bn == 160 && tall)
      launch_lds<2, 5, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
    else if (bn == 160)
      launch_lds<1, 5, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
    else if (bn == 128 && tall)
      launch_lds<2, 4, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
    else if (bn == 128)
      launch_lds<1, 4, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
    else if (tall)
      launch_lds<2, 2, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
    else
      launch_lds<1, 2, 2>(kg, grid, s, A, M, Kd, B, N, bias, C, epi);
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

int gemm_f32(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N, float* C,
             hipStream_t s) {
  return gemm_launch(A, M, Kd, B, N, nullptr, C, kEpiF32, s);
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
  return gemm_launch(x, n, d, w, E, nullptr, logits, kEpiF32, s);
}

ROUTE_API int route_est_hidden(const uint16_t* q, int64_t n, int32_t d, const uint16_t* w1,
                              const float* b1, int32_t hd, uint16_t* h, hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || hd < 8 || hd % 8 != 0) return ROUTE_ERR_SHAPE;
  if (hd > 4096) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!q || !w1 || !b1 || !h) return ROUTE_ERR_NULL;
  if (!aligned16(q) || !aligned16(w1) || !aligned16(h)) return ROUTE_ERR_ALIGN;
  return gemm_launch(q, n, d, w1, hd, b1, h, kEpiBiasGeluBf16, s);
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
  int st = gemm_launch(q, n, d, w1, hd, b1, h, kEpiBiasGeluBf16, s);
  if (st != ROUTE_OK) return st;
  return gemm_launch(h, n, hd, w2, E, b2, logits, kEpiBiasF32, s);
}
