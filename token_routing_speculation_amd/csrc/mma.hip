// Matrix-core product C = A . B^T (A [M][K], B [N][K], both K-contiguous bf16,
// binary32 accumulation) for the shapes where the matrix cores and the
// L2 -> CU operand stream, not HBM, set the pace: the estimator MLP of
// "Speculating Experts Accelerates Inference for Mixture-of-Experts"
// (item 2.C: 2048 -> 512 -> 128 for every token) and the router products
// (the "Federation of Experts (FoE)" article's router scores g[i]; the next
// gate on q_l, item 2.A), plus the router fused with the shuffled reduce that
// produces its input ("Speculative MoE" section 3.1; srs_gate160_kernel).
//
// gfx950 design (measured on MI355X, see the notes at each choice):
//  - v_mfma_f32_32x32x16_bf16. With one wave per SIMD the 16x16x32 form
//    reached 0.78 PFLOP/s and the 32x32x16 form 1.77 PFLOP/s (8 and 4
//    independent accumulators per wave).
//  - Operands go from global memory straight into LDS
//    (global_load_lds_dwordx4: 64 lanes x 16 bytes land as 1 KB at the
//    wave's LDS base), four stages deep, one barrier per 64-wide K step.
//    No register ring, no LDS store instructions.
//  - A workgroup of four waves owns BM x BN (2 x 2 waves); 128 x 128 when
//    that still gives a workgroup per CU, 64 x 64 otherwise; 129..160
//    columns get their own 64 x 160 variant (mma_nt160_kernel).
//  - Slab rows are 128 bytes, 16-byte pieces XOR-swizzled by (row / 2) % 8:
//    gfx950's LDS serves a 16-byte read for 16 lanes at a time from a
//    256-byte window of banks, so the 32 rows of a fragment read are
//    conflict-free (bank-conflict counter: zero).
//  - All fragments of step s + 1 are read right after its barrier, before the
//    MFMAs of step s are issued, so no MFMA waits on an LDS read; the loads of
//    step s + 4 are interleaved with those MFMAs (two MFMAs, one load), which
//    keeps a wave from stalling behind a full address queue.
#include "common.hpp"
#include "gemm.hpp"
#include "mfma.hpp"
#include "srs.hpp"
#include "topk.hpp"

namespace route {

namespace {

constexpr int kMmaThreads = 256;  // four waves, 2 x 2 over the tile
constexpr int kMmaStages = 4;     // LDS stages (K steps of 64) in the ring

// Waits until this wave's LDS reads have completed.
// Byte offset of logical 16-byte piece p (0..7) of 128-byte slab row r.
__device__ __forceinline__ int slab_off(int r, int p) { return r * 128 + ((p ^ ((r >> 1) & 7)) << 4); }

// The K step that pipeline step st loads when the walk over K starts at step
// rot (< nsteps); the sums then run in that rotated order. Used where every
// workgroup streams the same weight rows: when they are not cached, 256
// workgroups asking for the same lines at once wait on a few HBM channels.
__device__ __forceinline__ int k_step(int st, int rot, int nsteps) {
  const int k = st + rot;
  return k < nsteps ? k : k - nsteps;
}

template <int BM, int BN>
__global__ __launch_bounds__(kMmaThreads, 1) void mma_nt_kernel(
    const uint16_t* __restrict__ A, int64_t M, int Kd, const uint16_t* __restrict__ B, int N,
    const float* __restrict__ bias, void* __restrict__ C, int epi) {
  constexpr int MT = BM / 64, NT = BN / 64;       // 32 x 32 tiles per wave
  constexpr int STAGE = (BM + BN) * 128;          // one K step: BM + BN rows of 64 bf16
  constexpr int NI = (BM + BN) / 8 / 4;           // 1 KB loads per wave and step
  constexpr int NMF = 4 * MT * NT;                // MFMAs per wave and step
  constexpr int PER = NMF / NI > 0 ? NMF / NI : 1;
  static_assert(kMmaStages >= 3 && NI >= 1, "stage ring");
  __shared__ __attribute__((aligned(1024))) char lds[kMmaStages * STAGE];
  const int w = wave_id(), lane = lane_id();
  const int wr = w & 1, wc = w >> 1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int col0 = blockIdx.y * BN;
  const int nsteps = Kd / 64;  // even, >= 2

  // Load j of a stage (j = w + 4 i) fills slab rows 8 j .. 8 j + 7 (A rows
  // first, then B rows): lane l fetches the piece that the swizzle stores at
  // physical piece l % 8 of row 8 j + l / 8. Rows past M and columns past N
  // re-read the last valid one (their results are never stored).
  const char* src[NI];
  int dst[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = w + 4 * i;
    const int r = 8 * j + lane / 8;
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    if (r < BM) {
      const int64_t gr = row0 + r < M ? row0 + r : M - 1;
      src[i] = reinterpret_cast<const char*>(A + gr * Kd) + 16 * p;
    } else {
      const int gc = col0 + (r - BM) < N ? col0 + (r - BM) : N - 1;
      src[i] = reinterpret_cast<const char*>(B + static_cast<int64_t>(gc) * Kd) + 16 * p;
    }
    dst[i] = 8 * j * 128;
  }
  // a step past the end re-loads the last step into its own buffer (the same
  // bytes), which keeps every wave's count of pending loads uniform
  auto load_one = [&](int i, int st) {
    const int ks = st < nsteps ? st : nsteps - 1;
    lds_load16(src[i] + ks * 128, lds + (st % kMmaStages) * STAGE + dst[i]);
  };
  auto load_step = [&](int st) {
#pragma unroll
    for (int i = 0; i < NI; ++i) load_one(i, st);
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][t][e] = 0.f;

  // fragments of one step: chunk c (16 k) is pieces 2c, 2c + 1 of each row
  u32x4 fa[2][4][MT], fb[2][4][NT];
  auto read_frags = [&](int set, int st) {
    const char* base = lds + (st % kMmaStages) * STAGE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        fa[set][c][m] = *reinterpret_cast<const u32x4*>(
            base + slab_off(wr * 32 * MT + 32 * m + (lane & 31), 2 * c + (lane >> 5)));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        fb[set][c][t] = *reinterpret_cast<const u32x4*>(
            base + BM * 128 + slab_off(wc * 32 * NT + 32 * t + (lane & 31), 2 * c + (lane >> 5)));
    }
  };
  // the MFMAs of the step held in `set`, with the loads of step st_load
  // (none if negative) spread between them
  auto mfma_step = [&](int set, int st_load) {
    int q = 0, i = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[m][t] = mfma32x32x16(fa[set][c][m], fb[set][c][t], acc[m][t]);
          if (++q % PER == 0 && i < NI) {
            __builtin_amdgcn_sched_barrier(0);
            if (st_load >= 0) load_one(i, st_load);
            ++i;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
    for (; i < NI; ++i)
      if (st_load >= 0) load_one(i, st_load);
  };
  // step st's data is in LDS for every wave, and every wave has finished
  // reading step st - 1 (so its buffer may be refilled)
  auto sync_step = [&]() {
    wait_lgkm0();
    wait_vmcnt<(kMmaStages - 2) * NI>();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

#pragma unroll
  for (int s = 0; s < kMmaStages - 1; ++s) load_step(s);
  sync_step();
  load_step(kMmaStages - 1);
  read_frags(0, 0);
  for (int st = 0; st < nsteps - 2; st += 2) {
    sync_step();
    read_frags(1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0, st + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
    sync_step();
    read_frags(0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(1, st + 1 + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
  }
  sync_step();
  read_frags(1, nsteps - 1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(0, -1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(1, -1);

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = col0 + wc * 32 * NT + 32 * t + (lane & 31);
      if (col >= N) continue;
      const float bcol = epi != kEpiF32 ? bias[col] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + wr * 32 * MT + 32 * m + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= M) continue;
        const int64_t o = row * N + col;
        const float v = acc[m][t][e] + bcol;
        if (epi == kEpiBiasGeluBf16)
          static_cast<uint16_t*>(C)[o] = static_cast<uint16_t>(f32_to_bf16_bits(gelu_erf(v)));
        else
          static_cast<float*>(C)[o] = v;
      }
    }
}

// The same staging for 129..160 columns (the DeepSeek-V2 router's E = 160),
// where 32 x 32 tiles do not divide the width: a workgroup owns 64 rows x
// 160 columns, so A is read exactly once. Eight waves form two K groups of
// 2 x 2 waves (32 rows x 80 columns each, 2 x 5 tiles of
// v_mfma_f32_16x16x32_bf16); group g multiplies K chunk g of every 64-wide
// step, and the two groups' partial tiles are added once, in group order, at
// the end. A step's 28 loads of 1 KB are shared 4 / 3 over the eight waves.
// On the DeepSeek-V2 shape (16384 x 5120 x 160) it takes 41.5 us, against
// 47.2 us for the staged kernel of gate.hip.
constexpr int kM160Threads = 512;

__global__ __launch_bounds__(kM160Threads, 1) void mma_nt160_kernel(
    const uint16_t* __restrict__ A, int64_t M, int Kd, const uint16_t* __restrict__ B, int N,
    const float* __restrict__ bias, void* __restrict__ C, int epi) {
  constexpr int BM = 64, BN = 160;
  constexpr int MT = 2, NT = 5;                // 16 x 16 tiles per wave
  constexpr int STAGE = (BM + BN) * 128;       // 28 KB
  constexpr int NJ = (BM + BN) / 8;            // 1 KB loads per step (28)
  constexpr int NW = kM160Threads / kWave;     // 8
  constexpr int NI_MAX = (NJ + NW - 1) / NW;   // 4 (waves 0-3), 3 for waves 4-7
  static_assert(NJ == 4 * 4 + 3 * 4, "loads split 4 / 3 over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[kMmaStages * STAGE];
  const int w = wave_id(), lane = lane_id();
  const int g = w >> 2, w4 = w & 3;
  const int wr = w4 & 1, wc = w4 >> 1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int nsteps = Kd / 64;  // even, >= 2
  // workgroups are dealt to the eight XCDs in turn; each XCD's share starts
  // its walk over K an eighth of K further on (the workgroups of one XCD stay
  // in step, so each W line is fetched into that XCD's L2 once and used by
  // all of them)
  const int rot = static_cast<int>((blockIdx.x & 7) * nsteps / 8);
  const int ni = w < 4 ? 4 : 3;

  const char* src[NI_MAX];
  int dst[NI_MAX];
#pragma unroll
  for (int i = 0; i < NI_MAX; ++i) {
    const int j = w + NW * i < NJ ? w + NW * i : w;  // waves 4-7 have no fourth load
    const int r = 8 * j + lane / 8;
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    if (r < BM) {
      const int64_t gr = row0 + r < M ? row0 + r : M - 1;
      src[i] = reinterpret_cast<const char*>(A + gr * Kd) + 16 * p;
    } else {
      const int gc = r - BM < N ? r - BM : N - 1;
      src[i] = reinterpret_cast<const char*>(B + static_cast<int64_t>(gc) * Kd) + 16 * p;
    }
    dst[i] = 8 * j * 128;
  }
  auto load_one = [&](int i, int st) {
    const int ks = k_step(st < nsteps ? st : nsteps - 1, rot, nsteps);
    lds_load16(src[i] + ks * 128, lds + (st % kMmaStages) * STAGE + dst[i]);
  };
  auto load_step = [&](int st) {
#pragma unroll
    for (int i = 0; i < NI_MAX; ++i)
      if (i < ni) load_one(i, st);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's fragments of one step: K chunk g (32 k) is pieces 4g .. 4g + 3
  u32x4 fa[2][MT], fb[2][NT];
  auto read_frags = [&](int set, int st) {
    const char* base = lds + (st % kMmaStages) * STAGE;
    const int pc = 4 * g + (lane >> 4);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      fa[set][m] = *reinterpret_cast<const u32x4*>(
          base + slab_off(wr * 32 + 16 * m + (lane & 15), pc));
#pragma unroll
    for (int t = 0; t < NT; ++t)
      fb[set][t] = *reinterpret_cast<const u32x4*>(
          base + BM * 128 + slab_off(wc * 80 + 16 * t + (lane & 15), pc));
  };
  auto mfma_step = [&](int set, int st_load) {
    int q = 0, i = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[m][t] = mfma16x16x32(fa[set][m], fb[set][t], acc[m][t]);
        if (++q % 2 == 0 && i < NI_MAX) {  // a load after every second MFMA (measured best)
          __builtin_amdgcn_sched_barrier(0);
          if (st_load >= 0 && i < ni) load_one(i, st_load);
          ++i;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
    for (; i < NI_MAX; ++i)
      if (st_load >= 0 && i < ni) load_one(i, st_load);
  };
  auto sync_step = [&]() {
    wait_lgkm0();
    if (w < 4)
      wait_vmcnt<(kMmaStages - 2) * 4>();
    else
      wait_vmcnt<(kMmaStages - 2) * 3>();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

#pragma unroll
  for (int s2 = 0; s2 < kMmaStages - 1; ++s2) load_step(s2);
  sync_step();
  load_step(kMmaStages - 1);
  read_frags(0, 0);
  for (int st = 0; st < nsteps - 2; st += 2) {
    sync_step();
    read_frags(1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0, st + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
    sync_step();
    read_frags(0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(1, st + 1 + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
  }
  sync_step();
  read_frags(1, nsteps - 1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(0, -1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(1, -1);

  // group 1's partial tiles meet group 0's in LDS (the stages are free once
  // every wave's loads have landed and every wave is past its last read)
  wait_vmcnt<0>();
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  if (g == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) red[((w4 * MT + m) * NT + t) * kWave + lane] = acc[m][t];
  }
  __syncthreads();
  if (g == 1) return;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[m][t] += red[((w4 * MT + m) * NT + t) * kWave + lane];
      const int col = wc * 80 + 16 * t + (lane & 15);
      if (col >= N) continue;
      const float bcol = epi != kEpiF32 ? bias[col] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = row0 + wr * 32 + 16 * m + 4 * (lane >> 4) + j;
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

// ---------------------------------------------------------------------------
// The shuffled reduce fused with the router product on its output
// ("Speculative MoE" section 3.1 for the reduce and shuffle; the router
// scores of the "Federation of Experts (FoE)" article on the reduced rows):
// X[dst(i)] = bf16(sum_p partials[p][i]) and logits[dst(i)] = X[dst(i)] . W^T.
// The tile, the W stream and the MFMA schedule are mma_nt160_kernel's (64
// source rows, 160 columns, 16 x 16 x 32 tiles, two K groups, four LDS
// stages); the A slab of a step is not loaded from X but built. Thread t
// owns row t / 8, 16-byte piece t % 8 of each 128-byte step. Its pieces of
// the P partials go straight into LDS (global_load_lds), kSgLead(P) steps
// ahead, each lane's 16 bytes landing where that lane reads them back, so
// only the wave's own load count guards them. The thread then sums them in
// binary32 (partial order) and rounds once (the row mover's arithmetic, so X
// is the same bytes), writes the piece into the A slab and stores it to X.
// X is written once and never read back, and the W stream and matrix work
// hide under the partials' HBM stream.
//
// Wait accounting: every wait counts only this wave's loads issued after the
// awaited one. Vector-memory operations complete in issue order on gfx9
// (loads and stores alike), so the X stores, which the count leaves out,
// can only make a wait stricter.
// ---------------------------------------------------------------------------
// Steps of partials in flight: what the LDS holds beside the four stages
// (160 columns: 112 KB of stages, 48 KB of slots at P = 2; 64 columns: 64 KB
// of stages, the rest for slots, at most six steps).
template <int PT, int BN>
constexpr int sg_lead() {
  if constexpr (BN == 160) return PT <= 2 ? 3 : 1;
  else return (96 / (8 * PT)) < 6 ? (96 / (8 * PT)) : 6;
}

// One 16-byte piece per lane into LDS, as lds_load16, with the nontemporal
// (streaming) policy: the partials are read once.
__device__ __forceinline__ void lds_load16_nt(const void* g, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   2);
#endif
}

// BN = 160 (129..160 columns, DeepSeek-V2's router) or 64 (at most 64: the
// FoE router), the same pipeline: with 64 columns a step's W stage is 8 KB
// instead of 20, each wave multiplies 2 tiles of 16 columns instead of 5, and
// the LDS this frees holds more steps of partials in flight.
template <int PT, int BN = 160>
__global__ __launch_bounds__(kM160Threads, 1) void srs_gate160_kernel(
    const uint16_t* __restrict__ partials, int64_t n, int d, const int* __restrict__ row_of_src,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ W, int E, float* __restrict__ logits,
    SrsIdentity ident, GateTopk tk) {
  static_assert(BN == 160 || BN == 64, "the two tile widths");
  constexpr int BM = 64;
  constexpr int MT = 2, NT = BN / 32;       // 16 x 16 tiles per wave
  constexpr int WC = BN / 2;                // each wave's columns
  constexpr int STAGE = (BM + BN) * 128;    // 28 KB (16 KB at 64 columns)
  constexpr int NJW = BN / 8;               // 1 KB W loads per step (20, or 8)
  constexpr int NW = kM160Threads / kWave;  // 8
  constexpr int NIW = (NJW + NW - 1) / NW;  // 3 (waves 0-3) and 2 (waves 4-7), or 1
  constexpr int NIHI = NIW, NILO = BN == 160 ? 2 : 1;
  constexpr int LA = sg_lead<PT, BN>();
  constexpr int PSLOT = BM * 128;           // one partial's pieces of one step (8 KB)
  static_assert(BN == 64 || NJW == 3 * 4 + 2 * 4, "W loads split 3 / 2 over the waves");
  static_assert(BN == 160 || NJW == NW, "one W load per wave");
  static_assert(kMmaStages == 4, "the main loop stages two steps per pass");
  // loads a wave issues after the awaited ones (see above): its W loads (NIHI
  // for waves 0-3, NILO for 4-7) and PT partial loads per step
  constexpr int kWaitA3 = (LA - 1) * (NIHI + PT) + NIHI;
  constexpr int kWaitA2 = (LA - 1) * (NILO + PT) + NILO;
  constexpr int kWaitW3 = PT + 2 * (NIHI + PT), kWaitW2 = PT + 2 * (NILO + PT);
  static_assert(kWaitA3 < 64 && kWaitW3 < 64, "vmcnt range");
  // the four stages, then the partial slots
  __shared__ __attribute__((aligned(1024))) char lds[kMmaStages * STAGE + LA * PT * PSLOT];
  char* const pst = lds + kMmaStages * STAGE;
  const int w = wave_id(), lane = lane_id();
  const int g = w >> 2, w4 = w & 3;
  const int wr = w4 & 1, wc = w4 >> 1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int nsteps = d / 64;  // even, >= 2
  const int ni = w < 4 ? NIHI : NILO;

  // W: load j = w + 8 i fills slab rows BM + 8 j .. BM + 8 j + 7; lane l
  // fetches the piece that the swizzle stores at physical piece l % 8.
  // Columns past E re-read the last valid one (their results are not stored).
  const char* wsrc[NIW];
  int wdst[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int j = w + NW * i < NJW ? w + NW * i : w;  // waves 4-7 have no third load
    const int r = BM + 8 * j + lane / 8;
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    const int gc = r - BM < E ? r - BM : E - 1;
    wsrc[i] = reinterpret_cast<const char*>(W + static_cast<int64_t>(gc) * d) + 16 * p;
    wdst[i] = (BM + 8 * j) * 128;
  }
  auto load_w = [&](int t) {
    const int ks = t < nsteps ? t : nsteps - 1;
#pragma unroll
    for (int i = 0; i < NIW; ++i)
      if (i < ni) lds_load16(wsrc[i] + ks * 128, lds + (t % kMmaStages) * STAGE + wdst[i]);
  };

  // A: this thread's row and piece. Rows past n re-read row n - 1 and store
  // nothing.
  const int ar = threadIdx.x >> 3, apc = threadIdx.x & 7;
  const int64_t ai = row0 + ar;
  const bool alive = ai < n;
  const int adst = alive ? (row_of_src ? row_of_src[ai] : static_cast<int>(ai)) : -1;
  const bool astore = alive && adst >= 0 && adst < n && out != nullptr;  // out null: no X
  if (alive && apc == 0) write_identity_row(ident, ai, n);
  const size_t plane = static_cast<size_t>(n) * d;
  const uint16_t* asrc = partials + static_cast<size_t>(alive ? ai : n - 1) * d + 8 * apc;
  uint16_t* aout = astore ? out + static_cast<size_t>(adst) * d + 8 * apc : nullptr;
  const int alds = slab_off(ar, apc);
  char* pwave = pst + w * 1024;  // this wave's 1 KB of each partial slot
  auto load_a = [&](int t) {
    const int ks = t < nsteps ? t : nsteps - 1;
    char* slot = pwave + (t % LA) * PT * PSLOT;
#pragma unroll
    for (int p = 0; p < PT; ++p) lds_load16_nt(asrc + p * plane + 64 * ks, slot + p * PSLOT);
  };
  // step t's slab piece: sum, round, into the A slab and X
  auto build_a = [&](int t) {
    const char* slot = pst + (t % LA) * PT * PSLOT + 16 * threadIdx.x;
    float acc8[8];
    unpack8(*reinterpret_cast<const u32x4*>(slot), acc8);
#pragma unroll
    for (int p = 1; p < PT; ++p) {
      float f[8];
      unpack8(*reinterpret_cast<const u32x4*>(slot + p * PSLOT), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc8[e] += f[e];
    }
    const u32x4 x = pack8_cvt(acc8);
    *reinterpret_cast<u32x4*>(lds + (t % kMmaStages) * STAGE + alds) = x;
    if (astore) st16(aout + 64 * t, x);
  };
  // after the wave's count shows step t's partials landed: build step t's
  // piece, then load step t + LA's into the slot just read
  auto stage_a = [&](int t) {
    if (w < 4)
      wait_vmcnt<kWaitA3>();
    else
      wait_vmcnt<kWaitA2>();
    if (t < nsteps) build_a(t);
    load_a(t + LA);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's fragments of one step: K chunk g (32 k) is pieces 4g .. 4g + 3
  u32x4 fa[2][MT], fb[2][NT];
  auto read_frags = [&](int set, int st) {
    const char* base = lds + (st % kMmaStages) * STAGE;
    const int pc = 4 * g + (lane >> 4);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      fa[set][m] = *reinterpret_cast<const u32x4*>(
          base + slab_off(wr * 32 + 16 * m + (lane & 15), pc));
#pragma unroll
    for (int t = 0; t < NT; ++t)
      fb[set][t] = *reinterpret_cast<const u32x4*>(
          base + BM * 128 + slab_off(wc * WC + 16 * t + (lane & 15), pc));
  };
  // the MFMAs of one step with the staging of step tl (tl < 0: none): W's
  // loads after MFMAs 2, 4 and 6, the A piece after MFMA 8 (64 columns: the
  // W load after MFMA 1, the A piece after MFMA 3)
  constexpr int QW = BN == 160 ? 2 : 1, QA = BN == 160 ? 8 : 3;
  auto mfma_step = [&](int set, int tl) {
    int q = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[m][t] = mfma16x16x32(fa[set][m], fb[set][t], acc[m][t]);
        ++q;
        if (q % QW == 0 && q / QW <= NIW) {
          __builtin_amdgcn_sched_barrier(0);
          const int i = q / QW - 1;
          if (tl >= 0 && i < ni) {
            const int ks = tl < nsteps ? tl : nsteps - 1;
            lds_load16(wsrc[i] + ks * 128, lds + (tl % kMmaStages) * STAGE + wdst[i]);
          }
          __builtin_amdgcn_sched_barrier(0);
        } else if (q == QA) {
          __builtin_amdgcn_sched_barrier(0);
          if (tl >= 0) stage_a(tl);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };
  auto sync_step = [&]() {
    wait_lgkm0();
    if (w < 4)
      wait_vmcnt<kWaitW3>();
    else
      wait_vmcnt<kWaitW2>();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

  // prologue: partials of the first LA steps, then steps 0 .. 2 staged (the
  // first wait drains everything: the counts above hold from step 1 on)
#pragma unroll
  for (int t = 0; t < LA; ++t) load_a(t);
  load_w(0);
  wait_vmcnt<0>();
  build_a(0);
  load_a(LA);
  load_w(1);
  stage_a(1);
  load_w(2);
  stage_a(2);
  sync_step();
  load_w(3);
  stage_a(3);
  read_frags(0, 0);
  for (int st = 0; st < nsteps - 2; st += 2) {
    sync_step();
    read_frags(1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0, st + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
    sync_step();
    read_frags(0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(1, st + 1 + kMmaStages);
    __builtin_amdgcn_sched_barrier(0);
  }
  sync_step();
  read_frags(1, nsteps - 1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(0, -1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(1, -1);

  // group 1's partial tiles meet group 0's in LDS
  wait_vmcnt<0>();
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  if (g == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) red[((w4 * MT + m) * NT + t) * kWave + lane] = acc[m][t];
  }
  __syncthreads();
  // with the top-K, the finished tile also goes to LDS, after the partial
  // tiles: [BM][BN] binary32, the columns past E as -inf
  float* tile = reinterpret_cast<float*>(lds + MT * NT * 4 * kWave * sizeof(f32x4));
  if (g == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wr * 32 + 16 * m + 4 * (lane >> 4) + j;
        const int64_t row = row0 + r;
        int dst = -1;
        if (row < n) dst = row_of_src ? row_of_src[row] : static_cast<int>(row);
        const bool ok = dst >= 0 && dst < n;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = wc * WC + 16 * t + (lane & 15);
          const float v = acc[m][t][j] + red[((w4 * MT + m) * NT + t) * kWave + lane][j];
          if (logits && ok && col < E) logits[static_cast<int64_t>(dst) * E + col] = v;
          if (tk.idx) tile[r * BN + col] = col < E ? v : -__builtin_inff();
        }
      }
  }
  if (!tk.idx) return;
  __syncthreads();
  // Top-K of each row from the tile: one row per 16-lane segment (ten values
  // a lane), the eight waves taking 32 rows at a time.
  unsigned hits = 0;
  const int s16 = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = half * 32 + w * 4 + (lane >> 4);
    const int64_t row = row0 + r;
    float val[BN / 16];
    uint32_t key[BN / 16];
#pragma unroll
    for (int v = 0; v < BN / 16; ++v) {
      val[v] = tile[r * BN + s16 + 16 * v];
      key[v] = s16 + 16 * v < E ? order_key(val[v]) : 0u;
    }
    int dst = -1;
    if (row < n) dst = row_of_src ? row_of_src[row] : static_cast<int>(row);
    const bool keep = dst >= 0 && dst < n;
    if (tk.H <= 1) {
      int col;
      float wgt;
      seg_topk<16, BN / 16>(val, key, tk.K, tk.renorm, &col, &wgt);
      const bool pick = keep && s16 < tk.K;
      if (pick) {
        tk.idx[static_cast<int64_t>(dst) * tk.K + s16] = col;
        if (tk.weights) tk.weights[static_cast<int64_t>(dst) * tk.K + s16] = wgt;
      }
      if (tk.expert_cluster) {
        // (a NaN logit with every bit set has key 0 like the columns past E
        // and may tie with them: outside the contract, but no read past E)
        int cl = 0;
        if (row < n)
          cl = tk.lar_cluster ? static_cast<int>(tk.lar_cluster[row])
                              : (tk.dest ? static_cast<int>(tk.dest[row]) : 0);
        const int ec = pick && col < E ? static_cast<int>(tk.expert_cluster[col]) : -1;
        hits += __popcll(__ballot(ec == cl));
      }
    } else {
      // Grouped: group h's columns [h eg, (h + 1) eg) keep their keys, the
      // others are cleared, and the segment picks the group's kg; lane s < kg
      // holds group pick s, slot h kg + s. renorm = 1: the softmax over the
      // group's picks (seg_topk's); renorm = 0: over every column, from the
      // row's largest logit.
      const int H = tk.H, kg = tk.K / H, eg = E / H;
      float mall = 0.f, zall = 0.f;
      if (!tk.renorm) {
        uint32_t kmx = 0u;
#pragma unroll
        for (int v = 0; v < BN / 16; ++v) kmx = key[v] > kmx ? key[v] : kmx;
        mall = key_float(seg_max<16>(kmx));
        float zl = 0.f;
#pragma unroll
        for (int v = 0; v < BN / 16; ++v) zl += key[v] ? __expf(val[v] - mall) : 0.f;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) zl += __shfl_xor(zl, o, kWave);
        zall = zl;
      }
#pragma unroll 1
      for (int h = 0; h < H; ++h) {
        uint32_t kh[BN / 16];
#pragma unroll
        for (int v = 0; v < BN / 16; ++v) {
          const int c = s16 + 16 * v;
          kh[v] = c >= h * eg && c < (h + 1) * eg ? key[v] : 0u;
        }
        int col;
        float wgt;
        seg_topk<16, BN / 16>(val, kh, kg, 1, &col, &wgt);
        if (!tk.renorm) wgt = __fdividef(__expf(tile[r * BN + (col < BN ? col : 0)] - mall), zall);
        const bool pick = keep && s16 < kg;
        if (pick) {
          tk.idx[static_cast<int64_t>(dst) * tk.K + h * kg + s16] = col;
          if (tk.weights) tk.weights[static_cast<int64_t>(dst) * tk.K + h * kg + s16] = wgt;
        }
        if (tk.expert_cluster) {
          int cl = 0;
          if (row < n)
            cl = tk.lar_cluster ? static_cast<int>(tk.lar_cluster[row * H + h])
                                : (tk.dest ? static_cast<int>(tk.dest[row]) : 0);
          const int ec = pick && col < E ? static_cast<int>(tk.expert_cluster[col]) : -1;
          hits += __popcll(__ballot(ec == cl));
        }
      }
    }
  }
  if (tk.expert_cluster) {
    // the workgroup's count, one atomic: the partial tiles' LDS takes it
    __syncthreads();
    unsigned* cnt = reinterpret_cast<unsigned*>(lds);
    if (lane == 0) cnt[w] = hits;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long tot = 0;
#pragma unroll
      for (int v = 0; v < NW; ++v) tot += cnt[v];
      if (tot) atomicAdd(tk.local, tot);
    }
  }
}
}  // namespace

bool mma_fits(int64_t M, int Kd, int N) {
  return M > 0 && N > 32 && Kd >= 128 && Kd % 128 == 0;
}

int mma_launch(const uint16_t* A, int64_t M, int Kd, const uint16_t* B, int N, const float* bias,
               void* C, int epi, hipStream_t s) {
  if (!mma_fits(M, Kd, N)) return ROUTE_ERR_UNSUPPORTED;
  if (N > 128 && N <= 160) {
    mma_nt160_kernel<<<ceil_div(M, 64), kM160Threads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
    return launch_status();
  }
  const int64_t big = static_cast<int64_t>(ceil_div(M, 128)) * ceil_div(N, 128);
  if (N >= 128 && big >= 256) {
    dim3 grid(ceil_div(M, 128), ceil_div(N, 128));
    mma_nt_kernel<128, 128><<<grid, kMmaThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
  } else {
    dim3 grid(ceil_div(M, 64), ceil_div(N, 64));
    mma_nt_kernel<64, 64><<<grid, kMmaThreads, 0, s>>>(A, M, Kd, B, N, bias, C, epi);
  }
  return launch_status();
}

bool srs_gate_fits(int P, int d, int E) {
  return (P == 1 || P == 2 || P == 4) && d >= 128 && d % 128 == 0 && E >= 1 && E <= 160;
}

int srs_gate_launch(const uint16_t* partials, int P, int64_t n, int d, const int* row_of_src,
                    uint16_t* out, const uint16_t* w, int E, float* logits,
                    const SrsIdentity& ident, const GateTopk* topk, hipStream_t s) {
  if (!srs_gate_fits(P, d, E)) return ROUTE_ERR_UNSUPPORTED;
  const GateTopk tk =
      topk ? *topk : GateTopk{0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr};
  const unsigned grid = ceil_div(n, 64);
#define ROUTE_SG(PT, BN)                                                                      \
  srs_gate160_kernel<PT, BN><<<grid, kM160Threads, 0, s>>>(partials, n, d, row_of_src, out, w, \
                                                           E, logits, ident, tk)
  // at most 64 columns: the narrow tile (its LDS holds more partials in flight)
  if (E <= 64) {
    if (P == 1) ROUTE_SG(1, 64); else if (P == 2) ROUTE_SG(2, 64); else ROUTE_SG(4, 64);
  } else {
    if (P == 1) ROUTE_SG(1, 160); else if (P == 2) ROUTE_SG(2, 160); else ROUTE_SG(4, 160);
  }
#undef ROUTE_SG
  return launch_status();
}

}  // namespace route
