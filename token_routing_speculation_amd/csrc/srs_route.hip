// srs_shuffle_route: the shuffled reduce of "Speculative MoE" (section 3.1,
// s-TS) carried on through the router while each reduced row is still on
// chip: router logits ("Federation of Experts
// (FoE)" article, router scores g[i]), top-K with its softmax weights, and
// the local activation count ("Speculative MoE" glossary) against the row's
// predicted cluster. For a small expert set (this file's kernel) the router
// is a handful of dot products per row; run as separate launches it costs a
// re-read of the rows and three launches that each do almost nothing, so it
// rides along with the move. For 65..160 experts the matrix-core shuffle +
// router kernel (mma.hip) takes the top-K and the count in its epilogue.
//
// Layout of the work. The router rows w [E][d] are staged once per workgroup
// into LDS, each padded with zeros to a whole number of 64-lane vector sets
// (at most 64 KiB in all). Each wave owns one source row at a time:
// lane l holds the 16-byte vectors l, l + 64, ... of every partial, sums them
// in binary32 (partial order 0..P-1), rounds to bf16 and stores the row at its
// sorted position (the same bytes as srs_shuffle). The bf16 row is multiplied
// by each staged router row with v_dot2_f32_bf16 (binary32 accumulation of
// exact bf16 products) and summed over the wave; lane e keeps expert e's
// logit, so the top-K ranks one expert per lane on wave-uniform values.
//
// Two further modes of the same kernel, for at most 4096 tokens (one row per
// wave, sixteen consecutive tokens per workgroup):
//  - PRED (srs_predict_route): the route prediction ("Speculative MoE"
//    section 4.1) and the shuffle's order are made inside the kernel. Each
//    workgroup predicts and counts every token itself, from the token table
//    staged in its LDS where it fits, and places its own rows without a
//    separate sort.
//  - DISP (srs_predict_route_dispatch): each reduced row also goes straight
//    into its K expert slots (the dispatch, section 1), after a bounded grid
//    barrier at which every workgroup has published its pairs per (expert,
//    cluster).
#include "common.hpp"
#include "csort.hpp"
#include "mfma.hpp"
#include "predict.hpp"
#include "srs.hpp"
#include "topk.hpp"

#include <mutex>
#include <vector>

namespace route {
namespace {

// Sixteen waves per workgroup and at most one workgroup per CU: the router
// rows are staged once per CU, and every wave loops over rows.
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteWBytes = 64 * 1024;  // largest E * d * 2 staged in LDS
constexpr int kRouteMaxE = kWave;  // one lane per expert
constexpr int kRouteMaxGrid = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// (the pairs go through memcpy: a bit cast taken straight from a vector
// element has been seen to read element 0)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  bf16x2_t av, bv;
  __builtin_memcpy(&av, &a, 4);
  __builtin_memcpy(&bv, &b, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(av, bv, c, false);
}

// c + the dot product of eight bf16 pairs (binary32 accumulation)
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float c) {
  const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  const uint32_t b0 = b[0], b1 = b[1], b2 = b[2], b3 = b[3];
  c = dot2(a0, b0, c);
  c = dot2(a1, b1, c);
  c = dot2(a2, b2, c);
  return dot2(a3, b3, c);
}

// Sum over the wave, returned to every lane: DPP sums inside each row of
// 16 lanes, then the four row sums read through scalar registers.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += __uint_as_float(dpp<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppMirror>(__float_as_uint(v)));
  const uint32_t u = __float_as_uint(v);
  return (__uint_as_float(__builtin_amdgcn_readlane(u, 0)) +
          __uint_as_float(__builtin_amdgcn_readlane(u, 16))) +
         (__uint_as_float(__builtin_amdgcn_readlane(u, 32)) +
          __uint_as_float(__builtin_amdgcn_readlane(u, 48)));
}

struct RouteOut {
  float* logits;                  // [n][E], nullable
  int* idx;                       // [n][K]
  float* weights;                 // [n][K], nullable
  const uint8_t* expert_cluster;  // [E], nullable (then no count)
  unsigned long long* local;
};

// srs_predict_route: the route prediction ("Speculative MoE" notes, section
// 4.1) and the stable shuffle's order made inside the route kernel. Every
// workgroup predicts the cluster of every token outside its own sixteen and
// counts them by cluster (those before its rows, and all), predicts its own
// rows' clusters and ranks them, and so knows each of its rows' sorted
// position without a separate sort: the sort's results are written as
// route_predict_sort writes them. At most kPredRouteMax tokens (one row per
// wave, a wave's share of the others one batch of lane counters) and
// kPredRouteMaxG clusters (two registers of packed counters).
constexpr int64_t kPredRouteMax = kRouteMaxGrid * kRouteWaves;
constexpr int kPredRouteMaxG = 16;
constexpr int kPredOthers = 4;  // other tokens per lane: (4096 - 16) / 16 waves / 64 lanes
static_assert((kPredRouteMax - kRouteWaves + kRouteWaves - 1) / kRouteWaves <= kPredOthers * kWave,
              "one batch of others per wave");

// The dispatch made in the route kernel (srs_predict_route_dispatch): the
// rows go from registers to their expert slots after a grid barrier at which
// every workgroup has published its pairs per (cluster, expert).
struct DispOut {
  unsigned* arrive;     // the barrier's arrival count (a multiple of 256 between calls),
                        // then at +256 bytes [grid][G * E] each workgroup's pairs per
                        // (cluster, expert)
  int* expert_offsets;  // [E + 1]
  int* slot_of_pair;    // [n * K]
  int* pair_of_slot;    // [n * K]
  uint16_t* disp;       // [n * K][d]
};

struct PredSort {
  PredictArgs a;          // the prediction's inputs and the error word
  uint8_t* dest;          // [n] predicted clusters (out)
  int* offsets;           // [G + 1]
  int* row_of_src;        // [n]
  int* src_of_row;        // [n]
  uint8_t* row_cluster;   // [n]
  DispOut dp;             // with the dispatch (arrive non-null)
  int tables;             // the token table (and confidence bytes) staged in LDS
};

// Tables staged in LDS by the prediction prologue: each at most this many
// bytes (from its 16-byte aligned start), three 16-byte chunks per thread.
constexpr int kTabChunks = 3;
constexpr int kTabMaxBytes = kTabChunks * 1024 * 16;
// dynamic LDS the router rows and the staged tables may take together
constexpr int64_t kRouteTabLds = 144 * 1024;

// bytes a table of `len` bytes at `p` takes when staged (whole 16-byte chunks)
inline int tab_bytes(const void* p, int len) {
  return static_cast<int>(((reinterpret_cast<uintptr_t>(p) & 15) + len + 15) & ~uintptr_t(15));
}

// Bounded wait at the grid barrier: this many polls (each after a sleep of
// 2 x 64 cycles; a poll is a coherent load, about a microsecond), after which
// the workgroup flags ROUTE_EBIT_SYNC and skips the dispatch instead of
// waiting on. The workspace's second word, when not zero, replaces it (a
// caller's way to force the time-out).
constexpr unsigned kBarrierSpins = 1u << 19;
// the dispatch's LDS: per (cluster, expert) entry, the pairs before this
// workgroup, in all, and the entry's first slot, for up to kDispMaxGE entries
constexpr int kDispMaxGE = 256;
constexpr size_t kDispLds = 3 * kDispMaxGE * sizeof(int);

// A key source that never runs (the others' one batch is filled by hand).
struct NoKeys {
  template <int NB>
  __device__ __forceinline__ void batch(const int64_t (&)[NB], const bool (&)[NB],
                                        uint32_t (&k)[NB]) const {
#pragma unroll
    for (int q = 0; q < NB; ++q) k[q] = 0xffffffffu;
  }
};

template <int PT, int CPL, int EB, bool PRED, bool DISP = false>
__global__ __launch_bounds__(kRouteThreads) void srs_route_kernel(
    const uint16_t* __restrict__ partials, int64_t n, int d, const int* __restrict__ row_of_src,
    const uint8_t* __restrict__ dest, uint16_t* __restrict__ out, const uint16_t* __restrict__ w,
    int E, int K, int renorm, RouteOut ro, SrsIdentity ident, PredSort ps) {
  static_assert(EB * CPL <= 64, "staged router rows fit in 64 KiB");
  static_assert(PRED || !DISP, "the dispatch needs the workgroup-local order");
  static_assert(kRouteWaves == 16, "the dispatch's table sums take 16 workgroups per wave");
  extern __shared__ __align__(16) char wl[];
  __shared__ int ckey[kRouteWaves];  // with the prediction: the rows' clusters
  // with the dispatch: this workgroup's pairs per (cluster, expert), counted
  // as the rows are routed (cleared here, ahead of the prologue's barriers)
  __shared__ int lcnt[DISP ? kDispMaxGE : 1];
  if constexpr (DISP) {
    for (int t = threadIdx.x; t < ps.a.G * E; t += kRouteThreads) lcnt[t] = 0;
  }
  const int wv = wave_id();
  const int lane = lane_id();
  const int nv = d >> 3;  // 16-byte vectors per row
  const size_t plane = static_cast<size_t>(n) * d;

  // The router rows into LDS as EB rows of CPL * 64 vectors, zeros past the
  // row end and in the rows past E, so every lane's vectors meet a router
  // value without a guard: piece q (16 bytes) at byte 16 q. The pieces are
  // loaded into registers here and written to LDS once the first row's loads
  // are out too; only these older loads are waited for before the barrier.
  // (With the prediction's staged tables they go to LDS with the tables,
  // before the rows are issued.)
  constexpr int kRowV = CPL * kWave;  // vectors per staged router row
  constexpr int kPieces = EB * kRowV;
  constexpr int kStage = (kPieces + kRouteThreads - 1) / kRouteThreads;

  // With the prediction: the first loads of every token this wave predicts
  // (its own row's, and its share of the tokens outside the workgroup's
  // sixteen), then the router staging, then the tables' entries (or the
  // whole tables, staged); the rows go out after those, so waiting for the
  // predictions never waits for them.
  const int64_t clo = static_cast<int64_t>(blockIdx.x) * kRouteWaves;
  const int64_t chi = clo + kRouteWaves < n ? clo + kRouteWaves : n;
  const int64_t i_own = clo + wv;
  int64_t olo = 0, ohi = 0;
  PredictLoads so[kPredOthers], sm{};
  bool oin[kPredOthers];
  PredictArgs quiet = ps.a;
  quiet.err = nullptr;
  if constexpr (PRED) {
    others_share<kRouteWaves>(n, clo, chi, wv, &olo, &ohi);
#pragma unroll
    for (int q = 0; q < kPredOthers; ++q) {
      const int64_t jp = olo + q * kWave + lane;
      oin[q] = jp < ohi;
      so[q] = predict_stage1(quiet, oin[q] ? (jp < clo ? jp : jp + (chi - clo)) : 0);
    }
    sm = predict_stage1(ps.a, i_own < n ? i_own : 0);
  }
  // The token table (and with the fallback the confidence bytes) staged in
  // LDS after the router rows: each workgroup predicts every token, and as
  // random byte gathers from global memory every lookup is its own cache
  // line miss, which the CU serves a few hundred at a time. Staged, the
  // table is read as whole 16-byte chunks from its aligned start (entry t
  // at byte (table % 16) + t; a chunk never crosses a page).
  uint8_t* const ltab = reinterpret_cast<uint8_t*>(wl) + kPieces * 16;
  __shared__ uint8_t lng[PRED ? kPredRouteMaxG * kPredRouteMaxG : 1];  // the 2-gram table
  int lpre = 0, cpre = 0, lch = 0, cch = 0;
  u32x4 tl[kTabChunks], tcf[kTabChunks];
  int ngv = 0;
  if constexpr (PRED) {
    if (ps.tables) {
      const int gg = ps.a.G * ps.a.G;
      if (ps.a.conf && static_cast<int>(threadIdx.x) < gg) ngv = ps.a.ngram[threadIdx.x];
      const uintptr_t la = reinterpret_cast<uintptr_t>(ps.a.lut);
      lpre = static_cast<int>(la & 15);
      lch = (lpre + ps.a.vocab + 15) >> 4;
      const u32x4* lsrc = reinterpret_cast<const u32x4*>(la - lpre);
#pragma unroll
      for (int r = 0; r < kTabChunks; ++r) {
        const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
        tl[r] = lsrc[q < lch ? q : lch - 1];
      }
      if (ps.a.conf) {
        const uintptr_t ca = reinterpret_cast<uintptr_t>(ps.a.conf);
        cpre = static_cast<int>(ca & 15);
        cch = (cpre + ps.a.vocab + 15) >> 4;
        const u32x4* csrc = reinterpret_cast<const u32x4*>(ca - cpre);
#pragma unroll
        for (int r = 0; r < kTabChunks; ++r) {
          const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
          tcf[r] = csrc[q < cch ? q : cch - 1];
        }
      }
    }
  }
  u32x4 wst[kStage];
#pragma unroll
  for (int r = 0; r < kStage; ++r) {
    const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
    const int e = q / kRowV, v = q - e * kRowV;
    wst[r] = u32x4{0, 0, 0, 0};
    if (q < kPieces && e < E && v < nv) wst[r] = ld16(w + 8 * (static_cast<size_t>(e) * nv + v));
  }
  // Row loads: streaming (nt) buffer loads through a descriptor spanning the
  // one row, so vectors past the row end read as zeros without a per-vector
  // address. Issued vector by vector (every partial of vector c, then c + 1),
  // so the work on vector c waits only for its own loads.
  // (with the dispatch, x[0][c] keeps the reduced vector c to the end: the
  // row stays in the registers its loads landed in)
  u32x4 x[PT][CPL];
  // (valid false: an empty descriptor, every vector reads as zeros and no
  // memory is touched)
  auto load_row = [&](int64_t r, bool valid) {
    __amdgpu_buffer_rsrc_t rs[PT];
#pragma unroll
    for (int p = 0; p < PT; ++p)
      rs[p] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(partials + (valid ? p * plane + static_cast<size_t>(r) * d : 0)),
          static_cast<short>(0), valid ? d * 2 : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int p = 0; p < PT; ++p)
        x[p][c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[p], lane * 16, c * kWave * 16, 2));
  };
  // The first row's loads go out behind the staging loads, which retire
  // first (loads count down in issue order): the row's first vectors can be
  // reduced and stored while its later ones are in flight. (With the staged
  // tables the rows go out after the whole prediction; see below.)
  // A row's predicted cluster is loaded just before the row itself, so no
  // later load stands between the row and its first use. Both loads are
  // issued by every wave (a wave without a row reads zeros and a valid
  // byte), so the waits for the staging loads count the same on every path.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRouteWaves;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kRouteWaves + wv;
  int cl = 0;
  if constexpr (PRED) {
    if (ps.tables) {
      // Every load so far has landed and the rows are not out yet: the
      // tables and the router rows into LDS, then, past the barrier, the
      // lookups from there with no global load at all, so that no wave's
      // prediction waits in the CU's memory pipeline behind another wave's
      // rows.
      compiler_fence();
      wait_vmcnt<0>();
      compiler_fence();
#pragma unroll
      for (int r = 0; r < kTabChunks; ++r) {
        const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
        if (q < lch) *reinterpret_cast<u32x4*>(ltab + 16 * q) = tl[r];
        if (q < cch) *reinterpret_cast<u32x4*>(ltab + 16 * (lch + q)) = tcf[r];
      }
      if (ps.a.conf && static_cast<int>(threadIdx.x) < ps.a.G * ps.a.G)
        lng[threadIdx.x] = static_cast<uint8_t>(ngv);
#pragma unroll
      for (int r = 0; r < kStage; ++r) {
        const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
        if (q < kPieces) *reinterpret_cast<u32x4*>(wl + 16 * static_cast<size_t>(q)) = wst[r];
      }
      lds_barrier();
      const int G = ps.a.G;
      auto stage2_lds = [&](PredictLoads& s) {
        const bool fb = ps.a.conf != nullptr;
        const int tc = (s.t >= 0 && s.t < ps.a.vocab) ? s.t : 0;
        s.c = ltab[lpre + tc];
        s.cf = fb ? ltab[16 * lch + cpre + tc] : 0;
        s.g = fb ? lng[(s.p2 < G && s.p1 < G) ? s.p2 * G + s.p1 : 0] : 0;
      };
#pragma unroll
      for (int q = 0; q < kPredOthers; ++q) stage2_lds(so[q]);
      stage2_lds(sm);
    } else {
#pragma unroll
      for (int q = 0; q < kPredOthers; ++q) predict_stage2(quiet, so[q]);
      predict_stage2(ps.a, sm);
    }
  } else {
    cl = dest ? static_cast<int>(dest[i < n ? i : n - 1]) : 0;
  }
  // With the staged tables the prediction reads only LDS, so the rows go out
  // after it: a wave's row loads stall at issue until the CU's memory
  // pipeline takes them (waves issue oldest first), and a prediction behind
  // them would wait for other waves' rows.
  bool staged = false;  // the router rows already in LDS (with the staged tables)
  if constexpr (PRED) staged = ps.tables != 0;
  if (!staged) load_row(i, i < n);
  if (!staged) {
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int q = static_cast<int>(threadIdx.x) + r * kRouteThreads;
      if (q < kPieces) *reinterpret_cast<u32x4*>(wl + 16 * static_cast<size_t>(q)) = wst[r];
    }
  }
  int pdst = -1;  // with the prediction: this wave's row's sorted position
  if constexpr (PRED) {
    __shared__ int orow[kRouteWaves * kPredRouteMaxG];  // others before the rows, per wave
    __shared__ int prow[kRouteWaves * kPredRouteMaxG];  // and after them
    __shared__ int stot[kPredRouteMaxG];
    __shared__ int sbase[kPredRouteMaxG];
    __shared__ int stotal;
    const int G = ps.a.G;
    uint32_t ok[kPredOthers];
#pragma unroll
    for (int q = 0; q < kPredOthers; ++q) {
      uint32_t e = 0;
      const int c = predict_stage3(quiet, so[q], &e);
      ok[q] = oin[q] ? static_cast<uint32_t>(c) : 0xffffffffu;
    }
    const NoKeys none;
    if (G <= 8)
      others_count<1>(none, olo, ohi, clo, chi, G, ok, orow + wv * G, prow + wv * G);
    else
      others_count<2>(none, olo, ohi, clo, chi, G, ok, orow + wv * G, prow + wv * G);
    uint32_t e_own = 0;
    const int c_own = __builtin_amdgcn_readfirstlane(predict_stage3(ps.a, sm, &e_own));
    if (lane == 0) ckey[wv] = i_own < n ? c_own : -1;
    lds_barrier();
    for (int b = threadIdx.x; b < G; b += kRouteThreads) {
      int pre = 0, rest = 0;
#pragma unroll
      for (int v = 0; v < kRouteWaves; ++v) {
        pre += orow[v * G + b];
        rest += prow[v * G + b] + (ckey[v] == b ? 1 : 0);
      }
      sbase[b] = pre;
      stot[b] = pre + rest;
    }
    lds_barrier();
    if (wv == 0) scan_bins(stot, G, &stotal);
    lds_barrier();
    if (blockIdx.x == 0) {
      for (int b = threadIdx.x; b < G; b += kRouteThreads) ps.offsets[b] = stot[b];
      if (threadIdx.x == 0) ps.offsets[G] = stotal;
    }
    if (i_own < n) {
      // rank among the workgroup's rows of the same cluster before this one
      int rank = 0;
      for (int v = 0; v < wv; ++v) rank += ckey[v] == c_own ? 1 : 0;
      const bool valid = c_own < G;  // a table entry past G: no position, flagged
      pdst = valid ? stot[c_own] + sbase[c_own] + rank : -1;
      if (lane == 0) {
        const uint32_t e = e_own | (valid ? 0u : static_cast<uint32_t>(ROUTE_EBIT_DEST_RANGE));
        if (e) set_err(ps.a.err, e);
        ps.dest[i_own] = static_cast<uint8_t>(c_own);
        ps.row_of_src[i_own] = pdst;
        if (valid) {
          ps.src_of_row[pdst] = static_cast<int>(i_own);
          if (ps.row_cluster) ps.row_cluster[pdst] = static_cast<uint8_t>(c_own);
        }
      }
    }
    cl = c_own;
  }
  // (staged: the router rows were in LDS before the prediction's barriers,
  // so each wave goes on to its row as soon as its loads are out)
  if (staged) load_row(i, i < n);
  else lds_barrier();

  // lane e < E stands for expert e in the top-K and the count
  const int my_ec = (ro.expert_cluster && lane < E) ? static_cast<int>(ro.expert_cluster[lane]) : -1;
  unsigned lar = 0;
  // with the dispatch: this lane's pick and its rank, and the wave's picks
  // as a mask over the experts
  bool dpick = false;
  int drank = 0, ddst = -1;
  unsigned long long dpm = 0;

  for (; i < n; i += stride) {
    int dst;
    if constexpr (PRED)
      dst = pdst;  // one row per wave
    else
      dst = row_of_src ? row_of_src[i] : static_cast<int>(i);
    const bool keep = dst >= 0 && dst < n;  // key out of range (flagged by the sort): no outputs
    // The row's store through a descriptor spanning the destination row
    // (vectors past its end are dropped; for a row without a destination the
    // descriptor is empty and drops them all).
    const bool xst = keep && out != nullptr;  // out null (dispatch only): X is not written
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        xst ? out + static_cast<size_t>(dst) * d : const_cast<uint16_t*>(partials),
        static_cast<short>(0), xst ? d * 2 : 0, 0x00020000);
    // Vector by vector, as its loads land: reduce, round, store, and add its
    // products with every staged router row (binary32 dot products of exact
    // bf16 pairs) into one accumulator per expert. The work runs in steps of
    // (vector c, four router rows); each step's router reads are issued one
    // step ahead, into a ring of two. An empty asm statement after each step
    // takes the step's accumulators and the lane's LDS offset, and the next
    // reads address through that offset: the reads cannot run ahead of the
    // ring, and the products cannot sink past their step (left free, the
    // compiler hoists every router read and holds them all in registers).
    float acc[EB];
#pragma unroll
    for (int e = 0; e < EB; ++e) acc[e] = 0.f;
    constexpr int kGroups = EB / 4;
    constexpr int kSteps = CPL * kGroups;
    uint32_t off = 16u * lane;
    u32x4 wr[2][4];
    auto read_step = [&](int st, u32x4 (&dst)[4]) {
      const int c = st / kGroups, g = st - c * kGroups;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dst[k] = *reinterpret_cast<const u32x4*>(
            wl + off + 16 * (static_cast<size_t>(g * 4 + k) * kRowV + c * kWave));
    };
    read_step(0, wr[0]);
    u32x4 xb = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int c = st / kGroups, g = st - c * kGroups;
      if (g == 0) {
        // this vector's partials (waited for here, not before)
#pragma unroll
        for (int p = 0; p < PT; ++p) asm volatile("" : "+v"(x[p][c]));
        float f[8];
        unpack8(x[0][c], f);
#pragma unroll
        for (int p = 1; p < PT; ++p) {
          float h[8];
          unpack8(x[p][c], h);
#pragma unroll
          for (int k = 0; k < 8; ++k) f[k] += h[k];
        }
        xb = pack8_cvt(f);
        __builtin_amdgcn_raw_buffer_store_b128(xb, ors, lane * 16, c * kWave * 16, 0);
        if constexpr (DISP) x[0][c] = xb;
      }
      if (st + 1 < kSteps) read_step(st + 1, wr[(st + 1) & 1]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[g * 4 + k] = dot8(xb, wr[st & 1][k], acc[g * 4 + k]);
      asm volatile(""
                   : "+v"(off), "+v"(acc[g * 4]), "+v"(acc[g * 4 + 1]), "+v"(acc[g * 4 + 2]),
                     "+v"(acc[g * 4 + 3]));
    }
    // Expert e's logit, a wave-uniform sum, kept by lane e. The sums are
    // taken for every staged row (those past E hold zeros) and with no branch
    // around them: a guard would let the compiler sink each expert's products
    // to its sum, and every router read would stay live until then.
    float logit = 0.f;
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const float sum = wave_sum_uniform(acc[e]);
      logit = lane == e ? sum : logit;
    }
    // top-K on the order keys (lanes past E: key 0, below every logit)
    const uint32_t mykey = lane < E ? order_key(logit) : 0u;
    int rank = 0;  // experts ahead of this lane's: larger key, or equal key and lower index
    uint32_t kmax = 0;
    for (int e = 0; e < E; ++e) {
      const uint32_t k = __builtin_amdgcn_readlane(mykey, e);
      rank += (k > mykey || (k == mykey && e < lane)) ? 1 : 0;
      kmax = k > kmax ? k : kmax;
    }
    const bool pick = keep && lane < E && rank < K;
    const float ex = (renorm ? pick : lane < E) ? __expf(logit - key_float(kmax)) : 0.f;
    const float z = wave_sum_uniform(ex);
    if (keep) {
      if (ro.logits && lane < E) ro.logits[static_cast<size_t>(dst) * E + lane] = logit;
      const size_t base = static_cast<size_t>(dst) * K;
      if (pick) {
        ro.idx[base + rank] = lane;
        if (ro.weights) ro.weights[base + rank] = __fdividef(ex, z);
      }
      if (ro.expert_cluster) lar += __popcll(__ballot(pick && my_ec == cl));
    }
    if constexpr (DISP) {
      dpick = pick;
      drank = rank;
      ddst = dst;
      dpm = __ballot(pick);
      if (pick) atomicAdd(&lcnt[lane * ps.a.G + cl], 1);  // entry (expert, cluster)
    }
    if constexpr (!PRED) {
      if (lane == 0) write_identity_row(ident, i, n);
    }
    if (!PRED && i + stride < n) {
      cl = dest ? static_cast<int>(dest[i + stride]) : 0;
      load_row(i + stride, true);
    }
  }

  if constexpr (DISP) {
    // The dispatch ("Speculative MoE" section 1; the pair order of
    // moe_permute). Pair (X row r, rank k) with expert e goes to slot: the
    // pairs of experts before e, plus those of expert e in X rows before r.
    // X holds the clusters in order, each cluster's rows in source order, and
    // workgroup b's rows are sources 16 b .. 16 b + 15, so over the entries
    // u = e G + c (expert-major) the slot is: the pairs of all entries before
    // u, those of entry u in workgroups before b, and those of entry u in
    // this workgroup's earlier waves. Each workgroup publishes its pairs per
    // entry, meets every other at a grid barrier, then sums the table itself.
    __shared__ unsigned long long pmask[kRouteWaves];
    __shared__ int sflag;
    const int G = ps.a.G, GE = G * E;
    const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
    if (lane == 0) pmask[wv] = dpm;
    __syncthreads();  // (also: every wave is done with the router rows)
    // The table is entry-major (entry u of workgroup b' at u * 256 + b'),
    // written and read with agent-scope atomic accesses, which are coherent
    // across the XCDs' L2s without a cache write-back or invalidation.
    int* const table = reinterpret_cast<int*>(ps.dp.arrive) + 64;
    // The grid barrier. Wave 0 publishes the workgroup's counts and waits
    // until they have completed; its lane 0 then adds one arrival (workgroup
    // 0 adds 257 - grid, so one call adds 256 in all and the count, a
    // multiple of 256 before the call, moves from base to base + 256) and
    // waits for the last one. The host launches this kernel only where the
    // whole grid is resident at once.
    if (wv == 0) {
      for (int u = lane; u < GE; u += kWave)
        __hip_atomic_store(&table[u * kRouteMaxGrid + b], lcnt[u], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      compiler_fence();
      wait_vmcnt<0>();
      compiler_fence();
      if (lane == 0) {
        const unsigned inc = b == 0 ? 257u - static_cast<unsigned>(nb) : 1u;
        const unsigned old = __hip_atomic_fetch_add(ps.dp.arrive, inc, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        const unsigned base = old & ~255u;
        const unsigned cap_set = __hip_atomic_load(ps.dp.arrive + 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        // the bound word holds the polls allowed plus one (0: the default);
        // the first check is this workgroup's own arrival, so a word of 1
        // lets only the last workgroup to arrive through
        const unsigned cap = cap_set ? cap_set - 1 : kBarrierSpins;
        int ok = 1;
        for (unsigned it = 0;; ++it) {
          const unsigned now =
              it == 0 ? old + inc
                      : __hip_atomic_load(ps.dp.arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (now - base >= 256u) break;
          if (it >= cap) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        sflag = ok;
      }
    }
    __syncthreads();
    if (!sflag) {
      if (threadIdx.x == 0) set_err(ps.a.err, ROUTE_EBIT_SYNC);
    } else {
      int* const spre = reinterpret_cast<int*>(wl);  // [GE] pairs in earlier workgroups
      int* const stot = spre + GE;                   // [GE] pairs in all
      int* const sbase = stot + GE;                  // [GE] first slot of the entry here
      // wave w sums entries w, w + 16, ... (four at a time); lane l reads
      // workgroups l, l + 64, l + 128, l + 192
      for (int u0 = wv; u0 < GE; u0 += 4 * kRouteWaves) {
        int v[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = u0 + q * kRouteWaves;
          const int uc = u < GE ? u : GE - 1;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[q][j] = __hip_atomic_load(&table[uc * kRouteMaxGrid + lane + kWave * j],
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = u0 + q * kRouteWaves;
          int pre = 0, tot = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int bb = lane + kWave * j;
            tot += bb < nb ? v[q][j] : 0;
            pre += bb < b ? v[q][j] : 0;
          }
          tot = wave_sum_dpp(tot);
          pre = wave_sum_dpp(pre);
          if (u < GE && lane == 0) {
            spre[u] = pre;
            stot[u] = tot;
          }
        }
      }
      __syncthreads();
      // wave 0: exclusive scan of the entry totals (lane l holds entries
      // 4 l .. 4 l + 3); expert e's offset is the scan at entry e G
      if (wv == 0) {
        int s[4], run = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int u = 4 * lane + j;
          s[j] = run;
          run += u < GE ? stot[u] : 0;
        }
        int incl = run;  // inclusive scan of the lane sums
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          incl += lane >= o ? y : 0;
        }
        const int before = incl - run;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int u = 4 * lane + j;
          if (u < GE) {
            sbase[u] = before + s[j] + spre[u];
            if (b == 0 && u % G == 0) ps.dp.expert_offsets[u / G] = before + s[j];
          }
        }
        if (b == 0 && lane == kWave - 1) ps.dp.expert_offsets[E] = incl;
      }
      __syncthreads();
      if (ddst >= 0) {
        // this lane's pair: its slot, the maps, then the row into each slot
        // (a slot past the pairs, possible only with a broken table, is
        // flagged and not written)
        const int64_t npairs = n * K;
        int slot = 0;
        bool sok = false;
        if (dpick) {
          int before = 0;
          for (int v2 = 0; v2 < wv; ++v2)
            before += (ckey[v2] == cl && ((pmask[v2] >> lane) & 1ull)) ? 1 : 0;
          slot = sbase[lane * G + cl] + before;
          sok = slot >= 0 && slot < npairs;
          const int pair = ddst * K + drank;
          if (sok) {
            ps.dp.slot_of_pair[pair] = slot;
            ps.dp.pair_of_slot[slot] = pair;
          } else {
            set_err(ps.a.err, ROUTE_EBIT_INDEX_RANGE);
          }
        }
        for (int k = 0; k < K; ++k) {
          const unsigned long long m = __ballot(dpick && sok && drank == k);
          if (!m) continue;
          const int sl = __builtin_amdgcn_readlane(slot, __builtin_ctzll(m));
          const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
              ps.dp.disp + static_cast<size_t>(sl) * d, static_cast<short>(0), d * 2, 0x00020000);
          // streaming stores from four copies per row up (moe_permute's policy)
          if (K >= 4) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              __builtin_amdgcn_raw_buffer_store_b128(x[0][c], drs, lane * 16, c * kWave * 16, 2);
          } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              __builtin_amdgcn_raw_buffer_store_b128(x[0][c], drs, lane * 16, c * kWave * 16, 0);
          }
        }
      }
    }
  }

  if (ro.expert_cluster) {
    // every wave is done with the router rows: their LDS takes the counts
    __syncthreads();
    unsigned* cnt = reinterpret_cast<unsigned*>(wl);
    if (lane == 0) cnt[wv] = lar;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long tot = 0;
#pragma unroll
      for (int v = 0; v < kRouteWaves; ++v) tot += cnt[v];
      if (tot) atomicAdd(ro.local, tot);
    }
  }
}

int route_cpl(int nv) {
  const int need = (nv + kWave - 1) / kWave;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
}

// Whether `grid` workgroups of kRouteThreads with `lds` bytes of dynamic LDS
// are resident on the current device at once (workgroups per CU from the
// occupancy query times the CUs), cached per kernel, LDS size and device.
bool grid_resident(const void* kern, unsigned grid, size_t lds) {
  struct Entry {
    const void* kern;
    size_t lds;
    int dev;
    int64_t fits;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.kern == kern && e.lds == lds && e.dev == dev) return grid <= e.fits;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, kRouteThreads, lds) != hipSuccess)
    return false;
  cache.push_back(Entry{kern, lds, dev, static_cast<int64_t>(cus) * per});
  return grid <= static_cast<int64_t>(cus) * per;
}

// the smallest expert bound (8, 16, 32, 64) holding E
int route_eb(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }

template <int PT, int CPL, int EB>
bool launch_one(unsigned grid, size_t lds, hipStream_t s, const uint16_t* partials, int64_t n,
                int d, const int* fwd, const uint8_t* dest, uint16_t* out, const uint16_t* w,
                int E, int K, int renorm, const RouteOut& ro, const SrsIdentity& ident,
                const PredSort* ps) {
  if constexpr (EB * CPL > 64 || (PT == 4 && CPL == 8)) {
    return false;  // beyond the staged rows' 64 KiB, or the registers
  } else {
    if (ps && ps->dp.arrive) {
      // the grid barrier needs every workgroup resident at once
      auto* kern = &srs_route_kernel<PT, CPL, EB, true, true>;
      const size_t dl = lds > kDispLds ? lds : kDispLds;
      if (!grid_resident(reinterpret_cast<const void*>(kern), grid, dl)) return false;
      kern<<<grid, kRouteThreads, dl, s>>>(partials, n, d, fwd, dest, out, w, E, K, renorm, ro,
                                           ident, *ps);
    } else if (ps) {
      srs_route_kernel<PT, CPL, EB, true><<<grid, kRouteThreads, lds, s>>>(
          partials, n, d, fwd, dest, out, w, E, K, renorm, ro, ident, *ps);
    } else
      srs_route_kernel<PT, CPL, EB, false><<<grid, kRouteThreads, lds, s>>>(
          partials, n, d, fwd, dest, out, w, E, K, renorm, ro, ident, PredSort{});
    return true;
  }
}

template <int PT, int CPL>
bool launch_cpl(int eb, unsigned grid, size_t lds, hipStream_t s, const uint16_t* partials,
                int64_t n, int d, const int* fwd, const uint8_t* dest, uint16_t* out,
                const uint16_t* w, int E, int K, int renorm, const RouteOut& ro,
                const SrsIdentity& ident, const PredSort* ps) {
  switch (eb) {
#define ROUTE_EB(b)                                                                            \
  case b:                                                                                      \
    return launch_one<PT, CPL, b>(grid, lds, s, partials, n, d, fwd, dest, out, w, E, K,       \
                                  renorm, ro, ident, ps);
    ROUTE_EB(8) ROUTE_EB(16) ROUTE_EB(32) ROUTE_EB(64)
#undef ROUTE_EB
    default: return false;
  }
}

template <int PT>
bool launch_route(int cpl, int eb, unsigned grid, size_t lds, hipStream_t s,
                  const uint16_t* partials, int64_t n, int d, const int* fwd, const uint8_t* dest,
                  uint16_t* out, const uint16_t* w, int E, int K, int renorm, const RouteOut& ro,
                  const SrsIdentity& ident, const PredSort* ps) {
  switch (cpl) {
#define ROUTE_CPL(c)                                                                           \
  case c:                                                                                      \
    return launch_cpl<PT, c>(eb, grid, lds, s, partials, n, d, fwd, dest, out, w, E, K, renorm, \
                             ro, ident, ps);
    ROUTE_CPL(1) ROUTE_CPL(2) ROUTE_CPL(4) ROUTE_CPL(8)
#undef ROUTE_CPL
    default: return false;
  }
}

// bytes of the staged router rows: route_eb(E) rows of CPL * 64 vectors of
// 16 bytes (the expert bound times CPL is at most 64 exactly when E * CPL is)
int64_t route_lds(int d, int E) {
  return static_cast<int64_t>(route_eb(E)) * route_cpl(d / 8) * kWave * 16;
}

bool route_fits(int P, int d, int E) {
  if (E < 1 || E > kRouteMaxE) return false;
  const int cpl = route_cpl(d / 8);
  if (cpl == 0 || route_lds(d, E) > kRouteWBytes) return false;
  return P == 1 || P == 2 || (P == 4 && cpl <= 4);
}

size_t route_ws(int64_t n, int G) {
  return csort_ws_bytes(n, G) + align_up(static_cast<size_t>(n) * sizeof(int), 256) +
         align_up(static_cast<size_t>(n) * sizeof(int), 256);
}

}  // namespace
}  // namespace route

using namespace route;

// The row work of both entry points: the lane-per-expert kernel for small
// expert sets, else the matrix-core shuffle + router kernel with the top-K in
// its epilogue. fwd: each source row's sorted row (null: the identity).
static int route_rows(const uint16_t* partials, int P, int64_t n, int d, const int* fwd,
                      const uint8_t* dest, uint16_t* out, const uint16_t* w, int E,
                      float* logits, int K, int renorm, int* idx, float* weights,
                      const uint8_t* expert_cluster, unsigned long long* local,
                      const SrsIdentity& ident, hipStream_t s,
                      const PredSort* ps = nullptr) {
  if (!route_fits(P, d, E)) {
    if (ps) return ROUTE_ERR_UNSUPPORTED;
    const GateTopk tk{K, renorm != 0, idx, weights, dest, expert_cluster, local, 1, nullptr};
    return srs_gate_launch(partials, P, n, d, fwd, out, w, E, logits, ident, &tk, s);
  }
  const RouteOut ro{logits, idx, weights, expert_cluster, local};
  PredSort pst{};
  if (ps) {
    // with the prediction: stage the token table (and the confidence bytes)
    // in LDS where they fit beside the router rows
    pst = *ps;
    const int tb = tab_bytes(ps->a.lut, ps->a.vocab);
    const int cb = ps->a.conf ? tab_bytes(ps->a.conf, ps->a.vocab) : 0;
    pst.tables = tb <= kTabMaxBytes && cb <= kTabMaxBytes &&
                 route_lds(d, E) + tb + cb <= kRouteTabLds;
    ps = &pst;
  }
  const int64_t need = (n + kRouteWaves - 1) / kRouteWaves;
  const unsigned grid = static_cast<unsigned>(need < kRouteMaxGrid ? need : kRouteMaxGrid);
  // the padded router rows (room for the per-wave counts at the end too)
  size_t lds = static_cast<size_t>(route_lds(d, E));
  if (ps && ps->tables)
    lds += tab_bytes(ps->a.lut, ps->a.vocab) +
           (ps->a.conf ? tab_bytes(ps->a.conf, ps->a.vocab) : 0);
  if (lds < kRouteWaves * sizeof(unsigned)) lds = kRouteWaves * sizeof(unsigned);
  const int cpl = route_cpl(d / 8);
  const int eb = route_eb(E);
  bool done = false;
  if (P == 1)
    done = launch_route<1>(cpl, eb, grid, lds, s, partials, n, d, fwd, dest, out, w, E, K,
                           renorm != 0, ro, ident, ps);
  if (P == 2)
    done = launch_route<2>(cpl, eb, grid, lds, s, partials, n, d, fwd, dest, out, w, E, K,
                           renorm != 0, ro, ident, ps);
  if (P == 4)
    done = launch_route<4>(cpl, eb, grid, lds, s, partials, n, d, fwd, dest, out, w, E, K,
                           renorm != 0, ro, ident, ps);
  if (!done) return ROUTE_ERR_UNSUPPORTED;
  return launch_status();
}

// Shape checks shared by both entry points (SHAPE, then UNSUPPORTED).
static int route_shape(int P, int64_t n, int d, int E, int K) {
  if (n < 0 || P < 1 || d < 8 || d % 8 != 0 || E < 1 || K < 1 || K > E ||
      n >= (int64_t(1) << 31))
    return ROUTE_ERR_SHAPE;
  if (K > kMaxK || (!route_fits(P, d, E) && !srs_gate_fits(P, d, E)))
    return ROUTE_ERR_UNSUPPORTED;
  return ROUTE_OK;
}

ROUTE_API int srs_shuffle_route(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                                const uint8_t* dest, int32_t G, uint16_t* out,
                                int32_t* cluster_offsets, int32_t* row_of_src,
                                int32_t* src_of_row, uint8_t* row_cluster, const uint16_t* w,
                                int32_t E, float* logits, int32_t K, int32_t renorm,
                                int32_t* idx, float* weights, const uint8_t* expert_cluster,
                                unsigned long long* local, void* ws, size_t ws_bytes,
                                uint32_t* err, hipStream_t s) {
  if (G < 1) return ROUTE_ERR_SHAPE;
  const int chk = route_shape(P, n, d, E, K);
  if (chk != ROUTE_OK) return chk;
  if (G > kMaxClusters) return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    return launch_status();
  }
  if (!partials || !out || !w || !idx) return ROUTE_ERR_NULL;
  if ((expert_cluster == nullptr) != (local == nullptr)) return ROUTE_ERR_NULL;
  if (!dest && G != 1) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(out) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  const bool sort = dest != nullptr;
  if (sort && (!ws || ws_bytes < route_ws(n, G))) return ROUTE_ERR_WORKSPACE;
  const int* fwd = nullptr;
  if (sort) {
    char* wsp = static_cast<char*>(ws);
    const size_t ct = csort_ws_bytes(n, G);
    const size_t nt = align_up(static_cast<size_t>(n) * sizeof(int), 256);
    int* fwd_buf = row_of_src ? row_of_src : reinterpret_cast<int*>(wsp + ct);
    int* inv_buf = src_of_row ? src_of_row : reinterpret_cast<int*>(wsp + ct + nt);
    const int st = csort_launch<uint8_t>(dest, n, G, cluster_offsets, fwd_buf, inv_buf,
                                         row_cluster, wsp, err, ROUTE_EBIT_DEST_RANGE, s);
    if (st != ROUTE_OK) return st;
    fwd = fwd_buf;
  }
  const SrsIdentity ident = sort ? SrsIdentity{nullptr, nullptr, nullptr, nullptr}
                                 : SrsIdentity{cluster_offsets, row_of_src, src_of_row, row_cluster};
  return route_rows(partials, P, n, d, fwd, dest, out, w, E, logits, K, renorm, idx, weights,
                    expert_cluster, local, ident, s);
}

ROUTE_API int srs_route_sorted(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                               const int32_t* row_of_src, const uint8_t* dest, uint16_t* out,
                               const uint16_t* w, int32_t E, float* logits, int32_t K,
                               int32_t renorm, int32_t* idx, float* weights,
                               const uint8_t* expert_cluster, unsigned long long* local,
                               hipStream_t s) {
  const int chk = route_shape(P, n, d, E, K);
  if (chk != ROUTE_OK) return chk;
  if (n == 0) return ROUTE_OK;
  if (!partials || !out || !w || !idx || !row_of_src) return ROUTE_ERR_NULL;
  if ((expert_cluster == nullptr) != (local == nullptr)) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(out) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  const SrsIdentity none{nullptr, nullptr, nullptr, nullptr};
  return route_rows(partials, P, n, d, row_of_src, dest, out, w, E, logits, K, renorm, idx,
                    weights, expert_cluster, local, none, s);
}

ROUTE_API int srs_predict_route(const int32_t* tok, int64_t n, const uint8_t* lut,
                                const uint8_t* conf, int32_t vocab, const uint8_t* prev2,
                                const uint8_t* prev1, const uint8_t* ngram, int32_t G,
                                int32_t conf_thr, const uint16_t* partials, int32_t P, int32_t d,
                                const uint16_t* w, int32_t E, int32_t K, int32_t renorm,
                                uint8_t* dest, int32_t* cluster_offsets, int32_t* row_of_src,
                                int32_t* src_of_row, uint8_t* row_cluster, uint16_t* out,
                                float* logits, int32_t* idx, float* weights,
                                const uint8_t* expert_cluster, unsigned long long* local,
                                uint32_t* err, hipStream_t s) {
  if (vocab < 1 || G < 1) return ROUTE_ERR_SHAPE;
  const int chk = route_shape(P, n, d, E, K);
  if (chk != ROUTE_OK) return chk;
  if (n > kPredRouteMax || G > kPredRouteMaxG || !route_fits(P, d, E))
    return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    return launch_status();
  }
  if (!tok || !lut || !dest || !row_of_src || !src_of_row) return ROUTE_ERR_NULL;
  if (conf && (!prev2 || !prev1 || !ngram)) return ROUTE_ERR_NULL;
  if (!partials || !out || !w || !idx) return ROUTE_ERR_NULL;
  if ((expert_cluster == nullptr) != (local == nullptr)) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(out) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  const PredSort ps{PredictArgs{tok, lut, conf, vocab, prev2, prev1, ngram, G, conf_thr, err},
                    dest, cluster_offsets, row_of_src, src_of_row, row_cluster};
  const SrsIdentity none{nullptr, nullptr, nullptr, nullptr};
  return route_rows(partials, P, n, d, nullptr, dest, out, w, E, logits, K, renorm, idx, weights,
                    expert_cluster, local, none, s, &ps);
}

// the dispatch's workspace: the barrier count, then the count table
static size_t disp_ws(int G, int E) {
  return 256 + static_cast<size_t>(G) * E * kRouteMaxGrid * sizeof(int);
}

ROUTE_API int srs_predict_route_dispatch(
    const int32_t* tok, int64_t n, const uint8_t* lut, const uint8_t* conf, int32_t vocab,
    const uint8_t* prev2, const uint8_t* prev1, const uint8_t* ngram, int32_t G,
    int32_t conf_thr, const uint16_t* partials, int32_t P, int32_t d, const uint16_t* w,
    int32_t E, int32_t K, int32_t renorm, uint8_t* dest, int32_t* cluster_offsets,
    int32_t* row_of_src, int32_t* src_of_row, uint8_t* row_cluster, uint16_t* out,
    float* logits, int32_t* idx, float* weights, const uint8_t* expert_cluster,
    unsigned long long* local, int32_t* expert_offsets, int32_t* slot_of_pair,
    int32_t* pair_of_slot, uint16_t* disp, void* ws, size_t ws_bytes, uint32_t* err,
    hipStream_t s) {
  if (vocab < 1 || G < 1) return ROUTE_ERR_SHAPE;
  const int chk = route_shape(P, n, d, E, K);
  if (chk != ROUTE_OK) return chk;
  if (n > kPredRouteMax || G > kPredRouteMaxG || !route_fits(P, d, E) || G * E > kDispMaxGE)
    return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets || !expert_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    fill_i32<<<ceil_div(E + 1, 256), 256, 0, s>>>(expert_offsets, E + 1, 0);
    return launch_status();
  }
  if (!tok || !lut || !dest || !row_of_src || !src_of_row) return ROUTE_ERR_NULL;
  if (conf && (!prev2 || !prev1 || !ngram)) return ROUTE_ERR_NULL;
  if (!partials || !w || !idx || !weights || !slot_of_pair || !pair_of_slot || !disp)
    return ROUTE_ERR_NULL;
  if ((expert_cluster == nullptr) != (local == nullptr)) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(w) || !aligned16(disp) || (out && !aligned16(out)))
    return ROUTE_ERR_ALIGN;
  if (!ws || ws_bytes < disp_ws(G, E) || reinterpret_cast<uintptr_t>(ws) % 256)
    return ROUTE_ERR_WORKSPACE;
  char* wsp = static_cast<char*>(ws);
  const DispOut dp{reinterpret_cast<unsigned*>(wsp), expert_offsets, slot_of_pair, pair_of_slot,
                   disp};
  const PredSort ps{PredictArgs{tok, lut, conf, vocab, prev2, prev1, ngram, G, conf_thr, err},
                    dest, cluster_offsets, row_of_src, src_of_row, row_cluster, dp};
  const SrsIdentity none{nullptr, nullptr, nullptr, nullptr};
  return route_rows(partials, P, n, d, nullptr, dest, out, w, E, logits, K, renorm, idx, weights,
                    expert_cluster, local, none, s, &ps);
}

ROUTE_API size_t srs_predict_route_dispatch_workspace_size(int64_t n, int32_t G, int32_t E) {
  if (n < 0 || n > kPredRouteMax || G < 1 || E < 1 || G * E > kDispMaxGE) return 0;
  return disp_ws(G, E);
}

ROUTE_API int srs_route_grouped(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                                uint16_t* out, const uint16_t* w, int32_t E, float* logits,
                                int32_t K, int32_t H, int32_t renorm, int32_t* idx,
                                float* weights, const uint8_t* row_cluster,
                                const uint8_t* expert_cluster, unsigned long long* local,
                                hipStream_t s) {
  if (n < 0 || P < 1 || d < 8 || d % 8 != 0 || E < 1 || K < 1 || H < 1 || E % H != 0 ||
      K % H != 0 || K / H > E / H || n >= (int64_t(1) << 31))
    return ROUTE_ERR_SHAPE;
  if (K > kMaxK || !srs_gate_fits(P, d, E)) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!partials || !w || !idx) return ROUTE_ERR_NULL;
  if ((expert_cluster == nullptr) != (local == nullptr)) return ROUTE_ERR_NULL;
  if (expert_cluster && !row_cluster) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(w) || (out && !aligned16(out))) return ROUTE_ERR_ALIGN;
  const GateTopk tk{K, renorm != 0, idx, weights, nullptr, expert_cluster, local, H, row_cluster};
  const SrsIdentity none{nullptr, nullptr, nullptr, nullptr};
  return srs_gate_launch(partials, P, n, d, nullptr, out, w, E, logits, none, &tk, s);
}
