// moe_permute: expert-contiguous dispatch on one GPU. "Speculative MoE"
// notes, section 1: dispatch sends each token's activation to its K experts;
// on one device that is a stable counting sort of the (token, expert) pairs
// by expert (csort.hpp) followed by a row scatter. With H groups ("Federation
// of Experts (FoE)" article) pair (i, k) reads the group-(k / (K/H)) row of
// token i, so each source row is read once and written K/H times.
#include <mutex>

#include "common.hpp"
#include "csort.hpp"
#include "mfma.hpp"

namespace route {

// Two waves per workgroup. Measured on whole passes (graph replay, same box):
// the FoE-grouped pass 676.7-680.8 us against 687.7-692.8 us with four waves,
// the DeepSeek-V2-shaped pass unchanged; eight waves were no better.
constexpr int kPermThreads = 128;

// One wave per (token i, group h): read src[h][i], write it to the slots of
// the K/H pairs (i, h*kg .. h*kg + kg - 1). The row is loaded whole into
// registers (CPL 16-byte vectors per lane) before any store is issued.
// Cache policy: plain loads. The stores are streaming (nontemporal) when a
// row goes to many slots (STREAM) and plain otherwise; measured on whole
// passes (graph replay, same box), streaming stores won at six copies per
// row (DeepSeek-V2 shape: 573.5 against 587.9 us) and plain ones at two
// (FoE: 664.4-665.7 against 678.1-678.9 us; Mixtral: 94.6-95.2 against
// 99.0-99.5 us, where the combine then also finds disp in cache). Both
// streaming moved 4.9 TB/s against 6.0 TB/s in a probe of the six-copy case.
constexpr int kPermStreamCopies = 4;  // copies per row from which stores stream

template <int CPL, bool STREAM>
__global__ __launch_bounds__(kPermThreads) void permute_move(const uint16_t* __restrict__ src,
                                                             int64_t n, int K, int H, int d,
                                                             const int* __restrict__ slot_of_pair,
                                                             uint16_t* __restrict__ disp) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * (kPermThreads / kWave) + wave_id();
  if (g >= n * H) return;
  const int64_t i = g / H;
  const int h = static_cast<int>(g - i * H);
  const int kg = K / H;
  const int64_t nslots = n * K;
  const int lane = lane_id();
  const int nv = d >> 3;
  const uint16_t* row = src + (static_cast<size_t>(h) * n + i) * d;
  // vectors past the row end load vector 0 again (in bounds) and are never stored
  // the K/H destination slots first (scalar loads, all issued together)
  int slot[kMaxK];
#pragma unroll
  for (int t = 0; t < kMaxK; ++t) {
    slot[t] = -1;
    if (t < kg) {
      const int sl = slot_of_pair[i * K + h * kg + t];
      slot[t] = (sl >= 0 && sl < nslots) ? sl : -1;
    }
  }
  u32x4 x[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    x[c] = ld16(row + 8 * (v < nv ? v : 0));
  }
#pragma unroll
  for (int t = 0; t < kMaxK; ++t) {
    if (t >= kg || slot[t] < 0) continue;
    uint16_t* dst = disp + static_cast<size_t>(slot[t]) * d;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int v = lane + c * kWave;
      if (v < nv) {
        if constexpr (STREAM)
          st16_stream(dst + 8 * v, x[c]);
        else
          st16(dst + 8 * v, x[c]);
      }
    }
  }
}

// The dispatch in one launch, for small batches over few experts: workgroup
// b owns tokens [16 b, 16 b + 16), one wave each, and so the contiguous
// chunk of their pairs. Each wave issues, in this order, the loads of its
// share of the chunk's expert ids, of its share of all the other ids, and of
// its token's row; counts the others by expert (those before the chunk, and
// all of them), ranks the chunk as csort_rank does, keeps the chunk's slots
// in LDS and stores its row to them: the sort's two launches and the move's
// in one. The sort's ids are waited for alone (loads retire in issue order)
// and its barriers wait only for LDS, so the rows stay in flight throughout.
// Workgroup 0 writes the expert offsets. Every workgroup reads all n K
// expert ids (from L2 after the first), which bounds the form to small n K;
// rows of up to eight 16-byte vectors per lane (d <= 4096) keep it within
// the registers of sixteen waves.
constexpr int kFusedThreads = 1024;
constexpr int kFusedTokens = kFusedThreads / kWave;
constexpr int64_t kFusedMaxPairs = 16384;
constexpr int kFusedMaxE = 16;
constexpr int kFusedMaxK = kMaxK;
// Other ids per lane loaded ahead of counting (a wave's share of them is one
// batch up to 8192 pairs, two up to 16384); a lane meets at most
// kFusedMaxPairs / 1024 of them, within its 8-bit counters.
constexpr int kFusedOthers = 8;
static_assert(kFusedMaxPairs / kFusedThreads + 1 <= kCountMaxPerLane, "lane counters");
// the chunk (16 K pairs) is one tile per wave: ceil(16 K / 16) <= 64

template <int CPL, bool STREAM>
__global__ __launch_bounds__(kFusedThreads) void permute_fused(
    const int32_t* __restrict__ idx, int64_t n, int K, int E, int H, int nbits,
    const uint16_t* __restrict__ src, int d, int* __restrict__ offsets,
    int* __restrict__ slot_of_pair, int* __restrict__ pair_of_slot,
    uint16_t* __restrict__ disp, uint32_t* err) {
  constexpr int NW = kFusedTokens;
  __shared__ int stot[kFusedMaxE];
  __shared__ int sbase[kFusedMaxE];
  __shared__ int wrow[NW * kFusedMaxE];  // this chunk's counts per wave, then starts
  __shared__ int orow[NW * kFusedMaxE];  // the other pairs' counts: before the chunk
  __shared__ int prow[NW * kFusedMaxE];  // and after it
  __shared__ int spos[NW * kFusedMaxK];  // the chunk's slots
  __shared__ int stotal;
  const int t = threadIdx.x;
  const int w = wave_id();
  const int lane = lane_id();
  const int64_t b = blockIdx.x;
  const int64_t i = b * NW + w;  // this wave's token
  const int kg = K / H;
  const int nv = d >> 3;
  const int64_t nK = n * K;
  const ArrayKeys<int32_t> keys{idx};

  // this wave's share of the chunk's pairs (ranked as in csort_rank), then
  // its share of the other pairs, then its token's first group row
  const int64_t clo = b * NW * K;
  const int64_t chi = clo + NW * K < nK ? clo + NW * K : nK;
  const int64_t share = ((chi - clo + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int64_t qlo = clo + (w * share < chi - clo ? w * share : chi - clo);
  const int64_t qhi = qlo + share < chi ? qlo + share : chi;
  uint32_t first[1];
  load_batch(keys, first, qlo, qhi);
  int64_t olo, ohi;
  others_share<NW>(nK, clo, chi, w, &olo, &ohi);
  uint32_t ok[kFusedOthers];
  others_load(keys, olo, ohi, clo, chi, ok);
  u32x4 x[CPL];
  auto load_row = [&](int h) {
    const uint16_t* row = src + (static_cast<size_t>(h) * n + i) * d;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int v = lane + c * kWave;
      x[c] = ld16(row + 8 * (v < nv ? v : 0));  // past the row end: vector 0, never stored
    }
  };
  if (i < n) load_row(0);

  if (E <= 8)
    others_count<1>(keys, olo, ohi, clo, chi, E, ok, orow + w * E, prow + w * E);
  else
    others_count<2>(keys, olo, ohi, clo, chi, E, ok, orow + w * E, prow + w * E);
  int* myrow = wrow + w * E;
  if (lane < E) myrow[lane] = 0;  // each wave touches only its own rows, in order
  const bool bad = qlo < qhi && count_share(keys, qlo, qhi, E, nbits, first, myrow);
  if (bad) set_err(err, ROUTE_EBIT_EXPERT_RANGE);
  lds_barrier();
  for (int e = t; e < E; e += kFusedThreads) {
    int pre = 0, rest = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      pre += orow[v * E + e];
      rest += wrow[v * E + e] + prow[v * E + e];
    }
    sbase[e] = pre;
    stot[e] = pre + rest;
  }
  lds_barrier();
  if (w == 0) scan_bins(stot, E, &stotal);
  lds_barrier();
  for (int e = t; e < E; e += kFusedThreads) {
    if (b == 0) offsets[e] = stot[e];
    int run = stot[e] + sbase[e];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int cnt = wrow[v * E + e];
      wrow[v * E + e] = run;
      run += cnt;
    }
  }
  if (b == 0 && t == 0) offsets[E] = stotal;
  lds_barrier();
  if (qlo < qhi)
    place_share(keys, qlo, qhi, E, nbits, first, myrow, slot_of_pair, pair_of_slot,
                static_cast<uint8_t*>(nullptr), spos, clo);
  lds_barrier();
  if (i >= n) return;
  for (int h = 0; h < H; ++h) {
    if (h > 0) load_row(h);
    for (int q = 0; q < kg; ++q) {
      const int sl = spos[w * K + h * kg + q];
      if (sl < 0 || sl >= nK) continue;  // out-of-range expert: no slot
      uint16_t* dst = disp + static_cast<size_t>(sl) * d;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int v = lane + c * kWave;
        if (v < nv) {
          if constexpr (STREAM)
            st16_stream(dst + 8 * v, x[c]);
          else
            st16(dst + 8 * v, x[c]);
        }
      }
    }
  }
}

// vectors per lane for a row of nv 16-byte vectors: one of the instantiated sizes
inline int cpl_for(int nv) {
  const int need = (nv + kWave - 1) / kWave;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 10 ? 10 : 16;
}

// Scratch of moe_permute_noalloc: the sort's chunk-major histogram table at
// its largest, kMaxChunks chunks x kMaxExperts bins of int32 (512 KiB). Every
// GPU the library runs on holds its own copy until the process ends. In host
// code this name stands for the host-side shadow, not a device address: host
// code only ever uses the per-device address from hipGetSymbolAddress.
constexpr size_t kPermScratchBytes = static_cast<size_t>(kMaxChunks) * kMaxExperts * sizeof(int);
static __device__ __align__(256) unsigned char scratch[kPermScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that stream s runs on, looked up
// with that GPU current on the first call for it and kept afterwards.
int scratch_address(hipStream_t s, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ROUTE_ERR_HIP;
  int dev = cur;
  if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return ROUTE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ROUTE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ROUTE_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return ROUTE_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return ROUTE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ROUTE_OK;
}

}  // namespace route

using namespace route;

ROUTE_API size_t moe_permute_workspace_size(int64_t n, int32_t K, int32_t E) {
  if (n < 0 || K < 1 || E < 1 || E > kMaxExperts) return 0;
  return csort_ws_bytes(n * K, E);
}

// Host checks shared by both entry points (everything but the workspace).
static int permute_check(const int32_t* idx, int64_t n, int32_t K, int32_t E, int32_t H,
                         const uint16_t* src, int32_t d, const int32_t* expert_offsets,
                         const int32_t* slot_of_pair, const int32_t* pair_of_slot,
                         const uint16_t* disp) {
  if (n < 0 || K < 1 || E < 1 || H < 1 || K % H != 0) return ROUTE_ERR_SHAPE;
  if (n * static_cast<int64_t>(K) >= (int64_t(1) << 31)) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (!expert_offsets) return ROUTE_ERR_NULL;
  if (n == 0) return ROUTE_OK;
  if (!idx || !slot_of_pair || !pair_of_slot) return ROUTE_ERR_NULL;
  if ((src == nullptr) != (disp == nullptr)) return ROUTE_ERR_NULL;
  if (src) {
    if (d < 8 || d % 8 != 0) return ROUTE_ERR_SHAPE;
    if (d > 16 * 8 * kWave) return ROUTE_ERR_UNSUPPORTED;
    if (!aligned16(src) || !aligned16(disp)) return ROUTE_ERR_ALIGN;
  }
  return ROUTE_OK;
}

ROUTE_API int moe_permute(const int32_t* idx, int64_t n, int32_t K, int32_t E, int32_t H,
                          const uint16_t* src, int32_t d, int32_t* expert_offsets,
                          int32_t* slot_of_pair, int32_t* pair_of_slot, uint16_t* disp,
                          void* ws, size_t ws_bytes, uint32_t* err, hipStream_t s) {
  const int chk = permute_check(idx, n, K, E, H, src, d, expert_offsets, slot_of_pair,
                                pair_of_slot, disp);
  if (chk != ROUTE_OK) return chk;
  if (n == 0) {
    fill_i32<<<ceil_div(E + 1, 256), 256, 0, s>>>(expert_offsets, E + 1, 0);
    return launch_status();
  }
  const bool stream = K / H >= kPermStreamCopies;
  if (src && E <= kFusedMaxE && n * K <= kFusedMaxPairs && cpl_for(d / 8) <= 8) {
    // the sort and the move in one launch (no workspace used)
    const unsigned grid = ceil_div(n, kFusedTokens);
    switch (cpl_for(d / 8)) {
#define ROUTE_FUSED_CASE(c)                                                                   \
  case c:                                                                                     \
    if (stream)                                                                               \
      permute_fused<c, true><<<grid, kFusedThreads, 0, s>>>(idx, n, K, E, H, bits_for(E), src, \
                                                            d, expert_offsets, slot_of_pair,  \
                                                            pair_of_slot, disp, err);         \
    else                                                                                      \
      permute_fused<c, false><<<grid, kFusedThreads, 0, s>>>(idx, n, K, E, H, bits_for(E),    \
                                                             src, d, expert_offsets,          \
                                                             slot_of_pair, pair_of_slot, disp, \
                                                             err);                            \
    break;
      ROUTE_FUSED_CASE(1) ROUTE_FUSED_CASE(2) ROUTE_FUSED_CASE(4) ROUTE_FUSED_CASE(8)
#undef ROUTE_FUSED_CASE
      default: return ROUTE_ERR_UNSUPPORTED;
    }
    return launch_status();
  }
  if (!ws || ws_bytes < moe_permute_workspace_size(n, K, E)) return ROUTE_ERR_WORKSPACE;
  int st = csort_launch<int32_t>(idx, n * K, E, expert_offsets, slot_of_pair, pair_of_slot,
                                 nullptr, ws, err, ROUTE_EBIT_EXPERT_RANGE, s);
  if (st != ROUTE_OK || !src || n == 0) return st;
  if (d > 16 * 8 * kWave) return ROUTE_ERR_UNSUPPORTED;
  const unsigned grid = ceil_div(n * H, kPermThreads / kWave);
  switch (cpl_for(d / 8)) {
#define ROUTE_CPL_CASE(c)                                                                     \
  case c:                                                                                     \
    if (stream)                                                                               \
      permute_move<c, true><<<grid, kPermThreads, 0, s>>>(src, n, K, H, d, slot_of_pair, disp); \
    else                                                                                      \
      permute_move<c, false><<<grid, kPermThreads, 0, s>>>(src, n, K, H, d, slot_of_pair,     \
                                                           disp);                             \
    break;
    ROUTE_CPL_CASE(1) ROUTE_CPL_CASE(2) ROUTE_CPL_CASE(4) ROUTE_CPL_CASE(8) ROUTE_CPL_CASE(10)
    ROUTE_CPL_CASE(16)
#undef ROUTE_CPL_CASE
    default: return ROUTE_ERR_UNSUPPORTED;
  }
  return launch_status();
}

ROUTE_API int moe_permute_noalloc(const int32_t* idx, int64_t n, int32_t K, int32_t E, int32_t H,
                                  const uint16_t* src, int32_t d, int32_t* expert_offsets,
                                  int32_t* slot_of_pair, int32_t* pair_of_slot, uint16_t* disp,
                                  uint32_t* err, hipStream_t s) {
  // every host check before the scratch is looked up; n = 0 needs no scratch
  const int chk = permute_check(idx, n, K, E, H, src, d, expert_offsets, slot_of_pair,
                                pair_of_slot, disp);
  if (chk != ROUTE_OK) return chk;
  if (n == 0)
    return moe_permute(idx, n, K, E, H, src, d, expert_offsets, slot_of_pair, pair_of_slot, disp,
                       nullptr, 0, err, s);
  if (moe_permute_workspace_size(n, K, E) > kPermScratchBytes) return ROUTE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_address(s, &ws);
  if (st != ROUTE_OK) return st;
  return moe_permute(idx, n, K, E, H, src, d, expert_offsets, slot_of_pair, pair_of_slot, disp,
                     ws, kPermScratchBytes, err, s);
}
