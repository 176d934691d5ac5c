// moe_permute: expert-contiguous dispatch on one GPU. "Speculative MoE"
// notes, section 1: dispatch sends each token's activation to its K experts;
// on one device that is a stable counting sort of the (token, expert) pairs
// by expert (csort.hpp) followed by a row scatter. With H groups ("Federation
// of Experts (FoE)" article) pair (i, k) reads the group-(k / (K/H)) row of
// token i, so each source row is read once and written K/H times.
#include <mutex>

#include "common.hpp"
#include "csort.hpp"

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
  if (!ws || ws_bytes < moe_permute_workspace_size(n, K, E)) return ROUTE_ERR_WORKSPACE;
  int st = csort_launch<int32_t>(idx, n * K, E, expert_offsets, slot_of_pair, pair_of_slot,
                                 nullptr, ws, err, ROUTE_EBIT_EXPERT_RANGE, s);
  if (st != ROUTE_OK || !src || n == 0) return st;
  if (d > 16 * 8 * kWave) return ROUTE_ERR_UNSUPPORTED;
  const unsigned grid = ceil_div(n * H, kPermThreads / kWave);
  const bool stream = K / H >= kPermStreamCopies;
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
