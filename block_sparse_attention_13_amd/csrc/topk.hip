// Head-aware Top-k tile mask (Veda page, "Attention Structure Distillation",
// Execution: Top-k over the estimator's scores, per query tile and per head,
// yields the binary tile mask passed to the tile-skipping kernel).
//
// One wave per row (b, head, query tile). A row of up to 2048 scores that
// starts on a 16-byte boundary (every row when nT_max is a multiple of 4) is
// first copied into the wave's own LDS area in 1-KiB pieces with the gfx950
// LDS-DMA buffer loads (a per-row buffer, so pieces past the row read zeros),
// then read back one score per lane and chunk; other rows are read straight
// into registers with streaming loads. Each score becomes a 32-bit key
// whose unsigned order is the float order (-0 is first made +0, so signed
// zeros tie). The row's keys stay in registers (chunk i, lane l holds key
// tile j = 64*i + l). A bitwise search from the top bit finds a threshold t:
// the k-th largest key, or (stopping early) any t with exactly k keys >= t.
// One ascending pass over the chunks then keeps every key > t and the
// lowest-indexed keys == t until k are kept, which is exactly the
// lower-index tie rule. Ballots give output positions and bitmask words; each
// chunk's two bitmask words go into one lane each of a register, and the
// row's words are stored together at the end, instead of one single-lane store
// per word.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum over the 64 lanes of a wave, in registers: DPP butterflies inside each
// 16-lane row (quad swaps, then the half-row and row mirrors), then the four
// row sums read out as scalars. The result is wave-uniform.
template <int kCtrl>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(v, v, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum(int v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ uint32_t count_below(uint64_t mask) {  // set bits of lanes < this lane
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

template <int NCH>
__global__ __launch_bounds__(kThreads) void topk_kernel(GeoTable g, const float* __restrict__ scores, int32_t k_max,
                                                       int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask) {
  constexpr bool kStaged = NCH <= 32;   // rows of up to 2048 scores go through LDS
  // Each wave's area is whole 1-KiB pieces: a piece always writes all 64 lanes'
  // 16 bytes (zeros past the row), so a shorter area would spill into the next.
  constexpr int kRowWords = kStaged ? (NCH * 64 + 255) / 256 * 256 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t row_s[kRowsPerBlock][kRowWords];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int32_t tq = blockIdx.x * kRowsPerBlock + wave;
  const int hd = blockIdx.y, b = blockIdx.z;
  if (tq >= g.nT_max) return;
  const HeadGeo hg = g.h[hd];
  const int64_t row = (int64_t(b) * g.heads + hd) * g.nT_max + tq;
  int32_t* out = idx + row * k_max;
  const int n_words = (g.nT_max + 31) / 32;
  uint32_t* bm = bitmask ? bitmask + row * n_words : nullptr;

  if (tq >= hg.nT) {  // no such query tile for this head
    for (int i = lane; i < k_max; i += 64) out[i] = -1;
    if (bm)
      for (int i = lane; i < n_words; i += 64) bm[i] = 0u;
    return;
  }
  const int n = hg.nT, k = hg.k;
  const float* s = scores + row * g.nT_max;
  uint32_t key[NCH];  // key of score j = 64 i + lane in key[i]; 0 (below every finite score's key) past the row
  bool staged = false;
  if constexpr (kStaged) staged = (reinterpret_cast<uintptr_t>(s) & 15u) == 0;   // wave-uniform
  if (staged) {
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    lds_u32* dst = (lds_u32*)&row_s[wave][0];
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s), 0, n * 4, 0x00020000);
    const int pieces = (n * 4 + 1023) / 1024;
    for (int c = 0; c < pieces; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + c * 256, 16, 16 * lane, c * 1024, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's pieces have landed (only this wave reads them)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = i * 64 + lane;
      key[i] = j < n ? order_key(__uint_as_float(row_s[wave][j])) : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = i * 64 + lane;
      key[i] = j < n ? order_key(__builtin_nontemporal_load(s + j)) : 0u;
    }
  }
  // Largest t with #{key >= t} >= k: the k-th largest key. The search may
  // stop early at a t with exactly k keys >= t; those k keys are then the
  // k largest, and the selection below keeps exactly them.
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) c += key[i] >= cand;
    const int total = wave_sum(c);  // wave-uniform
    if (total >= k) {
      t = cand;
      if (total == k) break;
    }
  }
  int c_gt = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) c_gt += key[i] > t;
  const int need_eq = k - wave_sum(c_gt);  // keys equal to t still to keep, lowest index first

  constexpr int kWordRegs = (2 * NCH + 63) / 64;  // bitmask words of the row, 64 per register
  uint32_t bmw[kWordRegs];
#pragma unroll
  for (int r = 0; r < kWordRegs; ++r) bmw[r] = 0u;
  int kept = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const bool gt = key[i] > t;
    const bool eq = key[i] == t;
    const uint64_t eq_mask = __ballot(eq);
    const bool take = gt || (eq && eq_seen + int(count_below(eq_mask)) < need_eq);
    const uint64_t take_mask = __ballot(take);
    const int pos = kept + int(count_below(take_mask));
    if (take && pos < k) out[pos] = i * 64 + lane;   // exactly k are taken; the bound keeps writes in the row
    kept += __popcll(take_mask);
    eq_seen += __popcll(eq_mask);
    if (lane == (2 * i) % 64) bmw[(2 * i) / 64] = uint32_t(take_mask);
    if (lane == (2 * i + 1) % 64) bmw[(2 * i + 1) / 64] = uint32_t(take_mask >> 32);
  }
  if (bm) {
#pragma unroll
    for (int r = 0; r < kWordRegs; ++r)
      if (64 * r + lane < n_words) bm[64 * r + lane] = bmw[r];
  }
  for (int i = k + lane; i < k_max; i += 64) out[i] = -1;
}

template <int NCH>
hipError_t launch_nch(const GeoTable& g, const float* scores, int32_t k_max, int32_t* idx, uint32_t* bitmask,
                      hipStream_t s) {
  const dim3 grid((g.nT_max + kRowsPerBlock - 1) / kRowsPerBlock, g.heads, g.B);
  topk_kernel<NCH><<<grid, kThreads, 0, s>>>(g, scores, k_max, idx, bitmask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const GeoTable& g, const float* scores, int32_t k_max, int32_t* idx, uint32_t* bitmask,
                       hipStream_t s) {
  const int chunks = (g.nT_max + 63) / 64;
  if (chunks <= 1) return launch_nch<1>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 2) return launch_nch<2>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 4) return launch_nch<4>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 8) return launch_nch<8>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 16) return launch_nch<16>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 32) return launch_nch<32>(g, scores, k_max, idx, bitmask, s);
  if (chunks <= 64) return launch_nch<64>(g, scores, k_max, idx, bitmask, s);
  return launch_nch<128>(g, scores, k_max, idx, bitmask, s);
}

}  // namespace veda
