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
//
// score_topk_kernel runs the same selection on scores it computes itself
// from the estimator's features (Estimator: the products of the head-specific
// projections score each tile pair) and holds in LDS, so no score matrix goes
// through HBM.
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

// A row with no such query tile for its head: every index -1, no bit set.
__device__ __forceinline__ void empty_row(int32_t k_max, int n_words, int lane, int32_t* out, uint32_t* bm) {
  for (int i = lane; i < k_max; i += 64) out[i] = -1;
  if (bm)
    for (int i = lane; i < n_words; i += 64) bm[i] = 0u;
}

// The k largest of one row's keys (key of tile j = 64 i + lane in key[i]; 0,
// below every finite score's key, past the row): ascending tile indices into
// out[0..k), -1 in out[k..k_max), and the row's bitmask words when bm is set.
template <int NCH>
__device__ __forceinline__ void select_row(const uint32_t (&key)[NCH], int k, int32_t k_max, int n_words, int lane,
                                           int32_t* out, uint32_t* bm) {
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
    empty_row(k_max, n_words, lane, out, bm);
    return;
  }
  const int n = hg.nT;
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
  select_row<NCH>(key, hg.k, k_max, n_words, lane, out, bm);
}

constexpr int kStRows = 8;                  // query tiles per workgroup, one wave each in the selection
constexpr int kStThreads = 64 * kStRows;
constexpr int kStCols = 2;                  // key tiles a thread scores at once (each query read serves both)
constexpr int kStWavesPerSimd = 4;          // two workgroups per CU (64 KiB of keys each): at most 128 VGPRs

// Scores and Top-k in one pass: the ordered scores of kStRows query tiles
// against all key tiles of the head go to LDS as order keys, never to HBM,
// and each wave then selects one row from there. Score (i, j) is the same
// fp32 chain as the scores kernel's: FMA over the r channels in ascending
// order from +0, products of bf16 values exact, so the keys, and with them
// the lists and bitmasks, are the bytes of the two-kernel route.
// Thread t scores key tiles t + kStThreads * (kStCols m + u), u < kStCols,
// for all kStRows rows at once: the rows' features sit in LDS as fp32
// [channel][row], and each 16-byte broadcast read of four rows' values feeds
// 4 kStCols FMAs. The code avoids two things the compiler would otherwise
// do with it: the query reads take an offset the compiler cannot see is 0,
// so they are not hoisted out of the column loop (64 x 8 live values), and a
// column past the row still stores its keys (to a spare word past the row),
// so no branch sinks its FMA chain below the loop and keeps the query values
// live until then.
template <int R, int NCH>
__global__ __launch_bounds__(kStThreads, kStWavesPerSimd) void score_topk_kernel(
    GeoTable g, const uint16_t* __restrict__ feat_q, const uint16_t* __restrict__ feat_k, int32_t k_max,
    int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask) {
  constexpr int kRowWords = NCH * 64;
  __shared__ uint32_t key_s[kStRows][kRowWords + 1];   // word kRowWords: the spare
  __shared__ __attribute__((aligned(16))) float fq_s[R][kStRows];
  const int hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int n = hg.nT;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int i0 = blockIdx.x * kStRows;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  if (i0 < n) {  // workgroup-uniform
    for (int e = threadIdx.x; e < kStRows * R; e += kStThreads) {
      const int r = e % kStRows, c = e / kStRows;
      fq_s[c][r] = i0 + r < n ? bf16_to_f32(feat_q[(head_row + i0 + r) * R + c]) : 0.0f;
    }
    __syncthreads();
    // A key tile's feature row (R bf16, R / 8 pieces of 16 bytes) is loaded
    // whole, in back-to-back loads; a column past the row loads the last
    // row's features (a valid address) and its keys go to the spare word.
    constexpr int kPieces = R / 8;
    const uint16_t* fk_head = feat_k + head_row * R;
    const float4* fq4 = reinterpret_cast<const float4*>(&fq_s[0][0]);
    for (int jb = threadIdx.x; jb < n; jb += kStThreads * kStCols) {
      int32_t hidden_zero;
      asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
      uint4 kw[kStCols][kPieces];
#pragma unroll
      for (int u = 0; u < kStCols; ++u) {
        const int64_t j = min(jb + u * kStThreads, n - 1);
#pragma unroll
        for (int p = 0; p < kPieces; ++p) kw[u][p] = *reinterpret_cast<const uint4*>(fk_head + j * R + 8 * p);
      }
      float acc[kStCols][kStRows];
#pragma unroll
      for (int u = 0; u < kStCols; ++u)
#pragma unroll
        for (int r = 0; r < kStRows; ++r) acc[u][r] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < kPieces; ++cb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 8 * cb + e;
          float qv[kStRows];
#pragma unroll
          for (int r4 = 0; r4 < kStRows / 4; ++r4) {
            const float4 q4 = fq4[hidden_zero + (c * kStRows + 4 * r4) / 4];
            qv[4 * r4] = q4.x;
            qv[4 * r4 + 1] = q4.y;
            qv[4 * r4 + 2] = q4.z;
            qv[4 * r4 + 3] = q4.w;
          }
#pragma unroll
          for (int u = 0; u < kStCols; ++u) {
            const uint4 pc = kw[u][cb];
            const uint32_t wd = e / 2 == 0 ? pc.x : e / 2 == 1 ? pc.y : e / 2 == 2 ? pc.z : pc.w;
            const float kv = __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
#pragma unroll
            for (int r = 0; r < kStRows; ++r) acc[u][r] = __builtin_fmaf(qv[r], kv, acc[u][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one 8-channel group at a time
      }
#pragma unroll
      for (int u = 0; u < kStCols; ++u) {
        const int j = jb + u * kStThreads;
        const int js = j < n ? j : kRowWords;
#pragma unroll
        for (int r = 0; r < kStRows; ++r) key_s[r][js] = order_key(acc[u][r]);
      }
    }
    __syncthreads();
  }
  const int32_t tq = i0 + wave;
  if (tq >= g.nT_max) return;
  const int64_t row = head_row + tq;
  int32_t* out = idx + row * k_max;
  const int n_words = (g.nT_max + 31) / 32;
  uint32_t* bm = bitmask ? bitmask + row * n_words : nullptr;
  if (tq >= n) {
    empty_row(k_max, n_words, lane, out, bm);
    return;
  }
  uint32_t key[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int j = i * 64 + lane;
    key[i] = j < n ? key_s[wave][j] : 0u;
  }
  select_row<NCH>(key, hg.k, k_max, n_words, lane, out, bm);
}

template <int R, int NCH>
hipError_t launch_st(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t k_max, int32_t* idx,
                     uint32_t* bitmask, hipStream_t s) {
  const dim3 grid((g.nT_max + kStRows - 1) / kStRows, g.heads, g.B);
  score_topk_kernel<R, NCH><<<grid, kStThreads, 0, s>>>(g, feat_q, feat_k, k_max, idx, bitmask);
  return hipGetLastError();
}

template <int R>
hipError_t launch_st_r(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t k_max, int32_t* idx,
                       uint32_t* bitmask, hipStream_t s) {
  const int chunks = (g.nT_max + 63) / 64;
  if (chunks <= 1) return launch_st<R, 1>(g, feat_q, feat_k, k_max, idx, bitmask, s);
  if (chunks <= 2) return launch_st<R, 2>(g, feat_q, feat_k, k_max, idx, bitmask, s);
  if (chunks <= 4) return launch_st<R, 4>(g, feat_q, feat_k, k_max, idx, bitmask, s);
  if (chunks <= 8) return launch_st<R, 8>(g, feat_q, feat_k, k_max, idx, bitmask, s);
  if (chunks <= 16) return launch_st<R, 16>(g, feat_q, feat_k, k_max, idx, bitmask, s);
  return launch_st<R, 32>(g, feat_q, feat_k, k_max, idx, bitmask, s);
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

hipError_t launch_score_topk(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                             int32_t k_max, int32_t* idx, uint32_t* bitmask, hipStream_t s) {
  if (g.nT_max > kScoreTopkMaxTiles) return hipErrorInvalidValue;
  return r == 64 ? launch_st_r<64>(g, feat_q, feat_k, k_max, idx, bitmask, s)
                 : launch_st_r<32>(g, feat_q, feat_k, k_max, idx, bitmask, s);
}

}  // namespace veda
