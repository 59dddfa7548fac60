// Tile-skipping attention forward (Veda page, "Attention Structure
// Distillation", Execution: only the selected K/V tiles are fetched;
// Principle 03 "Tile-Sparse Kernel"; "Theoretical Rationale" 1 "Softmax
// Geometry": the row softmax over the kept keys, with its log-sum-exp).
//
// One workgroup (8 waves) computes one 128-query tile of one (batch, head).
// Wave (qg, half) owns queries 32qg..32qg+31 and keys 64half..64half+63 of
// each tile, so two compute waves share each SIMD and one's softmax runs under
// the other's MFMAs; the key halves are merged once at the end. For each
// selected key tile j:
//   S^T = K_j Q^T   32x32x16 bf16 MFMA, fp32 accumulate. Computing S
//                   transposed puts one query per lane (lanes l and l+32 hold
//                   the two halves of its logits), so row max and row sum are
//                   in-lane plus one exchange between the half-waves. Lane l
//                   of a 32-key block feeds key row pi(l) (bits 2 and 3 of l
//                   swapped), so each lane ends up holding runs of 8
//                   consecutive keys.
//   online softmax  base-2 with scale*log2(e) folded into one FMA; pad keys of
//                   border tiles get -inf through a branch-free bias. The
//                   running max only moves (and O is only rescaled) when a
//                   row's max grows by more than 2^8, so most tiles skip the
//                   rescale; P values up to 2^8 are exact in bf16's range.
//   O^T += V_j^T P^T  32x32x16 bf16 MFMA; P is rounded to bf16 (hardware
//                   pack) and used in the very registers the softmax produced
//                   it in: 8 consecutive keys, so each V^T operand is one
//                   16-byte chunk of a channel row.
// K (token-major) and V (channel-major) tiles go from global memory straight
// into LDS with the gfx950 LDS-DMA loads (no registers, no LDS store
// instructions): every wave copies eight 1-KiB chunks, four rows each, and
// picks each lane's source chunk so that the rows land XOR-swizzled (position
// = chunk ^ (row & 15)), which keeps the MFMA operand reads free of bank
// conflicts. The LDS tiles are double-buffered: the copy of tile i+1 runs
// under the compute of tile i. Query tiles of a head are dealt out so each XCD
// works on a contiguous run of neighbouring query tiles, whose key selections
// overlap, while all XCDs share the same head's K/V in the MALL.
// With a work queue (work_item) each XCD first works through the query tiles
// the fixed deal would have given it, then the last ones of every XCD are
// handed out through atomic counters to whichever XCD is free.
// The finished O rows go to the tiled output, or straight to each real
// token's row of a raster output (pad query slots are then not written), which
// spares the layer a separate unpermute pass. Q likewise comes from tiled Q,
// or straight from each real token's raster row (a pad slot gets a zero
// query, as tiled Q holds there), which spares the layer a tiled copy of Q.
#include <atomic>
#include <mutex>

#include "attn_tiles.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kRescaleSlack = 8.0f;   // log2 of the largest unnormalised P

// LDS-DMA copy plan of one wave. A tile is 32 (D = 128) or 16 (D = 64)
// chunks of 1 KiB; waves 0-3 copy K chunks, waves 4-7 V chunks, through
// buffer loads that write LDS directly (the tile's byte offset in a scalar
// register, one 32-bit offset per lane and chunk). In LDS, lane l of a chunk
// fills bytes 16l..16l+15; the lane loads the global 16-byte piece that
// belongs at its swizzled position, so row r holds its piece c at position
// c ^ (r mod positions-per-row, at most 16).
template <int D>
struct DmaPlan {
  const uint16_t* base;                         // this head's K or V tiles
  int32_t bytes;                                // their extent
  uint32_t off[4];                              // per-lane source byte offsets of chunks first..first+3
  int first;                                    // first chunk of this wave
  bool is_k;                                    // wave copies K (else V)
};

template <int D>
__device__ __forceinline__ DmaPlan<D> dma_plan(int wave, int lane, const uint16_t* k_head, const uint16_t* v_head,
                                               int32_t n_tiles) {
  using S = AttnShape<D>;
  DmaPlan<D> pl;
  pl.is_k = wave < kWaves / 2;
  pl.first = (pl.is_k ? wave : wave - kWaves / 2) * S::kChunksPerWave;
  pl.base = pl.is_k ? k_head : v_head;
  pl.bytes = n_tiles * S::kTileElems * 2;
  // The swizzle repeats every 16 rows = 4 chunks, so chunk first + 4q + s
  // starts 4096q bytes after chunk first + s.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = pl.first + i;
    if (pl.is_k) {  // token-major K: kKRowsPerChunk rows of D per chunk
      const int r = c * S::kKRowsPerChunk + lane / S::kKPos, p = lane % S::kKPos;
      pl.off[i] = uint32_t(r * D + ((p ^ (r & (S::kKPos - 1))) * 8)) * 2u;
    } else {        // channel-major V: 4 rows of 128 keys per chunk
      const int d = c * 4 + lane / 16, p = lane % 16;
      pl.off[i] = uint32_t(d * kTok + ((p ^ (d & 15)) * 8)) * 2u;
    }
  }
  return pl;
}

template <int D>
__device__ __forceinline__ void dma_issue(const DmaPlan<D>& pl, uint32_t tile_bytes, lds_u16* dst) {
#pragma unroll
  for (int i = 0; i < AttnShape<D>::kChunksPerWave; ++i)
    dma_copy(pl.base, pl.bytes, pl.off[i % 4], tile_bytes + 4096u * (i / 4), dst + (pl.first + i) * 512);
}

// Per-wave state of the online softmax for 32 queries x one key half.
template <int D>
struct WaveState {
  using S = AttnShape<D>;
  u32x4 qf[S::kDC];       // Q^T operand: d = 16dc + 8h .. +7 of query l32
  floatx16 oacc[S::kDB];  // O^T partial: d = 32db + 8(v/4) + 4h + v%4, query l32
  float m_run, l_run;     // running max (base 2, scaled) and partial sum
};

// S^T for this wave's 64 keys of one tile: block kb, row i = 8(v/4) + 4h + v%4
// is key 64half + 32kb + pi(i) = 64half + 32kb + 16(v/8) + 8h + 4((v/4)%2) + v%4.
template <int D>
__device__ __forceinline__ void s_tile(floatx16 (&sacc)[2], const WaveState<D>& w, const uint16_t* ks, int half,
                                       int h, int l32) {
  using S = AttnShape<D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
    const int r = 64 * half + 32 * kb + key_perm(l32);
    const uint16_t* krow = ks + r * D;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + (((2 * dc + h) ^ (r & (S::kKPos - 1))) * 8));
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(w.qf[dc]), sacc[kb], 0, 0, 0);
    }
  }
}

// Pad keys of a border tile get -inf through a branch-free bias (wm: this
// wave's 64 real-key bits; ~0 for a full tile, which is left untouched).
template <int D>
__device__ __forceinline__ void mask_tile(floatx16 (&sacc)[2], uint64_t wm) {
  if (wm != ~0ull) {
    const uint32_t wlo = uint32_t(wm), whi = uint32_t(wm >> 32);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int bit = 16 * (v / 8) + 4 * ((v / 4) % 2) + (v % 4);
        const uint32_t real = ((kb ? whi : wlo) >> bit) & 1u;
        sacc[kb][v] += __uint_as_float((real - 1u) & 0xFF800000u);
      }
  }
}

// Row max of a lane's 32 scores combined with the other half-wave's (lanes
// l and l + 32 hold the two halves of one query's keys), in base-2 units.
__device__ __forceinline__ float row_max_base2(float mx, float scale_log2) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
}

template <int D>
__device__ __forceinline__ float tile_max(const floatx16 (&sacc)[2], float scale_log2) {
  float mx = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
  return row_max_base2(mx, scale_log2);
}

// Running-max update of the online softmax (base 2), moved lazily: only when
// a row's max grows by more than 2^kRescaleSlack are m, l and O rescaled.
template <int D>
__device__ __forceinline__ void update_max(WaveState<D>& w, float mx) {
  using S = AttnShape<D>;
  if (__builtin_amdgcn_ballot_w64(mx > w.m_run + kRescaleSlack) != 0) {
    const float m_new = fmaxf(w.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) w.oacc[db][v] *= alpha;
  }
}

// V^T fragment of PV step t (block db = t / 4, kb = (t / 2) % 2, c2 = t % 2):
// 16 bytes of channel row 32db + l32, keys 64half + 32kb + 16c2 + 8h .. +7,
// i.e. chunk 8half + 4kb + 2c2 + h of the row, at its swizzled position.
template <int D>
__device__ __forceinline__ u32x4 v_frag(const uint16_t* vs, int t, int half, int h, int l32) {
  const int db = t / 4, kb = (t / 2) % 2, c2 = t % 2;
  const int d = 32 * db + l32;
  return *reinterpret_cast<const u32x4*>(vs + d * kTok + (((8 * half + 4 * kb + 2 * c2 + h) ^ (d & 15)) * 8));
}

// The hot part of one pipelined iteration. Step t issues one QK^T MFMA of
// the next tile (operand read kLook steps ahead) and, every other step, one
// LDS-DMA chunk, so no burst of copies fills the vector-memory queue; the PV
// MFMAs of this tile follow, their V^T reads kLook steps ahead. Scheduling
// fences keep each step's instructions together. The exponentials of this
// tile are written beside the QK^T steps, but the compiler sinks them below
// the next tile's mask code, toward their first use: the emitted order is a
// QK^T block, the exponentials, then PV. That order measured faster than
// exponentials kept inside the QK^T steps, and than the same order written
// out by hand. The next
// tile's pad-key bias and row max (VALU work) run under the PV MFMAs, two
// scores per step. The last iteration (kLast) has no next tile: it issues no
// QK^T MFMAs, no copies and no max.
template <int D, bool kLast, typename NextMask>
__device__ __forceinline__ void hot_tile(WaveState<D>& w, const floatx16 (&s_cur)[2], floatx16 (&s_next)[2],
                                         const uint16_t* ks_next, const uint16_t* vs_cur, const DmaPlan<D>& pl,
                                         uint32_t dma_tile_bytes, lds_u16* dma_dst, int half, int h, int l32,
                                         float scale_log2, const NextMask& next_mask, float& mx_next) {
  using S = AttnShape<D>;
  constexpr int kLook = 4;                 // LDS operand reads in flight ahead of the S MFMAs
  constexpr int kLookV = 4;                // ... and ahead of the PV MFMAs
  constexpr int kS = 2 * S::kDC;           // QK^T MFMAs per tile
  constexpr int kE = 16;                   // exponential pairs per tile
  constexpr int kPV = 4 * S::kDB;          // PV MFMAs per tile
  constexpr int kPer = 32 / kPV;           // next-tile scores whose max each PV step takes
  static_assert(kPer * kPV == 32, "the PV steps cover the 32 scores of a lane");
  constexpr int kSteps = kS > kE ? kS : kE;

  // A half that has seen only pad keys so far keeps m = -inf; its exponents
  // must then still be exp2(-inf) = 0, not NaN.
  const float m_use = w.m_run == -__builtin_inff() ? 0.0f : w.m_run;
  float psum = 0.0f;
  u32x4 pf[2][2];
  u32x4 kf[kS];
  if constexpr (!kLast) {
#pragma unroll
    for (int t = 0; t < kLook && t < kS; ++t) kf[t] = k_frag<D>(ks_next, t, half, h, l32);
  }
  const floatx16 zero = {};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    if (!kLast && t + kLook < kS) kf[t + kLook] = k_frag<D>(ks_next, t + kLook, half, h, l32);
    if (!kLast && t < kS) {
      const int kb = t / S::kDC, dc = t % S::kDC;
      s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[t]), as_bf16x8(w.qf[dc]),
                                                           dc == 0 ? zero : s_next[kb], 0, 0, 0);
    }
    if (t < kE) {  // keys v, v + 1 of block kb
      const int kb = t / 8, v = 2 * (t % 8);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][v], scale_log2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][v + 1], scale_log2, -m_use));
      psum += p0 + p1;
      pf[kb][v / 8][(v % 8) / 2] = pack_bf16x2(p0, p1);
    }
    if (!kLast && t % 2 == 1 && t / 2 < S::kChunksPerWave)
      dma_copy(pl.base, pl.bytes, pl.off[(t / 2) % 4], dma_tile_bytes + 4096u * (t / 8), dma_dst + (pl.first + t / 2) * 512);
    __builtin_amdgcn_sched_barrier(0);
  }
  w.l_run += psum;
  if constexpr (!kLast) mask_tile<D>(s_next, next_mask());  // real-key bits of the next tile

  u32x4 vf[kPV];
#pragma unroll
  for (int t = 0; t < kLookV; ++t) vf[t] = v_frag<D>(vs_cur, t, half, h, l32);
  float mx = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < kPV; ++t) {
    if (t + kLookV < kPV) vf[t + kLookV] = v_frag<D>(vs_cur, t + kLookV, half, h, l32);
    const int db = t / 4, kb = (t / 2) % 2, c2 = t % 2;
    w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[t]), as_bf16x8(pf[kb][c2]), w.oacc[db], 0, 0, 0);
    if (!kLast) {  // scores kPer*t .. kPer*t + kPer - 1 of the next tile's 32
#pragma unroll
      for (int e = 0; e < kPer; ++e) mx = fmaxf(mx, s_next[(kPer * t + e) / 16][(kPer * t + e) % 16]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!kLast) mx_next = row_max_base2(mx, scale_log2);
}

// kDense: dense attention. The kept tiles of query tile tq are all key
// tiles 0..nT_hd-1 in order, so the tile index is the loop counter and no
// index list is read (idx and k_max unused; the host sets k_hd = nT_hd).
template <int D, bool kDense>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_fwd_kernel(
    GeoTable g, const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, const int32_t* __restrict__ idx, int32_t k_max, float scale_log2,
    uint16_t* __restrict__ o_t, float* __restrict__ lse, uint16_t* __restrict__ o_r, int64_t osb, int64_t osn,
    int64_t osh, const uint16_t* __restrict__ q_r, int64_t qsb, int64_t qsn, int64_t qsh, int32_t* __restrict__ queue,
    int32_t n_static) {
  using S = AttnShape<D>;
  // K buffers lds[0..1], V buffers lds[2..3]; after the loop the space holds
  // the half merge.
  __shared__ __attribute__((aligned(16))) uint16_t lds[4][S::kTileElems];

  int32_t bx, hd, b;
  if (!work_item(g, queue, n_static, reinterpret_cast<int32_t*>(&lds[0][0]), &bx, &hd, &b)) return;
  const HeadGeo hg = g.h[hd];
  const int32_t tq = xcd_tile_order(bx, g.nT_max);
  const int64_t head_base = (int64_t(b) * g.heads + hd) * g.nT_max;
  const int64_t tile_elems = S::kTileElems;
  // Tiled output o_t, or (o_r non-null) raster output: then each real query
  // writes its token's row of o_r and pad query slots write nothing.
  uint16_t* o_tile = o_r ? nullptr : o_t + (head_base + tq) * tile_elems;
  float* lse_tile = lse ? lse + (head_base + tq) * kTok : nullptr;

  if (tq >= hg.nT) {  // no such query tile for this head: defined zeros / -inf
    if (o_tile)
      for (int e = threadIdx.x; e < kTok * D / 8; e += kThreads)
        reinterpret_cast<u32x4*>(o_tile)[e] = u32x4{0u, 0u, 0u, 0u};
    if (lse_tile)
      for (int e = threadIdx.x; e < kTok; e += kThreads) lse_tile[e] = -__builtin_inff();
    return;
  }

  // Wave (qg, half): queries 32qg..32qg+31 against keys 64half..64half+63 of
  // every selected tile; the two halves are merged at the end.
  // The two waves of a query group sit on different SIMDs (waves are dealt
  // to SIMDs round robin), so a tile whose only real queries form one group
  // keeps two SIMDs busy.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int qg = (wave >> 1) & 3, half = wave & 1;
  const int l32 = lane % 32, h = lane / 32;
  const int32_t* sel = kDense ? nullptr : idx + (head_base + tq) * k_max;
  const unsigned nT = unsigned(hg.nT);
  const int kh = kDense ? hg.nT : hg.k;
  // Key tile of iteration x (x < kh): the list's entry, or x itself when dense.
  auto tile_at = [&](int x) -> int32_t { return kDense ? x : sel[x]; };
  const DmaPlan<D> plan = dma_plan<D>(wave, lane, k_t + head_base * tile_elems, v_t + head_base * tile_elems, g.nT_max);
  // Byte offset of a copy source tile; entries outside [0, nT_hd) contribute
  // no keys and tile 0 stands in as a harmless source.
  auto tile_src = [&](int32_t jt) { return uint32_t(unsigned(jt) < nT ? jt : 0) * uint32_t(tile_elems * 2); };
  lds_u16* const lbuf = (lds_u16*)&lds[0][0];   // lds[b] is lbuf + b * kTileElems

  WaveState<D> w;
  if (q_r) {  // raster Q: this lane's query row, or a zero query for a pad slot (as in tiled Q)
    const int64_t n = raster_of_slot(g, hg, box_extent(g, hg, tq), qg * 32 + l32);
    if (n >= 0) {
      const uint16_t* qrow = q_r + int64_t(b) * qsb + n * qsn + int64_t(hd) * qsh + 8 * h;
#pragma unroll
      for (int dc = 0; dc < S::kDC; ++dc) w.qf[dc] = *reinterpret_cast<const u32x4*>(qrow + 16 * dc);
    } else {
#pragma unroll
      for (int dc = 0; dc < S::kDC; ++dc) w.qf[dc] = u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    const uint16_t* qrow = q_t + (head_base + tq) * tile_elems + (qg * 32 + l32) * D + 8 * h;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) w.qf[dc] = *reinterpret_cast<const u32x4*>(qrow + 16 * dc);
  }
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) w.oacc[db][v] = 0.0f;
  w.m_run = -__builtin_inff();
  w.l_run = 0.0f;

  // Software pipeline over the selected tiles. Iteration i computes S of
  // tile i+1 (its K landed during iteration i-1) while it runs the softmax
  // and PV of tile i; meanwhile K of tile i+2 and V of tile i+1 are copied.
  //   K of tile t in lds[t & 1]; V of tile t in lds[2 + (t & 1)].
  // A buffer is overwritten only after the barrier that ends the iteration
  // in which it was last read.
  // Tile indices of iterations i, i+1, i+2 (clamped to the last entry
  // past the end: such copies and products are never used). The next one is
  // loaded just before each iteration's closing barrier, so no scalar load is
  // in flight while the LDS operand reads are being waited for.
  int32_t j = tile_at(0), jn = tile_at(min(1, kh - 1)), jn2 = tile_at(min(2, kh - 1));
  if (plan.is_k) {
    dma_issue<D>(plan, tile_src(j), lbuf);
    dma_issue<D>(plan, tile_src(jn), lbuf + S::kTileElems);
  } else {
    dma_issue<D>(plan, tile_src(j), lbuf + 2 * S::kTileElems);
  }
  __builtin_amdgcn_s_waitcnt(0);  // Q and the first copies have landed
  __syncthreads();
  floatx16 sc[2];
  s_tile<D>(sc, w, lds[0], half, h, l32);
  mask_tile<D>(sc, real_key_bits(g, hg, j, half, h));
  float mx_cur = tile_max<D>(sc, scale_log2);  // row max of the tile the next iteration finishes
  __syncthreads();  // every wave has read lds[0] before tile 2 lands there

  // One pipelined iteration: s_cur holds S of tile i, s_next receives S of
  // tile i+1 (except in the last iteration, `last` = true_type, which only
  // finishes tile i).
  auto iteration = [&](auto last, int i, floatx16 (&s_cur)[2], floatx16 (&s_next)[2]) {
    constexpr bool kLast = decltype(last)::value;
    const int cur = i & 1;
    update_max<D>(w, mx_cur);
    // K of tile i+2 into lds[cur] (K of tile i, read in the previous
    // iteration) or V of tile i+1 into lds[2 + (cur ^ 1)] (V of tile i-1).
    // Tile i+1's scores are masked and their row max taken under the PV MFMAs.
    float mx_next = 0.0f;
    hot_tile<D, kLast>(w, s_cur, s_next, lds[cur ^ 1], lds[2 + cur], plan, tile_src(plan.is_k ? jn2 : jn),
                       lbuf + (plan.is_k ? cur : 2 + (cur ^ 1)) * S::kTileElems, half, h, l32, scale_log2,
                       [&] { return real_key_bits(g, hg, jn, half, h); }, mx_next);
    if constexpr (!kLast) {
      mx_cur = mx_next;
      j = jn;
      jn = jn2;
      jn2 = tile_at(min(i + 3, kh - 1));
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and the next index have landed
      __syncthreads();
    }
  };
  const std::false_type more{};
  const std::true_type last{};
  // With raster output, a query group made only of pad slots (border tiles)
  // computes nothing: its waves only make their copies and keep the barriers
  // (one per iteration but the last, as below), and nothing of it is written.
  bool pad_group = false;
  if (o_r && !hg.all_full) {
    const BoxExtent e = box_extent(g, hg, tq);
    if (!box_is_full(hg, e)) pad_group = uint32_t(box_slot_mask64(hg, e, 64 * (qg >> 1)) >> (32 * (qg & 1))) == 0u;
  }
  if (pad_group) {
    for (int i = 0; i + 1 < kh; ++i) {
      const int cur = i & 1;
      dma_issue<D>(plan, tile_src(plan.is_k ? jn2 : jn), lbuf + (plan.is_k ? cur : 2 + (cur ^ 1)) * S::kTileElems);
      jn = jn2;
      jn2 = tile_at(min(i + 3, kh - 1));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    floatx16 sn[2];
    int i = 0;
    for (; i + 2 < kh; i += 2) {
      iteration(more, i, sc, sn);
      iteration(more, i + 1, sn, sc);
    }
    if (i + 1 < kh) {
      iteration(more, i, sc, sn);
      iteration(last, i + 1, sn, sc);
    } else {
      iteration(last, i, sc, sn);
    }
  }
  __syncthreads();  // every wave is done with the tile buffers

  // Merge the two key halves through LDS (the tile buffers are free now):
  // m = max(m0, m1), O = O0 2^(m0-m) + O1 2^(m1-m), l likewise. Both halves
  // share the work: half 0 finishes O^T blocks 0..kDB/2-1 and half 1 blocks
  // kDB/2..kDB-1, each reading the other half's partials of its blocks, so
  // all eight waves combine and store O.
  constexpr int kOwn = S::kDB / 2;                           // O^T blocks each half finishes
  float* red = reinterpret_cast<float*>(&lds[0][0]);        // [4][kDB*16][64] partial O^T
  float* red_ml = red + 4 * S::kDB * 16 * 64;                // [4][2 halves][2][64] m, l
  static_assert(sizeof(lds) >= (4 * S::kDB * 16 * 64 + 4 * 2 * 2 * 64) * sizeof(float), "merge space");
  const float l_half = w.l_run + __shfl_xor(w.l_run, 32, 64);
  // The blocks the other half finishes (register indices fixed at compile time on each branch).
  auto give = [&](auto first) {
    constexpr int f = decltype(first)::value;
#pragma unroll
    for (int d2 = 0; d2 < kOwn; ++d2)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((qg * S::kDB + f + d2) * 16 + v) * 64 + lane] = w.oacc[f + d2][v];
  };
  if (half == 0)
    give(std::integral_constant<int, kOwn>{});
  else
    give(std::integral_constant<int, 0>{});
  red_ml[((qg * 2 + half) * 2 + 0) * 64 + lane] = w.m_run;
  red_ml[((qg * 2 + half) * 2 + 1) * 64 + lane] = l_half;
  __syncthreads();
  {
    // m, l of half 0 and half 1, in that order on both halves, so both compute the same l_tot.
    const float m0 = red_ml[((qg * 2 + 0) * 2 + 0) * 64 + lane], l0 = red_ml[((qg * 2 + 0) * 2 + 1) * 64 + lane];
    const float m1 = red_ml[((qg * 2 + 1) * 2 + 0) * 64 + lane], l1 = red_ml[((qg * 2 + 1) * 2 + 1) * 64 + lane];
    const float m = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float l_tot = l0 * a0 + l1 * a1;
    const float inv = 1.0f / l_tot;
    const float c0 = a0 * inv, c1 = a1 * inv;
    uint16_t* orow;
    if (o_tile) {
      orow = o_tile + (qg * 32 + l32) * D;
    } else {
      const int64_t n = raster_of_slot(g, hg, box_extent(g, hg, tq), qg * 32 + l32);
      orow = n >= 0 ? o_r + int64_t(b) * osb + n * osn + int64_t(hd) * osh : nullptr;
    }
    // Half 0's partial times c0 plus half 1's times c1, for the blocks this half finishes.
    auto finish = [&](auto first, auto is_half0) {
      constexpr int f = decltype(first)::value;
      constexpr bool h0 = decltype(is_half0)::value;
#pragma unroll
      for (int d2 = 0; d2 < kOwn; ++d2) {
        const int db = f + d2;
        float o[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float mine = w.oacc[db][v], theirs = red[((qg * S::kDB + db) * 16 + v) * 64 + lane];
          o[v] = h0 ? mine * c0 + theirs * c1 : theirs * c0 + mine * c1;
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 wd;
          wd[0] = pack_bf16x2(o[4 * g4 + 0], o[4 * g4 + 1]);
          wd[1] = pack_bf16x2(o[4 * g4 + 2], o[4 * g4 + 3]);
          if (orow) *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * h) = wd;
        }
      }
    };
    if (half == 0)
      finish(std::integral_constant<int, 0>{}, std::true_type{});
    else
      finish(std::integral_constant<int, kOwn>{}, std::false_type{});
    // A pad query slot has no token in a raster output: its LSE is -inf there.
    if (half == 0 && lse_tile && h == 0) {
      const bool pad_slot = o_r && !slot_is_real(hg, box_extent(g, hg, tq), qg * 32 + l32);
      lse_tile[qg * 32 + l32] = pad_slot ? -__builtin_inff() : (m + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

// The work queue of the allocation-free attention call: one queue's
// counters in a file-scope device array, so that a caller that cannot
// allocate needs no workspace. Each device holds its own copy; host code
// never passes the array's name to a kernel (in host code it only stands in
// for the symbol) but the address hipGetSymbolAddress gives on that device,
// looked up once per device with the device current.
static __device__ __align__(256) int32_t scratch[kAttnQueueInts];

}  // namespace

hipError_t attn_scratch_queue(int32_t** queue) {
  constexpr int kDevices = 64;
  static std::atomic<int32_t*> addr[kDevices];
  static std::mutex lock;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  int32_t* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(lock);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* sym = nullptr;
      e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<int32_t*>(sym);
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *queue = p;
  return hipSuccess;
}

hipError_t launch_sparse_attn(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const uint16_t* v_t,
                              const int32_t* idx, int32_t k_max, float scale, uint16_t* o_t, float* lse,
                              uint16_t* o_r, int64_t osb, int64_t osn, int64_t osh, const uint16_t* q_r, int64_t qsb,
                              int64_t qsn, int64_t qsh, int32_t* queue, hipStream_t s) {
  dim3 grid;
  int32_t n_static = 0;
  const hipError_t e = queue_launch(g, queue, &grid, &n_static, s);
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.44269504088896340736f;
  const bool dense = idx == nullptr;
  if (g.d == 128 && dense)
    sparse_attn_fwd_kernel<128, true><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse,
                                                               o_r, osb, osn, osh, q_r, qsb, qsn, qsh, queue, n_static);
  else if (g.d == 128)
    sparse_attn_fwd_kernel<128, false><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse,
                                                                o_r, osb, osn, osh, q_r, qsb, qsn, qsh, queue, n_static);
  else if (dense)
    sparse_attn_fwd_kernel<64, true><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse,
                                                              o_r, osb, osn, osh, q_r, qsb, qsn, qsh, queue, n_static);
  else
    sparse_attn_fwd_kernel<64, false><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse,
                                                               o_r, osb, osn, osh, q_r, qsb, qsn, qsh, queue, n_static);
  return hipGetLastError();
}

}  // namespace veda
