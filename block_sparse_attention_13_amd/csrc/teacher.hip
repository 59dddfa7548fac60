// Tile-level teacher of the distillation and the overlap of two tile masks
// (Veda page, "Attention Structure Distillation", Teacher: max-pooled full
// attention gives a tile-level target; Principle 01 "Full-Attention Structure
// Distillation"; "Empirical Study" 02: the oracle mask keeps each query
// tile's highest-response key tiles, and tile recall compares masks).
//
// Teacher: T[b, hd, tq, j] is the largest dense softmax probability between
// a real query of tile tq and a real key of tile j:
//   T = max_{i in tq, m in j} exp(scale q_i.k_m - lse_i),
// with lse_i the log-sum-exp of query i over every real key of the head (the
// LSE of the attention forward with every key tile kept). exp is monotone,
// so the block maximum is taken over the logits and exponentiated once.
//
// One workgroup (8 waves) handles one query tile and streams every key tile
// of its head through three LDS buffers (LDS-DMA copies two tiles ahead).
// Query tiles are dealt to the XCDs as in the attention forward, through the
// same optional work queue.
// Wave (qp, kq) computes S^T for queries 64qp..64qp+63 and keys
// 32kq..32kq+31 with 32x32x16 bf16 MFMAs (fp32 accumulation), each K
// fragment feeding two of them, takes the maximum of
// scale*log2(e)*s - log2(e)*lse per lane, reduces it over the wave, and the
// eight wave maxima of a key tile are combined through LDS.
#include "attn_tiles.hpp"

namespace veda {
namespace {

using namespace attn;

template <int D>
struct TeacherShape {
  static constexpr int kChunksPerWave = AttnShape<D>::kChunks / kWaves;  // K chunks each wave copies
};

// Largest value over the 64 lanes of a wave, in registers: DPP butterflies
// inside each 16-lane row (quad swaps, then the half-row and row mirrors),
// then the four row results read out as scalars.
template <int kCtrl>
__device__ __forceinline__ float dpp_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), kCtrl, 0xF, 0xF,
                                                              false)));
}
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_max<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_max<0x141>(x);  // row_half_mirror
  x = dpp_max<0x140>(x);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void teacher_kernel(GeoTable g, const uint16_t* __restrict__ q_t,
                                                             const uint16_t* __restrict__ k_t,
                                                             const float* __restrict__ lse, float scale_log2,
                                                             float* __restrict__ teacher, int32_t* __restrict__ queue,
                                                             int32_t n_static) {
  using S = AttnShape<D>;
  using TS = TeacherShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[3][S::kTileElems];
  __shared__ float red[2][kWaves];

  int32_t bx, hd, b;
  if (!work_item(g, queue, n_static, reinterpret_cast<int32_t*>(&kbuf[0][0]), &bx, &hd, &b)) return;
  const HeadGeo hg = g.h[hd];
  const int32_t tq = xcd_tile_order(bx, g.nT_max);
  const int64_t head_base = (int64_t(b) * g.heads + hd) * g.nT_max;
  const int64_t tile_elems = S::kTileElems;
  float* trow = teacher + (head_base + tq) * g.nT_max;
  const int32_t nT = hg.nT;

  // Key tiles past the head's last one, and whole rows of query tiles past
  // it, hold -inf.
  for (int j = (tq < nT ? nT : 0) + int(threadIdx.x); j < g.nT_max; j += kThreads) trow[j] = -__builtin_inff();
  if (tq >= nT) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  // Wave (qp, kq): queries 64qp..64qp+63 (two 32-query MFMA blocks) against
  // keys 32kq..32kq+31 of every key tile, i.e. block kq & 1 of key half
  // kq >> 1. Each K fragment read from LDS feeds two MFMAs (one per query
  // block), which halves the LDS reads of four 32-query groups.
  const int qp = wave & 1, kq = wave >> 1;
  const int khalf = kq >> 1, kblk = kq & 1;
  const int l32 = lane % 32, h = lane / 32;

  // Q^T operands of this lane's two queries, and their base-2 LSEs; a pad
  // query gets +inf so that it never raises a maximum.
  u32x4 qf[2][S::kDC];
  float lse2[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int slot = qp * 64 + qb * 32 + l32;
    const uint16_t* qrow = q_t + (head_base + tq) * tile_elems + slot * D + 8 * h;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) qf[qb][dc] = *reinterpret_cast<const u32x4*>(qrow + 16 * dc);
    const bool q_real = hg.all_full || slot_is_real(hg, box_extent(g, hg, tq), slot);
    lse2[qb] = q_real ? lse[(head_base + tq) * kTok + slot] * 1.44269504088896340736f : __builtin_inff();
  }

  // K-only LDS-DMA plan: wave w copies chunks w*cpw .. w*cpw + cpw - 1.
  uint32_t off[TS::kChunksPerWave];
#pragma unroll
  for (int i = 0; i < TS::kChunksPerWave; ++i) {
    const int c = wave * TS::kChunksPerWave + i;
    const int r = c * S::kKRowsPerChunk + lane / S::kKPos, p = lane % S::kKPos;
    off[i] = uint32_t(r * D + ((p ^ (r & (S::kKPos - 1))) * 8)) * 2u;
  }
  const uint16_t* k_head = k_t + head_base * tile_elems;
  const int32_t k_bytes = g.nT_max * S::kTileElems * 2;
  lds_u16* const lbuf = (lds_u16*)&kbuf[0][0];
  auto copy_tile = [&](int32_t jt, int buf) {
#pragma unroll
    for (int i = 0; i < TS::kChunksPerWave; ++i)
      dma_copy(k_head, k_bytes, off[i], uint32_t(jt) * uint32_t(S::kTileElems * 2),
               lbuf + buf * S::kTileElems + (wave * TS::kChunksPerWave + i) * 512);
  };

  copy_tile(0, 0);
  if (nT > 1) copy_tile(1, 1);
  __builtin_amdgcn_s_waitcnt(0);  // Q, the LSE and the first copies have landed
  __syncthreads();

  const floatx16 zero = {};
  int buf = 0;  // j % 3
  // K fragments of the current tile; those of tile j+1 are read right after
  // tile j's MFMAs are issued (tile j+1 has been resident since the previous
  // iteration's barrier), so the LDS latency hides under the MFMAs.
  u32x4 kf[S::kDC];
#pragma unroll
  for (int dc = 0; dc < S::kDC; ++dc) kf[dc] = k_frag<D>(&kbuf[0][0], kblk * S::kDC + dc, khalf, h, l32);
  for (int32_t j = 0; j < nT; ++j) {
    const int next = buf == 2 ? 0 : buf + 1;
    // K of tile j+2 into the buffer of tile j-1 (read in the previous iteration).
    if (j + 2 < nT) copy_tile(j + 2, next == 2 ? 0 : next + 1);
    floatx16 sacc[2];
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)  // alternate the two accumulators
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[dc]), as_bf16x8(qf[qb][dc]),
                                                           dc == 0 ? zero : sacc[qb], 0, 0, 0);
    if (j + 1 < nT) {
#pragma unroll
      for (int dc = 0; dc < S::kDC; ++dc) kf[dc] = k_frag<D>(&kbuf[next][0], kblk * S::kDC + dc, khalf, h, l32);
    }
    // Pad keys of a border tile never raise the maximum: this wave's 32 keys
    // are one word of its key half's real-key bits.
    const uint64_t wm = real_key_bits(g, hg, j, khalf, h);
    if (wm != ~0ull) {
      const uint32_t w32 = kblk ? uint32_t(wm >> 32) : uint32_t(wm);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int bit = 16 * (v / 8) + 4 * ((v / 4) % 2) + (v % 4);
          sacc[qb][v] += __uint_as_float((((w32 >> bit) & 1u) - 1u) & 0xFF800000u);
        }
    }
    // scale*log2(e)*s - log2(e)*lse is increasing in s, so each query's
    // maximum logit gives its maximum probability.
    float x = -__builtin_inff();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = sacc[qb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[qb][v]);
      x = fmaxf(x, __builtin_fmaf(mx, scale_log2, -lse2[qb]));
    }
    x = wave_max(x);
    if (lane == 0) red[j & 1][wave] = x;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copy of tile j+2 has landed
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = red[j & 1][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[j & 1][w]);
      trow[j] = __builtin_amdgcn_exp2f(m);
    }
    buf = next;
  }
}

// Common set bits of two tile masks, per (batch, head): the sum over the
// head's query tiles of popcount(a & b) over their words.
// Kept tiles two masks share per (batch, head), and optionally the tile
// recall: that count over the oracle mask's k_hd * nT_hd kept tiles.
__global__ __launch_bounds__(256) void mask_overlap_kernel(GeoTable g, const uint32_t* __restrict__ a,
                                                           const uint32_t* __restrict__ bmask,
                                                           unsigned long long* __restrict__ counts,
                                                           double* __restrict__ recall) {
  const int hd = blockIdx.x, b = blockIdx.y;
  const int32_t nT = g.h[hd].nT;
  const int words = (g.nT_max + 31) / 32;
  const int64_t base = (int64_t(b) * g.heads + hd) * g.nT_max * words;
  unsigned long long c = 0;
  for (int64_t e = threadIdx.x; e < int64_t(nT) * words; e += 256) c += __popc(a[base + e] & bmask[base + e]);
  __shared__ unsigned long long part[256];
  part[threadIdx.x] = c;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (counts) counts[int64_t(b) * g.heads + hd] = part[0];
    if (recall) recall[int64_t(b) * g.heads + hd] = double(part[0]) / (double(g.h[hd].k) * double(nT));
  }
}

}  // namespace

hipError_t launch_teacher(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const float* lse, float scale,
                          float* teacher, int32_t* queue, hipStream_t s) {
  dim3 grid;
  int32_t n_static = 0;
  const hipError_t e = queue_launch(g, queue, &grid, &n_static, s);
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.44269504088896340736f;
  if (g.d == 128)
    teacher_kernel<128><<<grid, kThreads, 0, s>>>(g, q_t, k_t, lse, scale_log2, teacher, queue, n_static);
  else
    teacher_kernel<64><<<grid, kThreads, 0, s>>>(g, q_t, k_t, lse, scale_log2, teacher, queue, n_static);
  return hipGetLastError();
}

hipError_t launch_mask_overlap(const GeoTable& g, const uint32_t* a, const uint32_t* b, unsigned long long* counts,
                               double* recall, hipStream_t s) {
  mask_overlap_kernel<<<dim3(g.heads, g.B), 256, 0, s>>>(g, a, b, counts, recall);
  return hipGetLastError();
}

}  // namespace veda
