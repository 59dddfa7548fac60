// Head-conditioned re-tiling and its inverse (Veda page, "Architecture",
// Principle 02 "Head-Conditioned Tile Geometry"; "Head-Aware Tile Search").
// Tiles are written token-major [.., 128, d] or channel-major [.., d, 128];
// the attention kernel takes V channel-major so its tiles can be copied into
// LDS as they are.
//
// Data movement, bound by HBM bandwidth (the Q/K variant also reduces each
// tile to its TripPool statistics on the way). One workgroup moves one
// 128-token box of one (batch, head): each token row is d bf16 values
// (256 B for d = 128), moved as 16-byte vectors so that every wave touches
// whole 256-byte segments on both sides. All loads of a thread are issued
// before its stores, which keeps 8 (d = 128) vector loads in flight per lane.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;

// Streaming (non-temporal) 16-byte loads and stores: every byte is touched
// once here and the tensors are far larger than L2 and MALL, so nothing is
// gained by keeping them there. Measured on the 245,760-token layer they move
// the gathers 4-10% closer to HBM bandwidth; the channel-major permute keeps
// ordinary loads (its eight-row reads per thread ran slower streamed).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_nt x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  const u32x4_nt x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(p));
}

template <int D>
struct RowMap {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per token row
  static constexpr int kRowsPerPass = kThreads / kChunks;
  static constexpr int kPasses = VEDA_TILE_TOKENS / kRowsPerPass;
};

template <int D>
__global__ __launch_bounds__(kThreads) void tile_permute_kernel(GeoTable g, const uint16_t* __restrict__ x,
                                                               int64_t sb, int64_t sn, int64_t sh,
                                                               uint16_t* __restrict__ xt) {
  using M = RowMap<D>;
  const int32_t tau = blockIdx.x, hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int chunk = threadIdx.x % M::kChunks;
  const int row0 = threadIdx.x / M::kChunks;
  uint4* dst = reinterpret_cast<uint4*>(xt + ((int64_t(b) * g.heads + hd) * g.nT_max + tau) * VEDA_TILE_TOKENS * D);
  uint4 val[M::kPasses];
  if (tau < hg.nT) {
    const BoxExtent e = box_extent(g, hg, tau);
    const uint16_t* src = x + int64_t(b) * sb + int64_t(hd) * sh + chunk * 8;
#pragma unroll
    for (int p = 0; p < M::kPasses; ++p) {
      const int64_t n = raster_of_slot(g, hg, e, row0 + p * M::kRowsPerPass);
      val[p] = n >= 0 ? load_stream(src + n * sn) : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int p = 0; p < M::kPasses; ++p) val[p] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < M::kPasses; ++p) store_stream(&dst[(row0 + p * M::kRowsPerPass) * M::kChunks + chunk], val[p]);
}

// The TripPool statistics of one tile held in LDS (tile_s: 128 slot rows of d
// bf16 values): threads 0..d-1 each sum one channel over the real slots in slot
// order (fp32 from +0, then a correctly rounded divide by the real-token count
// and a round to bf16); threads d..2d-1 take that channel's maximum and
// minimum (IEEE total order, -0 below +0). Writes the tile's 3d statistics.
template <int D>
__device__ __forceinline__ void tile_stats_from_lds(const HeadGeo& hg, const BoxExtent& e, const uint4* tile_s,
                                                    uint16_t* st_out) {
  const int c = threadIdx.x % D;
  const uint16_t* col = reinterpret_cast<const uint16_t*>(tile_s) + c;  // slot s of channel c at col[s * D]
  const bool full = box_is_full(hg, e);
  if (int(threadIdx.x) < D) {
    float sum = 0.0f;
    if (full) {
#pragma unroll 16
      for (int sl = 0; sl < VEDA_TILE_TOKENS; ++sl) sum = sum + bf16_to_f32(col[sl * D]);
    } else {
      for (int sl = 0; sl < VEDA_TILE_TOKENS; ++sl)
        if (slot_is_real(hg, e, sl)) sum = sum + bf16_to_f32(col[sl * D]);
    }
    // sum / n in double then to float is the correctly rounded float quotient
    // (53 >= 2*24 + 2, so the double rounding is innocuous).
    const int32_t n_real = e.vt * e.vh * e.vw;
    st_out[c] = f32_to_bf16_rne(float(double(sum) / double(n_real)));
  } else if (int(threadIdx.x) < 2 * D) {
    int32_t mx = -(1 << 20), mn = 1 << 20;
    if (full) {
#pragma unroll 16
      for (int sl = 0; sl < VEDA_TILE_TOKENS; ++sl) {
        const int32_t key = total_order_key(col[sl * D]);
        mx = max(mx, key);
        mn = min(mn, key);
      }
    } else {
      for (int sl = 0; sl < VEDA_TILE_TOKENS; ++sl) {
        if (!slot_is_real(hg, e, sl)) continue;
        const int32_t key = total_order_key(col[sl * D]);
        mx = max(mx, key);
        mn = min(mn, key);
      }
    }
    st_out[D + c] = from_total_order_key(mx);
    st_out[2 * D + c] = from_total_order_key(mn);
  }
}

// Token-major permute of Q or K fused with the TripPool statistics of each
// tile (Veda page, "Attention Structure Distillation", Estimator: average,
// maximum and minimum per tile; "Theoretical Rationale" 2): the tile is moved
// as above and also kept in LDS, where threads 0..d-1 each sum one channel
// over the real slots in slot order (fp32 from +0, then a correctly rounded
// divide by the real-token count and a round to bf16) and threads d..2d-1
// take that channel's maximum and minimum (IEEE total order, -0 below +0).
// This spares a second pass over the tiled tensor.
template <int D>
__global__ __launch_bounds__(kThreads) void tile_permute_stats_kernel(GeoTable g, const uint16_t* __restrict__ x,
                                                                     int64_t sb, int64_t sn, int64_t sh,
                                                                     uint16_t* __restrict__ xt,
                                                                     uint16_t* __restrict__ stats) {
  using M = RowMap<D>;
  static_assert(2 * D <= kThreads, "one thread per channel and statistic group");
  __shared__ uint4 tile_s[VEDA_TILE_TOKENS * M::kChunks];
  const int32_t tau = blockIdx.x, hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int chunk = threadIdx.x % M::kChunks;
  const int row0 = threadIdx.x / M::kChunks;
  const int64_t tile_row = (int64_t(b) * g.heads + hd) * g.nT_max + tau;
  uint4* dst = xt ? reinterpret_cast<uint4*>(xt + tile_row * VEDA_TILE_TOKENS * D) : nullptr;
  uint16_t* st_out = stats + tile_row * 3 * D;
  if (tau >= hg.nT) {  // tile beyond this head's grid: defined zeros
    if (dst)
#pragma unroll
      for (int p = 0; p < M::kPasses; ++p) dst[(row0 + p * M::kRowsPerPass) * M::kChunks + chunk] = make_uint4(0, 0, 0, 0);
    for (int c = threadIdx.x; c < 3 * D; c += kThreads) st_out[c] = 0;
    return;
  }
  const BoxExtent e = box_extent(g, hg, tau);
  const uint16_t* src = x + int64_t(b) * sb + int64_t(hd) * sh + chunk * 8;
  uint4 val[M::kPasses];
#pragma unroll
  for (int p = 0; p < M::kPasses; ++p) {
    const int64_t n = raster_of_slot(g, hg, e, row0 + p * M::kRowsPerPass);
    val[p] = n >= 0 ? load_stream(src + n * sn) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < M::kPasses; ++p) {
    const int r = row0 + p * M::kRowsPerPass;
    if (dst) store_stream(&dst[r * M::kChunks + chunk], val[p]);
    tile_s[r * M::kChunks + chunk] = val[p];
  }
  __syncthreads();

  tile_stats_from_lds<D>(hg, e, tile_s, st_out);
}

// Statistics only (no tiled copy, as for Q): a workgroup takes kStatTiles
// consecutive tiles of one (batch, head) and loads the next tile's rows into
// registers while the current tile's statistics are taken from LDS, so the
// loads of one tile run under the serial per-channel sums of the previous one.
// The statistics are the same code as above, so the bytes are identical.
constexpr int kStatTiles = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void tile_stats_kernel(GeoTable g, const uint16_t* __restrict__ x, int64_t sb,
                                                             int64_t sn, int64_t sh, uint16_t* __restrict__ stats) {
  using M = RowMap<D>;
  static_assert(2 * D <= kThreads, "one thread per channel and statistic group");
  __shared__ uint4 tile_s[VEDA_TILE_TOKENS * M::kChunks];
  const int hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int chunk = threadIdx.x % M::kChunks;
  const int row0 = threadIdx.x / M::kChunks;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  const uint16_t* src = x + int64_t(b) * sb + int64_t(hd) * sh + chunk * 8;
  const int32_t t0 = blockIdx.x * kStatTiles;
  const int32_t t_end = min(t0 + kStatTiles, g.nT_max);
  uint4 val[M::kPasses];
  auto load = [&](int32_t tau) {  // tau < nT_hd
    const BoxExtent e = box_extent(g, hg, tau);
#pragma unroll
    for (int p = 0; p < M::kPasses; ++p) {
      const int64_t n = raster_of_slot(g, hg, e, row0 + p * M::kRowsPerPass);
      val[p] = n >= 0 ? load_stream(src + n * sn) : make_uint4(0, 0, 0, 0);
    }
  };
  if (t0 < hg.nT) load(t0);
  for (int32_t tau = t0; tau < t_end; ++tau) {
    uint16_t* st_out = stats + (head_row + tau) * 3 * D;
    if (tau >= hg.nT) {  // tile beyond this head's grid: defined zeros
      for (int c = threadIdx.x; c < 3 * D; c += kThreads) st_out[c] = 0;
      continue;
    }
    __syncthreads();  // the previous tile's statistics are done with tile_s
#pragma unroll
    for (int p = 0; p < M::kPasses; ++p) tile_s[(row0 + p * M::kRowsPerPass) * M::kChunks + chunk] = val[p];
    __syncthreads();
    if (tau + 1 < t_end && tau + 1 < hg.nT) load(tau + 1);  // in flight during this tile's statistics
    tile_stats_from_lds<D>(hg, box_extent(g, hg, tau), tile_s, st_out);
  }
}

// Channel-major tiles [.., d, 128]: each thread moves an 8-slot x 8-channel
// block, read as 8 token rows of 16 bytes and written, transposed in
// registers, as 8 channel rows of 16 bytes. Lanes run along the slot groups,
// so each output row (128 slots, 256 bytes) is written by 16 adjacent lanes.
// For d = 128 the tile first goes through LDS so that the reads are whole
// token rows too (16 lanes a row, streaming loads): piece c of slot s sits at
// position c ^ ((s / 8) % 16) of its LDS row, which keeps both the row writes
// and the 8-row reads of a thread's block free of bank conflicts. Measured on
// the 245,760-token layer: 0.951 -> 0.865 ms, the rate of a plain copy.
template <int D>
__global__ __launch_bounds__(kThreads) void tile_permute_cm_kernel(GeoTable g, const uint16_t* __restrict__ x,
                                                                  int64_t sb, int64_t sn, int64_t sh,
                                                                  uint16_t* __restrict__ xt) {
  constexpr int kBlocks = (VEDA_TILE_TOKENS / 8) * (D / 8);
  const int32_t tau = blockIdx.x, hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  if (int(threadIdx.x) >= kBlocks) return;
  const int sg = threadIdx.x % 16, cg = threadIdx.x / 16;
  uint16_t* dst = xt + ((int64_t(b) * g.heads + hd) * g.nT_max + tau) * VEDA_TILE_TOKENS * D;
  uint4 in[8];
  if constexpr (D == 128) {  // every thread of the workgroup has a block, so all reach the barrier
    static_assert(kBlocks == kThreads, "one 8 x 8 block per thread");
    __shared__ uint4 tile_s[VEDA_TILE_TOKENS * 16];
    const int c = threadIdx.x % 16;
    if (tau < hg.nT) {
      const BoxExtent e = box_extent(g, hg, tau);
      const uint16_t* src = x + int64_t(b) * sb + int64_t(hd) * sh + c * 8;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int64_t n = raster_of_slot(g, hg, e, 16 * p + threadIdx.x / 16);
        in[p] = n >= 0 ? load_stream(src + n * sn) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) in[p] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int sl = 16 * p + threadIdx.x / 16;
      tile_s[sl * 16 + (c ^ ((sl >> 3) & 15))] = in[p];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int sl = 8 * sg + r;
      in[r] = tile_s[sl * 16 + (cg ^ ((sl >> 3) & 15))];
    }
  } else if (tau < hg.nT) {
    const BoxExtent e = box_extent(g, hg, tau);
    const uint16_t* src = x + int64_t(b) * sb + int64_t(hd) * sh + cg * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t n = raster_of_slot(g, hg, e, 8 * sg + r);
      in[r] = n >= 0 ? *reinterpret_cast<const uint4*>(src + n * sn) : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) in[r] = make_uint4(0, 0, 0, 0);
  }
  // in[r] holds channels 8cg..8cg+7 of slot 8sg + r; row i of the output is
  // channel 8cg + i over slots 8sg..8sg+7.
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = w[(2 * p) * 4 + i / 2], c = w[(2 * p + 1) * 4 + i / 2];
      o[p] = (i & 1) ? ((a >> 16) | (c & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c << 16));
    }
    store_stream(dst + (8 * cg + i) * VEDA_TILE_TOKENS + 8 * sg, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void tile_unpermute_kernel(GeoTable g, const uint16_t* __restrict__ xt,
                                                                 uint16_t* __restrict__ x, int64_t sb, int64_t sn,
                                                                 int64_t sh) {
  using M = RowMap<D>;
  const int32_t tau = blockIdx.x, hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  if (tau >= hg.nT) return;
  const int chunk = threadIdx.x % M::kChunks;
  const int row0 = threadIdx.x / M::kChunks;
  const uint4* src =
      reinterpret_cast<const uint4*>(xt + ((int64_t(b) * g.heads + hd) * g.nT_max + tau) * VEDA_TILE_TOKENS * D);
  const BoxExtent e = box_extent(g, hg, tau);
  uint4 val[M::kPasses];
#pragma unroll
  for (int p = 0; p < M::kPasses; ++p) val[p] = load_stream(&src[(row0 + p * M::kRowsPerPass) * M::kChunks + chunk]);
  uint16_t* dst = x + int64_t(b) * sb + int64_t(hd) * sh + chunk * 8;
#pragma unroll
  for (int p = 0; p < M::kPasses; ++p) {
    const int64_t n = raster_of_slot(g, hg, e, row0 + p * M::kRowsPerPass);
    if (n >= 0) store_stream(dst + n * sn, val[p]);
  }
}

}  // namespace

hipError_t launch_tile_permute(const GeoTable& g, const uint16_t* x, int64_t sb, int64_t sn, int64_t sh,
                               uint16_t* xt, bool channel_major, hipStream_t s) {
  const dim3 grid(g.nT_max, g.heads, g.B);
  if (channel_major) {
    if (g.d == 128)
      tile_permute_cm_kernel<128><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt);
    else
      tile_permute_cm_kernel<64><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt);
    return hipGetLastError();
  }
  if (g.d == 128)
    tile_permute_kernel<128><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt);
  else
    tile_permute_kernel<64><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt);
  return hipGetLastError();
}

hipError_t launch_tile_permute_stats(const GeoTable& g, const uint16_t* x, int64_t sb, int64_t sn, int64_t sh,
                                     uint16_t* xt, uint16_t* stats, hipStream_t s) {
  if (!xt) {  // statistics only
    const dim3 grid((g.nT_max + kStatTiles - 1) / kStatTiles, g.heads, g.B);
    if (g.d == 128)
      tile_stats_kernel<128><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, stats);
    else
      tile_stats_kernel<64><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, stats);
    return hipGetLastError();
  }
  const dim3 grid(g.nT_max, g.heads, g.B);
  if (g.d == 128)
    tile_permute_stats_kernel<128><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt, stats);
  else
    tile_permute_stats_kernel<64><<<grid, kThreads, 0, s>>>(g, x, sb, sn, sh, xt, stats);
  return hipGetLastError();
}

hipError_t launch_tile_unpermute(const GeoTable& g, const uint16_t* xt, uint16_t* x, int64_t sb, int64_t sn,
                                 int64_t sh, hipStream_t s) {
  const dim3 grid(g.nT_max, g.heads, g.B);
  if (g.d == 128)
    tile_unpermute_kernel<128><<<grid, kThreads, 0, s>>>(g, xt, x, sb, sn, sh);
  else
    tile_unpermute_kernel<64><<<grid, kThreads, 0, s>>>(g, xt, x, sb, sn, sh);
  return hipGetLastError();
}

}  // namespace veda
