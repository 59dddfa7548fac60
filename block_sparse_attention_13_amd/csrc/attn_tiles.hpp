// Tile-level building blocks shared by the attention kernels (the
// tile-skipping forward and the max-pooled dense teacher): vector types, the
// 8-wave decomposition of a 128-query tile, the LDS-DMA copy, the swizzled K
// fragment read that feeds the S^T MFMA, and the pad-key mask of a box.
//
// Eight waves share a 128-query tile: wave (qg, half) owns queries
// 32qg..32qg+31 and keys 64half..64half+63 of every key tile. K tiles sit in
// LDS as 128 rows of D bf16 values whose 16-byte pieces are XOR-swizzled
// (piece c of row r at position c ^ (r mod positions-per-row, at most 16)),
// which keeps the MFMA operand reads free of bank conflicts.
#pragma once

#include "veda_internal.hpp"

namespace veda {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;           // 8 waves: 4 query groups x 2 key halves
constexpr int kWaves = kThreads / 64;
constexpr int kTok = VEDA_TILE_TOKENS;  // 128 keys / queries per tile

template <int D>
struct AttnShape {
  static constexpr int kTileElems = kTok * D;           // one K or V tile (bf16 elements)
  static constexpr int kKPos = D / 8;                   // 16-byte positions per K row
  static constexpr int kKRowsPerChunk = 64 / kKPos;     // K rows per 1-KiB DMA chunk
  static constexpr int kChunks = kTileElems / 512;      // 1-KiB chunks per tile (K or V)
  static constexpr int kChunksPerWave = 2 * kChunks / kWaves;
  static constexpr int kDC = D / 16;                    // MFMA k-steps over the head dim
  static constexpr int kDB = D / 32;                    // 32-row blocks of O^T
  static_assert(kChunks % (kWaves / 2) == 0, "K and V chunks split over 4 waves each");
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Key row fed by lane l of a 32-key block: bits 2 and 3 of l swapped.
__device__ __forceinline__ int key_perm(int l) { return (l & ~12) | ((l & 4) << 1) | ((l & 8) >> 1); }

// Query tile handled by workgroup x of a head: the tiles of a head are split
// into 8 contiguous runs, run r going to the workgroups x with x % 8 == r
// (consecutive workgroups land on consecutive XCDs). Bijective for any n.
__device__ __forceinline__ int32_t xcd_tile_order(int32_t x, int32_t n) {
  const int32_t xcd = x % 8, pos = x / 8, q = n / 8, r = n % 8;
  return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

// Work queue. Under the power limit the XCDs run at different clocks, so a
// fixed deal of query tiles leaves the fastest XCDs idle while the slowest
// finishes. Work items are the linear indices bx + nT_max (hd + heads b) of
// a (nT_max, heads, B) grid. Queue x (x < 8) holds items x, x + 8, x + 16,
// ...: those a grid of that shape deals to XCD x, since workgroups go to the
// XCDs round robin. In the one-dimensional queue grid workgroup i is taken to
// sit on XCD i % 8 (only locality rests on this) and, for i / 8 < n_static,
// simply does item 8 (i / 8) + i % 8. Any other workgroup draws a ticket from
// counter 8; a ticket below the number of remaining items guarantees that an
// item is left somewhere, so it takes the next item of its own queue
// (counter x counts the draws past n_static from queue x) or else of the
// next queues in turn, and one pass finds it: a queue once exhausted stays
// exhausted. Workgroups with a ticket past the end have no item.
//
// Sets (bx, hd, b) and returns true, or returns false for no item. Without a
// queue the item is the workgroup's own grid position. `word` is LDS scratch
// for the broadcast; it must lie inside the kernel's tile buffers (a second
// LDS object makes the compiler wait for every LDS-DMA before each LDS read)
// and is free again when this returns.
__device__ __forceinline__ bool work_item(const GeoTable& g, int32_t* queue, int32_t n_static, int32_t* word,
                                          int32_t* bx, int32_t* hd, int32_t* b) {
  if (!queue) {
    *bx = blockIdx.x;
    *hd = blockIdx.y;
    *b = blockIdx.z;
    return true;
  }
  const int32_t total = g.nT_max * g.heads * g.B;
  const int home = blockIdx.x % 8;
  const int32_t n = blockIdx.x / 8;
  int32_t item = 8 * n + home;
  if (n >= n_static) {
    if (threadIdx.x == 0) {
      int32_t got = -1;
      if (atomicAdd(&queue[8], 1) < total - 8 * n_static) {
        for (int t = 0; t < 8; ++t) {
          const int x = (home + t) % 8;
          const int32_t m = n_static + atomicAdd(&queue[x], 1);
          if (m < (total - x + 7) / 8) {
            got = 8 * m + x;
            break;
          }
        }
      }
      *word = got;
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(*word);
    __syncthreads();  // every wave has read the word before the tile copies overwrite it
    if (item < 0) return false;
  }
  *bx = item % g.nT_max;
  *hd = (item / g.nT_max) % g.heads;
  *b = item / (g.nT_max * g.heads);
  return true;
}

namespace {

__global__ void queue_reset_kernel(int32_t* queue) {
  if (threadIdx.x < kAttnQueueInts) queue[threadIdx.x] = 0;
}

// Launch shape of a kernel over (nT_max, heads, B) query tiles: that grid
// without a queue, or the one-dimensional queue grid, after a one-workgroup
// kernel has cleared the counters on the stream (a kernel, not a memset, so
// the call can be captured in a graph). The last sixteenth of each XCD's
// share is handed out at run time, and each XCD has workgroups for a further
// sixteenth taken from the others (enough for clocks about 12% apart). A
// grid of fewer than 1024 tiles (4 per CU) has no tail worth balancing and
// does not use (or clear) the queue.
hipError_t queue_launch(const GeoTable& g, int32_t*& queue, dim3* grid, int32_t* n_static, hipStream_t s) {
  const int64_t total = int64_t(g.nT_max) * g.heads * g.B;
  *grid = dim3(g.nT_max, g.heads, g.B);
  *n_static = 0;
  if (total < 1024) queue = nullptr;
  if (!queue) return hipSuccess;
  const int32_t per = int32_t(total / 8), per_max = int32_t((total + 7) / 8);
  *n_static = per - per / 16;
  *grid = dim3(8 * (per_max + per / 16 + 1), 1, 1);
  queue_reset_kernel<<<1, 64, 0, s>>>(queue);
  return hipGetLastError();
}

}  // namespace

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// One 1-KiB LDS-DMA copy: lane l loads 16 bytes at byte tile_bytes + voff
// of a raw buffer over [base, base + bytes) (stride 0; reads past the end
// would return 0) into LDS bytes 16l..16l+15 of dst.
__device__ __forceinline__ void dma_copy(const uint16_t* base, int32_t bytes, uint32_t voff, uint32_t tile_bytes,
                                         lds_u16* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, tile_bytes, 0, 0);
}

// Real-key bits of this wave's 64 keys of tile j, shifted so bit
// 16(v/8) + 4((v/4)%2) + v%4 (+32 for kb = 1) is S^T element v of block kb;
// 0 for an index outside the head (the tile then contributes nothing).
__device__ __forceinline__ uint64_t real_key_bits(const GeoTable& g, const HeadGeo& hg, int32_t j, int half, int h) {
  if (unsigned(j) >= unsigned(hg.nT)) return 0ull;
  if (hg.all_full) return ~0ull;
  const BoxExtent e = box_extent(g, hg, j);
  if (box_is_full(hg, e)) return ~0ull;
  return box_slot_mask64(hg, e, 64 * half) >> (8 * h);
}

// K fragment of S^T step t (block kb = t / kDC, k-step dc = t % kDC) for
// this lane: 16 bytes of key row 64half + 32kb + pi(l32), channels
// 16dc + 8h .. +7, at its swizzled position.
template <int D>
__device__ __forceinline__ u32x4 k_frag(const uint16_t* ks, int t, int half, int h, int l32) {
  using S = AttnShape<D>;
  const int kb = t / S::kDC, dc = t % S::kDC;
  const int r = 64 * half + 32 * kb + key_perm(l32);
  return *reinterpret_cast<const u32x4*>(ks + r * D + (((2 * dc + h) ^ (r & (S::kKPos - 1))) * 8));
}

}  // namespace attn
}  // namespace veda
