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
