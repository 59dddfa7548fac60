// Internal declarations shared by the HIP translation units of libveda.
// Geometry travels to kernels by value (kernel arguments), so kernels need
// no device-side tables and the library holds no device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/veda.h"

namespace veda {

// Per-head tiling: edges are powers of two (their product is 128), stored as
// log2; box counts along h and w; total boxes; kept tiles per query tile.
struct HeadGeo {
  uint8_t lpt, lph, lpw, pad_;
  int32_t nTh, nTw, nT, k;
};

struct GeoTable {
  int32_t B, heads, d, T, H, W, nT_max;
  HeadGeo h[VEDA_MAX_HEADS];
};

// Decoded position of a box and the number of real tokens along each of its
// axes (smaller than the edge only for boxes on the padded border).
struct BoxExtent {
  int32_t t0, y0, x0;  // grid coordinates of the box origin
  int32_t vt, vh, vw;  // real extent along t, y, x
};

__device__ __forceinline__ BoxExtent box_extent(const GeoTable& g, const HeadGeo& hg, int32_t tau) {
  const int32_t pt = 1 << hg.lpt, ph = 1 << hg.lph, pw = 1 << hg.lpw;
  const int32_t bx = tau % hg.nTw;
  const int32_t rest = tau / hg.nTw;
  const int32_t by = rest % hg.nTh;
  const int32_t bt = rest / hg.nTh;
  BoxExtent e;
  e.t0 = bt * pt;
  e.y0 = by * ph;
  e.x0 = bx * pw;
  e.vt = min(pt, g.T - e.t0);
  e.vh = min(ph, g.H - e.y0);
  e.vw = min(pw, g.W - e.x0);
  return e;
}

__device__ __forceinline__ bool box_is_full(const HeadGeo& hg, const BoxExtent& e) {
  return e.vt == (1 << hg.lpt) && e.vh == (1 << hg.lph) && e.vw == (1 << hg.lpw);
}

// Slot sigma of a box is real iff each of its offsets lies inside the real extent.
__device__ __forceinline__ bool slot_is_real(const HeadGeo& hg, const BoxExtent& e, int32_t sigma) {
  const int32_t sx = sigma & ((1 << hg.lpw) - 1);
  const int32_t sy = (sigma >> hg.lpw) & ((1 << hg.lph) - 1);
  const int32_t st = sigma >> (hg.lpw + hg.lph);
  return st < e.vt && sy < e.vh && sx < e.vw;
}

// bf16 <-> fp32 (round to nearest even; inputs here are always finite).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Host-side launchers, one per kernel family (each defined next to its kernel).
hipError_t launch_tile_permute(const GeoTable& g, const uint16_t* x, int64_t sb, int64_t sn, int64_t sh,
                               uint16_t* xt, hipStream_t s);
hipError_t launch_tile_unpermute(const GeoTable& g, const uint16_t* xt, uint16_t* x, int64_t sb, int64_t sn,
                                 int64_t sh, hipStream_t s);
hipError_t launch_trippool_features(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t,
                                    const uint16_t* wq, const uint16_t* wk, int32_t r, uint16_t* stats_q,
                                    uint16_t* stats_k, uint16_t* feat_q, uint16_t* feat_k, hipStream_t s);
hipError_t launch_tile_scores(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                              float* scores, hipStream_t s);
hipError_t launch_topk(const GeoTable& g, const float* scores, int32_t k_max, int32_t* idx, uint32_t* bitmask,
                       hipStream_t s);
hipError_t launch_sparse_attn(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const uint16_t* v_t,
                              const int32_t* idx, int32_t k_max, float scale, uint16_t* o_t, float* lse,
                              hipStream_t s);

}  // namespace veda
