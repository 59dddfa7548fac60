// Internal declarations shared by the HIP translation units of libveda.
// Geometry travels to kernels by value (kernel arguments), so kernels need
// no device-side tables and the library holds no device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/veda.h"

namespace veda {

// Per-head tiling: edges are powers of two (their product is 128), stored as
// log2; whether every box is full (each grid edge a multiple of the tile
// edge: no pad slots anywhere); box counts along h and w; total boxes; kept
// tiles per query tile.
struct HeadGeo {
  uint8_t lpt, lph, lpw, all_full;
  int32_t nTh, nTw, nT, k;
};

// Counters of the attention work queue (int32 words of its workspace).
constexpr int kAttnQueueInts = VEDA_ATTN_QUEUE_BYTES / 4;

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

#define VEDA_HD __host__ __device__ __forceinline__

VEDA_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
VEDA_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

VEDA_HD BoxExtent box_extent(const GeoTable& g, const HeadGeo& hg, int32_t tau) {
  const int32_t pt = 1 << hg.lpt, ph = 1 << hg.lph, pw = 1 << hg.lpw;
  const int32_t bx = tau % hg.nTw;
  const int32_t rest = tau / hg.nTw;
  const int32_t by = rest % hg.nTh;
  const int32_t bt = rest / hg.nTh;
  BoxExtent e;
  e.t0 = bt * pt;
  e.y0 = by * ph;
  e.x0 = bx * pw;
  e.vt = imin(pt, g.T - e.t0);
  e.vh = imin(ph, g.H - e.y0);
  e.vw = imin(pw, g.W - e.x0);
  return e;
}

VEDA_HD bool box_is_full(const HeadGeo& hg, const BoxExtent& e) {
  return e.vt == (1 << hg.lpt) && e.vh == (1 << hg.lph) && e.vw == (1 << hg.lpw);
}

// Slot sigma of a box is real iff each of its offsets lies inside the real extent.
VEDA_HD bool slot_is_real(const HeadGeo& hg, const BoxExtent& e, int32_t sigma) {
  const int32_t sx = sigma & ((1 << hg.lpw) - 1);
  const int32_t sy = (sigma >> hg.lpw) & ((1 << hg.lph) - 1);
  const int32_t st = sigma >> (hg.lpw + hg.lph);
  return st < e.vt && sy < e.vh && sx < e.vw;
}

// Raster index n = (t*H + y)*W + x of slot sigma of a box, or -1 for a pad slot.
VEDA_HD int64_t raster_of_slot(const GeoTable& g, const HeadGeo& hg, const BoxExtent& e, int32_t sigma) {
  if (!slot_is_real(hg, e, sigma)) return -1;
  const int32_t sx = sigma & ((1 << hg.lpw) - 1);
  const int32_t sy = (sigma >> hg.lpw) & ((1 << hg.lph) - 1);
  const int32_t st = sigma >> (hg.lpw + hg.lph);
  return (int64_t(e.t0 + st) * g.H + (e.y0 + sy)) * g.W + (e.x0 + sx);
}

// 64 bits of a periodic slot pattern: bit b (slot base + b) is set iff
// (slot mod 2^lg_period) < lim. Slots are numbered 0..127 inside a box.
VEDA_HD uint64_t periodic_slot_bits(int lg_period, int lim, int base) {
  if (lg_period >= 6) {  // period 64 or 128: the condition is a plain prefix
    const int n = imin(imax(lim - (lg_period == 7 ? base : 0), 0), 64);
    return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
  }
  const int period = 1 << lg_period;
  uint64_t w = lim >= period ? ((1ull << period) - 1ull) : ((1ull << lim) - 1ull);
  for (int p = period; p < 64; p <<= 1) w |= w << p;
  return w;
}

// Bits base..base+63 of the box's real-slot mask (bit sigma set iff slot sigma
// holds a real token): x offset < vw, y offset < vh and t offset < vt.
VEDA_HD uint64_t box_slot_mask64(const HeadGeo& hg, const BoxExtent& e, int base) {
  const int lxy = hg.lpw + hg.lph;
  return periodic_slot_bits(hg.lpw, e.vw, base) & periodic_slot_bits(lxy, e.vh << hg.lpw, base) &
         periodic_slot_bits(7, e.vt << lxy, base);
}

// bf16 <-> fp32 (round to nearest even; inputs here are always finite).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Order-preserving integer key of a bf16 value in the IEEE total order (-0 < +0).
__device__ __forceinline__ int32_t total_order_key(uint32_t b) {
  const int32_t mag = int32_t(b & 0x7FFFu);
  return (b & 0x8000u) ? -mag - 1 : mag;
}
__device__ __forceinline__ uint16_t from_total_order_key(int32_t k) {
  return k >= 0 ? uint16_t(k) : uint16_t(0x8000u | uint32_t(-k - 1));
}

// Host-side launchers, one per kernel family (each defined next to its kernel).
hipError_t launch_tile_permute(const GeoTable& g, const uint16_t* x, int64_t sb, int64_t sn, int64_t sh,
                               uint16_t* xt, bool channel_major, hipStream_t s);
hipError_t launch_tile_permute_stats(const GeoTable& g, const uint16_t* x, int64_t sb, int64_t sn, int64_t sh,
                                     uint16_t* xt, uint16_t* stats, hipStream_t s);
hipError_t launch_tile_unpermute(const GeoTable& g, const uint16_t* xt, uint16_t* x, int64_t sb, int64_t sn,
                                 int64_t sh, hipStream_t s);
hipError_t launch_trippool_features(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t,
                                    const uint16_t* wq, const uint16_t* wk, int32_t r, uint16_t* stats_q,
                                    uint16_t* stats_k, uint16_t* feat_q, uint16_t* feat_k, hipStream_t s);
hipError_t launch_trippool_project(const GeoTable& g, const uint16_t* stats_q, const uint16_t* stats_k,
                                   const uint16_t* wq, const uint16_t* wk, int32_t r, uint16_t* feat_q,
                                   uint16_t* feat_k, hipStream_t s);
hipError_t launch_tile_scores(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                              float* scores, hipStream_t s);
hipError_t launch_tile_scores_mfma(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                                   float* scores, hipStream_t s);
hipError_t launch_avgpool_scores(const GeoTable& g, const uint16_t* stats_q, const uint16_t* stats_k, float* scores,
                                 hipStream_t s);
constexpr int kScoreTopkMaxTiles = 2048;   // key tiles per row the fused score + Top-k pass holds in LDS
hipError_t launch_score_topk(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                             int32_t k_max, int32_t* idx, uint32_t* bitmask, hipStream_t s);
hipError_t launch_topk(const GeoTable& g, const float* scores, int32_t k_max, int32_t* idx, uint32_t* bitmask,
                       hipStream_t s);
hipError_t launch_teacher(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const float* lse, float scale,
                          float* teacher, int32_t* queue, hipStream_t s);
hipError_t launch_mask_overlap(const GeoTable& g, const uint32_t* a, const uint32_t* b, unsigned long long* counts,
                               double* recall, hipStream_t s);
hipError_t launch_search_select(int32_t n_cand, int32_t B, int32_t heads, const double* err, double* err_sum,
                                int32_t* best, hipStream_t s);
hipError_t launch_distill_mean(const GeoTable& g, const float* kl_rows, double* mean, hipStream_t s);
hipError_t launch_head_sq_error(const GeoTable& g, const uint16_t* a, int64_t sab, int64_t san, int64_t sah,
                                const uint16_t* b, int64_t sbb, int64_t sbn, int64_t sbh, double* err,
                                hipStream_t s);
hipError_t launch_distill_kl(const GeoTable& g, const float* scores, const float* teacher, float grad_scale,
                             float* kl_rows, float* d_scores, hipStream_t s);
hipError_t launch_distill_grad(const GeoTable& g, int32_t r, const uint16_t* stats_q, const uint16_t* stats_k,
                               const uint16_t* feat_q, const uint16_t* feat_k, const float* d_scores,
                               float* d_feat_q, float* d_feat_k, float* d_wq, float* d_wk, hipStream_t s);
hipError_t launch_adam(int64_t n, float* w, const float* grad, float* m, float* v, float lr, float beta1, float beta2,
                       float eps, float bc1, float bc2, uint16_t* w_bf16, hipStream_t s);
// O goes to o_t (tiled) when o_r is null, else straight to raster o_r with
// element strides (osb, osn, osh).
// Address, on the current device, of the static work queue used by the
// allocation-free attention call (looked up once per device).
hipError_t attn_scratch_queue(int32_t** queue);
// Attention forward; idx == nullptr runs the dense kernel (every key tile of
// the head, in order; the table's k_hd must then be nT_hd).
hipError_t launch_sparse_attn(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const uint16_t* v_t,
                              const int32_t* idx, int32_t k_max, float scale, uint16_t* o_t, float* lse,
                              uint16_t* o_r, int64_t osb, int64_t osn, int64_t osh, const uint16_t* q_r,
                              int64_t qsb, int64_t qsn, int64_t qsh, int32_t* queue, hipStream_t s);

}  // namespace veda
