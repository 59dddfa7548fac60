// C ABI of libveda: argument validation, per-head geometry tables and kernel
// launches. Every argument check runs on the host before any HIP call, so an
// invalid call enqueues nothing and writes nothing. The library allocates no
// device memory; the only process-wide state is a per-device cache of the
// architecture check and, for the allocation-free attention call, of the
// address of its static work queue on each device.
#include <atomic>
#include <cmath>
#include <cstring>

#include "veda_internal.hpp"

namespace {

using veda::GeoTable;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int build_table(const veda_geom* g, GeoTable* t) {
  if (!g || !g->head_tile) return VEDA_ERR_NULL;
  if (g->B <= 0 || g->n_heads <= 0 || g->n_heads > VEDA_MAX_HEADS) return VEDA_ERR_SHAPE;
  if (g->head_dim != 64 && g->head_dim != 128) return VEDA_ERR_SHAPE;
  if (g->grid.T <= 0 || g->grid.H <= 0 || g->grid.W <= 0) return VEDA_ERR_SHAPE;
  if (g->B > 65535) return VEDA_ERR_SHAPE;
  std::memset(t, 0, sizeof(*t));
  t->B = g->B;
  t->heads = g->n_heads;
  t->d = g->head_dim;
  t->T = g->grid.T;
  t->H = g->grid.H;
  t->W = g->grid.W;
  int64_t nT_max = 0;
  for (int hd = 0; hd < g->n_heads; ++hd) {
    const veda_tile tl = g->head_tile[hd];
    if (tl.pt <= 0 || tl.ph <= 0 || tl.pw <= 0) return VEDA_ERR_TILE;
    if (int64_t(tl.pt) * tl.ph * tl.pw != VEDA_TILE_TOKENS) return VEDA_ERR_TILE;
    // Each edge divides 128, so it is a power of two.
    veda::HeadGeo& h = t->h[hd];
    h.lpt = uint8_t(__builtin_ctz(unsigned(tl.pt)));
    h.lph = uint8_t(__builtin_ctz(unsigned(tl.ph)));
    h.lpw = uint8_t(__builtin_ctz(unsigned(tl.pw)));
    h.all_full = uint8_t(g->grid.T % tl.pt == 0 && g->grid.H % tl.ph == 0 && g->grid.W % tl.pw == 0);
    const int64_t nTt = (int64_t(g->grid.T) + tl.pt - 1) / tl.pt;
    const int64_t nTh = (int64_t(g->grid.H) + tl.ph - 1) / tl.ph;
    const int64_t nTw = (int64_t(g->grid.W) + tl.pw - 1) / tl.pw;
    const int64_t nT = nTt * nTh * nTw;
    if (nT > VEDA_MAX_TILES) return VEDA_ERR_SHAPE;
    h.nTh = int32_t(nTh);
    h.nTw = int32_t(nTw);
    h.nT = int32_t(nT);
    h.k = 0;
    if (nT > nT_max) nT_max = nT;
  }
  t->nT_max = int32_t(nT_max);
  return VEDA_OK;
}

int set_k(const int32_t* k_per_head, int32_t k_max, GeoTable* t) {
  if (!k_per_head) return VEDA_ERR_NULL;
  if (k_max <= 0 || k_max > t->nT_max) return VEDA_ERR_K;
  for (int hd = 0; hd < t->heads; ++hd) {
    const int32_t k = k_per_head[hd];
    if (k < 1 || k > t->h[hd].nT || k > k_max) return VEDA_ERR_K;
    t->h[hd].k = k;
  }
  return VEDA_OK;
}

int check_strides(const veda_raster_strides& s) {
  if (s.b % 8 || s.n % 8 || s.h % 8) return VEDA_ERR_ALIGN;
  if (s.b < 0 || s.n < 0 || s.h < 0) return VEDA_ERR_SHAPE;
  return VEDA_OK;
}

// The current device must be a gfx950 (MI355X class). Cached per device id.
int check_device() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 ok, -1 not gfx950
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return VEDA_ERR_DEVICE;
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) {
      (void)hipGetLastError();  // clear a stale error so launch checks see only ours
      return c > 0 ? VEDA_OK : VEDA_ERR_DEVICE;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return VEDA_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? VEDA_OK : VEDA_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? VEDA_OK : VEDA_ERR_LAUNCH; }

#define VEDA_TRY(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != VEDA_OK) return rc_; \
  } while (0)

// The attention work queue: 16-byte aligned, and every item index (up to
// B * heads * nT_max) and the launch size stay far inside int32.
int check_queue(const GeoTable& t, const int32_t* queue) {
  if (!queue) return VEDA_OK;
  if (!aligned16(queue)) return VEDA_ERR_ALIGN;
  if (int64_t(t.B) * t.heads * t.nT_max > (int64_t(1) << 28)) return VEDA_ERR_SHAPE;
  return VEDA_OK;
}

}  // namespace

extern "C" {

const char* veda_status_str(int status) {
  switch (status) {
    case VEDA_OK: return "ok";
    case VEDA_ERR_NULL: return "null pointer argument";
    case VEDA_ERR_SHAPE: return "shape out of range";
    case VEDA_ERR_TILE: return "tile volume is not 128";
    case VEDA_ERR_K: return "k outside [1, tiles of the head] or above k_max";
    case VEDA_ERR_ALIGN: return "pointer not 16-byte aligned or stride not a multiple of 8";
    case VEDA_ERR_DEVICE: return "no gfx950 HIP device current";
    case VEDA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int veda_num_tiles(const veda_geom* g, int32_t head) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (head < 0 || head >= t.heads) return VEDA_ERR_SHAPE;
  return t.h[head].nT;
}

int veda_max_tiles(const veda_geom* g) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  return t.nT_max;
}

int veda_tile_permute(const veda_geom* g, const void* x_raster, veda_raster_strides s, void* x_tiled,
                      int32_t layout, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!x_raster || !x_tiled) return VEDA_ERR_NULL;
  if (layout != VEDA_TILED_TOKEN_MAJOR && layout != VEDA_TILED_CHANNEL_MAJOR) return VEDA_ERR_SHAPE;
  if (!aligned16(x_raster) || !aligned16(x_tiled)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_strides(s));
  VEDA_TRY(check_device());
  return launched(veda::launch_tile_permute(t, static_cast<const uint16_t*>(x_raster), s.b, s.n, s.h,
                                            static_cast<uint16_t*>(x_tiled), layout == VEDA_TILED_CHANNEL_MAJOR,
                                            static_cast<hipStream_t>(stream)));
}

int veda_tile_permute_stats(const veda_geom* g, const void* x_raster, veda_raster_strides s, void* x_tiled,
                            void* stats, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!x_raster || !stats) return VEDA_ERR_NULL;
  if (!aligned16(x_raster) || (x_tiled && !aligned16(x_tiled)) || !aligned16(stats)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_strides(s));
  VEDA_TRY(check_device());
  return launched(veda::launch_tile_permute_stats(t, static_cast<const uint16_t*>(x_raster), s.b, s.n, s.h,
                                                  static_cast<uint16_t*>(x_tiled), static_cast<uint16_t*>(stats),
                                                  static_cast<hipStream_t>(stream)));
}

int veda_tile_unpermute(const veda_geom* g, const void* x_tiled, void* x_raster, veda_raster_strides s,
                        void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!x_raster || !x_tiled) return VEDA_ERR_NULL;
  if (!aligned16(x_raster) || !aligned16(x_tiled)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_strides(s));
  VEDA_TRY(check_device());
  return launched(veda::launch_tile_unpermute(t, static_cast<const uint16_t*>(x_tiled),
                                              static_cast<uint16_t*>(x_raster), s.b, s.n, s.h,
                                              static_cast<hipStream_t>(stream)));
}

int veda_trippool_score(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* w_q,
                        const void* w_k, int32_t rank, void* stats_q, void* stats_k, void* feat_q, void* feat_k,
                        float* scores, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !w_q || !w_k || !stats_q || !stats_k || !feat_q || !feat_k || !scores)
    return VEDA_ERR_NULL;
  if (rank != 32 && rank != 64) return VEDA_ERR_SHAPE;
  for (const void* p : {q_tiled, k_tiled, w_q, w_k, static_cast<const void*>(stats_q),
                        static_cast<const void*>(stats_k), static_cast<const void*>(feat_q),
                        static_cast<const void*>(feat_k), static_cast<const void*>(scores)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  const hipStream_t st = static_cast<hipStream_t>(stream);
  VEDA_TRY(launched(veda::launch_trippool_features(
      t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
      static_cast<const uint16_t*>(w_q), static_cast<const uint16_t*>(w_k), rank, static_cast<uint16_t*>(stats_q),
      static_cast<uint16_t*>(stats_k), static_cast<uint16_t*>(feat_q), static_cast<uint16_t*>(feat_k), st)));
  return launched(veda::launch_tile_scores(t, static_cast<const uint16_t*>(feat_q),
                                           static_cast<const uint16_t*>(feat_k), rank, scores, st));
}

int veda_trippool_project_score(const veda_geom* g, const void* stats_q, const void* stats_k, const void* w_q,
                                const void* w_k, int32_t rank, void* feat_q, void* feat_k, float* scores,
                                void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!stats_q || !stats_k || !w_q || !w_k || !feat_q || !feat_k) return VEDA_ERR_NULL;
  if (rank != 32 && rank != 64) return VEDA_ERR_SHAPE;
  for (const void* p : {stats_q, stats_k, w_q, w_k, static_cast<const void*>(feat_q),
                        static_cast<const void*>(feat_k)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (scores && !aligned16(scores)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  const hipStream_t st = static_cast<hipStream_t>(stream);
  VEDA_TRY(launched(veda::launch_trippool_project(
      t, static_cast<const uint16_t*>(stats_q), static_cast<const uint16_t*>(stats_k),
      static_cast<const uint16_t*>(w_q), static_cast<const uint16_t*>(w_k), rank, static_cast<uint16_t*>(feat_q),
      static_cast<uint16_t*>(feat_k), st)));
  if (!scores) return VEDA_OK;  // features only (the fused score + Top-k call takes them from here)
  return launched(veda::launch_tile_scores(t, static_cast<const uint16_t*>(feat_q),
                                           static_cast<const uint16_t*>(feat_k), rank, scores, st));
}

int veda_tile_scores_mfma(const veda_geom* g, const void* feat_q, const void* feat_k, int32_t rank, float* scores,
                          void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!feat_q || !feat_k || !scores) return VEDA_ERR_NULL;
  if (rank != 32 && rank != 64) return VEDA_ERR_SHAPE;
  for (const void* p : {feat_q, feat_k, static_cast<const void*>(scores)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_tile_scores_mfma(t, static_cast<const uint16_t*>(feat_q),
                                                static_cast<const uint16_t*>(feat_k), rank, scores,
                                                static_cast<hipStream_t>(stream)));
}

int veda_avgpool_score(const veda_geom* g, const void* stats_q, const void* stats_k, float* scores, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!stats_q || !stats_k || !scores) return VEDA_ERR_NULL;
  for (const void* p : {stats_q, stats_k, static_cast<const void*>(scores)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_avgpool_scores(t, static_cast<const uint16_t*>(stats_q),
                                              static_cast<const uint16_t*>(stats_k), scores,
                                              static_cast<hipStream_t>(stream)));
}

int veda_topk_mask(const veda_geom* g, const float* scores, const int32_t* k_per_head, int32_t k_max,
                   int32_t* idx, uint32_t* bitmask, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!scores || !idx) return VEDA_ERR_NULL;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  if (!aligned16(scores) || !aligned16(idx) || (bitmask && !aligned16(bitmask))) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_topk(t, scores, k_max, idx, bitmask, static_cast<hipStream_t>(stream)));
}

int veda_score_topk(const veda_geom* g, const void* feat_q, const void* feat_k, int32_t rank,
                    const int32_t* k_per_head, int32_t k_max, int32_t* idx, uint32_t* bitmask, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!feat_q || !feat_k || !idx) return VEDA_ERR_NULL;
  if (rank != 32 && rank != 64) return VEDA_ERR_SHAPE;
  if (t.nT_max > veda::kScoreTopkMaxTiles) return VEDA_ERR_SHAPE;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  if (!aligned16(feat_q) || !aligned16(feat_k) || !aligned16(idx) || (bitmask && !aligned16(bitmask)))
    return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_score_topk(t, static_cast<const uint16_t*>(feat_q),
                                          static_cast<const uint16_t*>(feat_k), rank, k_max, idx, bitmask,
                                          static_cast<hipStream_t>(stream)));
}

int veda_sparse_attn_fwd(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                         const int32_t* idx, const int32_t* k_per_head, int32_t k_max, float softmax_scale,
                         void* o_tiled, float* lse, int32_t* work_queue, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !v_tiled || !idx || !o_tiled) return VEDA_ERR_NULL;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  for (const void* p : {q_tiled, k_tiled, v_tiled, static_cast<const void*>(idx), static_cast<const void*>(o_tiled)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_sparse_attn(
      t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
      static_cast<const uint16_t*>(v_tiled), idx, k_max, softmax_scale, static_cast<uint16_t*>(o_tiled), lse,
      nullptr, 0, 0, 0, nullptr, 0, 0, 0, work_queue, static_cast<hipStream_t>(stream)));
}

int veda_sparse_attn_fwd_raster(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                                const int32_t* idx, const int32_t* k_per_head, int32_t k_max, float softmax_scale,
                                void* o_raster, veda_raster_strides s, float* lse, int32_t* work_queue,
                                void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !v_tiled || !idx || !o_raster) return VEDA_ERR_NULL;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  for (const void* p : {q_tiled, k_tiled, v_tiled, static_cast<const void*>(idx), static_cast<const void*>(o_raster)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  VEDA_TRY(check_strides(s));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_sparse_attn(
      t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
      static_cast<const uint16_t*>(v_tiled), idx, k_max, softmax_scale, nullptr, lse,
      static_cast<uint16_t*>(o_raster), s.b, s.n, s.h, nullptr, 0, 0, 0, work_queue, static_cast<hipStream_t>(stream)));
}

int veda_sparse_attn_fwd_raster_io(const veda_geom* g, const void* q_raster, veda_raster_strides sq,
                                   const void* k_tiled, const void* v_tiled, const int32_t* idx,
                                   const int32_t* k_per_head, int32_t k_max, float softmax_scale, void* o_raster,
                                   veda_raster_strides so, float* lse, int32_t* work_queue, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_raster || !k_tiled || !v_tiled || !idx || !o_raster) return VEDA_ERR_NULL;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  for (const void* p : {q_raster, k_tiled, v_tiled, static_cast<const void*>(idx), static_cast<const void*>(o_raster)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  VEDA_TRY(check_strides(sq));
  VEDA_TRY(check_strides(so));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_sparse_attn(
      t, nullptr, static_cast<const uint16_t*>(k_tiled), static_cast<const uint16_t*>(v_tiled), idx, k_max,
      softmax_scale, nullptr, lse, static_cast<uint16_t*>(o_raster), so.b, so.n, so.h,
      static_cast<const uint16_t*>(q_raster), sq.b, sq.n, sq.h, work_queue, static_cast<hipStream_t>(stream)));
}

namespace {
// Dense attention keeps every key tile: k_hd = nT_hd for every head.
void set_dense(GeoTable* t) {
  for (int hd = 0; hd < t->heads; ++hd) t->h[hd].k = t->h[hd].nT;
}
}  // namespace

int veda_dense_attn_fwd(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                        float softmax_scale, void* o_tiled, float* lse, int32_t* work_queue, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !v_tiled || !o_tiled) return VEDA_ERR_NULL;
  set_dense(&t);
  for (const void* p : {q_tiled, k_tiled, v_tiled, static_cast<const void*>(o_tiled)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_sparse_attn(
      t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
      static_cast<const uint16_t*>(v_tiled), nullptr, t.nT_max, softmax_scale, static_cast<uint16_t*>(o_tiled), lse,
      nullptr, 0, 0, 0, nullptr, 0, 0, 0, work_queue, static_cast<hipStream_t>(stream)));
}

int veda_dense_attn_fwd_raster(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                               float softmax_scale, void* o_raster, veda_raster_strides s, float* lse,
                               int32_t* work_queue, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !v_tiled || !o_raster) return VEDA_ERR_NULL;
  set_dense(&t);
  for (const void* p : {q_tiled, k_tiled, v_tiled, static_cast<const void*>(o_raster)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  VEDA_TRY(check_strides(s));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_sparse_attn(
      t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
      static_cast<const uint16_t*>(v_tiled), nullptr, t.nT_max, softmax_scale, nullptr, lse,
      static_cast<uint16_t*>(o_raster), s.b, s.n, s.h, nullptr, 0, 0, 0, work_queue, static_cast<hipStream_t>(stream)));
}

int veda_sparse_attn_fwd_raster_io_noalloc(const veda_geom* g, const void* q_raster, veda_raster_strides sq,
                                           const void* k_tiled, const void* v_tiled, const int32_t* idx,
                                           const int32_t* k_per_head, int32_t k_max, float softmax_scale,
                                           void* o_raster, veda_raster_strides so, float* lse, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_raster || !k_tiled || !v_tiled || !idx || !o_raster) return VEDA_ERR_NULL;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  for (const void* p : {q_raster, k_tiled, v_tiled, static_cast<const void*>(idx), static_cast<const void*>(o_raster)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VEDA_ERR_ALIGN;
  // The static queue counts at most 2^28 work items, as a caller's workspace does.
  if (int64_t(t.B) * t.heads * t.nT_max > (int64_t(1) << 28)) return VEDA_ERR_SHAPE;
  VEDA_TRY(check_strides(sq));
  VEDA_TRY(check_strides(so));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  int32_t* queue = nullptr;
  if (veda::attn_scratch_queue(&queue) != hipSuccess) {
    (void)hipGetLastError();
    return VEDA_ERR_DEVICE;
  }
  return launched(veda::launch_sparse_attn(
      t, nullptr, static_cast<const uint16_t*>(k_tiled), static_cast<const uint16_t*>(v_tiled), idx, k_max,
      softmax_scale, nullptr, lse, static_cast<uint16_t*>(o_raster), so.b, so.n, so.h,
      static_cast<const uint16_t*>(q_raster), sq.b, sq.n, sq.h, queue, static_cast<hipStream_t>(stream)));
}

int veda_teacher_tile_max(const veda_geom* g, const void* q_tiled, const void* k_tiled, const float* lse_dense,
                          float softmax_scale, float* teacher, int32_t* work_queue, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!q_tiled || !k_tiled || !lse_dense || !teacher) return VEDA_ERR_NULL;
  for (const void* p : {q_tiled, k_tiled, static_cast<const void*>(lse_dense), static_cast<const void*>(teacher)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_queue(t, work_queue));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) softmax_scale = 1.0f / std::sqrt(float(t.d));
  VEDA_TRY(check_device());
  return launched(veda::launch_teacher(t, static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_tiled),
                                       lse_dense, softmax_scale, teacher, work_queue,
                                       static_cast<hipStream_t>(stream)));
}

int veda_mask_overlap(const veda_geom* g, const uint32_t* bitmask_a, const uint32_t* bitmask_b, uint64_t* counts,
                      void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!bitmask_a || !bitmask_b || !counts) return VEDA_ERR_NULL;
  for (const void* p : {static_cast<const void*>(bitmask_a), static_cast<const void*>(bitmask_b),
                        static_cast<const void*>(counts)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_mask_overlap(t, bitmask_a, bitmask_b, reinterpret_cast<unsigned long long*>(counts),
                                            nullptr, static_cast<hipStream_t>(stream)));
}

int veda_tile_recall(const veda_geom* g, const uint32_t* bitmask, const uint32_t* bitmask_oracle,
                     const int32_t* k_per_head, uint64_t* counts, double* recall, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!bitmask || !bitmask_oracle || !k_per_head || !recall) return VEDA_ERR_NULL;
  int32_t k_max = 0;
  for (int hd = 0; hd < t.heads; ++hd) k_max = k_per_head[hd] > k_max ? k_per_head[hd] : k_max;
  VEDA_TRY(set_k(k_per_head, k_max, &t));
  for (const void* p : {static_cast<const void*>(bitmask), static_cast<const void*>(bitmask_oracle),
                        static_cast<const void*>(recall)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (counts && !aligned16(counts)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_mask_overlap(t, bitmask, bitmask_oracle, reinterpret_cast<unsigned long long*>(counts),
                                            recall, static_cast<hipStream_t>(stream)));
}

int veda_tile_search_select(int32_t n_candidates, int32_t B, int32_t heads, const double* err, double* err_sum,
                            int32_t* best, void* stream) {
  if (!err || !best) return VEDA_ERR_NULL;
  if (n_candidates <= 0 || B <= 0 || B > 65535 || heads <= 0 || heads > VEDA_MAX_HEADS) return VEDA_ERR_SHAPE;
  if (!aligned16(err) || !aligned16(best) || (err_sum && !aligned16(err_sum))) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_search_select(n_candidates, B, heads, err, err_sum, best,
                                             static_cast<hipStream_t>(stream)));
}

int veda_candidate_tiles(veda_grid grid, veda_tile* tiles, int32_t capacity) {
  if (!tiles) return VEDA_ERR_NULL;
  if (grid.T <= 0 || grid.H <= 0 || grid.W <= 0 || capacity < 0) return VEDA_ERR_SHAPE;
  int n = 0;
  for (int a = 0; a < 8; ++a)
    for (int b = 0; a + b < 8; ++b) {
      const int32_t pt = 1 << a, ph = 1 << b, pw = 1 << (7 - a - b);
      if (pt > grid.T || ph > grid.H || pw > grid.W) continue;
      const int64_t nT = ((int64_t(grid.T) + pt - 1) / pt) * ((int64_t(grid.H) + ph - 1) / ph) *
                         ((int64_t(grid.W) + pw - 1) / pw);
      if (nT > VEDA_MAX_TILES) continue;
      if (n >= capacity) return VEDA_ERR_SHAPE;
      tiles[n++] = veda_tile{pt, ph, pw};
    }
  return n;
}

int veda_k_from_keep(const veda_geom* g, int32_t head, int64_t keep_num, int64_t keep_den) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (head < 0 || head >= t.heads) return VEDA_ERR_SHAPE;
  if (keep_den <= 0 || keep_num <= 0 || keep_num > keep_den) return VEDA_ERR_K;
  const __int128 n = t.h[head].nT;
  const __int128 k = (__int128(keep_num) * n + keep_den - 1) / keep_den;   // ceil(keep * nT_hd)
  return int(k < 1 ? 1 : (k > n ? n : k));
}

int veda_head_sq_error(const veda_geom* g, const void* a_raster, veda_raster_strides sa, const void* b_raster,
                       veda_raster_strides sb, double* err, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!a_raster || !b_raster || !err) return VEDA_ERR_NULL;
  if (!aligned16(a_raster) || !aligned16(b_raster) || !aligned16(err)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_strides(sa));
  VEDA_TRY(check_strides(sb));
  VEDA_TRY(check_device());
  return launched(veda::launch_head_sq_error(t, static_cast<const uint16_t*>(a_raster), sa.b, sa.n, sa.h,
                                             static_cast<const uint16_t*>(b_raster), sb.b, sb.n, sb.h, err,
                                             static_cast<hipStream_t>(stream)));
}

int veda_distill_kl(const veda_geom* g, const float* scores, const float* teacher, float grad_scale, float* kl_rows,
                    float* d_scores, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!scores || !teacher || !kl_rows || !d_scores) return VEDA_ERR_NULL;
  for (const void* p : {static_cast<const void*>(scores), static_cast<const void*>(teacher),
                        static_cast<const void*>(kl_rows), static_cast<const void*>(d_scores)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (!std::isfinite(grad_scale)) return VEDA_ERR_SHAPE;
  VEDA_TRY(check_device());
  return launched(veda::launch_distill_kl(t, scores, teacher, grad_scale, kl_rows, d_scores,
                                          static_cast<hipStream_t>(stream)));
}

int veda_distill_mean_kl(const veda_geom* g, const float* kl_rows, double* mean, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (!kl_rows || !mean) return VEDA_ERR_NULL;
  if (!aligned16(kl_rows) || (reinterpret_cast<uintptr_t>(mean) & 7u)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_distill_mean(t, kl_rows, mean, static_cast<hipStream_t>(stream)));
}

int veda_distill_grad(const veda_geom* g, int32_t rank, const void* stats_q, const void* stats_k, const void* feat_q,
                      const void* feat_k, const float* d_scores, float* d_feat_q, float* d_feat_k, float* d_w_q,
                      float* d_w_k, void* stream) {
  GeoTable t;
  VEDA_TRY(build_table(g, &t));
  if (rank != 32 && rank != 64) return VEDA_ERR_SHAPE;
  if (!stats_q || !stats_k || !feat_q || !feat_k || !d_scores || !d_feat_q || !d_feat_k || !d_w_q || !d_w_k)
    return VEDA_ERR_NULL;
  for (const void* p : {stats_q, stats_k, feat_q, feat_k, static_cast<const void*>(d_scores),
                        static_cast<const void*>(d_feat_q), static_cast<const void*>(d_feat_k),
                        static_cast<const void*>(d_w_q), static_cast<const void*>(d_w_k)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  return launched(veda::launch_distill_grad(
      t, rank, static_cast<const uint16_t*>(stats_q), static_cast<const uint16_t*>(stats_k),
      static_cast<const uint16_t*>(feat_q), static_cast<const uint16_t*>(feat_k), d_scores, d_feat_q, d_feat_k, d_w_q,
      d_w_k, static_cast<hipStream_t>(stream)));
}

int veda_adam_step(int64_t n, float* w_master, const float* grad, float* m, float* v, int32_t step, float lr,
                   float beta1, float beta2, float eps, void* w_bf16, void* stream) {
  if (!w_master || !grad || !m || !v) return VEDA_ERR_NULL;
  if (n <= 0 || step < 1 || !std::isfinite(lr) || !(beta1 >= 0.0f && beta1 < 1.0f) ||
      !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) || !std::isfinite(eps))
    return VEDA_ERR_SHAPE;
  for (const void* p : {static_cast<const void*>(w_master), static_cast<const void*>(grad),
                        static_cast<const void*>(m), static_cast<const void*>(v)})
    if (!aligned16(p)) return VEDA_ERR_ALIGN;
  if (w_bf16 && !aligned16(w_bf16)) return VEDA_ERR_ALIGN;
  VEDA_TRY(check_device());
  const float bc1 = float(1.0 - std::pow(double(beta1), double(step)));
  const float bc2 = float(1.0 - std::pow(double(beta2), double(step)));
  return launched(veda::launch_adam(n, w_master, grad, m, v, lr, beta1, beta2, eps, bc1, bc2,
                                    static_cast<uint16_t*>(w_bf16), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
