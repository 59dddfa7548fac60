// TripPool estimator (Veda page, "Attention Structure Distillation",
// Estimator: per-tile average, maximum and minimum of Q and K, mapped by
// head-specific Q/K projections to tile scores; "Theoretical Rationale" 2,
// "Tile Statistics").
//
// Three kernels:
//   trippool_features_kernel  one wave per tile: each lane owns d/64
//     channels and walks the 128 slots in order (fp32 sum, total-order
//     max/min over real slots); a wave load is one whole token row, so the
//     stream from HBM is coalesced. The 3d statistics are staged in LDS and
//     the same wave projects them with the head's W (held in LDS for the whole
//     workgroup, 2 workgroups per CU at d = 128): lane j owns output feature j and
//     accumulates over the 3d channels in order.
//   trippool_project_kernel  the projection alone, from statistics that the
//     fused permute (permute.hip) computed while it tiled Q and K.
//   tile_scores_kernel  S = feat_q . feat_k^T per head, 128 x 128 outputs per
//     workgroup, 8 x 8 per thread, fp32 accumulated over the r channels in order.
// Every accumulation runs in a fixed ascending order with one rounding per
// step (products of bf16 values are exact in fp32), so the results are
// reproducible bit for bit and independent of the launch shape.
//   tile_scores_mfma_kernel  the same S as the small bf16 GEMM the estimator
//     is (32x32x16 bf16 MFMA, fp32 accumulation in the matrix core's own
//     order): not bit-identical to the ordered sum, within its rounding bound.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTilesPerWave = 4;
constexpr int kTilesPerBlock = kWaves * kTilesPerWave;

// Head-specific projection of one tile's statistics st[0..C): lane j < R
// accumulates sum_c st[c] * W[c][j] in ascending c (fp32 FMA from +0; the
// products of bf16 values are exact) and rounds the sum to bf16.
template <int C, int R>
__device__ __forceinline__ void project_tile(const float* st, const uint16_t* w_s, int lane, uint16_t* f_out) {
  if (lane < R) {
    float acc = 0.0f;
    for (int c = 0; c < C; ++c) acc = __builtin_fmaf(st[c], bf16_to_f32(w_s[c * R + lane]), acc);
    f_out[lane] = f32_to_bf16_rne(acc);
  }
}

template <int D, int R>
__global__ __launch_bounds__(kThreads) void trippool_features_kernel(
    GeoTable g, const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk, uint16_t* __restrict__ stats_q,
    uint16_t* __restrict__ stats_k, uint16_t* __restrict__ feat_q, uint16_t* __restrict__ feat_k) {
  constexpr int C = 3 * D;           // statistic channels
  constexpr int CH = D / 64;         // channels per lane
  constexpr int kRowsPerLoad = 32;   // token rows held in registers at a time
  __shared__ uint16_t w_s[C * R];
  __shared__ float st_s[kWaves][C];

  const int hd = blockIdx.y;
  const int side = blockIdx.z & 1;  // 0 = Q, 1 = K
  const int b = blockIdx.z >> 1;
  const HeadGeo hg = g.h[hd];
  const uint16_t* xt = side ? k_t : q_t;
  const uint16_t* w = (side ? wk : wq) + int64_t(hd) * C * R;
  uint16_t* stats = side ? stats_k : stats_q;
  uint16_t* feat = side ? feat_k : feat_q;

  // Stage this head's projection matrix (3d x r bf16) in LDS.
  {
    const uint4* src = reinterpret_cast<const uint4*>(w);
    uint4* dst = reinterpret_cast<uint4*>(w_s);
    for (int i = threadIdx.x; i < C * R / 8; i += kThreads) dst[i] = src[i];
  }
  __syncthreads();

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int it = 0; it < kTilesPerWave; ++it) {
    const int32_t tau = blockIdx.x * kTilesPerBlock + it * kWaves + wave;
    if (tau >= g.nT_max) break;
    const int64_t row = (int64_t(b) * g.heads + hd) * g.nT_max + tau;
    uint16_t* st_out = stats + row * C;
    uint16_t* f_out = feat + row * R;
    if (tau >= hg.nT) {  // tile beyond this head's grid: defined zeros
      for (int c = lane; c < C; c += 64) st_out[c] = 0;
      if (lane < R) f_out[lane] = 0;
      continue;
    }
    const BoxExtent e = box_extent(g, hg, tau);
    const bool full = box_is_full(hg, e);
    // Lane owns channels [lane*CH, lane*CH + CH); one wave load reads a whole
    // token row (d bf16), so every load is a coalesced 128/256-byte segment.
    const uint16_t* src = xt + row * VEDA_TILE_TOKENS * D + lane * CH;
    float sum[CH];
    int32_t mx[CH], mn[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      sum[c] = 0.0f;
      mx[c] = -(1 << 20);
      mn[c] = 1 << 20;
    }
    int32_t n_real = 0;
    for (int s0 = 0; s0 < VEDA_TILE_TOKENS; s0 += kRowsPerLoad) {
      uint32_t v[kRowsPerLoad];
#pragma unroll
      for (int i = 0; i < kRowsPerLoad; ++i) {
        if constexpr (CH == 2)
          v[i] = *reinterpret_cast<const uint32_t*>(src + (s0 + i) * D);
        else
          v[i] = src[(s0 + i) * D];
      }
#pragma unroll
      for (int i = 0; i < kRowsPerLoad; ++i) {
        if (!full && !slot_is_real(hg, e, s0 + i)) continue;  // uniform over the wave
        ++n_real;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t bits = (v[i] >> (16 * c)) & 0xFFFFu;
          sum[c] = sum[c] + bf16_to_f32(uint16_t(bits));
          const int32_t key = total_order_key(bits);
          mx[c] = max(mx[c], key);
          mn[c] = min(mn[c], key);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // sum / n in double then to float is the correctly rounded float quotient
      // (53 >= 2*24 + 2, so the double rounding is innocuous).
      const float avg = float(double(sum[c]) / double(n_real));
      const uint16_t a = f32_to_bf16_rne(avg);
      const uint16_t hi = from_total_order_key(mx[c]);
      const uint16_t lo = from_total_order_key(mn[c]);
      const int ch = lane * CH + c;
      st_out[ch] = a;
      st_out[D + ch] = hi;
      st_out[2 * D + ch] = lo;
      st_s[wave][ch] = bf16_to_f32(a);
      st_s[wave][D + ch] = bf16_to_f32(hi);
      st_s[wave][2 * D + ch] = bf16_to_f32(lo);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    project_tile<C, R>(st_s[wave], w_s, lane, f_out);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Projections alone, from statistics already in HBM (written by the permute
// that computes them on the fly). r/8 lanes share a tile; each owns 8 of its
// r outputs for kProjTiles tiles (kLaneSlots apart) and keeps their sums in
// registers, so 8 kProjTiles FMA chains run side by side in every lane. All
// lanes walk the 3d channels in the same ascending order and read their 16
// bytes of W row c from LDS (the lanes of a wave read one contiguous row,
// free of bank conflicts); each W value is converted from bf16 once and
// serves all the lane's tiles. Each sum still takes one channel at a time in
// ascending order from +0, exactly as project_tile.
constexpr int kProjTiles = 4;   // tiles per lane: each W value, converted once, feeds kProjTiles FMAs
template <int D, int R>
__global__ __launch_bounds__(kThreads) void trippool_project_kernel(
    GeoTable g, const uint16_t* __restrict__ stats_q, const uint16_t* __restrict__ stats_k,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk, uint16_t* __restrict__ feat_q,
    uint16_t* __restrict__ feat_k) {
  constexpr int C = 3 * D;
  constexpr int kGroups = R / 8;                     // lanes per tile
  constexpr int kLaneSlots = kThreads / kGroups;     // tile slots per workgroup pass
  __shared__ __attribute__((aligned(16))) uint16_t w_s[C * R];

  const int hd = blockIdx.y;
  const int side = blockIdx.z & 1;  // 0 = Q, 1 = K
  const int b = blockIdx.z >> 1;
  const HeadGeo hg = g.h[hd];
  const uint16_t* stats = side ? stats_k : stats_q;
  const uint16_t* w = (side ? wk : wq) + int64_t(hd) * C * R;
  uint16_t* feat = side ? feat_k : feat_q;
  {
    const uint4* src = reinterpret_cast<const uint4*>(w);
    uint4* dst = reinterpret_cast<uint4*>(w_s);
    for (int i = threadIdx.x; i < C * R / 8; i += kThreads) dst[i] = src[i];
  }
  __syncthreads();

  const int grp = threadIdx.x % kGroups;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  int32_t tau[kProjTiles];
  const uint4* st[kProjTiles];
#pragma unroll
  for (int t = 0; t < kProjTiles; ++t) {
    tau[t] = (blockIdx.x * kProjTiles + t) * kLaneSlots + threadIdx.x / kGroups;
    st[t] = reinterpret_cast<const uint4*>(stats + (head_row + (tau[t] < hg.nT ? tau[t] : 0)) * C);
  }
  const uint16_t* wcol = w_s + 8 * grp;
  float acc[kProjTiles][8];
#pragma unroll
  for (int t = 0; t < kProjTiles; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.0f;
  for (int c8 = 0; c8 < C / 8; ++c8) {
    uint32_t sw[kProjTiles][4];
#pragma unroll
    for (int t = 0; t < kProjTiles; ++t) {
      const uint4 sv = st[t][c8];
      sw[t][0] = sv.x; sw[t][1] = sv.y; sw[t][2] = sv.z; sw[t][3] = sv.w;
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint4 wv = *reinterpret_cast<const uint4*>(wcol + (c8 * 8 + cc) * R);
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
      float wf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wf[e] = __uint_as_float((e & 1) ? (ww[e / 2] & 0xFFFF0000u) : (ww[e / 2] << 16));
#pragma unroll
      for (int t = 0; t < kProjTiles; ++t) {
        const float x = __uint_as_float((cc & 1) ? (sw[t][cc / 2] & 0xFFFF0000u) : (sw[t][cc / 2] << 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = __builtin_fmaf(x, wf[e], acc[t][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kProjTiles; ++t) {
    if (tau[t] >= g.nT_max) continue;
    const bool real = tau[t] < hg.nT;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = real ? (uint32_t(f32_to_bf16_rne(acc[t][2 * e])) | (uint32_t(f32_to_bf16_rne(acc[t][2 * e + 1])) << 16)) : 0u;
    *reinterpret_cast<uint4*>(feat + (head_row + tau[t]) * R + 8 * grp) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

constexpr int kScoreTile = 128;   // scores per workgroup: 128 x 128, 8 x 8 per thread
constexpr int kScorePad = 4;      // LDS row padding (floats): spreads the transposing stores over banks

// S[i, j] = sum over c < R of feat_q[i, c] * feat_k[j, c], fp32 FMA in
// ascending c from +0. Rows are `ld` elements apart: ld = R for the
// estimator's features; ld = 3d with R = d reads the avg block of the
// TripPool statistics, which gives the average-pooling scores.
template <int R>
__global__ __launch_bounds__(kThreads) void tile_scores_kernel(GeoTable g, const uint16_t* __restrict__ feat_q,
                                                              const uint16_t* __restrict__ feat_k, int32_t ld,
                                                              float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) float fq_s[R][kScoreTile + kScorePad];  // transposed: [channel][row]
  __shared__ __attribute__((aligned(16))) float fk_s[R][kScoreTile + kScorePad];
  const int hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int nb = (g.nT_max + kScoreTile - 1) / kScoreTile;
  const int i0 = blockIdx.x / nb * kScoreTile;
  const int j0 = blockIdx.x % nb * kScoreTile;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  // Stage both sides as fp32, transposed to [channel][row]; each thread
  // reads 8 features (16 bytes) of a row at a time.
  for (int e = threadIdx.x; e < kScoreTile * R / 8; e += kThreads) {
    const int r = e / (R / 8), c0 = (e % (R / 8)) * 8;
    const int i = i0 + r, j = j0 + r;
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    const uint4 qa = i < hg.nT ? *reinterpret_cast<const uint4*>(feat_q + (head_row + i) * ld + c0) : zero4;
    const uint4 ka = j < hg.nT ? *reinterpret_cast<const uint4*>(feat_k + (head_row + j) * ld + c0) : zero4;
    const uint32_t qw[4] = {qa.x, qa.y, qa.z, qa.w}, kw[4] = {ka.x, ka.y, ka.z, ka.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      fq_s[c0 + u][r] = __uint_as_float((u & 1) ? (qw[u / 2] & 0xFFFF0000u) : (qw[u / 2] << 16));
      fk_s[c0 + u][r] = __uint_as_float((u & 1) ? (kw[u / 2] & 0xFFFF0000u) : (kw[u / 2] << 16));
    }
  }
  __syncthreads();
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.0f;
#pragma unroll 4
  for (int c = 0; c < R; ++c) {
    const float4 q0 = *reinterpret_cast<const float4*>(&fq_s[c][ty * 8]);
    const float4 q1 = *reinterpret_cast<const float4*>(&fq_s[c][ty * 8 + 4]);
    const float4 k0 = *reinterpret_cast<const float4*>(&fk_s[c][tx * 8]);
    const float4 k1 = *reinterpret_cast<const float4*>(&fk_s[c][tx * 8 + 4]);
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) acc[a][k2] = __builtin_fmaf(qv[a], kv[k2], acc[a][k2]);
  }
  const float ninf = -__builtin_inff();
  const bool vec_ok = (g.nT_max % 4) == 0;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = i0 + ty * 8 + a;
    if (i >= g.nT_max) continue;
    float* out = scores + (head_row + i) * g.nT_max;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = j0 + tx * 8 + 4 * half;
      float v[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) v[k2] = (i < hg.nT && j + k2 < hg.nT) ? acc[a][4 * half + k2] : ninf;
      if (vec_ok && j + 3 < g.nT_max) {
        *reinterpret_cast<float4*>(out + j) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
          if (j + k2 < g.nT_max) out[j + k2] = v[k2];
      }
    }
  }
}

// S = feat_q . feat_k^T on the matrix cores. A workgroup of 4 waves takes a
// 128 x 128 block of one head; wave w owns rows 32w..32w+31 against all 128
// columns as four 32 x 32 MFMA outputs, each accumulated over r / 16 k-steps.
// Operands come straight from the bf16 feature rows: lane l of a k-step
// holds 8 consecutive channels (16 bytes) of row l % 32, channels 8 (l / 32)
// onward of the step. Output element v of lane l is row 8 (v / 4) + 4 (l / 32)
// + v % 4, column l % 32, so 32 lanes write 128 contiguous bytes of a row.
typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));
typedef float floatx16_s __attribute__((ext_vector_type(16)));
template <int R>
__global__ __launch_bounds__(256) void tile_scores_mfma_kernel(GeoTable g, const uint16_t* __restrict__ feat_q,
                                                              const uint16_t* __restrict__ feat_k,
                                                              float* __restrict__ scores) {
  constexpr int kSteps = R / 16;
  const int hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int nb = (g.nT_max + kScoreTile - 1) / kScoreTile;
  const int i0 = blockIdx.x / nb * kScoreTile, j0 = blockIdx.x % nb * kScoreTile;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, l32 = lane % 32, h = lane / 32;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  const int ia = i0 + 32 * wave + l32;   // rows past the head read as zeros and are written -inf
  uint4 qf[kSteps];
#pragma unroll
  for (int kk = 0; kk < kSteps; ++kk)
    qf[kk] = ia < hg.nT ? *reinterpret_cast<const uint4*>(feat_q + (head_row + ia) * R + 16 * kk + 8 * h) : zero4;
  floatx16_s acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int jb = j0 + 32 * n + l32;
    floatx16_s c = {};
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
      const uint4 kf =
          jb < hg.nT ? *reinterpret_cast<const uint4*>(feat_k + (head_row + jb) * R + 16 * kk + 8 * h) : zero4;
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_s, qf[kk]),
                                                  __builtin_bit_cast(bf16x8_s, kf), c, 0, 0, 0);
    }
    acc[n] = c;
  }
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int j = j0 + 32 * n + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + 32 * wave + 8 * (v / 4) + 4 * h + v % 4;
      if (i < g.nT_max && j < g.nT_max)
        scores[(head_row + i) * g.nT_max + j] = (i < hg.nT && j < hg.nT) ? acc[n][v] : ninf;
    }
  }
}

}  // namespace

hipError_t launch_trippool_features(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t,
                                    const uint16_t* wq, const uint16_t* wk, int32_t r, uint16_t* stats_q,
                                    uint16_t* stats_k, uint16_t* feat_q, uint16_t* feat_k, hipStream_t s) {
  const dim3 grid((g.nT_max + kTilesPerBlock - 1) / kTilesPerBlock, g.heads, 2 * g.B);
  if (g.d == 128 && r == 64)
    trippool_features_kernel<128, 64><<<grid, kThreads, 0, s>>>(g, q_t, k_t, wq, wk, stats_q, stats_k, feat_q, feat_k);
  else if (g.d == 128 && r == 32)
    trippool_features_kernel<128, 32><<<grid, kThreads, 0, s>>>(g, q_t, k_t, wq, wk, stats_q, stats_k, feat_q, feat_k);
  else if (g.d == 64 && r == 64)
    trippool_features_kernel<64, 64><<<grid, kThreads, 0, s>>>(g, q_t, k_t, wq, wk, stats_q, stats_k, feat_q, feat_k);
  else
    trippool_features_kernel<64, 32><<<grid, kThreads, 0, s>>>(g, q_t, k_t, wq, wk, stats_q, stats_k, feat_q, feat_k);
  return hipGetLastError();
}

hipError_t launch_trippool_project(const GeoTable& g, const uint16_t* stats_q, const uint16_t* stats_k,
                                   const uint16_t* wq, const uint16_t* wk, int32_t r, uint16_t* feat_q,
                                   uint16_t* feat_k, hipStream_t s) {
  const int tiles_per_block = kThreads / (r / 8) * kProjTiles;
  const dim3 grid((g.nT_max + tiles_per_block - 1) / tiles_per_block, g.heads, 2 * g.B);
  if (g.d == 128 && r == 64)
    trippool_project_kernel<128, 64><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, wq, wk, feat_q, feat_k);
  else if (g.d == 128 && r == 32)
    trippool_project_kernel<128, 32><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, wq, wk, feat_q, feat_k);
  else if (g.d == 64 && r == 64)
    trippool_project_kernel<64, 64><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, wq, wk, feat_q, feat_k);
  else
    trippool_project_kernel<64, 32><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, wq, wk, feat_q, feat_k);
  return hipGetLastError();
}

hipError_t launch_tile_scores(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                              float* scores, hipStream_t s) {
  const int nb = (g.nT_max + kScoreTile - 1) / kScoreTile;
  const dim3 grid(nb * nb, g.heads, g.B);
  if (r == 64)
    tile_scores_kernel<64><<<grid, kThreads, 0, s>>>(g, feat_q, feat_k, 64, scores);
  else
    tile_scores_kernel<32><<<grid, kThreads, 0, s>>>(g, feat_q, feat_k, 32, scores);
  return hipGetLastError();
}

hipError_t launch_tile_scores_mfma(const GeoTable& g, const uint16_t* feat_q, const uint16_t* feat_k, int32_t r,
                                   float* scores, hipStream_t s) {
  const int nb = (g.nT_max + kScoreTile - 1) / kScoreTile;
  const dim3 grid(nb * nb, g.heads, g.B);
  if (r == 64)
    tile_scores_mfma_kernel<64><<<grid, 256, 0, s>>>(g, feat_q, feat_k, scores);
  else
    tile_scores_mfma_kernel<32><<<grid, 256, 0, s>>>(g, feat_q, feat_k, scores);
  return hipGetLastError();
}

hipError_t launch_avgpool_scores(const GeoTable& g, const uint16_t* stats_q, const uint16_t* stats_k, float* scores,
                                 hipStream_t s) {
  const int nb = (g.nT_max + kScoreTile - 1) / kScoreTile;
  const dim3 grid(nb * nb, g.heads, g.B);
  if (g.d == 128)
    tile_scores_kernel<128><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, 3 * 128, scores);
  else
    tile_scores_kernel<64><<<grid, kThreads, 0, s>>>(g, stats_q, stats_k, 3 * 64, scores);
  return hipGetLastError();
}

}  // namespace veda
