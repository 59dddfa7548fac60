// Distillation of the tile estimator (Veda page, "Theoretical Rationale" 4,
// "Distillation Objective": the estimator's soft tile distribution is aligned
// with the max-pooled full-attention target by a KL divergence before the
// discrete Top-k; Principle 01 "Full-Attention Structure Distillation").
//
// For every (b, head, query tile) row over the head's key tiles:
//   A_tgt = T / sum_j T         (teacher row, max-pooled dense attention)
//   A_pred = softmax_j(S)       (estimator scores S = feat_q . feat_k)
//   KL = sum_j A_tgt (log A_tgt - log A_pred),  dKL/dS = A_pred - A_tgt.
// Back through S = F_q F_k^T and F = stats W (the bf16 rounding of F passed
// straight through): dF_q = dS F_k, dF_k = dS^T F_q, dW = stats^T dF summed
// over the batch. Then one Adam step on fp32 master weights, with the bf16
// copy the estimator reads.
//
// Everything accumulates in fp32 in a fixed order (rows split over lanes in a
// fixed pattern, GEMMs over the contraction index in ascending order), so the
// results are reproducible bit for bit.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = kRowThreads / 64;

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// One wave per row. Lane l handles key tiles j = l, l + 64, ... in order.
__global__ __launch_bounds__(kRowThreads) void kl_row_kernel(GeoTable g, const float* __restrict__ scores,
                                                            const float* __restrict__ teacher, float grad_scale,
                                                            float* __restrict__ kl_rows, float* __restrict__ d_scores) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int32_t tq = blockIdx.x * kRowsPerBlock + wave;
  const int hd = blockIdx.y, b = blockIdx.z;
  if (tq >= g.nT_max) return;
  const int32_t n = g.h[hd].nT;
  const int64_t row = (int64_t(b) * g.heads + hd) * g.nT_max + tq;
  const float* s = scores + row * g.nT_max;
  const float* t = teacher + row * g.nT_max;
  float* ds = d_scores + row * g.nT_max;
  if (tq >= n) {
    for (int j = lane; j < g.nT_max; j += 64) ds[j] = 0.0f;
    if (lane == 0) kl_rows[row] = 0.0f;
    return;
  }
  float smax = -__builtin_inff(), tsum = 0.0f;
  for (int j = lane; j < n; j += 64) {
    smax = fmaxf(smax, s[j]);
    tsum += t[j];
  }
  smax = wave_max_f(smax);
  tsum = wave_sum_f(tsum);
  float esum = 0.0f;
  for (int j = lane; j < n; j += 64) esum += __expf(s[j] - smax);
  esum = wave_sum_f(esum);
  const float lse = smax + __logf(esum);
  const float inv_t = 1.0f / tsum;
  float kl = 0.0f;
  for (int j = lane; j < g.nT_max; j += 64) {
    if (j < n) {
      const float lp = s[j] - lse;
      const float at = t[j] * inv_t;
      if (at > 0.0f) kl += at * (__logf(at) - lp);
      ds[j] = grad_scale * (__expf(lp) - at);
    } else {
      ds[j] = 0.0f;
    }
  }
  kl = wave_sum_f(kl);
  if (lane == 0) kl_rows[row] = kl;
}

// dF for one (b, head): mode 0: dF_q[i, c] = sum_j dS[i, j] F_k[j, c];
// mode 1: dF_k[j, c] = sum_i dS[i, j] F_q[i, c]. 64 output rows per
// workgroup, the contraction index staged through LDS in 64-wide slices and
// summed in ascending order.
constexpr int kGemmThreads = 256;
constexpr int kRowsBlk = 64;

template <int R>
__global__ __launch_bounds__(kGemmThreads) void grad_feat_kernel(GeoTable g, const uint16_t* __restrict__ feat_q,
                                                                const uint16_t* __restrict__ feat_k,
                                                                const float* __restrict__ d_scores,
                                                                float* __restrict__ d_feat_q,
                                                                float* __restrict__ d_feat_k) {
  constexpr int kColsPerThread = R / 16;                 // 16 column groups x 16 row groups of 4 rows
  __shared__ float a_s[kRowsBlk][kRowsBlk + 1];          // [output row][contraction]
  __shared__ float f_s[kRowsBlk][R];                     // [contraction][channel]
  const int mode = blockIdx.y % 2, hd = blockIdx.y / 2, b = blockIdx.z;
  const int32_t n = g.h[hd].nT;
  const int i0 = blockIdx.x * kRowsBlk;
  const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
  const float* dS = d_scores + head_row * g.nT_max;
  const uint16_t* F = mode == 0 ? feat_k : feat_q;
  float* out = mode == 0 ? d_feat_q : d_feat_k;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[4][kColsPerThread];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < kColsPerThread; ++c) acc[r][c] = 0.0f;
  for (int j0 = 0; j0 < n; j0 += kRowsBlk) {
    for (int e = threadIdx.x; e < kRowsBlk * kRowsBlk; e += kGemmThreads) {
      const int r = e / kRowsBlk, c = e % kRowsBlk;      // output row r, contraction c
      const int i = i0 + r, j = j0 + c;
      float v = 0.0f;
      if (i < n && j < n) v = mode == 0 ? dS[int64_t(i) * g.nT_max + j] : dS[int64_t(j) * g.nT_max + i];
      a_s[r][c] = v;
    }
    for (int e = threadIdx.x; e < kRowsBlk * R; e += kGemmThreads) {
      const int j = j0 + e / R, c = e % R;
      f_s[e / R][c] = j < n ? bf16_to_f32(F[(head_row + j) * R + c]) : 0.0f;
    }
    __syncthreads();
    for (int c = 0; c < kRowsBlk; ++c) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = a_s[4 * ty + r][c];
#pragma unroll
        for (int m = 0; m < kColsPerThread; ++m) acc[r][m] = __builtin_fmaf(a, f_s[c][tx + 16 * m], acc[r][m]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * ty + r;
    if (i >= g.nT_max) continue;
#pragma unroll
    for (int m = 0; m < kColsPerThread; ++m) out[(head_row + i) * R + tx + 16 * m] = i < n ? acc[r][m] : 0.0f;
  }
}

// dW[hd, a, c] = sum_b sum_i stats[b, hd, i, a] dF[b, hd, i, c] for both the
// query side (blockIdx.z == 0) and the key side. 64 rows a per workgroup.
template <int D, int R>
__global__ __launch_bounds__(kGemmThreads) void grad_w_kernel(GeoTable g, const uint16_t* __restrict__ stats_q,
                                                             const uint16_t* __restrict__ stats_k,
                                                             const float* __restrict__ d_feat_q,
                                                             const float* __restrict__ d_feat_k,
                                                             float* __restrict__ d_wq, float* __restrict__ d_wk) {
  constexpr int C = 3 * D;
  constexpr int kColsPerThread = R / 16;
  __shared__ float st_s[kRowsBlk][kRowsBlk + 1];         // [tile i][stat channel a]
  __shared__ float df_s[kRowsBlk][R];                    // [tile i][feature channel c]
  const int side = blockIdx.z, hd = blockIdx.y;
  const int a0 = blockIdx.x * kRowsBlk;
  const int32_t n = g.h[hd].nT;
  const uint16_t* stats = side == 0 ? stats_q : stats_k;
  const float* dF = side == 0 ? d_feat_q : d_feat_k;
  float* out = (side == 0 ? d_wq : d_wk) + int64_t(hd) * C * R;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[4][kColsPerThread];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < kColsPerThread; ++c) acc[r][c] = 0.0f;
  for (int b = 0; b < g.B; ++b) {
    const int64_t head_row = (int64_t(b) * g.heads + hd) * g.nT_max;
    for (int i0 = 0; i0 < n; i0 += kRowsBlk) {
      for (int e = threadIdx.x; e < kRowsBlk * kRowsBlk; e += kGemmThreads) {
        const int i = i0 + e / kRowsBlk, a = a0 + e % kRowsBlk;
        st_s[e / kRowsBlk][e % kRowsBlk] = (i < n && a < C) ? bf16_to_f32(stats[(head_row + i) * C + a]) : 0.0f;
      }
      for (int e = threadIdx.x; e < kRowsBlk * R; e += kGemmThreads) {
        const int i = i0 + e / R;
        df_s[e / R][e % R] = i < n ? dF[(head_row + i) * R + e % R] : 0.0f;
      }
      __syncthreads();
      for (int i = 0; i < kRowsBlk; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = st_s[i][4 * ty + r];
#pragma unroll
          for (int m = 0; m < kColsPerThread; ++m) acc[r][m] = __builtin_fmaf(s, df_s[i][tx + 16 * m], acc[r][m]);
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = a0 + 4 * ty + r;
    if (a >= C) continue;
#pragma unroll
    for (int m = 0; m < kColsPerThread; ++m) out[int64_t(a) * R + tx + 16 * m] = acc[r][m];
  }
}

// Adam on fp32 master weights; writes the bf16 copy (round to nearest even).
__global__ __launch_bounds__(256) void adam_kernel(int64_t n, float* __restrict__ w, const float* __restrict__ grad,
                                                   float* __restrict__ m, float* __restrict__ v, float lr,
                                                   float beta1, float beta2, float eps, float bc1, float bc2,
                                                   uint16_t* __restrict__ w_bf16) {
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    const float gr = grad[e];
    const float mm = beta1 * m[e] + (1.0f - beta1) * gr;
    const float vv = beta2 * v[e] + (1.0f - beta2) * gr * gr;
    m[e] = mm;
    v[e] = vv;
    const float ww = w[e] - lr * (mm / bc1) / (__fsqrt_rn(vv / bc2) + eps);
    w[e] = ww;
    if (w_bf16) w_bf16[e] = f32_to_bf16_rne(ww);
  }
}

}  // namespace

hipError_t launch_distill_kl(const GeoTable& g, const float* scores, const float* teacher, float grad_scale,
                             float* kl_rows, float* d_scores, hipStream_t s) {
  const dim3 grid((g.nT_max + kRowsPerBlock - 1) / kRowsPerBlock, g.heads, g.B);
  kl_row_kernel<<<grid, kRowThreads, 0, s>>>(g, scores, teacher, grad_scale, kl_rows, d_scores);
  return hipGetLastError();
}

hipError_t launch_distill_grad(const GeoTable& g, int32_t r, const uint16_t* stats_q, const uint16_t* stats_k,
                               const uint16_t* feat_q, const uint16_t* feat_k, const float* d_scores,
                               float* d_feat_q, float* d_feat_k, float* d_wq, float* d_wk, hipStream_t s) {
  const dim3 g1((g.nT_max + kRowsBlk - 1) / kRowsBlk, 2 * g.heads, g.B);
  if (r == 64)
    grad_feat_kernel<64><<<g1, kGemmThreads, 0, s>>>(g, feat_q, feat_k, d_scores, d_feat_q, d_feat_k);
  else
    grad_feat_kernel<32><<<g1, kGemmThreads, 0, s>>>(g, feat_q, feat_k, d_scores, d_feat_q, d_feat_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((3 * g.d + kRowsBlk - 1) / kRowsBlk, g.heads, 2);
  if (g.d == 128 && r == 64)
    grad_w_kernel<128, 64><<<g2, kGemmThreads, 0, s>>>(g, stats_q, stats_k, d_feat_q, d_feat_k, d_wq, d_wk);
  else if (g.d == 128)
    grad_w_kernel<128, 32><<<g2, kGemmThreads, 0, s>>>(g, stats_q, stats_k, d_feat_q, d_feat_k, d_wq, d_wk);
  else if (r == 64)
    grad_w_kernel<64, 64><<<g2, kGemmThreads, 0, s>>>(g, stats_q, stats_k, d_feat_q, d_feat_k, d_wq, d_wk);
  else
    grad_w_kernel<64, 32><<<g2, kGemmThreads, 0, s>>>(g, stats_q, stats_k, d_feat_q, d_feat_k, d_wq, d_wk);
  return hipGetLastError();
}

hipError_t launch_adam(int64_t n, float* w, const float* grad, float* m, float* v, float lr, float beta1, float beta2,
                       float eps, float bc1, float bc2, uint16_t* w_bf16, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  adam_kernel<<<dim3(unsigned(blocks < 4096 ? blocks : 4096)), 256, 0, s>>>(n, w, grad, m, v, lr, beta1, beta2, eps,
                                                                           bc1, bc2, w_bf16);
  return hipGetLastError();
}

}  // namespace veda
