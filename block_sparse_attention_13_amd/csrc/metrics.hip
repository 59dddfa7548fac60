// Squared error between two raster tensors per (batch, head): the objective
// of the head-aware tile search (Veda page, "Head-Aware Tile Search": each
// head takes the tiling that minimises the squared Frobenius norm of the
// difference between the full-attention output and the sparse output on
// calibration samples).
//
// One workgroup per (batch, head) reads both [N, d] slices with 16-byte loads
// and sums (a - b)^2 in fp64 per thread, then over the workgroup in a fixed
// tree order, so the result is deterministic. HBM-bound; the library keeps no
// scratch, so each head's sum stays inside one workgroup.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kSqThreads = 1024;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(kSqThreads) void head_sq_error_kernel(GeoTable g, const uint16_t* __restrict__ a,
                                                                  int64_t sab, int64_t san, int64_t sah,
                                                                  const uint16_t* __restrict__ b, int64_t sbb,
                                                                  int64_t sbn, int64_t sbh, double* __restrict__ err) {
  const int hd = blockIdx.x, bb = blockIdx.y;
  const int chunks = g.d / 8;                        // 16-byte pieces per token row
  const int64_t N = int64_t(g.T) * g.H * g.W;
  const int64_t total = N * chunks;
  const uint16_t* pa = a + bb * sab + hd * sah;
  const uint16_t* pb = b + bb * sbb + hd * sbh;
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < total; e += kSqThreads) {
    const int64_t n = e / chunks;
    const int c = int(e % chunks) * 8;
    const uint4 va = *reinterpret_cast<const uint4*>(pa + n * san + c);
    const uint4 vb = *reinterpret_cast<const uint4*>(pb + n * sbn + c);
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double d0 = double(bf16_lo(wa[i])) - double(bf16_lo(wb[i]));
      const double d1 = double(bf16_hi(wa[i])) - double(bf16_hi(wb[i]));
      acc = __builtin_fma(d0, d0, acc);
      acc = __builtin_fma(d1, d1, acc);
    }
  }
  __shared__ double part[kSqThreads];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kSqThreads / 2; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) err[int64_t(bb) * g.heads + hd] = part[0];
}

// Head-aware tile search, the choice (Veda page, "Head-Aware Tile Search"):
// per head, the candidate whose squared error summed over the batch (fp64,
// ascending batch index) is smallest; equal sums keep the lower candidate,
// and a NaN sum is never taken over a number. One thread per head.
__global__ void search_select_kernel(int32_t n_cand, int32_t B, int32_t heads, const double* __restrict__ err,
                                     double* __restrict__ err_sum, int32_t* __restrict__ best) {
  const int hd = blockIdx.x * blockDim.x + threadIdx.x;
  if (hd >= heads) return;
  int32_t pick = 0;
  double pick_s = __builtin_nan("");
  for (int32_t c = 0; c < n_cand; ++c) {
    double s = 0.0;
    for (int32_t b = 0; b < B; ++b) s += err[(int64_t(c) * B + b) * heads + hd];
    if (err_sum) err_sum[int64_t(c) * heads + hd] = s;
    if (s < pick_s || (pick_s != pick_s && s == s)) {
      pick = c;
      pick_s = s;
    }
  }
  best[hd] = pick;
}

// Mean of the per-query-tile KL over the rows that exist (b, hd, tq < nT_hd):
// one workgroup, fp64 per thread over a fixed stride, then a fixed tree
// order, so the value is reproducible.
constexpr int kMeanThreads = 1024;
__global__ __launch_bounds__(kMeanThreads) void distill_mean_kernel(GeoTable g, const float* __restrict__ kl_rows,
                                                                   double* __restrict__ mean) {
  double acc = 0.0;
  int64_t rows = 0;
  for (int b = 0; b < g.B; ++b)
    for (int hd = 0; hd < g.heads; ++hd) {
      const int32_t nT = g.h[hd].nT;
      const float* r = kl_rows + (int64_t(b) * g.heads + hd) * g.nT_max;
      for (int32_t t = threadIdx.x; t < nT; t += kMeanThreads) acc += double(r[t]);
      rows += nT;
    }
  __shared__ double part[kMeanThreads];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kMeanThreads / 2; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = part[0] / double(rows);
}

}  // namespace

hipError_t launch_search_select(int32_t n_cand, int32_t B, int32_t heads, const double* err, double* err_sum,
                                int32_t* best, hipStream_t s) {
  search_select_kernel<<<(heads + 63) / 64, 64, 0, s>>>(n_cand, B, heads, err, err_sum, best);
  return hipGetLastError();
}

hipError_t launch_distill_mean(const GeoTable& g, const float* kl_rows, double* mean, hipStream_t s) {
  distill_mean_kernel<<<1, kMeanThreads, 0, s>>>(g, kl_rows, mean);
  return hipGetLastError();
}

hipError_t launch_head_sq_error(const GeoTable& g, const uint16_t* a, int64_t sab, int64_t san, int64_t sah,
                                const uint16_t* b, int64_t sbb, int64_t sbn, int64_t sbh, double* err,
                                hipStream_t s) {
  head_sq_error_kernel<<<dim3(g.heads, g.B), kSqThreads, 0, s>>>(g, a, sab, san, sah, b, sbb, sbn, sbh, err);
  return hipGetLastError();
}

}  // namespace veda
