// Tile-skipping attention forward (Veda page, "Attention Structure
// Distillation", Execution: only the selected K/V tiles are fetched;
// Principle 03 "Tile-Sparse Kernel"; "Theoretical Rationale" 1 "Softmax
// Geometry": the row softmax over the kept keys, with its log-sum-exp).
//
// One workgroup (4 waves) computes one 128-query tile of one (batch, head).
// Wave w owns queries 32w..32w+31 and walks the tile's index list; for each
// selected key tile j:
//   S^T = K_j Q^T   32x32x16 bf16 MFMA, fp32 accumulate. Computing S
//                   transposed puts one query per lane (lanes l and l+32 hold
//                   the two halves of its 128 logits), so row max and row sum
//                   are in-lane plus one exchange between the half-waves.
//   online softmax  base-2 with scale*log2(e) folded into one FMA; pad keys of
//                   border tiles get -inf; rescale O by exp2(m_old - m_new).
//   O^T += V_j^T P^T  32x32x16 bf16 MFMA; P is rounded to bf16 and used in
//                   the very registers the softmax produced it in (the key
//                   order of the contraction is chosen to match them).
// K and V tiles (32 KiB each for d = 128) are double-buffered in LDS: the
// global loads of tile i+1 are in flight while tile i is computed. V is
// transposed on its way to LDS (an 8x8 register transpose per thread) so the
// PV operand reads are contiguous. Query tiles of a head are dealt out so that
// each XCD works on a contiguous run of neighbouring query tiles, whose key
// selections overlap, while all XCDs share the same head's K/V in the MALL.
#include "veda_internal.hpp"

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTok = VEDA_TILE_TOKENS;  // 128 keys / queries per tile
constexpr int kPadK = 8;                // LDS row padding (bf16 elements)

template <int D>
struct AttnShape {
  static constexpr int KS = D + kPadK;                 // K row stride in LDS (elements)
  static constexpr int VS = kTok + kPadK;              // V^T row stride in LDS (elements)
  static constexpr int kKPasses = kTok * D / 8 / kThreads;   // 16-byte K loads per thread
  static constexpr int kVBlocks = (kTok / 8) * (D / 8);      // 8x8 V blocks per tile
  static constexpr int kDC = D / 16;                   // MFMA k-steps over the head dim
  static constexpr int kDB = D / 32;                   // 32-row blocks of O^T
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16_rne(lo)) | (uint32_t(f32_to_bf16_rne(hi)) << 16);
}

// Query tile handled by workgroup x of a head: the tiles of a head are split
// into 8 contiguous runs, run r going to the workgroups x with x % 8 == r
// (consecutive workgroups land on consecutive XCDs). Bijective for any n.
__device__ __forceinline__ int32_t xcd_tile_order(int32_t x, int32_t n) {
  const int32_t xcd = x % 8, pos = x / 8, q = n / 8, r = n % 8;
  return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

template <int D>
__device__ __forceinline__ void load_kv(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                        u32x4 (&kreg)[AttnShape<D>::kKPasses], u32x4 (&vreg)[8]) {
  using S = AttnShape<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < S::kKPasses; ++p)
    kreg[p] = *reinterpret_cast<const u32x4*>(kt + (p * kThreads + t) * 8);
  if (t < S::kVBlocks) {
    const int kg = t / (D / 8), dg = t % (D / 8);
#pragma unroll
    for (int r = 0; r < 8; ++r) vreg[r] = *reinterpret_cast<const u32x4*>(vt + (kg * 8 + r) * D + dg * 8);
  }
}

template <int D>
__device__ __forceinline__ void store_kv(uint16_t* ks, uint16_t* vs, const u32x4 (&kreg)[AttnShape<D>::kKPasses],
                                         const u32x4 (&vreg)[8]) {
  using S = AttnShape<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < S::kKPasses; ++p) {
    const int e = (p * kThreads + t) * 8;  // element offset inside the dense tile
    *reinterpret_cast<u32x4*>(ks + (e / D) * S::KS + e % D) = kreg[p];
  }
  if (t < S::kVBlocks) {
    const int kg = t / (D / 8), dg = t % (D / 8);
    // vreg[r] holds V[8kg + r][8dg .. 8dg+7]; row i of the transpose is
    // V[8kg .. 8kg+7][8dg + i].
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = vreg[2 * p][i / 2], b = vreg[2 * p + 1][i / 2];
        o[p] = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(vs + (dg * 8 + i) * S::VS + kg * 8) = o;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_fwd_kernel(
    GeoTable g, const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, const int32_t* __restrict__ idx, int32_t k_max, float scale_log2,
    uint16_t* __restrict__ o_t, float* __restrict__ lse) {
  using S = AttnShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks_s[2][kTok * S::KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs_s[2][D * S::VS];

  const int hd = blockIdx.y, b = blockIdx.z;
  const HeadGeo hg = g.h[hd];
  const int32_t tq = xcd_tile_order(blockIdx.x, g.nT_max);
  const int64_t head_base = (int64_t(b) * g.heads + hd) * g.nT_max;
  const int64_t tile_elems = int64_t(kTok) * D;
  uint16_t* o_tile = o_t + (head_base + tq) * tile_elems;
  float* lse_tile = lse ? lse + (head_base + tq) * kTok : nullptr;

  if (tq >= hg.nT) {  // no such query tile for this head: defined zeros / -inf
    for (int e = threadIdx.x; e < kTok * D / 8; e += kThreads)
      reinterpret_cast<u32x4*>(o_tile)[e] = u32x4{0u, 0u, 0u, 0u};
    if (lse_tile)
      for (int e = threadIdx.x; e < kTok; e += kThreads) lse_tile[e] = -__builtin_inff();
    return;
  }

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int l32 = lane % 32, h = lane / 32;
  const int32_t* sel = idx + (head_base + tq) * k_max;
  const int kh = hg.k;
  const uint16_t* kbase = k_t + head_base * tile_elems;
  const uint16_t* vbase = v_t + head_base * tile_elems;

  // Q^T operand: lane (query 32w + l32, half h) holds d = 16dc + 8h .. +7.
  u32x4 qf[S::kDC];
  {
    const uint16_t* qrow = q_t + (head_base + tq) * tile_elems + (wave * 32 + l32) * D + 8 * h;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) qf[dc] = *reinterpret_cast<const u32x4*>(qrow + 16 * dc);
  }

  floatx16 oacc[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;

  // Entries outside [0, nT_hd) are skipped (they contribute no keys).
  u32x4 kreg[S::kKPasses], vreg[8];
  int32_t j = sel[0];
  if (unsigned(j) < unsigned(hg.nT)) {
    load_kv<D>(kbase + int64_t(j) * tile_elems, vbase + int64_t(j) * tile_elems, kreg, vreg);
    store_kv<D>(ks_s[0], vs_s[0], kreg, vreg);
  }
  __syncthreads();

  for (int i = 0; i < kh; ++i) {
    const int cur = i & 1;
    const int32_t jn = (i + 1 < kh) ? sel[i + 1] : -1;
    const bool jn_ok = unsigned(jn) < unsigned(hg.nT);
    if (jn_ok) load_kv<D>(kbase + int64_t(jn) * tile_elems, vbase + int64_t(jn) * tile_elems, kreg, vreg);
    if (unsigned(j) < unsigned(hg.nT)) {
    // S^T[kb]: keys 32kb + (8(v/4) + 4h + v%4), query l32.
    const uint16_t* ks = ks_s[cur];
    floatx16 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
#pragma unroll
      for (int dc = 0; dc < S::kDC; ++dc) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + (32 * kb + l32) * S::KS + 16 * dc + 8 * h);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[dc]), sacc[kb], 0, 0, 0);
      }
    }

    // Pad keys of a border tile take no part.
    const BoxExtent e = box_extent(g, hg, j);
    // Branch-free: the bias is +0 for a real key and -inf for a pad key,
    // built from integer compares (no per-element control flow).
    if (!box_is_full(hg, e)) {
      const int pwm = (1 << hg.lpw) - 1, phm = (1 << hg.lph) - 1, sh = hg.lpw + hg.lph;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int sig = 32 * kb + 8 * (v / 4) + 4 * h + (v % 4);
          const uint32_t real = uint32_t((sig & pwm) < e.vw) & uint32_t(((sig >> hg.lpw) & phm) < e.vh) &
                                uint32_t((sig >> sh) < e.vt);
          sacc[kb][v] += __uint_as_float((real - 1u) & 0xFF800000u);
        }
    }

    // Online softmax in base 2.
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    u32x4 pf[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], scale_log2, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v + 1], scale_log2, -m_new));
        psum += p0 + p1;
        pf[kb][v / 8][(v % 8) / 2] = pack_bf16x2(p0, p1);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

    // O^T[db] += V^T P^T over the 128 keys, 16 at a time: k-slot v' of half h
    // is key 32kb + 16c2 + 8(v'/4) + 4h + v'%4.
    const uint16_t* vs = vs_s[cur];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
        for (int db = 0; db < S::kDB; ++db) {
          const uint16_t* vrow = vs + (32 * db + l32) * S::VS + 32 * kb + 16 * c2 + 4 * h;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[kb][c2]), oacc[db], 0, 0, 0);
        }
      }
    }

    }  // valid tile
    if (jn_ok) store_kv<D>(ks_s[cur ^ 1], vs_s[cur ^ 1], kreg, vreg);
    j = jn;
    __syncthreads();
  }

  // Epilogue: combine the half-wave partial sums, normalise, write O and LSE.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  uint16_t* orow = o_tile + (wave * 32 + l32) * D;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * h) = w;
    }
  }
  if (lse_tile && h == 0) lse_tile[wave * 32 + l32] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
}

}  // namespace

hipError_t launch_sparse_attn(const GeoTable& g, const uint16_t* q_t, const uint16_t* k_t, const uint16_t* v_t,
                              const int32_t* idx, int32_t k_max, float scale, uint16_t* o_t, float* lse,
                              hipStream_t s) {
  const dim3 grid(g.nT_max, g.heads, g.B);
  const float scale_log2 = scale * 1.44269504088896340736f;
  if (g.d == 128)
    sparse_attn_fwd_kernel<128><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse);
  else
    sparse_attn_fwd_kernel<64><<<grid, kThreads, 0, s>>>(g, q_t, k_t, v_t, idx, k_max, scale_log2, o_t, lse);
  return hipGetLastError();
}

}  // namespace veda
