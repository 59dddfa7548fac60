// Tile-skipping attention forward (Veda page, "Attention Structure
// Distillation", Execution: only the selected K/V tiles are fetched;
// Principle 03 "Tile-Sparse Kernel"; "Theoretical Rationale" 1 "Softmax
// Geometry": the row softmax over the kept keys, with its log-sum-exp).
//
// One workgroup (8 waves) computes one 128-query tile of one (batch, head).
// Wave (qg, half) owns queries 32qg..32qg+31 and keys 64half..64half+63 of
// each tile, so two compute waves share each SIMD and one's softmax runs under
// the other's MFMAs; the key halves are merged once at the end. For each
// selected key tile j:
//   S^T = K_j Q^T   32x32x16 bf16 MFMA, fp32 accumulate. Computing S
//                   transposed puts one query per lane (lanes l and l+32 hold
//                   the two halves of its 128 logits), so row max and row sum
//                   are in-lane plus one exchange between the half-waves.
//   online softmax  base-2 with scale*log2(e) folded into one FMA; pad keys of
//                   border tiles get -inf through a branch-free bias. The
//                   running max only moves (and O is only rescaled) when a
//                   row's max grows by more than 2^8, so most tiles skip the
//                   rescale; P values up to 2^8 are exact in bf16's range.
//   O^T += V_j^T P^T  32x32x16 bf16 MFMA; P is rounded to bf16 (hardware
//                   pack) and used in the very registers the softmax produced
//                   it in (the key order of the contraction is chosen to match).
// K and V tiles (32 KiB each for d = 128) go global -> registers -> LDS; V is
// transposed on the way (each thread turns 16 keys x 4 channels into eight
// 16-byte chunks of V^T in MFMA key order) so each PV operand is one 16-byte
// read; the V^T rows are XOR-swizzled so chunk writes and operand reads are
// free of bank conflicts. The LDS tiles are double-buffered and the staging
// is pipelined two tiles deep (loads get a whole iteration to land; LDS
// stores run under the PV MFMAs). Query tiles of a head are dealt out so
// each XCD works on a contiguous run of neighbouring query tiles, whose key
// selections overlap, while all XCDs share the same head's K/V in the MALL.
#include "veda_internal.hpp"

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;           // 8 waves: 4 query groups x 2 key halves
constexpr int kHalfThreads = kThreads / 2;
constexpr int kTok = VEDA_TILE_TOKENS;  // 128 keys / queries per tile
constexpr int kPadK = 8;                // LDS row padding (bf16 elements)
constexpr float kRescaleSlack = 8.0f;   // log2 of the largest unnormalised P

template <int D>
struct AttnShape {
  static constexpr int KS = D + kPadK;                  // K row stride in LDS (elements)
  static constexpr int kKPasses = kTok * D / 8 / kHalfThreads;  // 16-byte K loads per K-staging thread
  static constexpr int kVQuads = D / 4;                 // 4-channel groups of V
  static constexpr int kVBlocks = (kTok / 16) * kVQuads;        // 16-key x 4-channel V blocks per tile
  static constexpr int kDC = D / 16;                    // MFMA k-steps over the head dim
  static constexpr int kDB = D / 32;                    // 32-row blocks of O^T
  static_assert(kKPasses <= 8 && kVBlocks <= kHalfThreads, "staging layout");
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// V^T in LDS: row d (a channel) holds the tile's 128 keys as 16 chunks of 16
// bytes. Chunk c = 2G + h holds keys 16G + 4h + {0..3} and 16G + 8 + 4h + {0..3},
// exactly the eight keys lane half h feeds to one PV MFMA; it is stored at
// position c ^ swz(d). swz makes both the chunk writes (rows 4q + i, 16 or 8
// consecutive q) and the operand reads (16 or 8 consecutive rows) hit distinct
// bank groups for 64 and for 32 LDS banks.
__device__ __forceinline__ int vt_swizzle(int d) {
  return ((d ^ (d >> 3)) & 3) | (d & 4) | ((((d >> 3) ^ (d >> 5)) & 1) << 3);
}

// Query tile handled by workgroup x of a head: the tiles of a head are split
// into 8 contiguous runs, run r going to the workgroups x with x % 8 == r
// (consecutive workgroups land on consecutive XCDs). Bijective for any n.
__device__ __forceinline__ int32_t xcd_tile_order(int32_t x, int32_t n) {
  const int32_t xcd = x % 8, pos = x / 8, q = n / 8, r = n % 8;
  return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

// Staging of the next K/V tile, specialised by role so that the staging
// registers are written on one path only: waves 0-3 stage K (kKPasses
// 16-byte row pieces per thread), waves 4-7 stage V as 16-key x 4-channel
// blocks (16 rows of 8 bytes; rows 2m and 2m+1 share st[m]).
template <int D, bool kStageK>
struct Stager {
  using S = AttnShape<D>;
  u32x4 st[8];
  int t;  // thread index within the staging half (0..255)

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt) {
    if constexpr (kStageK) {
#pragma unroll
      for (int p = 0; p < S::kKPasses; ++p) st[p] = *reinterpret_cast<const u32x4*>(kt + (p * kHalfThreads + t) * 8);
    } else if (t < S::kVBlocks) {
      const int dq = t % S::kVQuads, kg = t / S::kVQuads;
      const uint16_t* src = vt + (16 * kg) * D + 4 * dq;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(src + (2 * m) * D);
        const u32x2 c = *reinterpret_cast<const u32x2*>(src + (2 * m + 1) * D);
        st[m] = u32x4{a[0], a[1], c[0], c[1]};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* ks, uint16_t* vs) const {
    if constexpr (kStageK) {
#pragma unroll
      for (int p = 0; p < S::kKPasses; ++p) {
        const int e = (p * kHalfThreads + t) * 8;  // element offset inside the dense tile
        *reinterpret_cast<u32x4*>(ks + (e / D) * S::KS + e % D) = st[p];
      }
    } else if (t < S::kVBlocks) {
      const int dq = t % S::kVQuads, kg = t / S::kVQuads;
      // Channel 4dq + i of key row r (0..15) is 16-bit half i%2 of dword
      // 2(r%2) + i/2 of st[r/2].
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 4 * dq + i;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 o;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int ra = (p < 2 ? 4 * hh : 8 + 4 * hh) + 2 * (p % 2), rb = ra + 1;
            const uint32_t a = st[ra / 2][2 * (ra % 2) + i / 2], c = st[rb / 2][2 * (rb % 2) + i / 2];
            o[p] = (i & 1) ? ((a >> 16) | (c & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c << 16));
          }
          *reinterpret_cast<u32x4*>(vs + d * kTok + (((2 * kg + hh) ^ vt_swizzle(d)) * 8)) = o;
        }
      }
    }
  }
};

// Per-wave state of the online softmax for 32 queries x one key half.
template <int D>
struct WaveState {
  using S = AttnShape<D>;
  u32x4 qf[S::kDC];      // Q^T operand: d = 16dc + 8h .. +7 of query l32
  floatx16 oacc[S::kDB];  // O^T partial: d = 32db + 8(v/4) + 4h + v%4, query l32
  float m_run, l_run;     // running max (base 2, scaled) and partial sum
};

// One selected key tile j for one wave: S^T, mask, online softmax, PV.
// after_s() runs once the S^T MFMAs are issued and after_pv() once the PV
// MFMAs are issued, so staging work placed there overlaps the matrix cores.
template <int D, class AfterS, class AfterPV>
__device__ __forceinline__ void attend_tile(WaveState<D>& w, const uint16_t* ks, const uint16_t* vs,
                                            const GeoTable& g, const HeadGeo& hg, int32_t j, int half, int h,
                                            int l32, float scale_log2, AfterS&& after_s, AfterPV&& after_pv) {
  using S = AttnShape<D>;
  // S^T[kb]: keys 64half + 32kb + (8(v/4) + 4h + v%4), query l32.
  floatx16 sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
    const uint16_t* krow = ks + (64 * half + 32 * kb + l32) * S::KS + 8 * h;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 16 * dc);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(w.qf[dc]), sacc[kb], 0, 0, 0);
    }
  }
  after_s();

  // Pad keys of a border tile get -inf: the box's real-slot mask is built
  // once per tile with uniform ops; each lane pulls its bits (its keys are
  // bits 32kb + 8(v/4) + v%4 of the mask shifted by 64half + 4h).
  const BoxExtent e = box_extent(g, hg, j);
  if (!box_is_full(hg, e)) {
    const uint64_t wm = box_slot_mask64(hg, e, 64 * half) >> (4 * h);
    const uint32_t wlo = uint32_t(wm), whi = uint32_t(wm >> 32);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t real = ((kb ? whi : wlo) >> (8 * (v / 4) + (v % 4))) & 1u;
        sacc[kb][v] += __uint_as_float((real - 1u) & 0xFF800000u);
      }
  }

  // Online softmax in base 2 with a lazily moved running max.
  float mx = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mx > w.m_run + kRescaleSlack) != 0) {
    const float m_new = fmaxf(w.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) w.oacc[db][v] *= alpha;
  }
  // A half that has seen only pad keys so far keeps m = -inf; its exponents
  // must then still be exp2(-inf) = 0, not NaN.
  const float m_use = w.m_run == -__builtin_inff() ? 0.0f : w.m_run;
  float psum = 0.0f;
  u32x4 pf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], scale_log2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v + 1], scale_log2, -m_use));
      psum += p0 + p1;
      pf[kb][v / 8][(v % 8) / 2] = pack_bf16x2(p0, p1);
    }
  }
  w.l_run += psum;

  // O^T[db] += V^T P^T over this half's 64 keys, 16 at a time: k-slot v' of
  // half-wave h is key 64half + 32kb + 16c2 + 8(v'/4) + 4h + v'%4, i.e.
  // chunk 2G + h of group G = 4half + 2kb + c2 in the V^T rows.
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    const int d = 32 * db + l32;
    const int t0 = (8 * half + h) ^ vt_swizzle(d);
    const uint16_t* vrow = vs + d * kTok;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vrow + ((t0 ^ (4 * kb + 2 * c2)) * 8));
        w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[kb][c2]), w.oacc[db], 0, 0, 0);
      }
    }
  }
  after_pv();
}

// The tile loop of one wave; kStageK selects which half of each tile this
// wave stages. Staging is pipelined two tiles deep: during iteration i the
// staging registers hold tile i+1, loaded at the end of iteration i-1; once
// the PV MFMAs of tile i are issued they go to the free LDS buffer and the
// loads of tile i+2 start, so every load has a whole iteration to land and
// the LDS stores run under the PV MFMAs. Every thread runs the same number of iterations and barriers.
template <int D, bool kStageK>
__device__ __forceinline__ void attend_all(WaveState<D>& w, uint16_t (&ks_s)[2][kTok * AttnShape<D>::KS],
                                           uint16_t (&vs_s)[2][D * kTok], const GeoTable& g, const HeadGeo& hg,
                                           const int32_t* sel, const uint16_t* kbase, const uint16_t* vbase,
                                           int half, int h, int l32, float scale_log2) {
  const int64_t tile_elems = int64_t(kTok) * D;
  const unsigned nT = unsigned(hg.nT);
  const int kh = hg.k;
  Stager<D, kStageK> stg;
  stg.t = threadIdx.x % kHalfThreads;
  // Entries outside [0, nT_hd) contribute no keys; tile 0 stands in as a
  // harmless load source so every load is unconditional.
  auto src = [&](int32_t jt) { return unsigned(jt) < nT ? jt : 0; };
  int32_t j = sel[0];
  stg.load(kbase + int64_t(src(j)) * tile_elems, vbase + int64_t(src(j)) * tile_elems);
  stg.store(ks_s[0], vs_s[0]);
  int32_t jn = kh > 1 ? sel[1] : 0;
  stg.load(kbase + int64_t(src(jn)) * tile_elems, vbase + int64_t(src(jn)) * tile_elems);
  __syncthreads();
  for (int i = 0; i < kh; ++i) {
    const int cur = i & 1;
    const bool has_next = i + 1 < kh;
    const int32_t jnn = i + 2 < kh ? sel[i + 2] : 0;
    auto nothing = [] {};
    auto restage = [&] {  // tile i+1 -> free LDS buffer, then start loading tile i+2
      if (has_next) stg.store(ks_s[cur ^ 1], vs_s[cur ^ 1]);
      stg.load(kbase + int64_t(src(jnn)) * tile_elems, vbase + int64_t(src(jnn)) * tile_elems);
    };
    if (unsigned(j) < nT)
      attend_tile<D>(w, ks_s[cur], vs_s[cur], g, hg, j, half, h, l32, scale_log2, nothing, restage);
    else
      restage();
    j = jn;
    jn = jnn;
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_fwd_kernel(
    GeoTable g, const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, const int32_t* __restrict__ idx, int32_t k_max, float scale_log2,
    uint16_t* __restrict__ o_t, float* __restrict__ lse) {
  using S = AttnShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks_s[2][kTok * S::KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs_s[2][D * kTok];

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

  // Wave (qg, half): queries 32qg..32qg+31 against keys 64half..64half+63 of
  // every selected tile; the two halves are merged at the end.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int qg = wave & 3, half = wave >> 2;
  const int l32 = lane % 32, h = lane / 32;
  const int32_t* sel = idx + (head_base + tq) * k_max;
  const uint16_t* kbase = k_t + head_base * tile_elems;
  const uint16_t* vbase = v_t + head_base * tile_elems;

  WaveState<D> w;
  {
    const uint16_t* qrow = q_t + (head_base + tq) * tile_elems + (qg * 32 + l32) * D + 8 * h;
#pragma unroll
    for (int dc = 0; dc < S::kDC; ++dc) w.qf[dc] = *reinterpret_cast<const u32x4*>(qrow + 16 * dc);
  }
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) w.oacc[db][v] = 0.0f;
  w.m_run = -__builtin_inff();
  w.l_run = 0.0f;
  // Let Q land before the loop, so no wait on it inside the loop can drain
  // the in-order counter that the staging loads share.
  __builtin_amdgcn_s_waitcnt(0);

  if (wave < 4)
    attend_all<D, true>(w, ks_s, vs_s, g, hg, sel, kbase, vbase, half, h, l32, scale_log2);
  else
    attend_all<D, false>(w, ks_s, vs_s, g, hg, sel, kbase, vbase, half, h, l32, scale_log2);

  // Merge the two key halves through LDS (the K/V buffers are free now):
  // m = max(m0, m1), O = O0 2^(m0-m) + O1 2^(m1-m), l likewise.
  float* red = reinterpret_cast<float*>(&ks_s[0][0]);       // [4][kDB*16][64] partial O^T
  float* red_ml = red + 4 * S::kDB * 16 * 64;                // [4][2][64] m, l
  static_assert(sizeof(ks_s) >= (4 * S::kDB * 16 * 64 + 4 * 2 * 64) * sizeof(float), "merge space");
  const float l_half = w.l_run + __shfl_xor(w.l_run, 32, 64);
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((qg * S::kDB + db) * 16 + v) * 64 + lane] = w.oacc[db][v];
    red_ml[(qg * 2 + 0) * 64 + lane] = w.m_run;
    red_ml[(qg * 2 + 1) * 64 + lane] = l_half;
  }
  __syncthreads();
  if (half == 0) {
    const float m1 = red_ml[(qg * 2 + 0) * 64 + lane];
    const float l1 = red_ml[(qg * 2 + 1) * 64 + lane];
    const float m = fmaxf(w.m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(w.m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float l_tot = l_half * a0 + l1 * a1;
    const float inv = 1.0f / l_tot;
    const float c0 = a0 * inv, c1 = a1 * inv;
    uint16_t* orow = o_tile + (qg * 32 + l32) * D;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) {
      float o[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) o[v] = w.oacc[db][v] * c0 + red[((qg * S::kDB + db) * 16 + v) * 64 + lane] * c1;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 wd;
        wd[0] = pack_bf16x2(o[4 * g4 + 0], o[4 * g4 + 1]);
        wd[1] = pack_bf16x2(o[4 * g4 + 2], o[4 * g4 + 3]);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * h) = wd;
      }
    }
    if (lse_tile && h == 0) lse_tile[qg * 32 + l32] = (m + __log2f(l_tot)) * 0.69314718055994530942f;
  }
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
