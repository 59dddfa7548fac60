"""CPU oracle for the Veda tile-sparse self-attention forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry
point and the CPU-baseline leg of the benchmark may import or run this module.
It shares no code with the HIP path (no kernels, headers, helpers or tables):
it is plain numpy, written from the method's definition, slow on purpose, and
each function names the passage it follows. Sources:

  [Veda]  "Veda: Scalable Video Diffusion via Distilled Sparse Attention"
          project page (veda-sparse.github.io)
  [News]  mlllm.io article on Veda, section "What happened"

Where the pages leave a step open, the reading used is stated in the function
that implements it. Numerics: inputs are bfloat16 values held in float32/64;
attention runs in float64; the tile statistics, projections and scores follow
the fp32 evaluation order stated below, so that the tile mask is reproducible
bit for bit.

Parity pins: every function here is checked by the CPU test suite against
hand-derived fixtures, brute force, closed forms, library routines or the
pages' inequalities; none is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

Grid = Tuple[int, int, int]
Tile = Tuple[int, int, int]


# --------------------------------------------------------------------------
# bfloat16 helpers (own implementation; the oracle holds bf16 values in f32)
# --------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value reached bf16 rounding")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit pattern of values that are already bf16-representable."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value is not representable in bfloat16")
    return (u >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# O1: head-conditioned tiling ([Veda] "Architecture", Principle 02
# "Head-Conditioned Tile Geometry"; "Head-Aware Tile Search": p_t*p_h*p_w = B;
# [News] "What happened": 128-token key tiles)
# --------------------------------------------------------------------------

def tile_counts(grid: Grid, tile: Tile) -> Tuple[int, int, int]:
    """Boxes along (t, h, w) when each axis is padded up to a multiple of the
    tile edge (reading: per-axis padding; flat padding cannot form 3D boxes)."""
    (T, H, W), (pt, ph, pw) = grid, tile
    return (-(-T // pt), -(-H // ph), -(-W // pw))


def num_tiles(grid: Grid, tile: Tile) -> int:
    a, b, c = tile_counts(grid, tile)
    return a * b * c


def tiled_position(grid: Grid, tile: Tile) -> np.ndarray:
    """For every token n of the raster (n = (t*H + y)*W + x), its position
    p = vol*tau + sigma in the tiled sequence.

    Readings: tiles are numbered in raster order of their box coordinates,
    tau = ((t//pt)*nTh + y//ph)*nTw + x//pw, and tokens inside a box in raster
    order of their offsets, sigma = ((t%pt)*ph + y%ph)*pw + x%pw.
    """
    T, H, W = grid
    pt, ph, pw = tile
    _, nTh, nTw = tile_counts(grid, tile)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    tau = ((t // pt) * nTh + y // ph) * nTw + x // pw
    sigma = ((t % pt) * ph + y % ph) * pw + x % pw
    return (tau * (pt * ph * pw) + sigma).astype(np.int64)


def tile_permute(x: np.ndarray, grid: Grid, tile: Tile) -> Tuple[np.ndarray, np.ndarray]:
    """Gather a raster sequence x[N, ...] into tiled order [nT*vol, ...].

    Pad slots (positions no real token maps to) hold 0. Returns the tiled
    array and the boolean validity of each tiled slot.
    """
    vol = tile[0] * tile[1] * tile[2]
    nT = num_tiles(grid, tile)
    pos = tiled_position(grid, tile)
    out = np.zeros((nT * vol,) + x.shape[1:], dtype=x.dtype)
    valid = np.zeros(nT * vol, dtype=bool)
    out[pos] = x
    valid[pos] = True
    return out, valid


def tile_unpermute(xt: np.ndarray, grid: Grid, tile: Tile) -> np.ndarray:
    """Inverse of tile_permute: raster x[n] = xt[p(n)]; pad slots are dropped."""
    return xt[tiled_position(grid, tile)]


# --------------------------------------------------------------------------
# O2: TripPool ([Veda] "Attention Structure Distillation", Estimator: average,
# maximum and minimum statistics; "Theoretical Rationale" 2, "Tile Statistics")
# --------------------------------------------------------------------------

def trippool(xt: np.ndarray, valid: np.ndarray, vol: int = 128) -> np.ndarray:
    """Per tile and channel: [avg | max | min] over the tile's real tokens.

    xt: tiled values [nT*vol, d] (bf16 values in float32); valid: [nT*vol].
    Readings: the three statistics are concatenated along channels (3d
    features). The mean is a float32 sum taken slot by slot in ascending slot
    order starting from +0, divided (correctly rounded, float32) by the
    number of real tokens, and rounded to bfloat16. Max and min are exact.
    Pad slots take no part.
    """
    xt = np.asarray(xt, dtype=np.float32)
    d = xt.shape[1]
    nT = xt.shape[0] // vol
    x3 = xt.reshape(nT, vol, d)
    v3 = valid.reshape(nT, vol)
    s = np.zeros((nT, d), dtype=np.float32)
    for sigma in range(vol):
        add = (s + x3[:, sigma, :]).astype(np.float32)
        s = np.where(v3[:, sigma, None], add, s)
    n = v3.sum(axis=1).astype(np.float32)
    if np.any(n == 0):
        raise ValueError("tile without real tokens")
    avg = bf16_round((s / n[:, None]).astype(np.float32))
    # Max and min in the IEEE total order, so that -0 < +0 (only the sign of
    # a zero extremum depends on this reading).
    key = _total_order_key(x3)
    big = np.int32(1 << 20)
    mx = _from_total_order_key(np.where(v3[:, :, None], key, -big).max(axis=1))
    mn = _from_total_order_key(np.where(v3[:, :, None], key, big).min(axis=1))
    return np.concatenate([avg, mx, mn], axis=1)


def _total_order_key(x: np.ndarray) -> np.ndarray:
    """Integer key of bf16 values that orders them like the IEEE total order
    (-0 just below +0)."""
    b = float_to_bf16_bits(x).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag - 1, mag).astype(np.int32)


def _from_total_order_key(key: np.ndarray) -> np.ndarray:
    bits = np.where(key >= 0, key, 0x8000 | (-key - 1)).astype(np.uint16)
    return bf16_bits_to_float(bits)


# --------------------------------------------------------------------------
# O3/O4: head-specific projections and tile scores ([Veda] "Attention
# Structure Distillation", Estimator: TripPool + head-specific Q/K projections
# give the tile scores; "Theoretical Rationale" 4: the estimator's scores
# define the distribution that Top-k thresholds)
# --------------------------------------------------------------------------

def fp32_dot_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C[i, j] = sum_c a[i, c] * b[c, j], accumulated in float32 one term at a
    time in ascending c, starting from +0.

    With bfloat16 operands every product is exact in float32, so each step is
    a single float32 rounding of (partial sum + product).
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    acc = np.zeros((a.shape[0], b.shape[1]), dtype=np.float32)
    for c in range(a.shape[1]):
        prod = (a[:, c:c + 1] * b[c:c + 1, :]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    return acc


def project(stats: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Features P = bf16(stats @ W) for one head; stats [nT, 3d], W [3d, r].
    Reading: a plain linear map per head and per side (Q or K), no bias."""
    return bf16_round(fp32_dot_rows(stats, w))


def tile_scores(feat_q: np.ndarray, feat_k: np.ndarray) -> np.ndarray:
    """S[i, j] = <P^Q_i, P^K_j> in float32 (reading: no scale, no bias)."""
    return fp32_dot_rows(feat_q, np.ascontiguousarray(np.asarray(feat_k, np.float32).T))


def avgpool_scores(stats_q: np.ndarray, stats_k: np.ndarray) -> np.ndarray:
    """Average-pooling tile scores, the baseline the pages set Veda's mask
    against at the same budget ([Veda] "Empirical Study", 02 "Controlled Mask
    Intervention"): S[i, j] = <mean of query tile i, mean of key tile j> over
    all d channels, i.e. the avg block of the TripPool statistics alone, with
    no projection. Reading: the same float32 evaluation order as the
    estimator's scores (ascending channel, from +0), so that its Top-k mask is
    reproducible bit for bit."""
    d = np.asarray(stats_q).shape[1] // 3
    mq = np.asarray(stats_q, np.float32)[:, :d]
    mk = np.asarray(stats_k, np.float32)[:, :d]
    return fp32_dot_rows(mq, np.ascontiguousarray(mk.T))


# --------------------------------------------------------------------------
# O5: head-aware Top-k ([Veda] "Attention Structure Distillation", Execution:
# Top-k selection per query tile gives the tile mask)
# --------------------------------------------------------------------------

def topk_row_bruteforce(row: Sequence[float], k: int) -> List[int]:
    """The k key tiles with the largest scores, ties to the lower index, in
    ascending index order. Python float comparison treats -0.0 == +0.0."""
    order = sorted(range(len(row)), key=lambda j: (-float(row[j]), j))
    return sorted(order[:k])


def topk(S: np.ndarray, k: int) -> np.ndarray:
    """Row-wise Top-k of S[nQ, nK] -> int64 [nQ, k], ascending per row.

    A stable sort on the negated score keeps equal scores (and -0 vs +0) in
    index order, which is the lower-index tie rule.
    """
    S = np.asarray(S, dtype=np.float32)
    order = np.argsort(-S, axis=1, kind="stable")[:, :k]
    return np.sort(order, axis=1)


def bitmask(idx: np.ndarray, n_keys: int) -> np.ndarray:
    """Pack selected key-tile indices into uint32 words: bit j%32 of word j//32."""
    words = -(-n_keys // 32)
    out = np.zeros((idx.shape[0], words), dtype=np.uint64)
    for row in range(idx.shape[0]):
        for j in idx[row]:
            if j >= 0:
                out[row, j // 32] |= np.uint64(1) << np.uint64(j % 32)
    return out.astype(np.uint32)


# --------------------------------------------------------------------------
# O6: tile-skipping attention ([Veda] "Attention Structure Distillation",
# Execution: only the selected K/V tiles are fetched; "Theoretical Rationale"
# 1, "Softmax Geometry": each row is a softmax over the kept keys, which
# renormalises them by Z / Z_hat; the log-sum-exp potential gives the LSE)
# --------------------------------------------------------------------------

def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, grid: Grid, tile: Tile,
                     sel: np.ndarray, scale: float, query_tiles: Sequence[int] = None
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Raster-order attention in which a query of tile i sees exactly the real
    keys whose tile is listed in sel[i] (sel entries < 0 are ignored).

    q, k, v: [N, d] raster order (any float dtype; upcast to float64).
    Returns o [N, d] float64 and lse [N] float64 (natural log, logits already
    multiplied by `scale`). Only the queries of `query_tiles` (default: all)
    are computed; the other rows are NaN.
    Readings: no causal mask; softmax base e with temperature 1; pad tokens
    are not keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    vol = tile[0] * tile[1] * tile[2]
    tile_of = tiled_position(grid, tile) // vol           # tile index of each raster token
    nT = num_tiles(grid, tile)
    members = [np.flatnonzero(tile_of == t) for t in range(nT)]
    o = np.full((q.shape[0], v.shape[1]), np.nan)
    lse = np.full(q.shape[0], np.nan)
    tiles = range(nT) if query_tiles is None else query_tiles
    for i in tiles:
        qi = members[i]
        keys = np.concatenate([members[j] for j in sel[i] if j >= 0])
        u = (q[qi] @ k[keys].T) * scale
        m = u.max(axis=1, keepdims=True)
        e = np.exp(u - m)
        z = e.sum(axis=1, keepdims=True)
        o[qi] = (e @ v[keys]) / z
        lse[qi] = (m + np.log(z))[:, 0]
    return o, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Full softmax attention over all N keys (the case the sparse layer
    reduces to when every key tile is kept)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    u = (q @ k.T) * scale
    m = u.max(axis=1, keepdims=True)
    e = np.exp(u - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ v) / z, (m + np.log(z))[:, 0]


# --------------------------------------------------------------------------
# Teacher, oracle mask and tile recall ([Veda] "Attention Structure
# Distillation", Teacher: max-pooling the full attention map gives tile-level
# supervision; Principle 01 "Full-Attention Structure Distillation";
# "Empirical Study" 02: the oracle mask keeps each query tile's
# highest-response key tiles, and tile recall measures how many of them a
# mask keeps)
# --------------------------------------------------------------------------

def teacher_tile_max(q: np.ndarray, k: np.ndarray, grid: Grid, tile: Tile, scale: float,
                     query_tiles: Sequence[int] = None) -> np.ndarray:
    """Max-pooled full attention: T[i, j] is the largest dense softmax
    probability between a real query of tile i and a real key of tile j.

    q, k: [N, d] raster order. Each query's softmax runs over all N real
    keys (no mask), in float64. Rows of tiles not in `query_tiles` (default:
    all) are NaN. Reading: the pooling window is one (query tile, key tile)
    block of the attention map, and pad slots take no part.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vol = tile[0] * tile[1] * tile[2]
    tile_of = tiled_position(grid, tile) // vol
    nT = num_tiles(grid, tile)
    T = np.full((nT, nT), np.nan)
    tiles = range(nT) if query_tiles is None else query_tiles
    for i in tiles:
        qi = np.flatnonzero(tile_of == i)
        u = (q[qi] @ k.T) * scale
        m = u.max(axis=1, keepdims=True)
        p = np.exp(u - m)
        p /= p.sum(axis=1, keepdims=True)
        best = p.max(axis=0)                       # per key: its largest probability over the tile's queries
        for j in range(nT):
            T[i, j] = best[tile_of == j].max()
    return T


def mask_overlap(bitmask_a: np.ndarray, bitmask_b: np.ndarray) -> int:
    """Number of (query tile, key tile) pairs kept by both masks."""
    both = np.asarray(bitmask_a, dtype=np.uint32) & np.asarray(bitmask_b, dtype=np.uint32)
    return int(np.unpackbits(both.view(np.uint8)).sum())


def tile_recall(idx_mask: np.ndarray, idx_oracle: np.ndarray) -> float:
    """Share of the oracle mask's kept tiles that the mask also keeps
    (index lists [nT, k]; entries < 0 ignored)."""
    hit = total = 0
    for row_m, row_o in zip(idx_mask, idx_oracle):
        o = set(int(x) for x in row_o if x >= 0)
        hit += len(o & set(int(x) for x in row_m if x >= 0))
        total += len(o)
    return hit / total


# --------------------------------------------------------------------------
# Head-aware tile search ([Veda] "Head-Aware Tile Search": candidate tile
# shapes keep p_t*p_h*p_w = 128; each head takes the one that minimises the
# squared Frobenius norm of O_full - O_sparse on calibration samples;
# Principle 02 "Head-Conditioned Tile Geometry")
# --------------------------------------------------------------------------

def tile_search_errors(q: np.ndarray, k: np.ndarray, v: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                       grid: Grid, candidates: Sequence[Tile], k_of, scale: float = None) -> np.ndarray:
    """||O_dense - O_sparse(tile)||_F^2 of one head for every candidate tile,
    where O_sparse runs the whole layer (tiling, TripPool estimator, Top-k
    with k = k_of(nT)) and O_dense is full softmax attention."""
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_dense, _ = dense_attention(q, k, v, scale)
    errs = []
    for tile in candidates:
        r = head_forward(q, k, v, wq, wk, grid, tile, k_of(num_tiles(grid, tile)), scale)
        errs.append(float(((r["o"] - o_dense) ** 2).sum()))
    return np.array(errs)


# --------------------------------------------------------------------------
# Distillation objective ([Veda] "Theoretical Rationale" 4, "Distillation
# Objective": the estimator's soft tile distribution is aligned with the
# max-pooled full-attention target by D_KL(A_tgt || A_pred) before Top-k;
# Principle 01 "Full-Attention Structure Distillation")
# --------------------------------------------------------------------------

def distill_kl(S: np.ndarray, T: np.ndarray, grad_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One head's rows (query tiles) over its key tiles: A_tgt = T row
    normalised to sum 1, A_pred = softmax(S row); returns the per-row KL
    divergence and grad_scale * dKL/dS = grad_scale * (A_pred - A_tgt).
    Readings: the target is the teacher row normalised (the pages give no
    other normalisation); the estimator's distribution is the softmax of its
    scores at temperature 1."""
    S = np.asarray(S, np.float64)
    T = np.asarray(T, np.float64)
    a_t = T / T.sum(axis=1, keepdims=True)
    m = S.max(axis=1, keepdims=True)
    log_p = S - m - np.log(np.exp(S - m).sum(axis=1, keepdims=True))
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(a_t > 0, a_t * (np.log(a_t) - log_p), 0.0)
    return terms.sum(axis=1), grad_scale * (np.exp(log_p) - a_t)


def distill_grad(stats_q: np.ndarray, stats_k: np.ndarray, feat_q: np.ndarray, feat_k: np.ndarray,
                 dS: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Back from dL/dS through S = F_q F_k^T and F = stats W to dL/dW_q and
    dL/dW_k (one head, one batch element), in float64."""
    dS = np.asarray(dS, np.float64)
    dFq = dS @ np.asarray(feat_k, np.float64)
    dFk = dS.T @ np.asarray(feat_q, np.float64)
    return np.asarray(stats_q, np.float64).T @ dFq, np.asarray(stats_k, np.float64).T @ dFk


def distill_loss(stats_q: np.ndarray, stats_k: np.ndarray, wq: np.ndarray, wk: np.ndarray, T: np.ndarray) -> float:
    """Summed KL of one head with the features computed exactly (no bf16
    rounding): the function whose derivative distill_kl + distill_grad give."""
    S = (np.asarray(stats_q, np.float64) @ wq) @ (np.asarray(stats_k, np.float64) @ wk).T
    return float(distill_kl(S, T)[0].sum())


def adam_step(w: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, step: int, lr: float,
              beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8):
    """Bias-corrected Adam (Kingma and Ba), float64; returns new (w, m, v)."""
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    mh = m / (1 - beta1 ** step)
    vh = v / (1 - beta2 ** step)
    return w - lr * mh / (np.sqrt(vh) + eps), m, v


# --------------------------------------------------------------------------
# The whole layer, one head at a time
# --------------------------------------------------------------------------

def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                 grid: Grid, tile: Tile, topk_k: int, scale: float = None,
                 query_tiles: Sequence[int] = None) -> Dict[str, np.ndarray]:
    """Run O1-O7 for one (batch, head): raster q/k/v [N, d] (bf16 values as
    float32), W [3d, r]. Returns every intermediate the layer produces:

      qt, kt, vt  tiled inputs [nT*128, d]; valid [nT*128]
      stats_q, stats_k [nT, 3d]; feat_q, feat_k [nT, r]; scores [nT, nT]
      idx [nT, k] ascending; bitmask [nT, ceil(nT/32)]
      o [N, d], lse [N] in raster order (float64)
    """
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vol = tile[0] * tile[1] * tile[2]
    nT = num_tiles(grid, tile)
    qt, valid = tile_permute(q, grid, tile)
    kt, _ = tile_permute(k, grid, tile)
    vt, _ = tile_permute(v, grid, tile)
    stats_q = trippool(qt, valid, vol)
    stats_k = trippool(kt, valid, vol)
    feat_q = project(stats_q, wq)
    feat_k = project(stats_k, wk)
    S = tile_scores(feat_q, feat_k)
    idx = topk(S, topk_k)
    o, lse = sparse_attention(q, k, v, grid, tile, idx, scale, query_tiles)
    return dict(qt=qt, kt=kt, vt=vt, valid=valid, stats_q=stats_q, stats_k=stats_k,
                feat_q=feat_q, feat_k=feat_k, scores=S, idx=idx,
                bitmask=bitmask(idx, nT), o=o, lse=lse)
