"""Veda tile-sparse self-attention forward on AMD MI355X (gfx950).

Python face of libveda.so. Each function allocates its outputs with torch on
the inputs' device, passes raw pointers and torch's current HIP stream to the
C ABI, and raises VedaError on a non-zero status. No computation happens in
Python: the five steps of the layer are HIP kernels.

  tile_permute     raster [B, N, heads, d] -> tiled [B, heads, nT_max, 128, d]
                   (token-major) or [B, heads, nT_max, d, 128] (channel-major)
  trippool_score   tiled Q, K + W_q, W_k  -> stats, features, tile scores
  topk_mask        scores -> ascending index lists (+ bitmask) per query tile
  sparse_attn_fwd  tiled Q, K, V + index lists -> tiled O (+ LSE)
  tile_unpermute   tiled -> raster
  tile_permute_stats      raster Q or K -> token-major tiles + TripPool stats, one pass
  trippool_project_score  stats + W_q, W_k -> features, tile scores (or the features alone)
  score_topk       features -> the tile scores and their Top-k in one pass, with no score matrix
  tile_scores_mfma the same scores from the features on the matrix cores (within rounding, not
                   bit-identical; the layer keeps the ordered scores)
  sparse_attn_fwd_raster  sparse_attn_fwd writing raster O (no unpermute pass)
  tile_stats       the TripPool statistics of raster Q or K alone (no tiled copy)
  sparse_attn_fwd_raster_io  sparse_attn_fwd_raster reading raster Q (no tiled Q)
  sparse_attn_fwd_raster_io_noalloc  the same with the library's static work queue: allocates nothing
  attn_queue       workspace of the attention calls' work queue (query tiles handed out at run time)
  layer_forward    the layer: tile_stats of Q, tile_permute_stats of K, tile_permute
                   of V, trippool_project_score (features), score_topk, sparse_attn_fwd_raster_io

Dense attention (the baseline) and measuring a mask against the method's own target:
  dense_attn_fwd   every key tile kept, no index list (tiled O + LSE; dense_attn_fwd_raster: raster O)
  dense_index      index lists that keep every key tile (dense attention through sparse_attn_fwd)
  teacher_tile_max max-pooled dense attention per (query tile, key tile); topk_mask of it is the
                   oracle tile mask
  avgpool_score    average-pooling tile scores (the pages' baseline mask at the same budget)
  mask_overlap     kept tiles two masks have in common, per (batch, head)
  tile_recall      those kept tiles over the oracle mask's k_hd * nT_hd, per (batch, head)

Head-aware tile search:
  head_sq_error    per-head squared difference of two raster tensors
  candidate_tiles  tile shapes (power-of-two edges, product 128) that fit a grid
  tile_search      per head, the candidate tiling whose sparse output is closest to dense attention
  k_from_keep      k per head from a keep fraction

Distilling the estimator toward the teacher:
  distill_kl       KL(teacher row || softmax(scores)) per query tile, and d/d scores
  distill_grad     the gradient back to W_q, W_k
  adam_step        one Adam update of fp32 master weights and their bf16 copy
  distill_train    estimator -> KL -> gradient -> Adam, for a number of steps
"""

from __future__ import annotations

import dataclasses
import fractions
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import VedaError

__all__ = ["Geometry", "VedaError", "tile_permute", "tile_permute_stats", "tile_unpermute", "trippool_score",
           "trippool_project_score", "topk_mask", "score_topk", "sparse_attn_fwd_raster", "tile_stats",
           "sparse_attn_fwd_raster_io", "sparse_attn_fwd_raster_io_noalloc",
           "sparse_attn_fwd", "attn_queue", "layer_forward",
           "dense_attn_fwd", "dense_attn_fwd_raster", "dense_index", "teacher_tile_max", "avgpool_score", "tile_scores_mfma", "mask_overlap", "tile_recall",
           "head_sq_error", "candidate_tiles", "tile_search", "distill_kl", "distill_grad", "adam_step",
           "distill_train", "k_from_keep", "TILE_TOKENS", "TOKEN_MAJOR", "CHANNEL_MAJOR"]

TILE_TOKENS = _lib.VEDA_TILE_TOKENS
TOKEN_MAJOR = _lib.VEDA_TILED_TOKEN_MAJOR
CHANNEL_MAJOR = _lib.VEDA_TILED_CHANNEL_MAJOR


@dataclasses.dataclass
class Geometry:
    """Batch, heads, head dim, latent grid (T, H, W) and one tile shape per head."""
    B: int
    n_heads: int
    head_dim: int
    grid: Tuple[int, int, int]
    head_tiles: Sequence[Tuple[int, int, int]]

    def __post_init__(self):
        if len(self.head_tiles) != self.n_heads:
            raise ValueError("need one tile shape per head")
        self._tiles = (_lib.VedaTile * self.n_heads)(*[_lib.VedaTile(*map(int, t)) for t in self.head_tiles])
        self._c = _lib.VedaGeom(int(self.B), int(self.n_heads), int(self.head_dim), _lib.VedaGrid(*map(int, self.grid)),
                                self._tiles)

    @property
    def c(self):
        return self._c

    @property
    def tokens(self) -> int:
        T, H, W = self.grid
        return T * H * W

    def num_tiles(self, head: int) -> int:
        return _lib.check(_lib.lib.veda_num_tiles(self._c, int(head)), "veda_num_tiles")

    def max_tiles(self) -> int:
        return _lib.check(_lib.lib.veda_max_tiles(self._c), "veda_max_tiles")


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, shape=None, name="tensor"):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raster_strides(x: torch.Tensor, geom: Geometry, name: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 device tensor")
    if tuple(x.shape) != (geom.B, geom.tokens, geom.n_heads, geom.head_dim):
        raise ValueError(f"{name} must have shape [B, N, heads, d] = "
                         f"{(geom.B, geom.tokens, geom.n_heads, geom.head_dim)}, got {tuple(x.shape)}")
    if x.stride(3) != 1:
        raise ValueError(f"{name} must have unit channel stride")
    return _lib.VedaRasterStrides(x.stride(0), x.stride(1), x.stride(2))


def _tiled_shape(geom: Geometry, last: int):
    return (geom.B, geom.n_heads, geom.max_tiles(), TILE_TOKENS, last)


def _tiled_cm_shape(geom: Geometry):
    return (geom.B, geom.n_heads, geom.max_tiles(), geom.head_dim, TILE_TOKENS)


def tile_permute(x: torch.Tensor, geom: Geometry, out: Optional[torch.Tensor] = None,
                 layout: int = TOKEN_MAJOR) -> torch.Tensor:
    """Gather a raster tensor [B, N, heads, d] (bf16, any strides with unit
    channel stride) into head-tiled order: [B, heads, nT_max, 128, d] for
    TOKEN_MAJOR, [B, heads, nT_max, d, 128] for CHANNEL_MAJOR (each tile
    transposed; the layout sparse_attn_fwd takes V in)."""
    s = _raster_strides(x, geom, "x")
    if layout == TOKEN_MAJOR:
        shape = _tiled_shape(geom, geom.head_dim)
    elif layout == CHANNEL_MAJOR:
        shape = _tiled_cm_shape(geom)
    else:
        raise ValueError("layout must be TOKEN_MAJOR or CHANNEL_MAJOR")
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, shape, "out")
    _lib.check(_lib.lib.veda_tile_permute(geom.c, x.data_ptr(), s, out.data_ptr(), int(layout), _stream(x)),
               "veda_tile_permute")
    return out


def tile_permute_stats(x: torch.Tensor, geom: Geometry, out: Optional[torch.Tensor] = None,
                       stats: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token-major tile_permute of Q or K and the TripPool statistics of each
    tile in one pass: (x_tiled [B, heads, nT_max, 128, d], stats [B, heads,
    nT_max, 3d] bf16), the same bytes as tile_permute and trippool_score's
    stats_q / stats_k."""
    s = _raster_strides(x, geom, "x")
    shape = _tiled_shape(geom, geom.head_dim)
    sshape = (geom.B, geom.n_heads, geom.max_tiles(), 3 * geom.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    if stats is None:
        stats = torch.empty(sshape, dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, shape, "out")
    _need(stats, torch.bfloat16, sshape, "stats")
    _lib.check(_lib.lib.veda_tile_permute_stats(geom.c, x.data_ptr(), s, out.data_ptr(), stats.data_ptr(),
                                                _stream(x)), "veda_tile_permute_stats")
    return out, stats


def tile_stats(x: torch.Tensor, geom: Geometry, stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The TripPool statistics of each tile of Q or K ([B, heads, nT_max, 3d]
    bf16, the same bytes as tile_permute_stats gives) in a pass that only
    reads the raster tensor: no tiled copy is written."""
    s = _raster_strides(x, geom, "x")
    sshape = (geom.B, geom.n_heads, geom.max_tiles(), 3 * geom.head_dim)
    if stats is None:
        stats = torch.empty(sshape, dtype=torch.bfloat16, device=x.device)
    _need(stats, torch.bfloat16, sshape, "stats")
    _lib.check(_lib.lib.veda_tile_permute_stats(geom.c, x.data_ptr(), s, None, stats.data_ptr(), _stream(x)),
               "veda_tile_permute_stats")
    return stats


def tile_unpermute(xt: torch.Tensor, geom: Geometry, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Scatter a tiled tensor back to raster order [B, N, heads, d]."""
    _need(xt, torch.bfloat16, _tiled_shape(geom, geom.head_dim), "x_tiled")
    if out is None:
        out = torch.empty((geom.B, geom.tokens, geom.n_heads, geom.head_dim), dtype=torch.bfloat16, device=xt.device)
    s = _raster_strides(out, geom, "out")
    _lib.check(_lib.lib.veda_tile_unpermute(geom.c, xt.data_ptr(), out.data_ptr(), s, _stream(xt)),
               "veda_tile_unpermute")
    return out


def trippool_score(q_t: torch.Tensor, k_t: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, geom: Geometry,
                   out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """TripPool statistics, head-specific projections and tile scores.
    Returns stats_q, stats_k [B, heads, nT_max, 3d], feat_q, feat_k
    [B, heads, nT_max, r] (bf16) and scores [B, heads, nT_max, nT_max] (fp32)."""
    d, nT = geom.head_dim, geom.max_tiles()
    tshape = _tiled_shape(geom, d)
    _need(q_t, torch.bfloat16, tshape, "q_tiled")
    _need(k_t, torch.bfloat16, tshape, "k_tiled")
    if w_q.dim() != 3:
        raise ValueError("w_q must be [heads, 3d, r]")
    r = w_q.shape[2]
    _need(w_q, torch.bfloat16, (geom.n_heads, 3 * d, r), "w_q")
    _need(w_k, torch.bfloat16, (geom.n_heads, 3 * d, r), "w_k")
    dev = q_t.device
    B, Hh = geom.B, geom.n_heads
    if out is None:
        out = {
            "stats_q": torch.empty((B, Hh, nT, 3 * d), dtype=torch.bfloat16, device=dev),
            "stats_k": torch.empty((B, Hh, nT, 3 * d), dtype=torch.bfloat16, device=dev),
            "feat_q": torch.empty((B, Hh, nT, r), dtype=torch.bfloat16, device=dev),
            "feat_k": torch.empty((B, Hh, nT, r), dtype=torch.bfloat16, device=dev),
            "scores": torch.empty((B, Hh, nT, nT), dtype=torch.float32, device=dev),
        }
    for name, shape, dt in (("stats_q", (B, Hh, nT, 3 * d), torch.bfloat16), ("stats_k", (B, Hh, nT, 3 * d), torch.bfloat16),
                            ("feat_q", (B, Hh, nT, r), torch.bfloat16), ("feat_k", (B, Hh, nT, r), torch.bfloat16),
                            ("scores", (B, Hh, nT, nT), torch.float32)):
        _need(out[name], dt, shape, name)
    _lib.check(_lib.lib.veda_trippool_score(
        geom.c, q_t.data_ptr(), k_t.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), int(r),
        out["stats_q"].data_ptr(), out["stats_k"].data_ptr(), out["feat_q"].data_ptr(), out["feat_k"].data_ptr(),
        out["scores"].data_ptr(), _stream(q_t)), "veda_trippool_score")
    return out


def trippool_project_score(stats_q: torch.Tensor, stats_k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                           geom: Geometry, out: Optional[Dict[str, torch.Tensor]] = None,
                           with_scores: bool = True) -> Dict[str, torch.Tensor]:
    """Projections and tile scores from statistics already computed (by
    tile_permute_stats): feat_q, feat_k [B, heads, nT_max, r] bf16 and scores
    [B, heads, nT_max, nT_max] fp32, as trippool_score. With `with_scores`
    false only the features are computed (score_topk takes the mask from
    them)."""
    d, nT = geom.head_dim, geom.max_tiles()
    B, Hh = geom.B, geom.n_heads
    _need(stats_q, torch.bfloat16, (B, Hh, nT, 3 * d), "stats_q")
    _need(stats_k, torch.bfloat16, (B, Hh, nT, 3 * d), "stats_k")
    if w_q.dim() != 3:
        raise ValueError("w_q must be [heads, 3d, r]")
    r = w_q.shape[2]
    _need(w_q, torch.bfloat16, (Hh, 3 * d, r), "w_q")
    _need(w_k, torch.bfloat16, (Hh, 3 * d, r), "w_k")
    dev = stats_q.device
    shapes = {"feat_q": ((B, Hh, nT, r), torch.bfloat16), "feat_k": ((B, Hh, nT, r), torch.bfloat16)}
    if with_scores:
        shapes["scores"] = ((B, Hh, nT, nT), torch.float32)
    out = dict(out) if out is not None else {}
    for name, (shape, dt) in shapes.items():
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=dt, device=dev)
        _need(out[name], dt, shape, name)
    _lib.check(_lib.lib.veda_trippool_project_score(
        geom.c, stats_q.data_ptr(), stats_k.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), int(r),
        out["feat_q"].data_ptr(), out["feat_k"].data_ptr(), out["scores"].data_ptr() if with_scores else None,
        _stream(stats_q)), "veda_trippool_project_score")
    return {n: out[n] for n in shapes}


def avgpool_score(stats_q: torch.Tensor, stats_k: torch.Tensor, geom: Geometry,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Average-pooling tile scores [B, heads, nT_max, nT_max] fp32: the dot
    product of the tile means (the avg block of the statistics) over all d
    channels; -inf outside each head's block. topk_mask of it is the pages'
    average-pooling baseline mask."""
    nT = geom.max_tiles()
    shp = (geom.B, geom.n_heads, nT, 3 * geom.head_dim)
    _need(stats_q, torch.bfloat16, shp, "stats_q")
    _need(stats_k, torch.bfloat16, shp, "stats_k")
    if out is None:
        out = torch.empty((geom.B, geom.n_heads, nT, nT), dtype=torch.float32, device=stats_q.device)
    _need(out, torch.float32, (geom.B, geom.n_heads, nT, nT), "scores")
    _lib.check(_lib.lib.veda_avgpool_score(geom.c, stats_q.data_ptr(), stats_k.data_ptr(), out.data_ptr(),
                                           _stream(stats_q)), "veda_avgpool_score")
    return out


def tile_scores_mfma(feat_q: torch.Tensor, feat_k: torch.Tensor, geom: Geometry,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The estimator's tile scores [B, heads, nT_max, nT_max] fp32 from the
    projected features, computed with bf16 MFMA (fp32 accumulation in the
    matrix core's order): within fp32 rounding of trippool_project_score's
    ordered scores, not always bit-identical to them."""
    nT = geom.max_tiles()
    r = feat_q.shape[-1] if feat_q.dim() == 4 else -1
    shp = (geom.B, geom.n_heads, nT, r)
    _need(feat_q, torch.bfloat16, shp, "feat_q")
    _need(feat_k, torch.bfloat16, shp, "feat_k")
    if out is None:
        out = torch.empty((geom.B, geom.n_heads, nT, nT), dtype=torch.float32, device=feat_q.device)
    _need(out, torch.float32, (geom.B, geom.n_heads, nT, nT), "scores")
    _lib.check(_lib.lib.veda_tile_scores_mfma(geom.c, feat_q.data_ptr(), feat_k.data_ptr(), int(r), out.data_ptr(),
                                              _stream(feat_q)), "veda_tile_scores_mfma")
    return out


def topk_mask(scores: torch.Tensor, geom: Geometry, k_per_head: Sequence[int], k_max: Optional[int] = None,
              with_bitmask: bool = True, idx: Optional[torch.Tensor] = None,
              bitmask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Head-aware Top-k: idx [B, heads, nT_max, k_max] int32 (ascending, -1
    padded) and optionally bitmask [B, heads, nT_max, ceil(nT_max/32)] uint32."""
    nT = geom.max_tiles()
    _need(scores, torch.float32, (geom.B, geom.n_heads, nT, nT), "scores")
    ks = list(k_per_head)
    if len(ks) != geom.n_heads:
        raise ValueError("need one k per head")
    if k_max is None:
        k_max = max(ks)
    dev = scores.device
    if idx is None:
        idx = torch.empty((geom.B, geom.n_heads, nT, k_max), dtype=torch.int32, device=dev)
    _need(idx, torch.int32, (geom.B, geom.n_heads, nT, k_max), "idx")
    if with_bitmask and bitmask is None:
        bitmask = torch.empty((geom.B, geom.n_heads, nT, (nT + 31) // 32), dtype=torch.uint32, device=dev)
    if bitmask is not None:
        _need(bitmask, torch.uint32, (geom.B, geom.n_heads, nT, (nT + 31) // 32), "bitmask")
    _lib.check(_lib.lib.veda_topk_mask(geom.c, scores.data_ptr(), _lib.int_array(ks), int(k_max), idx.data_ptr(),
                                       bitmask.data_ptr() if bitmask is not None else None, _stream(scores)),
               "veda_topk_mask")
    return idx, bitmask


SCORE_TOPK_MAX_TILES = 2048   # longest score row score_topk holds on chip


def score_topk(feat_q: torch.Tensor, feat_k: torch.Tensor, geom: Geometry, k_per_head: Sequence[int],
               k_max: Optional[int] = None, with_bitmask: bool = True, idx: Optional[torch.Tensor] = None,
               bitmask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Tile scores and head-aware Top-k in one pass, from the projections
    (no score matrix): the idx and bitmask topk_mask gives for the scores
    trippool_project_score writes, bit for bit. nT_max <= 2048."""
    nT = geom.max_tiles()
    if feat_q.dim() != 4:
        raise ValueError("feat_q must be [B, heads, nT_max, r]")
    r = feat_q.shape[3]
    _need(feat_q, torch.bfloat16, (geom.B, geom.n_heads, nT, r), "feat_q")
    _need(feat_k, torch.bfloat16, (geom.B, geom.n_heads, nT, r), "feat_k")
    ks = list(k_per_head)
    if len(ks) != geom.n_heads:
        raise ValueError("need one k per head")
    if k_max is None:
        k_max = max(ks)
    dev = feat_q.device
    if idx is None:
        idx = torch.empty((geom.B, geom.n_heads, nT, k_max), dtype=torch.int32, device=dev)
    _need(idx, torch.int32, (geom.B, geom.n_heads, nT, k_max), "idx")
    if with_bitmask and bitmask is None:
        bitmask = torch.empty((geom.B, geom.n_heads, nT, (nT + 31) // 32), dtype=torch.uint32, device=dev)
    if bitmask is not None:
        _need(bitmask, torch.uint32, (geom.B, geom.n_heads, nT, (nT + 31) // 32), "bitmask")
    _lib.check(_lib.lib.veda_score_topk(geom.c, feat_q.data_ptr(), feat_k.data_ptr(), int(r), _lib.int_array(ks),
                                        int(k_max), idx.data_ptr(),
                                        bitmask.data_ptr() if bitmask is not None else None, _stream(feat_q)),
               "veda_score_topk")
    return idx, bitmask


ATTN_QUEUE_BYTES = 64


def attn_queue(device) -> torch.Tensor:
    """Workspace of the attention work queue (each attention call clears it
    on its stream first; calls that may overlap need separate ones)."""
    return torch.empty(ATTN_QUEUE_BYTES // 4, dtype=torch.int32, device=device)


def _queue_ptr(work_queue, dynamic, device):
    """Device pointer of the work-queue workspace: None (fixed per-XCD shares)
    unless `dynamic`; a fresh workspace when none is given."""
    if not dynamic:
        return None
    if work_queue is None:
        work_queue = attn_queue(device)
    if (work_queue.dtype != torch.int32 or work_queue.device != device or not work_queue.is_contiguous()
            or work_queue.numel() * 4 < ATTN_QUEUE_BYTES):
        raise ValueError(f"work_queue must be a contiguous int32 tensor of {ATTN_QUEUE_BYTES // 4} elements "
                         f"on {device}")
    return work_queue.data_ptr()


def _attn_args(q_t, k_t, v_t, idx, geom, k_per_head, with_lse, lse):
    """Checks of the attention calls' tensors (q_t None: Q comes in raster
    order and is checked by the caller); returns (k list, k_max, lse)."""
    tshape = _tiled_shape(geom, geom.head_dim)
    for name, t in (("q_tiled", q_t), ("k_tiled", k_t)):
        if t is not None:
            _need(t, torch.bfloat16, tshape, name)
    _need(v_t, torch.bfloat16, _tiled_cm_shape(geom), "v_tiled")
    if idx.dim() != 4:
        raise ValueError("idx must be [B, heads, nT_max, k_max]")
    k_max = idx.shape[3]
    _need(idx, torch.int32, (geom.B, geom.n_heads, tshape[2], k_max), "idx")
    ks = list(k_per_head)
    if len(ks) != geom.n_heads:
        raise ValueError("need one k per head")
    if with_lse and lse is None:
        lse = torch.empty(tshape[:4], dtype=torch.float32, device=k_t.device)
    if lse is not None:
        _need(lse, torch.float32, tshape[:4], "lse")
    return ks, k_max, lse


def sparse_attn_fwd_raster(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, idx: torch.Tensor,
                           geom: Geometry, k_per_head: Sequence[int], scale: Optional[float] = None,
                           with_lse: bool = True, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, work_queue: Optional[torch.Tensor] = None,
                           dynamic: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sparse_attn_fwd writing O straight into raster order [B, N, heads, d]
    (`out` may be any strided view with unit channel stride): the bytes
    tile_unpermute of the tiled O would give, without that pass. `work_queue`
    and `dynamic` as in sparse_attn_fwd."""
    ks, k_max, lse = _attn_args(q_t, k_t, v_t, idx, geom, k_per_head, with_lse, lse)
    if out is None:
        out = torch.empty((geom.B, geom.tokens, geom.n_heads, geom.head_dim), dtype=torch.bfloat16,
                          device=q_t.device)
    s = _raster_strides(out, geom, "out")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_sparse_attn_fwd_raster(
        geom.c, q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), idx.data_ptr(), _lib.int_array(ks), int(k_max), sc,
        out.data_ptr(), s, lse.data_ptr() if lse is not None else None, _queue_ptr(work_queue, dynamic, q_t.device),
        _stream(q_t)), "veda_sparse_attn_fwd_raster")
    return out, lse


def sparse_attn_fwd_raster_io(q: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, idx: torch.Tensor,
                              geom: Geometry, k_per_head: Sequence[int], scale: Optional[float] = None,
                              with_lse: bool = True, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, work_queue: Optional[torch.Tensor] = None,
                              dynamic: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sparse_attn_fwd_raster reading Q in raster order too ([B, N, heads, d],
    any strided view with unit channel stride): the bytes it gives with the
    tiled Q of tile_permute(q), with no tiled copy of Q."""
    sq = _raster_strides(q, geom, "q")
    ks, k_max, lse = _attn_args(None, k_t, v_t, idx, geom, k_per_head, with_lse, lse)
    if out is None:
        out = torch.empty((geom.B, geom.tokens, geom.n_heads, geom.head_dim), dtype=torch.bfloat16,
                          device=q.device)
    so = _raster_strides(out, geom, "out")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_sparse_attn_fwd_raster_io(
        geom.c, q.data_ptr(), sq, k_t.data_ptr(), v_t.data_ptr(), idx.data_ptr(), _lib.int_array(ks), int(k_max), sc,
        out.data_ptr(), so, lse.data_ptr() if lse is not None else None, _queue_ptr(work_queue, dynamic, q.device),
        _stream(q)), "veda_sparse_attn_fwd_raster_io")
    return out, lse


def sparse_attn_fwd_raster_io_noalloc(q: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, idx: torch.Tensor,
                                      geom: Geometry, k_per_head: Sequence[int], out: torch.Tensor,
                                      lse: Optional[torch.Tensor] = None,
                                      scale: Optional[float] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sparse_attn_fwd_raster_io for callers that cannot allocate: `out`
    (and `lse`, if wanted) come from the caller and the work queue is the
    library's static one, so the call allocates nothing. Calls that may
    overlap in time on one device race on that queue."""
    sq = _raster_strides(q, geom, "q")
    ks, k_max, lse = _attn_args(None, k_t, v_t, idx, geom, k_per_head, False, lse)
    so = _raster_strides(out, geom, "out")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_sparse_attn_fwd_raster_io_noalloc(
        geom.c, q.data_ptr(), sq, k_t.data_ptr(), v_t.data_ptr(), idx.data_ptr(), _lib.int_array(ks), int(k_max), sc,
        out.data_ptr(), so, lse.data_ptr() if lse is not None else None, _stream(q)),
        "veda_sparse_attn_fwd_raster_io_noalloc")
    return out, lse


def sparse_attn_fwd(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, idx: torch.Tensor, geom: Geometry,
                    k_per_head: Sequence[int], scale: Optional[float] = None, with_lse: bool = True,
                    o_t: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    work_queue: Optional[torch.Tensor] = None, dynamic: bool = True
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Tile-skipping attention over the selected key tiles. Q and K are
    token-major tiles, V channel-major ([B, heads, nT_max, d, 128]); returns
    tiled O (bf16, token-major) and LSE [B, heads, nT_max, 128] (fp32,
    natural log). With `dynamic` the query tiles are handed out through a
    work queue (`work_queue`, from attn_queue, or a fresh one), which keeps
    XCDs at different clocks busy to the end; the outputs are the same bytes
    either way."""
    tshape = _tiled_shape(geom, geom.head_dim)
    for name, t in (("q_tiled", q_t), ("k_tiled", k_t)):
        _need(t, torch.bfloat16, tshape, name)
    _need(v_t, torch.bfloat16, _tiled_cm_shape(geom), "v_tiled")
    if idx.dim() != 4:
        raise ValueError("idx must be [B, heads, nT_max, k_max]")
    k_max = idx.shape[3]
    _need(idx, torch.int32, (geom.B, geom.n_heads, tshape[2], k_max), "idx")
    ks = list(k_per_head)
    if len(ks) != geom.n_heads:
        raise ValueError("need one k per head")
    if o_t is None:
        o_t = torch.empty(tshape, dtype=torch.bfloat16, device=q_t.device)
    _need(o_t, torch.bfloat16, tshape, "o_tiled")
    if with_lse and lse is None:
        lse = torch.empty(tshape[:4], dtype=torch.float32, device=q_t.device)
    if lse is not None:
        _need(lse, torch.float32, tshape[:4], "lse")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_sparse_attn_fwd(geom.c, q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), idx.data_ptr(),
                                             _lib.int_array(ks), int(k_max), sc, o_t.data_ptr(),
                                             lse.data_ptr() if lse is not None else None,
                                             _queue_ptr(work_queue, dynamic, q_t.device), _stream(q_t)),
               "veda_sparse_attn_fwd")
    return o_t, lse


def layer_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                  geom: Geometry, k_per_head: Sequence[int], scale: Optional[float] = None,
                  buffers: Optional[Dict[str, torch.Tensor]] = None, tiled_q: bool = False,
                  keep_scores: bool = False) -> Dict[str, torch.Tensor]:
    """One Veda attention layer: the TripPool statistics of Q (a read-only
    pass), K permuted with its statistics in the same pass, V permuted,
    projections, tile scores and their Top-k mask in one pass, and
    tile-skipping attention that reads Q and writes O in raster order.
    `buffers` (from a previous call) reuses every output allocation. Returns
    all intermediates, `o` and the attention's work-queue workspace `queue`;
    there is no tiled Q or O (tile_permute, sparse_attn_fwd and
    tile_unpermute give the same `o`). With `tiled_q` the layer tiles Q as
    well (output `q_t`) and the attention reads that. With `keep_scores`, or
    when rows are longer than score_topk holds (SCORE_TOPK_MAX_TILES), the
    score matrix is written (output `scores`) and topk_mask reads it. Every
    other output is the same bytes on each route."""
    b = buffers if buffers is not None else {}
    if tiled_q:
        b["q_t"], b["stats_q"] = tile_permute_stats(q, geom, b.get("q_t"), b.get("stats_q"))
    else:
        b["stats_q"] = tile_stats(q, geom, b.get("stats_q"))
    b["k_t"], b["stats_k"] = tile_permute_stats(k, geom, b.get("k_t"), b.get("stats_k"))
    b["v_t"] = tile_permute(v, geom, b.get("v_t"), layout=CHANNEL_MAJOR)
    fused = not keep_scores and geom.max_tiles() <= SCORE_TOPK_MAX_TILES
    if fused:
        b.pop("scores", None)
    est = trippool_project_score(b["stats_q"], b["stats_k"], w_q, w_k, geom,
                                 {n: b.get(n) for n in ("feat_q", "feat_k", "scores")}, with_scores=not fused)
    b.update(est)
    if fused:
        b["idx"], b["bitmask"] = score_topk(b["feat_q"], b["feat_k"], geom, k_per_head, idx=b.get("idx"),
                                            bitmask=b.get("bitmask"))
    else:
        b["idx"], b["bitmask"] = topk_mask(b["scores"], geom, k_per_head, idx=b.get("idx"),
                                           bitmask=b.get("bitmask"))
    if b.get("queue") is None:
        b["queue"] = attn_queue(q.device)
    if tiled_q:
        b["o"], b["lse"] = sparse_attn_fwd_raster(b["q_t"], b["k_t"], b["v_t"], b["idx"], geom, k_per_head, scale,
                                                  out=b.get("o"), lse=b.get("lse"), work_queue=b["queue"])
    else:
        b["o"], b["lse"] = sparse_attn_fwd_raster_io(q, b["k_t"], b["v_t"], b["idx"], geom, k_per_head, scale,
                                                     out=b.get("o"), lse=b.get("lse"), work_queue=b["queue"])
    return b


def dense_attn_fwd(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, geom: Geometry,
                   scale: Optional[float] = None, with_lse: bool = True, o_t: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, work_queue: Optional[torch.Tensor] = None,
                   dynamic: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense attention (every key tile kept, no index list) on tiled Q, K
    and channel-major V: tiled O and LSE, the bytes sparse_attn_fwd gives
    with dense_index."""
    tshape = _tiled_shape(geom, geom.head_dim)
    _need(q_t, torch.bfloat16, tshape, "q_tiled")
    _need(k_t, torch.bfloat16, tshape, "k_tiled")
    _need(v_t, torch.bfloat16, _tiled_cm_shape(geom), "v_tiled")
    if o_t is None:
        o_t = torch.empty(tshape, dtype=torch.bfloat16, device=q_t.device)
    _need(o_t, torch.bfloat16, tshape, "o_tiled")
    if with_lse and lse is None:
        lse = torch.empty(tshape[:4], dtype=torch.float32, device=q_t.device)
    if lse is not None:
        _need(lse, torch.float32, tshape[:4], "lse")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_dense_attn_fwd(geom.c, q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), sc, o_t.data_ptr(),
                                            lse.data_ptr() if lse is not None else None,
                                            _queue_ptr(work_queue, dynamic, q_t.device), _stream(q_t)),
               "veda_dense_attn_fwd")
    return o_t, lse


def dense_attn_fwd_raster(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, geom: Geometry,
                          scale: Optional[float] = None, with_lse: bool = True, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, work_queue: Optional[torch.Tensor] = None,
                          dynamic: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """dense_attn_fwd writing O in raster order [B, N, heads, d]."""
    tshape = _tiled_shape(geom, geom.head_dim)
    _need(q_t, torch.bfloat16, tshape, "q_tiled")
    _need(k_t, torch.bfloat16, tshape, "k_tiled")
    _need(v_t, torch.bfloat16, _tiled_cm_shape(geom), "v_tiled")
    if out is None:
        out = torch.empty((geom.B, geom.tokens, geom.n_heads, geom.head_dim), dtype=torch.bfloat16, device=q_t.device)
    so = _raster_strides(out, geom, "out")
    if with_lse and lse is None:
        lse = torch.empty(tshape[:4], dtype=torch.float32, device=q_t.device)
    if lse is not None:
        _need(lse, torch.float32, tshape[:4], "lse")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_dense_attn_fwd_raster(geom.c, q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), sc,
                                                   out.data_ptr(), so, lse.data_ptr() if lse is not None else None,
                                                   _queue_ptr(work_queue, dynamic, q_t.device), _stream(q_t)),
               "veda_dense_attn_fwd_raster")
    return out, lse


def dense_index(geom: Geometry, device) -> Tuple[torch.Tensor, List[int]]:
    """Index lists that keep every key tile of every head (idx[..., j] = j)
    and the matching k per head: sparse_attn_fwd with these is dense
    attention, and its LSE is the one teacher_tile_max needs."""
    nT = geom.max_tiles()
    idx = torch.arange(nT, dtype=torch.int32, device=device).expand(geom.B, geom.n_heads, nT, nT).contiguous()
    return idx, [geom.num_tiles(hd) for hd in range(geom.n_heads)]


def teacher_tile_max(q_t: torch.Tensor, k_t: torch.Tensor, lse_dense: torch.Tensor, geom: Geometry,
                     scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     work_queue: Optional[torch.Tensor] = None, dynamic: bool = True) -> torch.Tensor:
    """Max-pooled dense attention: [B, heads, nT_max, nT_max] fp32, the
    largest dense softmax probability between each query tile and key tile
    (-inf outside the head's block). lse_dense is the LSE of dense_attn_fwd
    (or of sparse_attn_fwd with dense_index). `work_queue` and `dynamic` as in sparse_attn_fwd."""
    tshape = _tiled_shape(geom, geom.head_dim)
    _need(q_t, torch.bfloat16, tshape, "q_tiled")
    _need(k_t, torch.bfloat16, tshape, "k_tiled")
    _need(lse_dense, torch.float32, tshape[:4], "lse_dense")
    nT = tshape[2]
    if out is None:
        out = torch.empty((geom.B, geom.n_heads, nT, nT), dtype=torch.float32, device=q_t.device)
    _need(out, torch.float32, (geom.B, geom.n_heads, nT, nT), "teacher")
    sc = float(scale) if scale is not None else 0.0
    _lib.check(_lib.lib.veda_teacher_tile_max(geom.c, q_t.data_ptr(), k_t.data_ptr(), lse_dense.data_ptr(), sc,
                                              out.data_ptr(), _queue_ptr(work_queue, dynamic, q_t.device),
                                              _stream(q_t)), "veda_teacher_tile_max")
    return out


def mask_overlap(bitmask_a: torch.Tensor, bitmask_b: torch.Tensor, geom: Geometry,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Common kept tiles of two masks: [B, heads] (int64 here; the counts are
    far below 2^63), the sum over each head's query tiles of popcount(a & b)."""
    nT = geom.max_tiles()
    shape = (geom.B, geom.n_heads, nT, (nT + 31) // 32)
    _need(bitmask_a, torch.uint32, shape, "bitmask_a")
    _need(bitmask_b, torch.uint32, shape, "bitmask_b")
    if out is None:
        out = torch.empty((geom.B, geom.n_heads), dtype=torch.int64, device=bitmask_a.device)
    _need(out, torch.int64, (geom.B, geom.n_heads), "counts")
    _lib.check(_lib.lib.veda_mask_overlap(geom.c, bitmask_a.data_ptr(), bitmask_b.data_ptr(), out.data_ptr(),
                                          _stream(bitmask_a)), "veda_mask_overlap")
    return out


def tile_recall(bitmask: torch.Tensor, bitmask_oracle: torch.Tensor, geom: Geometry, k_per_head: Sequence[int],
                out: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tile recall per (batch, head), fp64 [B, heads] on the device: kept
    tiles the mask shares with the oracle mask over the oracle mask's
    k_hd * nT_hd (k_per_head is the oracle mask's k). `counts` (int64
    [B, heads]), when given, receives the numerators."""
    nT = geom.max_tiles()
    shape = (geom.B, geom.n_heads, nT, (nT + 31) // 32)
    _need(bitmask, torch.uint32, shape, "bitmask")
    _need(bitmask_oracle, torch.uint32, shape, "bitmask_oracle")
    ks = list(k_per_head)
    if len(ks) != geom.n_heads:
        raise ValueError("need one k per head")
    if out is None:
        out = torch.empty((geom.B, geom.n_heads), dtype=torch.float64, device=bitmask.device)
    _need(out, torch.float64, (geom.B, geom.n_heads), "recall")
    if counts is not None:
        _need(counts, torch.int64, (geom.B, geom.n_heads), "counts")
    _lib.check(_lib.lib.veda_tile_recall(geom.c, bitmask.data_ptr(), bitmask_oracle.data_ptr(), _lib.int_array(ks),
                                         counts.data_ptr() if counts is not None else None, out.data_ptr(),
                                         _stream(bitmask)), "veda_tile_recall")
    return out


def head_sq_error(a: torch.Tensor, b: torch.Tensor, geom: Geometry,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp64 [B, heads]: sum over tokens and channels of (a - b)^2 for two raster
    bf16 tensors [B, N, heads, d] (any strides with unit channel stride)."""
    sa = _raster_strides(a, geom, "a")
    sb = _raster_strides(b, geom, "b")
    if out is None:
        out = torch.empty((geom.B, geom.n_heads), dtype=torch.float64, device=a.device)
    _need(out, torch.float64, (geom.B, geom.n_heads), "err")
    _lib.check(_lib.lib.veda_head_sq_error(geom.c, a.data_ptr(), sa, b.data_ptr(), sb, out.data_ptr(), _stream(a)),
               "veda_head_sq_error")
    return out


def candidate_tiles(grid: Sequence[int]) -> List[Tuple[int, int, int]]:
    """Every (pt, ph, pw) of powers of two with pt * ph * pw = 128 whose edges
    do not exceed the grid's (T, H, W) and whose tile count stays within the
    library's limit (veda_candidate_tiles)."""
    out = (_lib.VedaTile * 36)()
    n = _lib.check(_lib.lib.veda_candidate_tiles(_lib.VedaGrid(*map(int, grid)), out, 36), "veda_candidate_tiles")
    return [(out[i].pt, out[i].ph, out[i].pw) for i in range(n)]


def _k_of(keep, geom: Geometry, head: int) -> int:
    """k_hd = ceil(keep * nT_hd) (veda_k_from_keep, exact in integers)."""
    f = keep if isinstance(keep, fractions.Fraction) else fractions.Fraction(str(keep))
    return _lib.check(_lib.lib.veda_k_from_keep(geom.c, int(head), f.numerator, f.denominator), "veda_k_from_keep")


def k_from_keep(geom: Geometry, keep) -> List[int]:
    """k per head for a keep fraction (e.g. 0.05 for 95% sparsity)."""
    return [_k_of(keep, geom, hd) for hd in range(geom.n_heads)]


def tile_search(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                grid: Sequence[int], keep, candidates: Optional[Sequence[Tuple[int, int, int]]] = None,
                scale: Optional[float] = None) -> Dict[str, object]:
    """Head-aware tile search on calibration inputs: for every candidate tile
    shape, run the whole layer with that shape on every head (k_hd =
    ceil(keep * nT_hd)) and measure each head's ||O_dense - O_sparse||_F^2
    against dense attention; each head takes the candidate with the smallest
    error summed over the batch.

    Returns {"candidates", "err" (fp64 [n_candidates, B, heads], host),
    "best" (one tile shape per head), "o_dense"}."""
    B, N, Hh, d = q.shape
    cands = list(candidates) if candidates is not None else candidate_tiles(grid)
    if not cands:
        raise ValueError("no candidate tile shape fits the grid")
    g0 = Geometry(B, Hh, d, tuple(grid), [cands[0]] * Hh)
    q_t = tile_permute(q, g0)
    k_t = tile_permute(k, g0)
    v_t = tile_permute(v, g0, layout=CHANNEL_MAJOR)
    o_dense, _ = dense_attn_fwd_raster(q_t, k_t, v_t, g0, scale, with_lse=False)
    del q_t, k_t, v_t
    err = torch.empty((len(cands), B, Hh), dtype=torch.float64, device=q.device)
    for ci, tile in enumerate(cands):
        g = Geometry(B, Hh, d, tuple(grid), [tuple(tile)] * Hh)
        ks = k_from_keep(g, keep)
        o = layer_forward(q, k, v, w_q, w_k, g, ks, scale)["o"]
        head_sq_error(o, o_dense, g, out=err[ci])
    best = torch.empty((Hh,), dtype=torch.int32, device=q.device)
    _lib.check(_lib.lib.veda_tile_search_select(len(cands), B, Hh, err.data_ptr(), None, best.data_ptr(),
                                                _stream(q)), "veda_tile_search_select")
    return {"candidates": cands, "err": err.cpu().numpy(), "best": [tuple(cands[i]) for i in best.cpu().tolist()],
            "o_dense": o_dense}


def distill_kl(scores: torch.Tensor, teacher: torch.Tensor, geom: Geometry, grad_scale: float = 1.0,
               kl_rows: Optional[torch.Tensor] = None, d_scores: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per query tile: KL(teacher row normalised || softmax(scores row)) over
    the head's key tiles ([B, heads, nT_max] fp32) and grad_scale times its
    gradient with respect to the scores ([B, heads, nT_max, nT_max])."""
    nT = geom.max_tiles()
    shape = (geom.B, geom.n_heads, nT, nT)
    _need(scores, torch.float32, shape, "scores")
    _need(teacher, torch.float32, shape, "teacher")
    if kl_rows is None:
        kl_rows = torch.empty(shape[:3], dtype=torch.float32, device=scores.device)
    if d_scores is None:
        d_scores = torch.empty(shape, dtype=torch.float32, device=scores.device)
    _need(kl_rows, torch.float32, shape[:3], "kl_rows")
    _need(d_scores, torch.float32, shape, "d_scores")
    _lib.check(_lib.lib.veda_distill_kl(geom.c, scores.data_ptr(), teacher.data_ptr(), float(grad_scale),
                                        kl_rows.data_ptr(), d_scores.data_ptr(), _stream(scores)), "veda_distill_kl")
    return kl_rows, d_scores


def distill_grad(est: Dict[str, torch.Tensor], d_scores: torch.Tensor, geom: Geometry,
                 out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Gradient of the distillation loss with respect to W_q and W_k ([heads,
    3d, r] fp32), through the estimator outputs `est` (stats_q, stats_k,
    feat_q, feat_k from trippool_score). Also returns d_feat_q, d_feat_k."""
    r = est["feat_q"].shape[-1]
    d, nT, B, Hh = geom.head_dim, geom.max_tiles(), geom.B, geom.n_heads
    _need(d_scores, torch.float32, (B, Hh, nT, nT), "d_scores")
    dev = d_scores.device
    if out is None:
        out = {"d_feat_q": torch.empty((B, Hh, nT, r), dtype=torch.float32, device=dev),
               "d_feat_k": torch.empty((B, Hh, nT, r), dtype=torch.float32, device=dev),
               "d_w_q": torch.empty((Hh, 3 * d, r), dtype=torch.float32, device=dev),
               "d_w_k": torch.empty((Hh, 3 * d, r), dtype=torch.float32, device=dev)}
    for n, shp in (("d_feat_q", (B, Hh, nT, r)), ("d_feat_k", (B, Hh, nT, r)), ("d_w_q", (Hh, 3 * d, r)),
                   ("d_w_k", (Hh, 3 * d, r))):
        _need(out[n], torch.float32, shp, n)
    for n, shp in (("stats_q", (B, Hh, nT, 3 * d)), ("stats_k", (B, Hh, nT, 3 * d)), ("feat_q", (B, Hh, nT, r)),
                   ("feat_k", (B, Hh, nT, r))):
        _need(est[n], torch.bfloat16, shp, n)
    _lib.check(_lib.lib.veda_distill_grad(
        geom.c, int(r), est["stats_q"].data_ptr(), est["stats_k"].data_ptr(), est["feat_q"].data_ptr(),
        est["feat_k"].data_ptr(), d_scores.data_ptr(), out["d_feat_q"].data_ptr(), out["d_feat_k"].data_ptr(),
        out["d_w_q"].data_ptr(), out["d_w_k"].data_ptr(), _stream(d_scores)), "veda_distill_grad")
    return out


def adam_step(w: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, step: int, lr: float,
              betas: Tuple[float, float] = (0.9, 0.999), eps: float = 1e-8,
              w_bf16: Optional[torch.Tensor] = None) -> None:
    """One bias-corrected Adam step on fp32 master weights (in place), and
    their bf16 copy when given."""
    for name, t in (("w", w), ("grad", grad), ("m", m), ("v", v)):
        _need(t, torch.float32, tuple(w.shape), name)
    if w_bf16 is not None:
        _need(w_bf16, torch.bfloat16, tuple(w.shape), "w_bf16")
    _lib.check(_lib.lib.veda_adam_step(w.numel(), w.data_ptr(), grad.data_ptr(), m.data_ptr(), v.data_ptr(),
                                       int(step), float(lr), float(betas[0]), float(betas[1]), float(eps),
                                       w_bf16.data_ptr() if w_bf16 is not None else None, _stream(w)),
               "veda_adam_step")


def distill_train(q_t: torch.Tensor, k_t: torch.Tensor, teacher: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                  geom: Geometry, steps: int, lr: float = 1e-2, betas: Tuple[float, float] = (0.9, 0.999),
                  eps: float = 1e-8) -> Dict[str, object]:
    """Distil the head-specific projections toward the teacher on fixed
    calibration tiles: each step runs the estimator with the bf16 weights,
    the KL objective (mean over query tiles) and its gradient, then Adam on
    fp32 master copies. Returns the trained bf16 weights and the loss after
    each step (mean KL per query tile, from the step's forward)."""
    wq_m, wk_m = w_q.float().contiguous(), w_k.float().contiguous()
    wq_b, wk_b = w_q.clone(), w_k.clone()
    mq, vq, mk, vk = (torch.zeros_like(wq_m) for _ in range(4))
    rows = sum(geom.num_tiles(hd) for hd in range(geom.n_heads)) * geom.B
    losses = torch.empty((steps,), dtype=torch.float64, device=q_t.device)
    est = trippool_score(q_t, k_t, wq_b, wk_b, geom)   # the statistics do not depend on W: taken once
    grads, kl, ds = None, None, None
    for step in range(1, steps + 1):
        if step > 1:
            est.update(trippool_project_score(est["stats_q"], est["stats_k"], wq_b, wk_b, geom,
                                              {n: est[n] for n in ("feat_q", "feat_k", "scores")}))
        kl, ds = distill_kl(est["scores"], teacher, geom, 1.0 / rows, kl, ds)
        grads = distill_grad(est, ds, geom, grads)
        adam_step(wq_m, grads["d_w_q"], mq, vq, step, lr, betas, eps, wq_b)
        adam_step(wk_m, grads["d_w_k"], mk, vk, step, lr, betas, eps, wk_b)
        _lib.check(_lib.lib.veda_distill_mean_kl(geom.c, kl.data_ptr(), losses[step - 1:step].data_ptr(),
                                                 _stream(kl)), "veda_distill_mean_kl")
    return {"w_q": wq_b, "w_k": wk_b, "loss": losses.cpu().tolist()}
