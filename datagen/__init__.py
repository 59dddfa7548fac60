"""Seeded synthetic inputs for the Veda tile-sparse attention forward.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
the workload table and the input generator only: no step of the attention
method (no tiling, pooling, projection, scoring, selection or softmax) is
computed here. Both the HIP path and the oracle receive the same host bytes.

Workloads (shapes follow the video latents the Veda pages measure on: the
245K-token long-video layer of "Scaling Law in Practice", the 720P and 480P
grids of "Inference Latency" and "Evaluation" on veda-sparse.github.io):

  tiny  : B=1, 2 heads,  d=64,  grid 4x16x16  (1,024 tok), tile (2,8,8),  k=4 of 8
  480p  : B=1, 12 heads, d=128, grid 21x30x52 (32,760 tok), tile (4,4,8), keep 10%
  720p  : B=1, 40 heads, d=128, grid 21x45x80 (75,600 tok), tile (4,4,8), keep 5%
  hc    : as 720p, tile per head (4,4,8)/(1,8,16)/(8,4,4) round robin, keep 10%
  long  : B=1, 40 heads, d=128, grid 64x48x80 (245,760 tok), tile (4,4,8), k=96 of 1920

Each token of Q, K and V is a low-frequency field of the (t, y, x) position plus
unit Gaussian noise, rounded to bfloat16:

  field[n, c] = A_hd * sum_f a[f, c] * cos(2*pi*<k_f, pos_n> + phi_f)

with 8 frequency vectors k_f ~ U(-2, 2)^3 (cycles over the whole grid span),
phases phi_f ~ U(0, 2*pi), and each channel's loading a[:, c] a random unit
vector of R^8. pos_n = (t/T, y/H, x/W). The field is nearly constant inside a
128-token tile, which is the regime the pages' tile-statistics argument
(Theoretical Rationale 2, "Tile Statistics") assumes. The per-head amplitude
A_hd is 1, or U(0.5, 2) for the 720p and hc workloads.

Projection weights W_q, W_k [heads, 3d, r] are N(0, 1) / sqrt(3d), rounded to
bfloat16.

The field is summed in a fixed order without BLAS, so the same workload
gives the same bytes on every call, whatever the thread count.

Random streams: numpy PCG64 seeded by SeedSequence([seed, tensor_id, b, hd])
for tensor_id 0/1/2 = Q/K/V; [seed, 99, hd] for A_hd; [seed, 100, hd] and
[seed, 101, hd] for W_q and W_k. A workload with `noise_seed` set draws the
noise from [noise_seed, tensor_id, b, hd] instead (the field, amplitudes and
weights keep `seed`): the same positional structure with other content, the
held-out sample of the distillation report.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction
from typing import Dict, List, Optional, Tuple

import numpy as np

TILE_TOKENS = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    d: int
    r: int
    grid: Tuple[int, int, int]
    tile_cycle: Tuple[Tuple[int, int, int], ...]   # head hd uses tile_cycle[hd % len]
    keep: Optional[Fraction]                        # fraction of key tiles kept, or None
    k_fixed: Optional[int]                          # explicit k when keep is None
    amp_uniform: bool                               # A_hd ~ U(0.5, 2) instead of 1
    seed: int
    description: str
    noise_seed: Optional[int] = None                # noise from its own stream (the field keeps `seed`)

    @property
    def tokens(self) -> int:
        T, H, W = self.grid
        return T * H * W

    def head_tiles(self) -> List[Tuple[int, int, int]]:
        return [self.tile_cycle[h % len(self.tile_cycle)] for h in range(self.heads)]

    def tiles_per_head(self) -> List[int]:
        """Number of 128-token boxes per head when every axis is padded up."""
        T, H, W = self.grid
        out = []
        for pt, ph, pw in self.head_tiles():
            out.append(-(-T // pt) * -(-H // ph) * -(-W // pw))
        return out

    def k_per_head(self) -> List[int]:
        """Key tiles kept per query tile: ceil(keep * tiles), or the fixed k."""
        if self.keep is None:
            return [self.k_fixed] * self.heads
        num, den = self.keep.numerator, self.keep.denominator
        return [(n * num + den - 1) // den for n in self.tiles_per_head()]

    def with_heads(self, heads: int) -> "Workload":
        """The first `heads` heads of this workload (same seeds, so each head's
        inputs are the bytes it has in the full workload)."""
        if heads == self.heads:
            return self
        desc = self.description.replace(f"{self.heads} heads", f"heads 0-{heads - 1} of {self.heads}", 1)
        return dataclasses.replace(self, heads=heads, description=desc)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 2, 64, 32, (4, 16, 16), ((2, 8, 8),), None, 4, False, 0,
                     "Tiny: B=1, 2 heads, d=64, grid 4x16x16 (1,024 tokens), tile (2,8,8), k=4 of 8 (50% sparse)"),
    "480p": Workload("480p", 1, 12, 128, 64, (21, 30, 52), ((4, 4, 8),), Fraction(1, 10), None, False, 1,
                     "480P-short: B=1, 12 heads, d=128, grid 21x30x52 (32,760 tokens, padded per axis), tile (4,4,8), keep 10% (90% sparse)"),
    "720p": Workload("720p", 1, 40, 128, 64, (21, 45, 80), ((4, 4, 8),), Fraction(1, 20), None, True, 2,
                     "720P-81f: B=1, 40 heads, d=128, grid 21x45x80 (75,600 tokens, padded per axis), tile (4,4,8), keep 5% (95% sparse)"),
    "hc": Workload("hc", 1, 40, 128, 64, (21, 45, 80), ((4, 4, 8), (1, 8, 16), (8, 4, 4)), Fraction(1, 10), None, True, 3,
                   "Head-conditioned: B=1, 40 heads, d=128, grid 21x45x80, tiles (4,4,8)/(1,8,16)/(8,4,4) by head mod 3, keep 10% (90% sparse)"),
    "long": Workload("long", 1, 40, 128, 64, (64, 48, 80), ((4, 4, 8),), None, 96, False, 4,
                     "Long video: B=1, 40 heads, d=128, grid 64x48x80 (245,760 tokens), tile (4,4,8) -> 1920 tiles, k=96 (95% sparse)"),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns (round to nearest even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def head_amplitudes(w: Workload) -> np.ndarray:
    out = np.ones(w.heads, dtype=np.float64)
    if w.amp_uniform:
        for hd in range(w.heads):
            out[hd] = _rng(w.seed, 99, hd).uniform(0.5, 2.0)
    return out


def _positions(grid: Tuple[int, int, int]) -> np.ndarray:
    T, H, W = grid
    t, y, x = np.meshgrid(np.arange(T) / T, np.arange(H) / H, np.arange(W) / W, indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)  # [N, 3], raster order


def _fill_head(out: np.ndarray, w: Workload, tensor_id: int, b: int, hd: int,
               pos: np.ndarray, amp: float) -> None:
    rng = _rng(w.seed, tensor_id, b, hd)
    kf = rng.uniform(-2.0, 2.0, size=(8, 3))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=8)
    a = rng.standard_normal((8, w.d))
    a /= np.linalg.norm(a, axis=0, keepdims=True)
    # Sums in a fixed order without BLAS (whose summation order can change
    # with its threading), so the bytes are the same on every call: the
    # 3-term phase elementwise, the 8-term field with numpy's own einsum loop.
    arg = pos[:, 0:1] * kf[:, 0] + pos[:, 1:2] * kf[:, 1] + pos[:, 2:3] * kf[:, 2]   # [N, 8]
    c = amp * np.cos(2.0 * math.pi * arg + phi)
    field = np.einsum("nf,fd->nd", c, a, optimize=False)                         # [N, d] float64
    if w.noise_seed is not None:
        rng = _rng(w.noise_seed, tensor_id, b, hd)
    noise = rng.standard_normal((pos.shape[0], w.d), dtype=np.float32)
    out[b, :, hd, :] = to_bf16_bits(field.astype(np.float32) + noise)


def generate_qkv(w: Workload, threads: Optional[int] = None,
                 heads: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
    """Q, K, V as bf16 bit patterns, raster layout [B, N, heads, d] (uint16).

    `heads` restricts generation to a subset of heads (others stay zero); the
    bytes of a generated head do not depend on which other heads are made.
    """
    N = w.tokens
    pos = _positions(w.grid)
    amps = head_amplitudes(w)
    hs = list(range(w.heads)) if heads is None else list(heads)
    out = {name: np.zeros((w.B, N, w.heads, w.d), dtype=np.uint16) for name in ("q", "k", "v")}
    jobs = [(name, tid, b, hd) for tid, name in enumerate(("q", "k", "v"))
            for b in range(w.B) for hd in hs]
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_fill_head, out[name], w, tid, b, hd, pos, float(amps[hd]))
                for name, tid, b, hd in jobs]
        for f in futs:
            f.result()
    return out


def generate_weights(w: Workload) -> Dict[str, np.ndarray]:
    """W_q, W_k as bf16 bit patterns [heads, 3d, r] (uint16), row-major (stats @ W)."""
    out = {}
    for name, tid in (("wq", 100), ("wk", 101)):
        arr = np.zeros((w.heads, 3 * w.d, w.r), dtype=np.uint16)
        for hd in range(w.heads):
            g = _rng(w.seed, tid, hd).standard_normal((3 * w.d, w.r)) / math.sqrt(3 * w.d)
            arr[hd] = to_bf16_bits(g.astype(np.float32))
        out[name] = arr
    return out


def generate(w: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    d = generate_qkv(w, threads)
    d.update(generate_weights(w))
    return d
