"""Helpers for the GPU parity tests: move seeded host bytes to the device, run
the HIP path through the C ABI, and compare with the CPU oracle computed from
the same host bytes."""

from __future__ import annotations

import math
import sys
from typing import Dict, List, Sequence

import numpy as np
import torch

import oracle as O

# Tolerances for attention output and LSE (bf16 inputs, fp32 MFMA accumulate,
# P rounded to bf16 before the PV product, fp32 online softmax). O is stored
# in bf16, whose half-ulp alone exceeds 1e-2 once |o| >= 4 (1.5625e-2 on
# [4, 8)) and is 7.8e-3 on [2, 4), where the path's own fp32 error can push
# the rounding to the other neighbour. So:
#   |o| <  2: the literal bound |got - want| <= 1e-2;
#   |o| >= 2: the error beyond the output's own quantisation,
#             |got - want| <= 1e-2 + half_ulp_bf16(want);
#   relative L2 <= 5e-3 everywhere.
# Every comparison is recorded with its raw max-abs error beside the
# beyond-rounding figure (RECORD; written out by conftest when
# VEDA_PARITY_LOG names a file).
O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
O_LITERAL_BELOW = 2.0
LSE_MAX_ABS = 2e-3

RECORD: List[dict] = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def f32_of_bf16(t: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_float(bits_of(t))


def geometry(w, heads: Sequence[int] = None):
    import block_sparse_attention_13_amd as V
    return V.Geometry(w.B, w.heads, w.d, w.grid, w.head_tiles())


def oracle_head(data: Dict[str, np.ndarray], w, b: int, hd: int, k: int, query_tiles=None, scale=None):
    """The oracle's whole layer for one (batch, head) from the host bytes."""
    q, k_, v = (O.bf16_bits_to_float(data[n][b, :, hd, :]) for n in ("q", "k", "v"))
    wq, wk = (O.bf16_bits_to_float(data[n][hd]) for n in ("wq", "wk"))
    return O.head_forward(q, k_, v, wq, wk, w.grid, w.head_tiles()[hd], k, scale=scale, query_tiles=query_tiles)


def compare_o(got: np.ndarray, want: np.ndarray, what: str):
    """Element-wise attention check: max-abs (literal below |o| = 2, beyond
    the bf16 half-ulp above) and relative L2. Returns (raw max-abs, rel-L2)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(np.max(err)) if err.size else 0.0
    beyond = err - half_ulp_bf16(want)
    excess = float(np.max(beyond)) if err.size else 0.0
    small = np.abs(want) < O_LITERAL_BELOW
    max_abs_small = float(np.max(err[small])) if np.any(small) else 0.0
    over = err > O_MAX_ABS
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    rec = {"what": what, "elements": int(err.size), "o_max_abs": max_abs, "o_max_abs_beyond_bf16_rounding": excess,
           "o_max_abs_where_abs_o_below_2": max_abs_small, "elements_over_1e-2": int(over.sum()),
           "abs_o_of_those_min": float(np.abs(want[over]).min()) if np.any(over) else None,
           "o_rel_l2": rel, "max_abs_o": float(np.max(np.abs(want))) if err.size else 0.0}
    RECORD.append(rec)
    assert max_abs_small <= O_MAX_ABS and excess <= O_MAX_ABS and rel <= O_REL_L2, \
        (f"{what}: max-abs {max_abs:.3e} ({max_abs_small:.3e} where |o| < 2, {excess:.3e} beyond bf16 output "
         f"rounding), rel-L2 {rel:.3e}")
    return max_abs, rel


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def compare_lse(got: np.ndarray, want: np.ndarray, what: str):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))
    assert err <= LSE_MAX_ABS, f"{what}: LSE max-abs {err:.3e}"
    return err
