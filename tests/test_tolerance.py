"""The attention tolerance used by the GPU parity tests, exercised on the CPU:
the exact output rounded to bf16 passes it, and a single wrong tile in the
mask (a planted mistake in the oracle's input) fails it."""

import math

import numpy as np
import pytest

import datagen
import oracle as O
from gpu_harness import compare_o, half_ulp_bf16


def _tiny_head():
    w = datagen.WORKLOADS["tiny"]
    data = datagen.generate(w)
    q, k, v = (O.bf16_bits_to_float(data[n][0, :, 0, :]) for n in ("q", "k", "v"))
    wq, wk = (O.bf16_bits_to_float(data[n][0]) for n in ("wq", "wk"))
    return w, q, k, v, O.head_forward(q, k, v, wq, wk, w.grid, (2, 8, 8), 4)


def test_rounded_exact_output_passes():
    w, q, k, v, r = _tiny_head()
    compare_o(O.bf16_round(r["o"].astype(np.float32)), r["o"], "bf16-rounded oracle")


def test_one_flipped_mask_entry_fails():
    w, q, k, v, r = _tiny_head()
    idx = r["idx"].copy()
    row = 3
    missing = [j for j in range(8) if j not in idx[row]][0]
    idx[row, 0] = missing                          # swap one kept tile for a dropped one
    o_bad, _ = O.sparse_attention(q, k, v, w.grid, (2, 8, 8), np.sort(idx, axis=1), 1 / math.sqrt(64))
    with pytest.raises(AssertionError):
        compare_o(O.bf16_round(o_bad.astype(np.float32)), r["o"], "one tile swapped")


def test_half_ulp_values():
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([5.1]))[0] == 2.0 ** -6
