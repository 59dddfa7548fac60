"""The CPU oracle checked against what the pages and the mathematics fix."""

import numpy as np
import pytest

import oracle as O
import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_SMALL_CHECKS, ids=lambda c: getattr(c, "__name__", "check"))
def test_oracle_pin(check):
    check(O)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: goes up to 1 + 2^-6.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    assert O.bf16_round(x).tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def test_workload_shapes_match_the_configs():
    """Box counts and k per head as the workload descriptions state them."""
    import datagen
    W = datagen.WORKLOADS
    assert W["tiny"].tiles_per_head() == [8, 8] and W["tiny"].k_per_head() == [4, 4]
    assert W["long"].tiles_per_head() == [1920] * 40 and W["long"].k_per_head() == [96] * 40
    assert W["480p"].tiles_per_head() == [336] * 12 and W["480p"].k_per_head() == [34] * 12
    assert W["720p"].tiles_per_head() == [720] * 40 and W["720p"].k_per_head() == [36] * 40
    hc = W["hc"]
    assert hc.tiles_per_head()[:3] == [720, 630, 720] and hc.k_per_head()[:3] == [72, 63, 72]
    for w in W.values():
        for hd, tile in enumerate(w.head_tiles()):
            assert tile[0] * tile[1] * tile[2] == 128
            assert O.num_tiles(w.grid, tile) == w.tiles_per_head()[hd]


def test_oracle_head_forward_tiny_is_consistent():
    import datagen
    w = datagen.WORKLOADS["tiny"]
    data = datagen.generate(w)
    q, k, v = (O.bf16_bits_to_float(data[n][0, :, 0, :]) for n in ("q", "k", "v"))
    wq, wk = (O.bf16_bits_to_float(data[n][0]) for n in ("wq", "wk"))
    r = O.head_forward(q, k, v, wq, wk, w.grid, w.head_tiles()[0], w.k_per_head()[0])
    assert r["idx"].shape == (8, 4) and np.all(np.diff(r["idx"], axis=1) > 0)
    assert np.all(np.isfinite(r["o"])) and np.all(np.isfinite(r["lse"]))
    assert np.array_equal(O.tile_unpermute(r["qt"], w.grid, (2, 8, 8)), q)
    # keeping every tile reproduces dense attention
    o_all, lse_all = O.sparse_attention(q, k, v, w.grid, (2, 8, 8), np.tile(np.arange(8), (8, 1)), 0.125)
    od, lsed = O.dense_attention(q, k, v, 0.125)
    assert np.max(np.abs(o_all - od)) < 1e-12 and np.all(r["lse"] <= lsed + 1e-12)


def test_products_stay_normal_on_generated_data():
    """The fp32 evaluation order is exact per step only if no product of two
    bf16 operands is subnormal; check that on a generated workload."""
    import datagen
    w = datagen.WORKLOADS["tiny"]
    data = datagen.generate(w)
    q = O.bf16_bits_to_float(data["q"][0, :, 0, :])
    qt, valid = O.tile_permute(q, w.grid, (2, 8, 8))
    st = O.trippool(qt, valid).astype(np.float64)
    wq = O.bf16_bits_to_float(data["wq"][0]).astype(np.float64)
    prods = np.abs(st[:, :, None] * wq[None, :, :])
    assert prods[prods > 0].min() > 2.0 ** -126


def test_input_generator_bytes_are_pinned():
    """The seeded inputs are the bytes recorded in tests/golden/datagen_sha256.json."""
    import json
    import os
    import importlib.util
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("make_datagen_hashes",
                                                  os.path.join(here, "golden", "make_datagen_hashes.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(here, "golden", "datagen_sha256.json")) as f:
        want = json.load(f)["hashes"]
    assert mod.hashes() == want
