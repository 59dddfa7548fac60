"""Tile scores and their Top-k in one pass (veda_score_topk) against the CPU
oracle.

The inputs are seeded bf16 features; the expected lists and bitmasks are the
oracle's: its ordered fp32 scores of those features (tile_scores), then its
Top-k (a stable sort: equal scores keep the lower tile, -0 equals +0) and
bitmask, bit for bit. Feature rows past a head's own tiles are filled with
NaN patterns: the call must not read them. The two-call route
(trippool_project_score's scores, then topk_mask) must give the same bytes
on the layer's own features."""

import dataclasses

import numpy as np
import pytest
import torch

import datagen
import oracle as O
from gpu_harness import bits_of, geometry, say, to_dev_bf16

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
NAN_BITS = 0x7FC1


def _features(rng, B, heads, n_tiles, nT_max, r, kind):
    """bf16 bits [B, heads, nT_max, r]: N(0, 1) features, or (kind "ties")
    half-integers in [-2, 2] with signed zeros, whose scores tie often; rows
    past each head's tiles hold NaN patterns."""
    f = np.full((B, heads, nT_max, r), NAN_BITS, np.uint16)
    for b in range(B):
        for hd in range(heads):
            n = n_tiles[hd]
            if kind == "ties":
                x = rng.integers(-4, 5, size=(n, r)).astype(np.float32) * np.float32(0.5)
                x[x == 0] = np.where(rng.random(int((x == 0).sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
            else:
                x = rng.standard_normal((n, r)).astype(np.float32)
            f[b, hd, :n] = O.float_to_bf16_bits(O.bf16_round(x))
    return f


def _check(V, g, fq, fk, ks, with_bitmask=True):
    B, heads, nT_max, r = fq.shape
    kmax = max(ks)
    idx, bm = V.score_topk(to_dev_bf16(fq), to_dev_bf16(fk), g, ks, with_bitmask=with_bitmask)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    bm = bits_of(bm) if bm is not None else None
    words = (nT_max + 31) // 32
    for b in range(B):
        for hd in range(heads):
            n, k = g.num_tiles(hd), ks[hd]
            S = O.tile_scores(O.bf16_bits_to_float(fq[b, hd, :n]), O.bf16_bits_to_float(fk[b, hd, :n]))
            want = O.topk(S, k)
            got = idx[b, hd]
            assert np.array_equal(got[:n, :k], want), (b, hd)
            assert np.all(got[:n, k:] == -1) and np.all(got[n:] == -1), (b, hd, "pad")
            if bm is not None:
                want_bm = np.zeros((nT_max, words), np.uint32)
                ob = O.bitmask(want, n)
                want_bm[:n, :ob.shape[1]] = ob
                assert np.array_equal(bm[b, hd], want_bm), (b, hd, "bitmask")
    return idx


@pytest.mark.parametrize("grid,tiles,B,r,kind", [
    ((4, 16, 16), [(2, 8, 8)], 1, 32, "normal"),                             # 8 tiles
    ((21, 30, 52), [(4, 4, 8)], 1, 64, "normal"),                            # 1,008: ragged last chunk
    ((21, 45, 80), [(4, 4, 8), (1, 8, 16), (8, 4, 4)], 2, 64, "normal"),     # 720 / 630 / 720 tiles
    ((64, 48, 80), [(4, 4, 8)], 1, 64, "normal"),                            # 1,920: the long layer's rows
    ((21, 45, 80), [(4, 4, 8), (1, 8, 16), (8, 4, 4)], 1, 64, "ties"),
    ((7, 48, 40), [(1, 16, 8)], 1, 32, "ties"),                              # 105 tiles
])
def test_score_topk_matches_oracle(grid, tiles, B, r, kind):
    V = __import__("block_sparse_attention_13_amd")
    heads = len(tiles)
    g = V.Geometry(B, heads, 128, grid, tiles)
    n_tiles = [g.num_tiles(hd) for hd in range(heads)]
    nT = g.max_tiles()
    say(f"[score-topk] grid {grid} tiles {n_tiles} B {B} r {r} {kind}")
    rng = np.random.default_rng(sum(grid) + r)
    fq = _features(rng, B, heads, n_tiles, nT, r, kind)
    fk = _features(rng, B, heads, n_tiles, nT, r, kind)
    ks = [max(1, n // 20) + hd for hd, n in enumerate(n_tiles)]
    _check(V, g, fq, fk, ks)


def test_score_topk_extreme_k_and_no_bitmask():
    """k = 1, k = every tile and a middle k in one call; no bitmask output."""
    V = __import__("block_sparse_attention_13_amd")
    tiles = [(4, 4, 8), (1, 8, 16), (8, 4, 4)]
    g = V.Geometry(1, 3, 64, (9, 33, 70), tiles)
    n_tiles = [g.num_tiles(hd) for hd in range(3)]
    rng = np.random.default_rng(5)
    fq = _features(rng, 1, 3, n_tiles, g.max_tiles(), 32, "ties")
    fk = _features(rng, 1, 3, n_tiles, g.max_tiles(), 32, "ties")
    ks = [1, n_tiles[1], n_tiles[2] // 2]
    say(f"[score-topk] tiles {n_tiles}, k {ks}")
    _check(V, g, fq, fk, ks)
    _check(V, g, fq, fk, ks, with_bitmask=False)


def test_score_topk_longest_rows_and_beyond():
    """2,048 key tiles per row (the most the call holds on chip) match the
    oracle; 2,176 are refused with nothing written."""
    V = __import__("block_sparse_attention_13_amd")
    g = V.Geometry(1, 1, 128, (32, 64, 128), [(4, 4, 8)])
    assert g.max_tiles() == 2048 == V.SCORE_TOPK_MAX_TILES
    rng = np.random.default_rng(7)
    fq = _features(rng, 1, 1, [2048], 2048, 64, "normal")
    fk = _features(rng, 1, 1, [2048], 2048, 64, "normal")
    _check(V, g, fq, fk, [102])
    g2 = V.Geometry(1, 1, 128, (32, 64, 132), [(4, 4, 8)])
    n2 = g2.max_tiles()
    assert n2 == 2176
    f2 = to_dev_bf16(_features(rng, 1, 1, [n2], n2, 64, "normal"))
    idx = torch.full((1, 1, n2, 8), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(V.VedaError):
        V.score_topk(f2, f2, g2, [8], idx=idx, with_bitmask=False)
    torch.cuda.synchronize()
    assert bool((idx == 7).all())


@pytest.mark.parametrize("name,heads,B", [("hc", 6, 2), ("long", 40, 1)])   # long: the benchmarked layer, every head
def test_score_topk_equals_two_call_route(name, heads, B):
    """On the layer's own features, the one-pass call and the two calls
    (scores written by trippool_project_score, then topk_mask) give the
    same bytes in every row, into outputs with 4 KiB guards that stay
    untouched."""
    V = __import__("block_sparse_attention_13_amd")
    w = dataclasses.replace(W[name].with_heads(heads), B=B)
    data = datagen.generate(w)
    g = geometry(w)
    ks = w.k_per_head()
    q, k = to_dev_bf16(data["q"]), to_dev_bf16(data["k"])
    wq, wk = to_dev_bf16(data["wq"]), to_dev_bf16(data["wk"])
    stats_q = V.tile_stats(q, g)
    _, stats_k = V.tile_permute_stats(k, g)
    est = V.trippool_project_score(stats_q, stats_k, wq, wk, g)
    idx2, bm2 = V.topk_mask(est["scores"], g, ks)
    nT, kmax = g.max_tiles(), max(ks)
    guard = 4096
    n_idx, n_bm = B * heads * nT * kmax * 4, B * heads * nT * ((nT + 31) // 32) * 4
    buf_i = torch.full((n_idx + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    buf_b = torch.full((n_bm + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    idx1 = buf_i[guard:guard + n_idx].view(torch.int32).view(B, heads, nT, kmax)
    bm1 = buf_b[guard:guard + n_bm].view(torch.uint32).view(B, heads, nT, (nT + 31) // 32)
    feats = V.trippool_project_score(stats_q, stats_k, wq, wk, g, with_scores=False)
    assert set(feats) == {"feat_q", "feat_k"}
    V.score_topk(feats["feat_q"], feats["feat_k"], g, ks, idx=idx1, bitmask=bm1)
    torch.cuda.synchronize()
    say(f"[score-topk] {w.name} heads {heads} B {B}: {B * heads * nT} rows")
    assert torch.equal(feats["feat_q"].view(torch.int16), est["feat_q"].view(torch.int16))
    assert torch.equal(idx1, idx2)
    assert torch.equal(bm1.view(torch.int32), bm2.view(torch.int32))
    for buf in (buf_i, buf_b):
        assert bool((buf[:guard] == 0xA5).all()) and bool((buf[-guard:] == 0xA5).all())
