"""The estimator's tile scores on the matrix cores (veda_tile_scores_mfma)
against the CPU oracle's ordered fp32 scores.

Expected values come from the oracle alone, computed from the seeded inputs
(tile permute, TripPool statistics, projections, ordered scores); the HIP
path supplies only the features it scores, which a layer call makes and
which other tests hold bit-exact to the oracle's.

Bound: every product of two bf16 values is exact in fp32, and both sides
sum r of them in fp32, in different orders. Each differs from the exact sum
by at most gamma_r * sum |products| (gamma_n = n u / (1 - n u), u = 2^-24), so
the two differ by at most twice that. Top-k: where the lists differ, every
tile the MFMA list keeps and the oracle's drops must score, exactly, within
the two tiles' combined bounds of every tile the oracle keeps and the MFMA
list drops (a near-tie); elsewhere the lists are equal."""

import numpy as np
import pytest
import torch

import datagen
import oracle as O
from gpu_harness import geometry, say, to_dev_bf16

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def _oracle_features(data, w, hd):
    tile = w.head_tiles()[hd]
    out = {}
    for side, wname in (("q", "wq"), ("k", "wk")):
        x = O.bf16_bits_to_float(data[side][0, :, hd, :])
        xt, valid = O.tile_permute(x, w.grid, tile)
        stats = O.trippool(xt, valid)
        out[side] = O.project(stats, O.bf16_bits_to_float(data[wname][hd]))
    return out["q"], out["k"]


@pytest.mark.parametrize("name,heads", [("tiny", None), ("480p", 3), ("hc", 3), ("long", 2)])
def test_mfma_scores_within_rounding_and_masks_valid(name, heads):
    import block_sparse_attention_13_amd as V
    w = W[name] if heads is None else W[name].with_heads(heads)
    say(f"[scores-mfma] {w.name} heads {w.heads}")
    data = datagen.generate(w)
    g = geometry(w)
    ks = w.k_per_head()
    q, k, wq, wk = (to_dev_bf16(data[n]) for n in ("q", "k", "wq", "wk"))
    stats_q = V.tile_stats(q, g)
    _, stats_k = V.tile_permute_stats(k, g)
    est = V.trippool_project_score(stats_q, stats_k, wq, wk, g)
    s_mf = V.tile_scores_mfma(est["feat_q"], est["feat_k"], g)
    idx_mf, _ = V.topk_mask(s_mf, g, ks)
    torch.cuda.synchronize()
    s_mf = s_mf.cpu().numpy()
    idx_mf = idx_mf.cpu().numpy()
    r = w.r
    rows_differ = 0
    for hd in range(w.heads):
        nT = w.tiles_per_head()[hd]
        fq, fk = _oracle_features(data, w, hd)
        want = O.tile_scores(fq, fk)
        exact = fq.astype(np.float64) @ fk.astype(np.float64).T
        mag = np.abs(fq.astype(np.float64)) @ np.abs(fk.astype(np.float64)).T
        bound = 2 * gamma(r) * mag
        got = s_mf[0, hd, :nT, :nT]
        assert np.all(np.isneginf(s_mf[0, hd, nT:, :])) and np.all(np.isneginf(s_mf[0, hd, :, nT:])), hd
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.all(err <= bound), (hd, float((err - bound).max()))
        same = float(np.mean(got.view(np.uint32) == want.view(np.uint32)))
        kk = ks[hd]
        want_idx = O.topk(want, kk)
        e = 2 * gamma(r) * mag   # each MFMA score's distance from the exact one is within gamma_r * mag
        for i in range(nT):
            a = set(idx_mf[0, hd, i, :kk].tolist())
            b = set(want_idx[i].tolist())
            if a == b:
                continue
            rows_differ += 1
            for j in a - b:
                for j2 in b - a:
                    assert exact[i, j2] - exact[i, j] <= e[i, j] + e[i, j2], (hd, i, j, j2)
        say(f"[scores-mfma] head {hd}: bit-equal {same:.3f}, max error / bound {float((err / np.maximum(bound, 1e-300)).max()):.3f}")
    say(f"[scores-mfma] {w.name}: Top-k rows that differ from the ordered scores' {rows_differ}")


def test_mfma_scores_reject_bad_rank():
    import block_sparse_attention_13_amd as V
    from block_sparse_attention_13_amd import _lib
    w = W["tiny"]
    g = geometry(w)
    nT = g.max_tiles()
    f = torch.zeros((1, w.heads, nT, 48), dtype=torch.bfloat16, device="cuda")
    s = torch.full((1, w.heads, nT, nT), 7.0, device="cuda")
    rc = _lib.lib.veda_tile_scores_mfma(g.c, f.data_ptr(), f.data_ptr(), 48, s.data_ptr(), None)
    assert rc != 0
    torch.cuda.synchronize()
    assert bool((s == 7.0).all())
