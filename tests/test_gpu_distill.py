"""Distillation of the estimator: KL objective and gradient, the gradient
back to W_q/W_k, and Adam, HIP path vs the CPU oracle.

The oracle runs in float64 on the GPU's own inputs (its scores, teacher,
stats and features, read back bit for bit), so the comparison isolates each
kernel's fp32 arithmetic:
  * KL rows: fp32 softmax and logs over <= 720 terms: relative 1e-4;
  * d_scores: elementwise A_pred - A_tgt, absolute 1e-4 of the row's
    largest entry;
  * d_W: fp32 sums over <= 720 tiles of products: relative 1e-4 of the
    largest entry;
  * Adam: fp32 elementwise: relative 1e-5; the bf16 copy is exactly the
    round-to-nearest-even of the fp32 master."""

import dataclasses

import numpy as np
import pytest
import torch

import datagen
import oracle as O
from gpu_harness import bits_of, geometry, say, to_dev_bf16

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS


def _lib():
    import block_sparse_attention_13_amd as V
    return V


def _setup(w):
    V = _lib()
    data = datagen.generate(w)
    g = geometry(w)
    q, k, v, wq, wk = (to_dev_bf16(data[n]) for n in ("q", "k", "v", "wq", "wk"))
    out = V.layer_forward(q, k, v, wq, wk, g, w.k_per_head(), tiled_q=True, keep_scores=True)
    idx_d, ks_d = V.dense_index(g, q.device)
    _, lse = V.sparse_attn_fwd(out["q_t"], out["k_t"], out["v_t"], idx_d, g, ks_d)
    T = V.teacher_tile_max(out["q_t"], out["k_t"], lse, g)
    return g, out, T, wq, wk


@pytest.mark.parametrize("wname,heads,B", [("480p", 2, 2), ("hc", 3, 1)])
def test_distill_kl_and_grad_match_oracle(wname, heads, B):
    V = _lib()
    w = dataclasses.replace(W[wname].with_heads(heads), B=B)
    say(f"[distill] workload {w.name} heads {heads} B {B}")
    g, out, T, wq, wk = _setup(w)
    rows = sum(g.num_tiles(hd) for hd in range(heads)) * B
    kl, ds = V.distill_kl(out["scores"], T, g, 1.0 / rows)
    grads = V.distill_grad(out, ds, g)
    torch.cuda.synchronize()
    f32 = lambda t: t.float().cpu().numpy().astype(np.float64)
    S, Tc, klc, dsc = (x.cpu().numpy() for x in (out["scores"], T, kl, ds))
    sq, sk, fq, fk = (f32(out[n]) for n in ("stats_q", "stats_k", "feat_q", "feat_k"))
    dwq, dwk = grads["d_w_q"].cpu().numpy(), grads["d_w_k"].cpu().numpy()
    for hd in range(heads):
        n = g.num_tiles(hd)
        want_wq = np.zeros_like(dwq[hd], dtype=np.float64)
        want_wk = np.zeros_like(want_wq)
        for b in range(B):
            kl_ref, ds_ref = O.distill_kl(S[b, hd, :n, :n], Tc[b, hd, :n, :n], 1.0 / rows)
            rel = np.abs(klc[b, hd, :n] - kl_ref) / np.maximum(np.abs(kl_ref), 1e-6)
            assert rel.max() <= 1e-4, ("kl", hd, b, rel.max())
            assert np.all(klc[b, hd, n:] == 0) and not dsc[b, hd, n:].any() and not dsc[b, hd, :n, n:].any()
            err = np.abs(dsc[b, hd, :n, :n] - ds_ref).max(axis=1) / np.abs(ds_ref).max(axis=1)
            assert err.max() <= 1e-4, ("d_scores", hd, b, err.max())
            gq, gk = O.distill_grad(sq[b, hd, :n], sk[b, hd, :n], fq[b, hd, :n], fk[b, hd, :n],
                                    dsc[b, hd, :n, :n].astype(np.float64))
            want_wq += gq
            want_wk += gk
        for got, want, name in ((dwq[hd], want_wq, "d_w_q"), (dwk[hd], want_wk, "d_w_k")):
            e = np.abs(got - want).max() / np.abs(want).max()
            assert e <= 1e-4, (name, hd, e)
        say(f"[distill] head {hd}: KL rows, d_scores and d_W within tolerance")


def test_adam_step_matches_oracle():
    V = _lib()
    rng = np.random.default_rng(4)
    n = 40 * 384 * 64 + 7
    w0 = rng.standard_normal(n).astype(np.float32)
    w = torch.from_numpy(w0.copy()).cuda()
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    wb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    wr, mr, vr = w0.astype(np.float64), np.zeros(n), np.zeros(n)
    for step in range(1, 4):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1, n)).astype(np.float32)
        V.adam_step(w, torch.from_numpy(g).cuda(), m, v, step, 1e-2, (0.9, 0.99), 1e-8, wb)
        wr, mr, vr = O.adam_step(wr, g.astype(np.float64), mr, vr, step, 1e-2, 0.9, 0.99, 1e-8)
    torch.cuda.synchronize()
    got = w.cpu().numpy()
    assert np.max(np.abs(got - wr) / np.maximum(np.abs(wr), 1e-3)) <= 1e-5
    want_b = O.float_to_bf16_bits(O.bf16_round(got))
    assert np.array_equal(bits_of(wb), want_b)


def test_distillation_lowers_the_loss():
    """A few Adam steps on the 480p workload's calibration tiles lower the
    mean KL per query tile by an order of magnitude; the training is
    deterministic (fixed summation orders), so two runs agree bit for bit."""
    V = _lib()
    w = W["480p"].with_heads(2)
    g, out, T, wq, wk = _setup(w)
    r1 = V.distill_train(out["q_t"], out["k_t"], T, wq, wk, g, 60, 3e-3)
    r2 = V.distill_train(out["q_t"], out["k_t"], T, wq, wk, g, 60, 3e-3)
    say(f"[distill] loss {r1['loss'][0]:.3f} -> {r1['loss'][-1]:.3f}")
    assert r1["loss"][-1] < 0.1 * r1["loss"][0]
    assert r1["loss"] == r2["loss"] and torch.equal(r1["w_q"].view(torch.int16), r2["w_q"].view(torch.int16))


def test_distill_mean_kl_over_existing_rows():
    """veda_distill_mean_kl: the mean of kl_rows over the query tiles that
    exist (padded rows of shorter heads excluded), against numpy's fp64 mean
    of the same rows; B = 2 and three tile shapes give rows of different
    lengths. Rows past nT_hd are filled with garbage that must not count."""
    from block_sparse_attention_13_amd import _lib
    w = dataclasses.replace(W["hc"].with_heads(3), B=2)
    g = geometry(w)
    nT = g.max_tiles()
    rng = np.random.default_rng(17)
    rows = rng.uniform(0, 5, size=(w.B, w.heads, nT)).astype(np.float32)
    want = np.mean(np.concatenate([rows[b, hd, :g.num_tiles(hd)].astype(np.float64)
                                   for b in range(w.B) for hd in range(w.heads)]))
    for hd in range(w.heads):
        rows[:, hd, g.num_tiles(hd):] = 1e30
    t = torch.from_numpy(rows).cuda()
    mean = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    assert _lib.lib.veda_distill_mean_kl(g.c, t.data_ptr(), mean.data_ptr(), None) == 0
    got = mean.item()
    say(f"[distill] mean KL {got:.12f} vs {want:.12f}")
    assert abs(got - want) <= 1e-12 * want
