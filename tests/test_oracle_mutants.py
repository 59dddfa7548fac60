"""Plant a mistake in a copy of the oracle (on the CPU) and check that the pins
catch it. Each mutation is a textual edit of the oracle source; the copy is
executed as a separate module and every small pin is run against it: at least
one must fail, otherwise the pins do not bite on that part of the oracle."""

import os
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "veda_oracle.py")

MUTANTS = {
    "slot order transposed inside a box":
        ("sigma = ((t % pt) * ph + y % ph) * pw + x % pw", "sigma = ((x % pw) * ph + y % ph) * pt + t % pt"),
    "tile numbering column-major":
        ("tau = ((t // pt) * nTh + y // ph) * nTw + x // pw", "tau = ((x // pw) * nTh + y // ph) * (-(-grid[0] // pt)) + t // pt"),
    "floor instead of ceil box counts":
        ("return (-(-T // pt), -(-H // ph), -(-W // pw))", "return (max(1, T // pt), max(1, H // ph), max(1, W // pw))"),
    "mean summed in reverse slot order":
        ("for sigma in range(vol):", "for sigma in reversed(range(vol)):"),
    "mean divided by the box volume":
        ("n = v3.sum(axis=1).astype(np.float32)", "n = np.full(nT, vol, dtype=np.float32)"),
    "mean not rounded to bf16":
        ("avg = bf16_round((s / n[:, None]).astype(np.float32))", "avg = (s / n[:, None]).astype(np.float32)"),
    "max and min swapped":
        ("return np.concatenate([avg, mx, mn], axis=1)", "return np.concatenate([avg, mn, mx], axis=1)"),
    "pads count in max":
        ("mx = _from_total_order_key(np.where(v3[:, :, None], key, -big).max(axis=1))",
         "mx = _from_total_order_key(key.max(axis=1))"),
    "dot accumulated in float64":
        [("acc = np.zeros((a.shape[0], b.shape[1]), dtype=np.float32)", "acc = np.zeros((a.shape[0], b.shape[1]), dtype=np.float64)"),
         ("acc = (acc + prod).astype(np.float32)", "acc = acc + prod.astype(np.float64)")],
    "dot accumulated in descending order":
        ("for c in range(a.shape[1]):", "for c in reversed(range(a.shape[1])):"),
    "scores with the key side transposed wrongly":
        ("return fp32_dot_rows(feat_q, np.ascontiguousarray(np.asarray(feat_k, np.float32).T))",
         "return fp32_dot_rows(feat_k, np.ascontiguousarray(np.asarray(feat_q, np.float32).T))"),
    "top-k ties to the higher index":
        ("order = np.argsort(-S, axis=1, kind=\"stable\")[:, :k]",
         "order = (S.shape[1] - 1 - np.argsort(-S[:, ::-1], axis=1, kind=\"stable\"))[:, :k]"),
    "top-k keeps the smallest":
        ("order = np.argsort(-S, axis=1, kind=\"stable\")[:, :k]", "order = np.argsort(S, axis=1, kind=\"stable\")[:, :k]"),
    "top-k orders signed zeros by bit pattern":
        ("order = np.argsort(-S, axis=1, kind=\"stable\")[:, :k]",
         "order = np.argsort(-(S + np.where(np.signbit(S) & (S == 0), np.float32(-1e-30), np.float32(0))), axis=1, kind=\"stable\")[:, :k]"),
    "bitmask bit order reversed":
        ("out[row, j // 32] |= np.uint64(1) << np.uint64(j % 32)", "out[row, j // 32] |= np.uint64(1) << np.uint64(31 - j % 32)"),
    "softmax scale dropped":
        ("u = (q[qi] @ k[keys].T) * scale", "u = (q[qi] @ k[keys].T)"),
    "lse without the max":
        ("lse[qi] = (m + np.log(z))[:, 0]", "lse[qi] = np.log(z)[:, 0]"),
    "query tile reads the wrong mask row":
        ("keys = np.concatenate([members[j] for j in sel[i] if j >= 0])",
         "keys = np.concatenate([members[j] for j in sel[(i + 1) % len(sel)] if j >= 0])"),
    "output not normalised":
        ("o[qi] = (e @ v[keys]) / z", "o[qi] = (e @ v[keys]) / z.max()"),
    "teacher averages the block instead of its maximum":
        ("T[i, j] = best[tile_of == j].max()", "T[i, j] = best[tile_of == j].mean()"),
    "teacher skips the softmax normalisation":
        ("p /= p.sum(axis=1, keepdims=True)", "p = p"),
    "teacher pools over query tiles by the key's tile":
        ("qi = np.flatnonzero(tile_of == i)", "qi = np.flatnonzero(tile_of == (i + 1) % nT)"),
    "tile search sums absolute differences":
        ("errs.append(float(((r[\"o\"] - o_dense) ** 2).sum()))", "errs.append(float(np.abs(r[\"o\"] - o_dense).sum()))"),
    "distillation gradient with the wrong sign":
        ("return terms.sum(axis=1), grad_scale * (np.exp(log_p) - a_t)", "return terms.sum(axis=1), grad_scale * (a_t - np.exp(log_p))"),
    "distillation target not normalised":
        ("a_t = T / T.sum(axis=1, keepdims=True)", "a_t = T"),
    "distillation gradient through the wrong feature side":
        ("dFq = dS @ np.asarray(feat_k, np.float64)", "dFq = dS @ np.asarray(feat_q, np.float64)"),
    "adam without bias correction":
        ("mh = m / (1 - beta1 ** step)", "mh = m"),
    "layer projects Q with W_k and K with W_q":
        [("feat_q = project(stats_q, wq)", "feat_q = project(stats_q, wk)"),
         ("feat_k = project(stats_k, wk)", "feat_k = project(stats_k, wq)")],
    "layer pools K's statistics from Q's tiles":
        ("stats_k = trippool(kt, valid, vol)", "stats_k = trippool(qt, valid, vol)"),
    "layer default scale 1/d":
        ("scale = 1.0 / math.sqrt(d)\n    vol = tile[0]", "scale = 1.0 / d\n    vol = tile[0]"),
    "tile search default scale 1/d":
        ("scale = 1.0 / math.sqrt(d)\n    o_dense", "scale = 1.0 / d\n    o_dense"),
    "layer scores key tiles against query tiles":
        ("S = tile_scores(feat_q, feat_k)", "S = tile_scores(feat_k, feat_q)"),
    "layer attends to K in place of V":
        ("o, lse = sparse_attention(q, k, v, grid, tile, idx, scale, query_tiles)",
         "o, lse = sparse_attention(q, k, k, grid, tile, idx, scale, query_tiles)"),
    "average pooling scores the max block":
        ("mq = np.asarray(stats_q, np.float32)[:, :d]", "mq = np.asarray(stats_q, np.float32)[:, d:2 * d]"),
    "average pooling over half the channels":
        ("mk = np.asarray(stats_k, np.float32)[:, :d]", "mk = np.asarray(stats_k, np.float32)[:, :d // 2]; mq = mq[:, :d // 2]"),
    "average pooling scores transposed":
        ("return fp32_dot_rows(mq, np.ascontiguousarray(mk.T))", "return fp32_dot_rows(mk, np.ascontiguousarray(mq.T))"),
    "mask overlap counts either mask":
        ("both = np.asarray(bitmask_a, dtype=np.uint32) & np.asarray(bitmask_b, dtype=np.uint32)",
         "both = np.asarray(bitmask_a, dtype=np.uint32) | np.asarray(bitmask_b, dtype=np.uint32)"),
}


def _mutant(edits):
    with open(SRC) as f:
        src = f.read()
    for old, new in ([edits] if isinstance(edits, tuple) else edits):
        assert src.count(old) == 1, f"mutation anchor must occur exactly once: {old!r}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    M = _mutant(MUTANTS[name])
    failures = 0
    for check in P.ALL_SMALL_CHECKS:
        try:
            check(M)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught the mutant '{name}'"
