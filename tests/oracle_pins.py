"""Pins of the CPU oracle to things other than itself.

Every check takes the oracle namespace `O` as an argument, so that the mutant
tests can run the same checks against oracles with a planted mistake and
confirm that each mistake is caught. Sources of truth used here:

  * hand-derived fixtures under tests/golden/ (each cites its passage);
  * brute-force enumeration written independently of the oracle's index math;
  * closed forms (Q = 0, one-hot values, two-key softmax);
  * library routines (torch scaled_dot_product_attention / logsumexp on CPU,
    numpy float64 dot products);
  * the pages' relations: the Z / Z_hat renormalisation of kept keys and the
    log-sum-exp potential (Theoretical Rationale 1, "Softmax Geometry"), the
    Bhatia-Davis bound (Theoretical Rationale 2, "Tile Statistics").
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_vals(rng, shape, scale=1.0):
    """Random bf16-representable float32 values (truncation of random floats)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


# ------------------------------------------------------------------ O1 / O7

def brute_force_positions(grid, tile):
    """Enumerate boxes in raster order of box coordinates and slots in raster
    order inside each box, handing out consecutive tiled positions; record
    which raster token (if any) sits at each position."""
    T, H, W = grid
    pt, ph, pw = tile
    nTt, nTh, nTw = -(-T // pt), -(-H // ph), -(-W // pw)
    pos = {}
    p = 0
    for bt in range(nTt):
        for by in range(nTh):
            for bx in range(nTw):
                for st in range(pt):
                    for sy in range(ph):
                        for sx in range(pw):
                            t, y, x = bt * pt + st, by * ph + sy, bx * pw + sx
                            if t < T and y < H and x < W:
                                pos[(t * H + y) * W + x] = p
                            p += 1
    return np.array([pos[n] for n in range(T * H * W)]), p


def check_permutation_golden(O):
    g = _golden("permutation_grid2x3x4_tile1x2x2.json")
    grid, tile = tuple(g["grid"]), tuple(g["tile"])
    assert O.num_tiles(grid, tile) == g["num_tiles"]
    assert list(O.tiled_position(grid, tile)) == g["tiled_position_of_raster_token"]
    x = np.arange(1, 25, dtype=np.float32)[:, None]
    xt, valid = O.tile_permute(x, grid, tile)
    assert sorted(np.flatnonzero(~valid).tolist()) == g["pad_slots"]
    assert np.all(xt[~valid] == 0)


def check_permutation_bruteforce(O, shapes):
    for grid, tile in shapes:
        want, total = brute_force_positions(grid, tile)
        got = O.tiled_position(grid, tile)
        assert O.num_tiles(grid, tile) * tile[0] * tile[1] * tile[2] == total
        assert np.array_equal(got, want), (grid, tile)
        # bijection onto the valid slots, inverse, pad count
        N = grid[0] * grid[1] * grid[2]
        x = np.arange(N, dtype=np.int64)[:, None] + 1
        xt, valid = O.tile_permute(x, grid, tile)
        assert valid.sum() == N and len(np.unique(got)) == N
        assert (~valid).sum() == total - N
        assert np.array_equal(O.tile_unpermute(xt, grid, tile), x)


# ------------------------------------------------------------------ O2

def check_trippool_golden(O):
    g = _golden("trippool_slot_order.json")
    for case in g["cases"]:
        vals = np.array(case["values"], dtype=np.float32)
        n = len(vals)
        vol = 8                                   # pad the box: only n slots are real
        xt = np.zeros((vol, 1), dtype=np.float32)
        xt[:n, 0] = vals
        valid = np.zeros(vol, dtype=bool)
        valid[:n] = True
        st = O.trippool(xt, valid, vol)[0]
        for got, key in zip(st, ("avg", "max", "min")):
            want = np.float32(case[key])
            assert got == want and np.signbit(got) == np.signbit(want), (case["comment"], key, got, want)


def check_trippool_bruteforce(O, grid, tile, d=6, seed=0):
    """Gather each box's real tokens straight from raster coordinates and check
    the statistics against their definitions."""
    rng = np.random.default_rng(seed)
    T, H, W = grid
    pt, ph, pw = tile
    vol = pt * ph * pw
    x = _bf16_vals(rng, (T * H * W, d), 2.0)
    xt, valid = O.tile_permute(x, grid, tile)
    st = O.trippool(xt, valid, vol)
    nTt, nTh, nTw = -(-T // pt), -(-H // ph), -(-W // pw)
    tau = 0
    for bt in range(nTt):
        for by in range(nTh):
            for bx in range(nTw):
                rows = []
                for t in range(bt * pt, min(T, bt * pt + pt)):
                    for y in range(by * ph, min(H, by * ph + ph)):
                        for xx in range(bx * pw, min(W, bx * pw + pw)):
                            rows.append(x[(t * H + y) * W + xx])
                g = np.array(rows, dtype=np.float64)
                mean = g.mean(axis=0)
                M, m = g.max(axis=0), g.min(axis=0)
                avg, mx, mn = st[tau, :d], st[tau, d:2 * d], st[tau, 2 * d:]
                assert np.array_equal(mx, M.astype(np.float32)) and np.array_equal(mn, m.astype(np.float32))
                assert np.all(mn <= avg) and np.all(avg <= mx)
                # float32 sum error + one bf16 rounding (relative 2^-8)
                err = 1.01 * len(rows) * 2.0 ** -24 * np.abs(g).sum(axis=0) / len(rows)
                assert np.all(np.abs(avg - mean) <= err + np.abs(mean) * 2.0 ** -8 + 1e-30)
                # Bhatia-Davis (Tile Statistics): var <= (M - mu)(mu - m)
                var = g.var(axis=0)
                assert np.all(var <= (M - mean) * (mean - m) * (1 + 1e-12) + 1e-12)
                tau += 1


def check_trippool_constant(O):
    xt = np.full((16, 3), np.float32(0.375))
    valid = np.ones(16, dtype=bool)
    valid[11:] = False
    xt[11:] = 0
    st = O.trippool(xt, valid, 16)[0]
    assert np.all(st == np.float32(0.375))


# ------------------------------------------------------------------ O3 / O4

def check_dot_golden(O):
    g = _golden("fp32_dot_order.json")
    for case in g["cases"]:
        a = np.array([case["a"]], dtype=np.float32)
        b = np.array(case["b"], dtype=np.float32)[:, None]
        got = O.fp32_dot_rows(a, b)[0, 0]
        assert got == np.float32(case["result"]), case["comment"]


def check_dot_error_bound(O, seed=1):
    """|fl32 sum - exact| <= gamma_n * sum |a_c b_c| (Higham's bound for a
    recursive sum of exact products), against a float64 (exact here) dot."""
    rng = np.random.default_rng(seed)
    for n in (1, 7, 64, 384):
        a = _bf16_vals(rng, (9, n), 3.0)
        b = _bf16_vals(rng, (n, 5), 0.05)
        got = O.fp32_dot_rows(a, b).astype(np.float64)
        exact = a.astype(np.float64) @ b.astype(np.float64)
        u = 2.0 ** -24
        gam = n * u / (1 - n * u)
        bound = gam * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
        assert np.all(np.abs(got - exact) <= bound)


def check_projection_rounds_to_bf16(O, seed=2):
    rng = np.random.default_rng(seed)
    st = _bf16_vals(rng, (11, 24))
    w = _bf16_vals(rng, (24, 8), 0.2)
    p = O.project(st, w)
    assert np.all((p.view(np.uint32) & np.uint32(0xFFFF)) == 0)
    exact = st.astype(np.float64) @ w.astype(np.float64)
    assert np.all(np.abs(p - exact) <= np.abs(exact) * 2.0 ** -8 + 24 * 2.0 ** -24 * (np.abs(st) @ np.abs(w)) * 2)


def check_average_pooling_special_case(O, seed=3):
    """With W = [I_r; 0; 0] the estimator reduces to the average-pooling score
    (the mean-only baseline the pages compare against), a plain dot product
    of the tile means."""
    rng = np.random.default_rng(seed)
    grid, tile, d, r = (2, 4, 8), (1, 2, 4), 8, 4
    vol = 8
    q = _bf16_vals(rng, (64, d))
    k = _bf16_vals(rng, (64, d))
    qt, valid = O.tile_permute(q, grid, tile)
    kt, _ = O.tile_permute(k, grid, tile)
    W = np.zeros((3 * d, r), dtype=np.float32)
    W[np.arange(r), np.arange(r)] = 1.0
    S = O.tile_scores(O.project(O.trippool(qt, valid, vol), W), O.project(O.trippool(kt, valid, vol), W))
    mq = qt.reshape(-1, vol, d).astype(np.float64).mean(axis=1)[:, :r]
    mk = kt.reshape(-1, vol, d).astype(np.float64).mean(axis=1)[:, :r]
    want = mq @ mk.T
    # two bf16 roundings of the means (2^-8 relative each) and a float32 dot
    tol = 3 * 2.0 ** -8 * (np.abs(mq) @ np.abs(mk).T) + 1e-6
    assert np.all(np.abs(S - want) <= tol)


def check_avgpool_scores(O, seed=14):
    """Average-pooling scores three ways. (1) Small-integer tokens in full
    boxes of 16 make every tile mean exact in bf16 and every score exact in
    float32, so the scores equal the dot products of tile means gathered by
    brute force from raster coordinates (all d channels; query means on the
    left, key means on the right, so a transposed or max-pooled score fails).
    (2) On a ragged grid with general bf16 values they equal the estimator
    with rank d and W = [I; 0; 0], bit for bit (same evaluation order).
    (3) They stay within the float32 accumulation bound of the exact dot
    product of the bf16 means."""
    rng = np.random.default_rng(seed)
    grid, tile, d = (2, 4, 8), (1, 2, 8), 8                 # 64 tokens, 4 full boxes of 16
    N = 64
    q = rng.integers(-8, 9, size=(N, d)).astype(np.float32)
    k = rng.integers(-8, 9, size=(N, d)).astype(np.float32)
    qt, valid = O.tile_permute(q, grid, tile)
    kt, _ = O.tile_permute(k, grid, tile)
    S = O.avgpool_scores(O.trippool(qt, valid, 16), O.trippool(kt, valid, 16))
    pos, _ = brute_force_positions(grid, tile)
    tile_of = pos // 16
    mq = np.stack([q[tile_of == j].astype(np.float64).mean(axis=0) for j in range(4)])
    mk = np.stack([k[tile_of == j].astype(np.float64).mean(axis=0) for j in range(4)])
    assert np.array_equal(S.astype(np.float64), mq @ mk.T)
    assert not np.array_equal(mq @ mk.T, (mq @ mk.T).T)            # the check sees a transposition
    grid, tile, d = (3, 5, 6), (2, 2, 4), 8                 # ragged: 2 x 3 x 2 boxes of 16
    q = _bf16_vals(rng, (90, d))
    k = _bf16_vals(rng, (90, d))
    qt, valid = O.tile_permute(q, grid, tile)
    kt, _ = O.tile_permute(k, grid, tile)
    sq, sk = O.trippool(qt, valid, 16), O.trippool(kt, valid, 16)
    W = np.zeros((3 * d, d), np.float32)
    W[np.arange(d), np.arange(d)] = 1.0
    S = O.avgpool_scores(sq, sk)
    assert np.array_equal(S, O.tile_scores(O.project(sq, W), O.project(sk, W)))
    a = sq[:, :d].astype(np.float64)
    b = sk[:, :d].astype(np.float64)
    gamma = d * 2.0 ** -24 / (1 - d * 2.0 ** -24)
    assert np.all(np.abs(S - a @ b.T) <= gamma * (np.abs(a) @ np.abs(b).T) + 1e-30)


# ------------------------------------------------------------------ O5

def check_topk_golden(O):
    g = _golden("topk_ties.json")
    S = np.array([g["scores"]], dtype=np.float32)
    for case in g["cases"]:
        idx = O.topk(S, case["k"])
        assert idx[0].tolist() == case["idx"], case
        assert O.bitmask(idx, S.shape[1])[0].tolist() == case["bitmask"], case
        assert O.topk_row_bruteforce(S[0], case["k"]) == case["idx"]


def check_topk_bruteforce(O, seed=4):
    rng = np.random.default_rng(seed)
    for n, k in ((1, 1), (5, 3), (33, 7), (70, 70), (129, 10)):
        S = rng.integers(-3, 4, size=(6, n)).astype(np.float32) * np.float32(0.5)
        S[S == 0] = np.where(rng.random((S == 0).sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
        S[-1] = rng.standard_normal(n).astype(np.float32)
        idx = O.topk(S, k)
        for r in range(S.shape[0]):
            row = [float(v) for v in S[r]]
            # independent brute force: repeatedly take the best remaining
            left = list(range(n))
            keep = []
            for _ in range(k):
                best = left[0]
                for j in left[1:]:
                    if row[j] > row[best]:
                        best = j
                keep.append(best)
                left.remove(best)
            assert idx[r].tolist() == sorted(keep), (n, k, r)
        if k < n:
            small = O.topk(S, k - 1) if k > 1 else np.zeros((S.shape[0], 0), dtype=np.int64)
            for r in range(S.shape[0]):
                assert set(small[r].tolist()) <= set(idx[r].tolist())


# ------------------------------------------------------------------ O6

def check_attention_two_keys(O):
    """Closed form: logits (0, 2) give p = (1/(1+e^2), e^2/(1+e^2)) and
    LSE = log(1 + e^2)."""
    grid, tile = (1, 1, 4), (1, 1, 2)
    q = np.zeros((4, 4))
    q[:, 0] = 2.0                                   # scale 1/sqrt(4): u = q.k / 2
    k = np.array([[0, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [2, 0, 0, 0]], dtype=np.float64)
    v = np.array([[5, 5, 5, 5], [7, 7, 7, 7], [1, 0, 0, 0], [0, 1, 0, 0]], dtype=np.float64)
    sel = np.array([[1], [1]])
    o, lse = O.sparse_attention(q, k, v, grid, tile, sel, 0.5)
    p0 = 1.0 / (1.0 + math.exp(2.0))
    want = np.array([p0, 1 - p0, 0, 0])
    assert np.allclose(o, want[None, :], rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(1 + math.exp(2.0)), rtol=0, atol=1e-14)


def check_attention_dense_matches_sdpa(O, seed=5):
    """Keeping every tile gives plain softmax attention; compare with torch's
    scaled_dot_product_attention and logsumexp in float64 on the CPU."""
    import torch
    rng = np.random.default_rng(seed)
    grid, tile, d = (2, 3, 8), (1, 2, 4), 16          # padded: 8 boxes of 8, 48 tokens
    N = 48
    q, k, v = (_bf16_vals(rng, (N, d)) for _ in range(3))
    nT = O.num_tiles(grid, tile)
    sel = np.tile(np.arange(nT), (nT, 1))
    scale = 1.0 / math.sqrt(d)
    o, lse = O.sparse_attention(q, k, v, grid, tile, sel, scale)
    tq, tk, tv = (torch.from_numpy(a.astype(np.float64))[None, None] for a in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    want_lse = torch.logsumexp((tq @ tk.transpose(-1, -2))[0, 0] * scale, dim=-1).numpy()
    assert np.max(np.abs(o - want)) < 1e-12
    assert np.max(np.abs(lse - want_lse)) < 1e-12
    od, lsed = O.dense_attention(q, k, v, scale)
    assert np.max(np.abs(od - want)) < 1e-12 and np.max(np.abs(lsed - want_lse)) < 1e-12


def _random_sel(rng, nT, k):
    return np.sort(np.stack([rng.choice(nT, size=k, replace=False) for _ in range(nT)]), axis=1)


def check_attention_renormalisation(O, seed=6):
    """With V = identity the output row is the probability row itself. Kept
    keys then satisfy P_sparse = P_dense * Z / Z_hat, and Z / Z_hat =
    exp(LSE_dense - LSE_sparse) >= 1 (Softmax Geometry)."""
    rng = np.random.default_rng(seed)
    grid, tile = (2, 2, 6), (1, 2, 2)                  # 24 tokens, 6 boxes of 4
    N, d = 24, 8
    q = _bf16_vals(rng, (N, d))
    k = _bf16_vals(rng, (N, d))
    v = np.eye(N)
    nT = O.num_tiles(grid, tile)
    scale = 1.0 / math.sqrt(d)
    sel = _random_sel(rng, nT, 2)
    ps, lses = O.sparse_attention(q, k, v, grid, tile, sel, scale)
    pd, lsed = O.dense_attention(q, k, v, scale)
    assert np.allclose(ps.sum(axis=1), 1.0, atol=1e-12)
    ratio = np.exp(lsed - lses)
    assert np.all(ratio >= 1.0 - 1e-12) and np.all(lses <= lsed + 1e-12)
    tile_of = O.tiled_position(grid, tile) // 4
    for n in range(N):
        kept = np.isin(tile_of, sel[tile_of[n]])
        assert np.allclose(ps[n, kept], pd[n, kept] * ratio[n], rtol=1e-10, atol=1e-15)
        assert np.all(ps[n, ~kept] == 0)


def check_attention_zero_query(O, seed=7):
    """Q = 0 makes every logit 0, so each output is the plain mean of the real
    value rows in the selected tiles (pad slots must not count)."""
    rng = np.random.default_rng(seed)
    grid, tile = (3, 3, 5), (2, 2, 2)                  # heavily padded
    N, d = 45, 4
    q = np.zeros((N, d))
    k = _bf16_vals(rng, (N, d))
    v = _bf16_vals(rng, (N, d))
    nT = O.num_tiles(grid, tile)
    sel = _random_sel(rng, nT, 3)
    o, lse = O.sparse_attention(q, k, v, grid, tile, sel, 0.5)
    T, H, W = grid
    for n in range(N):
        t, y, x = n // (H * W), (n // W) % H, n % W
        my = ((t // 2) * 2 + y // 2) * 3 + x // 2         # box of token n, computed directly
        rows = []
        for m in range(N):
            tm, ym, xm = m // (H * W), (m // W) % H, m % W
            if ((tm // 2) * 2 + ym // 2) * 3 + xm // 2 in sel[my]:
                rows.append(v[m])
        assert np.allclose(o[n], np.mean(rows, axis=0), atol=1e-12)
        assert abs(lse[n] - math.log(len(rows))) < 1e-12


def check_attention_monotone_and_bounded(O, seed=8):
    rng = np.random.default_rng(seed)
    grid, tile = (2, 4, 4), (1, 2, 4)                 # 4 boxes of 8
    N, d = 32, 8
    q, k, v = (_bf16_vals(rng, (N, d), 2.0) for _ in range(3))
    nT = O.num_tiles(grid, tile)
    S = rng.standard_normal((nT, nT)).astype(np.float32)
    prev = None
    for kk in range(1, nT + 1):
        sel = O.topk(S, kk)
        o, lse = O.sparse_attention(q, k, v, grid, tile, sel, 0.3)
        if prev is not None:
            assert np.all(lse >= prev - 1e-12)
        prev = lse
        tile_of = O.tiled_position(grid, tile) // 8
        for n in range(N):
            rows = v[np.isin(tile_of, sel[tile_of[n]])]
            assert np.all(o[n] <= rows.max(axis=0) + 1e-12) and np.all(o[n] >= rows.min(axis=0) - 1e-12)


# ------------------------------------------------------- teacher and recall

def check_teacher_matches_pooled_softmax(O, seed=9):
    """Teacher = block max-pooling of the full softmax map: build the dense
    probability matrix with torch.softmax (float64, CPU), lay it out in tiled
    order with the brute-force positions (pad rows and columns -inf), and
    max-pool each (query tile, key tile) block with amax; compare."""
    import torch
    rng = np.random.default_rng(seed)
    grid, tile, d = (2, 3, 8), (1, 2, 4), 16            # padded: 8 boxes of 8 slots, 48 tokens
    N, vol = 48, 8
    q, k = (_bf16_vals(rng, (N, d), 2.0) for _ in range(2))
    scale = 0.7
    P = torch.softmax(torch.from_numpy(q.astype(np.float64)) @ torch.from_numpy(k.astype(np.float64)).T * scale,
                      dim=-1)
    pos, total = brute_force_positions(grid, tile)
    nT = total // vol
    Pt = torch.full((total, total), -math.inf, dtype=torch.float64)
    idx = torch.from_numpy(pos)
    Pt[idx[:, None], idx[None, :]] = P
    want = Pt.reshape(nT, vol, nT, vol).amax(dim=(1, 3)).numpy()
    got = O.teacher_tile_max(q, k, grid, tile, scale)
    assert got.shape == (nT, nT)
    assert np.max(np.abs(got - want)) < 1e-14
    sub = O.teacher_tile_max(q, k, grid, tile, scale, query_tiles=[3])
    assert np.array_equal(sub[3], got[3]) and np.all(np.isnan(np.delete(sub, 3, axis=0)))


def check_teacher_uniform_keys(O):
    """Identical keys give every query the uniform distribution 1/N, so every
    block maximum is exactly 1/N; a key that dominates every query's logits
    gives probability ~1 in its tile's column and ~0 elsewhere."""
    grid, tile, d = (2, 4, 4), (1, 4, 4), 4              # 2 full boxes of 16 slots, 32 tokens
    N = 32
    q = np.linspace(-1, 1, N * d).reshape(N, d).astype(np.float32)
    k = np.tile(np.array([[0.5, -0.25, 1.0, 2.0]], np.float32), (N, 1))
    T = O.teacher_tile_max(q, k, grid, tile, 1.0)
    assert np.allclose(T, 1.0 / N, rtol=1e-13, atol=0)
    k2 = np.zeros((N, d), np.float32)
    k2[5] = 40.0                                         # raster token 5 = (t 0, y 1, x 1): box 0
    q2 = np.ones((N, d), np.float32)
    T2 = O.teacher_tile_max(q2, k2, grid, tile, 1.0)
    # logits: 160 for token 5, 0 for the 31 others: p = 1 / (1 + 31 e^-160) and e^-160 / (1 + 31 e^-160)
    assert np.all(T2[:, 0] == 1.0)
    assert np.allclose(T2[:, 1], math.exp(-160.0) / (1 + 31 * math.exp(-160.0)), rtol=1e-12, atol=0)


def check_recall_golden(O):
    """Tile recall and mask overlap on hand-made masks: query tile 0 keeps
    {0, 1} against an oracle {1, 2}; tile 1 keeps {2, 3} against {2, 3}: 3 of
    the oracle's 4 kept tiles, so recall 3/4 and overlap 3."""
    m = np.array([[0, 1], [2, 3]])
    o = np.array([[1, 2], [2, 3]])
    assert O.tile_recall(m, o) == 0.75
    assert O.tile_recall(o, o) == 1.0
    assert O.mask_overlap(O.bitmask(m, 4), O.bitmask(o, 4)) == 3
    assert O.mask_overlap(O.bitmask(m, 40), O.bitmask(np.array([[2, 3], [0, 1]]), 40)) == 0


# --------------------------------------------------------------- tile search

def check_tile_search_errors(O, seed=10):
    """The search objective through an independent route: for one candidate,
    keep the oracle's own tile lists but redo the attention as torch
    scaled_dot_product_attention with a boolean token mask built from the
    brute-force tiled positions, against unmasked SDPA, and sum the squared
    difference. With every tile kept the error vanishes for every candidate."""
    import torch
    rng = np.random.default_rng(seed)
    grid, d, r = (2, 4, 16), 16, 8                         # 128 tokens
    N = 128
    q, k, v = (_bf16_vals(rng, (N, d)) for _ in range(3))
    wq, wk = (_bf16_vals(rng, (3 * d, r), 0.2) for _ in range(2))
    cands = [(1, 4, 8), (2, 2, 8), (1, 1, 16)]             # volume 32 boxes: tile volume need not be 128 here
    keep = lambda n: max(1, n // 2)
    errs = O.tile_search_errors(q, k, v, wq, wk, grid, cands, keep)
    t = lambda a: torch.from_numpy(a.astype(np.float64))[None, None]
    dense = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0]
    for ci, tile in enumerate(cands):
        vol = tile[0] * tile[1] * tile[2]
        res = O.head_forward(q, k, v, wq, wk, grid, tile, keep(O.num_tiles(grid, tile)))
        pos, _ = brute_force_positions(grid, tile)
        tile_of = pos // vol
        allowed = np.zeros((N, N), bool)
        for n in range(N):
            allowed[n] = np.isin(tile_of, res["idx"][tile_of[n]])
        o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v),
                                                             attn_mask=torch.from_numpy(allowed)[None, None])[0, 0]
        want = float(((o - dense) ** 2).sum())
        assert abs(errs[ci] - want) <= 1e-9 * max(want, 1e-30), (tile, errs[ci], want)
    assert np.all(O.tile_search_errors(q, k, v, wq, wk, grid, cands, lambda n: n) < 1e-20)


# ------------------------------------------------------------ whole layer

def _tile_members(grid, tile):
    """Raster tokens of each tile, from the brute-force enumeration."""
    pos, _ = brute_force_positions(grid, tile)
    vol = tile[0] * tile[1] * tile[2]
    return pos // vol, pos % vol


def check_head_forward_wiring(O):
    """The whole layer of one head, wired step by step, against an independent
    route from raster coordinates. Inputs are small integers, so the mean,
    max, projections and scores are exact; W_q picks the avg block and W_k
    the max block, so swapping the projections or pooling the wrong tensor
    changes the scores. The expected tile statistics come from the
    brute-force tile membership (torch float32 divide, then torch's
    round-to-nearest-even to bfloat16); the mask from an exhaustive sort;
    O and LSE from torch scaled_dot_product_attention with a boolean token
    mask at its own default scale 1/sqrt(d) (the oracle's default must agree)."""
    import torch
    rng = np.random.default_rng(13)
    grid, tile, d, r, k_keep = (3, 4, 7), (2, 2, 4), 4, 4, 3      # ragged on two axes: 8 boxes of 16
    N = grid[0] * grid[1] * grid[2]
    q = rng.integers(-8, 9, size=(N, d)).astype(np.float32)
    k = rng.integers(-8, 9, size=(N, d)).astype(np.float32)
    v = rng.integers(-8, 9, size=(N, d)).astype(np.float32) / np.float32(4)
    wq = np.zeros((3 * d, r), np.float32)
    wk = np.zeros((3 * d, r), np.float32)
    wq[np.arange(r), np.arange(r)] = 1.0                          # avg block of Q
    wk[d + np.arange(r), np.arange(r)] = 1.0                      # max block of K
    res = O.head_forward(q, k, v, wq, wk, grid, tile, k_keep)
    tile_of, _ = _tile_members(grid, tile)
    nT = int(tile_of.max()) + 1
    assert O.num_tiles(grid, tile) == nT == 8

    def stats(x):
        out = np.zeros((nT, 3 * d), np.float64)
        for j in range(nT):
            rows = x[tile_of == j]
            mean = (torch.tensor(rows.sum(axis=0), dtype=torch.float32) / len(rows)).to(torch.bfloat16)
            out[j] = np.concatenate([mean.double().numpy(), rows.max(axis=0), rows.min(axis=0)])
        return out

    sq, sk = stats(q), stats(k)
    assert np.array_equal(res["stats_q"].astype(np.float64), sq)
    assert np.array_equal(res["stats_k"].astype(np.float64), sk)
    assert np.array_equal(res["feat_q"].astype(np.float64), sq[:, :r])
    assert np.array_equal(res["feat_k"].astype(np.float64), sk[:, d:d + r])
    S = sq[:, :r] @ sk[:, d:d + r].T
    assert np.array_equal(res["scores"].astype(np.float64), S)
    for i in range(nT):
        best = sorted(range(nT), key=lambda j: (-S[i, j], j))[:k_keep]
        assert res["idx"][i].tolist() == sorted(best), i
    allowed = np.zeros((N, N), bool)
    for n in range(N):
        allowed[n] = np.isin(tile_of, res["idx"][tile_of[n]])
    t = lambda a: torch.from_numpy(a.astype(np.float64))[None, None]
    mask = torch.from_numpy(allowed)[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)[0, 0].numpy()
    logits = (t(q) @ t(k).transpose(-1, -2))[0, 0] / math.sqrt(d)
    want_lse = torch.logsumexp(logits.masked_fill(~torch.from_numpy(allowed), -math.inf), dim=-1).numpy()
    assert np.max(np.abs(res["o"] - want)) < 1e-12
    assert np.max(np.abs(res["lse"] - want_lse)) < 1e-12
    assert np.array_equal(O.tile_unpermute(res["vt"], grid, tile), v)


# ------------------------------------------------------------- distillation

def check_distill_gradient_finite_differences(O, seed=11):
    """dL/dW from distill_kl + distill_grad against central finite differences
    of the exact loss (float64, features unrounded)."""
    rng = np.random.default_rng(seed)
    n, c, r = 7, 12, 4
    sq, sk = rng.standard_normal((n, c)), rng.standard_normal((n, c))
    wq, wk = 0.5 * rng.standard_normal((c, r)), 0.5 * rng.standard_normal((c, r))
    T = rng.uniform(0.01, 1.0, (n, n))
    fq, fk = sq @ wq, sk @ wk
    _, dS = O.distill_kl(fq @ fk.T, T)
    gq, gk = O.distill_grad(sq, sk, fq, fk, dS)
    h = 1e-6
    for w, g, which in ((wq, gq, 0), (wk, gk, 1)):
        num = np.zeros_like(w)
        for idx in np.ndindex(*w.shape):
            wp, wm = w.copy(), w.copy()
            wp[idx] += h
            wm[idx] -= h
            lp = O.distill_loss(sq, sk, wp, wk, T) if which == 0 else O.distill_loss(sq, sk, wq, wp, T)
            lm = O.distill_loss(sq, sk, wm, wk, T) if which == 0 else O.distill_loss(sq, sk, wq, wm, T)
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-6 * max(1.0, np.max(np.abs(g))), (which, np.max(np.abs(num - g)))


def check_distill_kl_closed_forms(O):
    """KL vanishes when the scores are the teacher's logarithm plus a per-row
    constant; a two-tile row has KL = a log(a/p) + (1-a) log((1-a)/(1-p));
    gradient rows sum to zero; grad_scale scales only the gradient."""
    T = np.array([[0.2, 0.5, 0.3], [1e-3, 2.0, 0.7]])
    S = np.log(T) + np.array([[4.0], [-1.5]])
    kl, dS = O.distill_kl(S, T)
    assert np.all(np.abs(kl) < 1e-14) and np.max(np.abs(dS)) < 1e-14
    a, p = 0.25, 1 / (1 + math.exp(-0.7))
    kl2, dS2 = O.distill_kl(np.array([[0.7, 0.0]]), np.array([[1.0, 3.0]]), grad_scale=2.0)
    want = a * math.log(a / p) + (1 - a) * math.log((1 - a) / (1 - p))
    assert abs(kl2[0] - want) < 1e-14 and abs(dS2[0, 0] - 2 * (p - a)) < 1e-14
    rng = np.random.default_rng(12)
    _, d3 = O.distill_kl(rng.standard_normal((5, 9)), rng.uniform(0.1, 1, (5, 9)))
    assert np.max(np.abs(d3.sum(axis=1))) < 1e-14


def check_adam_first_steps(O):
    """First Adam step moves every weight by lr * g / (|g| + eps) (bias
    correction makes m_hat = g, v_hat = g^2); a second step with the same
    gradient moves it by the same amount again."""
    g = np.array([0.3, -2.0, 1e-3])
    w0 = np.array([1.0, 2.0, 3.0])
    w1, m, v = O.adam_step(w0, g, np.zeros(3), np.zeros(3), 1, 0.1, eps=1e-8)
    assert np.allclose(w1, w0 - 0.1 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-15)
    w2, _, _ = O.adam_step(w1, g, m, v, 2, 0.1, eps=1e-8)
    assert np.allclose(w2, w1 - 0.1 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-12)


ALL_SMALL_CHECKS = [
    check_permutation_golden,
    lambda O: check_permutation_bruteforce(O, [((2, 3, 4), (1, 2, 2)), ((4, 16, 16), (2, 8, 8)),
                                               ((5, 7, 9), (2, 2, 4)), ((3, 9, 17), (1, 8, 16)),
                                               ((9, 5, 5), (8, 4, 4))]),
    check_trippool_golden,
    lambda O: check_trippool_bruteforce(O, (3, 5, 6), (2, 2, 4)),
    check_trippool_constant,
    check_dot_golden,
    check_dot_error_bound,
    check_projection_rounds_to_bf16,
    check_average_pooling_special_case,
    check_avgpool_scores,
    check_topk_golden,
    check_topk_bruteforce,
    check_attention_two_keys,
    check_attention_dense_matches_sdpa,
    check_attention_renormalisation,
    check_attention_zero_query,
    check_attention_monotone_and_bounded,
    check_teacher_matches_pooled_softmax,
    check_teacher_uniform_keys,
    check_recall_golden,
    check_tile_search_errors,
    check_head_forward_wiring,
    check_distill_gradient_finite_differences,
    check_distill_kl_closed_forms,
    check_adam_first_steps,
]
