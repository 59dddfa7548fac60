"""HIP path vs the CPU oracle, through the C ABI, on the same seeded host bytes.

Bit-exact: tiled Q/K/V, TripPool stats, features, tile scores, index lists,
bitmasks, unpermuted layouts. Within tolerance (max-abs 1e-2, rel-L2 5e-3 for
O; 2e-3 for LSE): attention outputs. Large workloads run in full on the GPU
and are checked on sampled heads and query tiles."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import datagen
import oracle as O
from gpu_harness import (bits_of, compare_lse, compare_o, f32_of_bf16, geometry, oracle_head, say, to_dev_bf16)

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS


def _lib():
    import block_sparse_attention_13_amd as V
    return V


def run_layer(w, data, k_per_head=None, buffers=None, tiled_q=False, keep_scores=False):
    V = _lib()
    geom = geometry(w)
    ks = k_per_head or w.k_per_head()
    q, k, v = (to_dev_bf16(data[n]) for n in ("q", "k", "v"))
    wq, wk = to_dev_bf16(data["wq"]), to_dev_bf16(data["wk"])
    out = V.layer_forward(q, k, v, wq, wk, geom, ks, buffers=buffers, tiled_q=tiled_q, keep_scores=keep_scores)
    torch.cuda.synchronize()
    return geom, out, (q, k, v, wq, wk)


def _tiled_q(out, data, geom):
    """The layer's tiled Q, or (the layer reads Q in raster order) a tiled
    copy made by tile_permute."""
    return out["q_t"] if "q_t" in out else _lib().tile_permute(to_dev_bf16(data["q"]), geom)


def _sample_tiles(nT, count, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, nT // 2, nT - 2, nT - 1]
    extra = rng.choice(nT, size=min(nT, count), replace=False).tolist()
    return sorted(set(t for t in fixed + extra if 0 <= t < nT))


def _layer_scores(out, data, geom):
    """The layer's tile scores: written by the layer (keep_scores, or rows
    too long for the one-pass call), else recomputed from its statistics by
    trippool_project_score, whose scores the one-pass Top-k selects from."""
    if "scores" in out:
        return out["scores"]
    wq, wk = to_dev_bf16(data["wq"]), to_dev_bf16(data["wk"])
    return _lib().trippool_project_score(out["stats_q"], out["stats_k"], wq, wk, geom)["scores"]


def check_head(w, data, out, hd, ks, tiles, b=0, check_attention=True):
    """Full bit-exact check of one head's tiling and estimator, and attention
    on the sampled query tiles."""
    d, nT = w.d, w.tiles_per_head()[hd]
    nT_max = max(w.tiles_per_head())
    tile = w.head_tiles()[hd]
    r = oracle_head(data, w, b, hd, ks[hd], query_tiles=tiles if check_attention else [])
    q_t = _tiled_q(out, data, geometry(w))
    for name in ("q_t", "k_t", "v_t"):
        got = bits_of((q_t if name == "q_t" else out[name])[b, hd])
        if name == "v_t":  # channel-major tiles [nT_max, d, 128]
            got = np.ascontiguousarray(got.swapaxes(1, 2))
        assert np.array_equal(got[:nT].reshape(-1, d), O.float_to_bf16_bits(r[name[0] + "t"])), (name, hd)
        assert not got[nT:].any(), (name, hd, "tiles beyond the head must be zero")
    for name in ("stats_q", "stats_k", "feat_q", "feat_k"):
        got = bits_of(out[name][b, hd])
        assert np.array_equal(got[:nT], O.float_to_bf16_bits(r[name])), (name, hd)
        assert not got[nT:].any(), (name, hd)
    S = _layer_scores(out, data, geometry(w))[b, hd].cpu().numpy()
    assert np.array_equal(S[:nT, :nT].view(np.uint32), r["scores"].view(np.uint32)), ("scores", hd)
    assert np.all(np.isneginf(S[nT:, :])) and np.all(np.isneginf(S[:, nT:])), ("scores pad", hd)
    idx = out["idx"][b, hd].cpu().numpy()
    k = ks[hd]
    assert np.array_equal(idx[:nT, :k], r["idx"]), ("idx", hd)
    assert np.all(idx[:nT, k:] == -1) and np.all(idx[nT:] == -1), ("idx pad", hd)
    bm = bits_of(out["bitmask"][b, hd])
    words = (nT_max + 31) // 32
    want_bm = np.zeros((nT_max, words), np.uint32)
    want_bm[:nT, :r["bitmask"].shape[1]] = r["bitmask"]
    assert np.array_equal(bm, want_bm), ("bitmask", hd)
    if not check_attention:
        return r
    # The layer writes raster O directly; the tiled route (pre-filled with
    # garbage, so every byte it leaves is checked) must give the same bytes.
    V = _lib()
    geom = geometry(w)
    o_tiled = torch.full(q_t.shape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    o_tiled, lse_tiled = V.sparse_attn_fwd(q_t, out["k_t"], out["v_t"], out["idx"], geom, ks, o_t=o_tiled)
    o_back = V.tile_unpermute(o_tiled, geom)
    torch.cuda.synchronize()
    assert torch.equal(o_back[b, :, hd].view(torch.int16), out["o"][b, :, hd].view(torch.int16)), ("raster O", hd)
    pos = O.tiled_position(w.grid, tile)
    real = np.zeros(nT_max * 128, bool)
    real[pos] = True
    lse_r, lse_tl = out["lse"][b, hd].cpu().numpy().reshape(-1), lse_tiled[b, hd].cpu().numpy().reshape(-1)
    assert np.array_equal(lse_r[real].view(np.int32), lse_tl[real].view(np.int32)), ("lse", hd)
    assert np.all(np.isneginf(lse_r[~real])), ("raster lse of pad slots", hd)
    rows = np.flatnonzero(np.isfinite(r["lse"]))
    o_gpu = f32_of_bf16(out["o"][b, :, hd, :])
    compare_o(o_gpu[rows], r["o"][rows], f"{w.name} head {hd} O")
    lse_t = out["lse"][b, hd].cpu().numpy().reshape(-1)
    compare_lse(lse_t[pos[rows]], r["lse"][rows], f"{w.name} head {hd}")
    # pad query slots hold the output of a zero query: the mean of the real
    # value rows of the selected tiles
    valid = np.zeros(nT * 128, bool)
    valid[pos] = True
    v_t = O.bf16_bits_to_float(bits_of(out["v_t"][b, hd])).reshape(nT_max, d, 128).swapaxes(1, 2).astype(np.float64)
    o_t = f32_of_bf16(o_tiled[b, hd]).reshape(nT_max, 128, d)
    for t in tiles:
        pads = np.flatnonzero(~valid[t * 128:(t + 1) * 128])
        if len(pads):
            sel = r["idx"][t]
            keys = np.concatenate([v_t[j][valid[j * 128:(j + 1) * 128]] for j in sel])
            want = keys.mean(axis=0)
            compare_o(o_t[t, pads], np.broadcast_to(want, (len(pads), d)), f"pad queries of tile {t}")
    if nT < nT_max:
        assert not bits_of(o_tiled[b, hd])[nT:].any()
        assert np.all(np.isneginf(out["lse"][b, hd, nT:].cpu().numpy()))
    return r


@pytest.mark.parametrize("name,heads,tiles_per_head", [
    ("tiny", None, None),
    ("480p", None, 24),
    ("720p", [0, 1, 2, 21, 39], 12),
    ("hc", [0, 1, 2, 3, 4, 5, 38, 39], 12),
    ("long", [0, 17, 39], 8),     # the benchmarked 245,760-token layer, full size
])
def test_layer_matches_oracle(name, heads, tiles_per_head):
    w = W[name]
    say(f"[parity] workload {name}: {w.description}")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data)
    ks = w.k_per_head()
    for hd in (heads if heads is not None else range(w.heads)):
        nT = w.tiles_per_head()[hd]
        tiles = list(range(nT)) if tiles_per_head is None else _sample_tiles(nT, tiles_per_head, seed=hd)
        check_head(w, data, out, hd, ks, tiles)
    # every head: lists are ascending, in range, k_hd long
    idx = out["idx"].cpu().numpy()
    for hd in range(w.heads):
        nT, k = w.tiles_per_head()[hd], ks[hd]
        row = idx[0, hd, :nT, :k]
        assert np.all(np.diff(row, axis=1) > 0) and row.min() >= 0 and row.max() < nT


def test_batched_layer_matches_oracle():
    """Batch 2 against the oracle, per batch entry: 720p geometry with 4 heads
    (5,760 query tiles, so the attention hands tiles out through the work
    queue), sampled heads and query tiles of both entries."""
    w = dataclasses.replace(W["720p"].with_heads(4), B=2)
    say(f"[parity] {w.description} B {w.B}")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data)
    assert "queue" in out
    ks = w.k_per_head()
    for b, hd in ((0, 1), (1, 0), (1, 3)):
        nT = w.tiles_per_head()[hd]
        check_head(w, data, out, hd, ks, _sample_tiles(nT, 6, seed=10 * b + hd), b=b)
    assert not torch.equal(out["o"][0], out["o"][1])


def test_head_dim_64_layer_matches_oracle():
    """d = 64, r = 64 against the oracle: grid 9 x 27 x 33 with (2, 4, 16)
    tiles leaves every axis ragged (105 tiles per head, k = 3), and B = 4
    x 3 heads gives 1,260 query tiles, so the attention runs through the
    work queue. Every query tile of four (batch, head) pairs is checked."""
    w = dataclasses.replace(_random_workload((9, 27, 33), [(2, 4, 16)], 64, 64, heads=3, seed=4, k=3), B=4)
    say(f"[parity] d 64: grid {w.grid} B {w.B} heads {w.heads} items {max(w.tiles_per_head()) * w.heads * w.B}")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data)
    assert "queue" in out
    ks = w.k_per_head()
    for b, hd in ((0, 0), (1, 2), (3, 1), (3, 2)):
        check_head(w, data, out, hd, ks, list(range(w.tiles_per_head()[hd])), b=b)


def test_estimator_is_deterministic():
    V = _lib()
    w = W["480p"]
    data = datagen.generate(w)
    geom, out, (q, k, v, wq, wk) = run_layer(w, data, keep_scores=True)
    first = out["scores"].clone()
    q_t = V.tile_permute(q, geom)
    for _ in range(2):
        again = V.trippool_score(q_t, out["k_t"], wq, wk, geom)
        torch.cuda.synchronize()
        assert torch.equal(again["scores"].view(torch.int32), first.view(torch.int32))


def test_unpermute_inverts_permute_with_strided_raster():
    """Q taken as a strided slice of a packed [B, N, 3, heads, d] tensor."""
    V = _lib()
    w = dataclasses.replace(W["480p"], heads=4, B=2)
    g = geometry(w)
    rng = np.random.default_rng(11)
    packed = rng.integers(0, 1 << 16, size=(w.B, w.tokens, 3, w.heads, w.d), dtype=np.uint16)
    packed &= np.uint16(0x7F7F)  # finite bf16 patterns
    dev = to_dev_bf16(packed)
    x = dev[:, :, 1]                                     # strides (N*3*H*d, 3*H*d, d, 1)
    xt = V.tile_permute(x, g)
    back = V.tile_unpermute(xt, g)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x.contiguous().view(torch.int16))
    want, _ = O.tile_permute(packed[1, :, 1, 3, :], w.grid, w.head_tiles()[3])
    assert np.array_equal(bits_of(xt[1, 3]).reshape(-1, w.d), want)
    # channel-major tiles are the token-major ones transposed, tile by tile
    xc = V.tile_permute(x, g, layout=V.CHANNEL_MAJOR)
    torch.cuda.synchronize()
    assert xc.shape == (w.B, w.heads, g.max_tiles(), w.d, 128)
    assert torch.equal(xc.view(torch.int16), xt.transpose(3, 4).contiguous().view(torch.int16))
    # the one-pass permute + statistics on the same strided input
    xs, st = V.tile_permute_stats(x, g)
    wz = torch.zeros((w.heads, 3 * w.d, 64), dtype=torch.bfloat16, device="cuda")
    two = V.trippool_score(xt, xt, wz, wz, g)
    torch.cuda.synchronize()
    assert torch.equal(xs.view(torch.int16), xt.view(torch.int16))
    assert torch.equal(st.view(torch.int16), two["stats_q"].view(torch.int16))


@pytest.mark.parametrize("wname,heads,B,custom", [
    ("hc", 6, 2, None),                                            # three tile shapes, ragged boxes
    ("tiny", None, 1, None),                                       # d = 64, r = 32
    (None, None, 1, ((3, 9, 17), [(1, 8, 16), (8, 4, 4)], 64, 64)),  # d = 64, r = 64, mostly pad
])
def test_fused_layer_matches_unfused(wname, heads, B, custom):
    """layer_forward takes the statistics of Q alone and of K while it
    permutes K (tile_stats, tile_permute_stats + trippool_project_score),
    and its attention reads raster Q and writes raster O
    (sparse_attn_fwd_raster_io); with tiled_q it tiles Q too and reads that
    (sparse_attn_fwd_raster). Both, and the unfused route (tile_permute,
    trippool_score, topk_mask, sparse_attn_fwd, tile_unpermute), must give
    the same bytes. Raster O also goes into strided views (and raster Q
    comes from one) whose neighbouring bytes must stay untouched."""
    V = _lib()
    if custom is None:
        w = W[wname] if heads is None else W[wname].with_heads(heads)
        w = dataclasses.replace(w, B=B)
    else:
        grid, tiles, d, r = custom
        w = _random_workload(grid, tiles, d, r, heads=2 * len(tiles), seed=5, k=1)
    say(f"[one-pass] {w.description} B {w.B}")
    data = datagen.generate(w)
    geom, out, (q, k, v, wq, wk) = run_layer(w, data)
    _, out_t, _ = run_layer(w, data, tiled_q=True)
    _, out_s, _ = run_layer(w, data, keep_scores=True)   # scores written, then topk_mask
    assert "q_t" not in out and "scores" not in out and "scores" in out_s
    for name in ("k_t", "v_t", "stats_q", "stats_k", "feat_q", "feat_k", "idx", "bitmask", "lse", "o"):
        for other in (out_t, out_s):
            assert torch.equal(out[name].contiguous().view(torch.uint8), other[name].contiguous().view(torch.uint8)), name
    q_t, k_t = V.tile_permute(q, geom), V.tile_permute(k, geom)
    two = V.trippool_score(q_t, k_t, wq, wk, geom)
    torch.cuda.synchronize()
    assert torch.equal(out_t["q_t"].view(torch.int16), q_t.view(torch.int16))
    assert torch.equal(out["k_t"].view(torch.int16), k_t.view(torch.int16))
    for name in ("stats_q", "stats_k", "feat_q", "feat_k"):
        assert torch.equal(out[name].view(torch.int16), two[name].view(torch.int16)), name
    assert torch.equal(out_s["scores"].view(torch.int32), two["scores"].view(torch.int32))
    ks = w.k_per_head()
    idx, bm = V.topk_mask(two["scores"], geom, ks)
    v_t = V.tile_permute(v, geom, layout=V.CHANNEL_MAJOR)
    o_t, lse = V.sparse_attn_fwd(q_t, k_t, v_t, idx, geom, ks)
    o = V.tile_unpermute(o_t, geom)
    torch.cuda.synchronize()
    assert torch.equal(out["idx"], idx)
    assert torch.equal(out["bitmask"].view(torch.int32), bm.view(torch.int32))
    assert torch.equal(out["o"].view(torch.int16), o.view(torch.int16))
    real = torch.zeros(lse.shape, dtype=torch.bool, device=lse.device)
    for hd, tile in enumerate(w.head_tiles()):
        pos = torch.from_numpy(O.tiled_position(w.grid, tile)).to(lse.device)
        real[:, hd].view(w.B, -1)[:, pos] = True
    assert torch.equal(out["lse"][real].view(torch.int32), lse[real].view(torch.int32))
    assert torch.all(torch.isneginf(out["lse"][~real]))
    packed = torch.full((w.B, w.tokens, 2, w.heads, w.d), 0x7FC0, dtype=torch.int16, device="cuda")
    view = packed.view(torch.bfloat16)[:, :, 1]
    V.sparse_attn_fwd_raster(q_t, k_t, v_t, idx, geom, ks, out=view, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(packed[:, :, 1], o.view(torch.int16))
    assert torch.all(packed[:, :, 0] == 0x7FC0)
    # raster Q from a strided view (Q in slot 0 of a packed [B, N, 3, heads, d] tensor)
    qkv = torch.stack([q, k, v], dim=2)
    packed.fill_(0x7FC0)
    V.sparse_attn_fwd_raster_io(qkv[:, :, 0], k_t, v_t, idx, geom, ks, out=view, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(packed[:, :, 1], o.view(torch.int16))
    assert torch.all(packed[:, :, 0] == 0x7FC0)


def _random_workload(grid, tiles, d, r, heads, seed, keep=None, k=None):
    return datagen.Workload("custom", 1, heads, d, r, grid, tuple(tiles), keep, k, False, seed, "custom")


def test_work_queue_matches_fixed_deal():
    """Handing query tiles out through the work queue changes only which
    workgroup computes a tile: tiled O, raster O and LSE are the same bytes
    as with fixed per-XCD shares. One workspace, filled with garbage first,
    serves every call, the later workloads smaller (d 128 then 64, item
    counts B * heads * nT_max of 2688, 1700, 1260 and exactly 1024, two not
    multiples of 8): each call clears it itself. Below 1024 items (1008
    and 36 here) the fixed deal is used and the workspace is not touched."""
    V = _lib()
    queue = torch.full((V.ATTN_QUEUE_BYTES // 4,), 123456, dtype=torch.int32, device="cuda")
    cases = [dataclasses.replace(W["480p"].with_heads(4), B=2),
             dataclasses.replace(_random_workload((5, 37, 66), [(1, 8, 16), (8, 4, 4)], 128, 32, heads=2, seed=3,
                                                  k=2), B=5),
             dataclasses.replace(_random_workload((9, 27, 33), [(2, 4, 16)], 64, 64, heads=3, seed=4, k=3), B=4),
             dataclasses.replace(W["tiny"], B=64), dataclasses.replace(W["tiny"], B=63),
             _random_workload((5, 6, 20), [(2, 4, 16)], 64, 64, heads=3, seed=4, k=3)]
    for w in cases:
        say(f"[queue] {w.description} B {w.B} items {max(w.tiles_per_head()) * w.heads * w.B}")
        data = datagen.generate(w)
        geom, out, (q, _, _, _, _) = run_layer(w, data)
        ks = w.k_per_head()
        args = (V.tile_permute(q, geom), out["k_t"], out["v_t"], out["idx"], geom, ks)
        rio = (q, out["k_t"], out["v_t"], out["idx"], geom, ks)
        io_f, iol_f = V.sparse_attn_fwd_raster_io(*rio, dynamic=False)
        o_f, lse_f = V.sparse_attn_fwd(*args, dynamic=False)
        r_f, rl_f = V.sparse_attn_fwd_raster(*args, dynamic=False)
        for _ in range(2):
            o_d, lse_d = V.sparse_attn_fwd(*args, work_queue=queue)
            r_d, rl_d = V.sparse_attn_fwd_raster(*args, work_queue=queue)
            io_d, iol_d = V.sparse_attn_fwd_raster_io(*rio, work_queue=queue)
            torch.cuda.synchronize()
            assert torch.equal(io_d.view(torch.int16), r_f.view(torch.int16))
            assert torch.equal(io_f.view(torch.int16), r_f.view(torch.int16))
            assert torch.equal(iol_d.view(torch.int32), rl_f.view(torch.int32))
            assert torch.equal(iol_f.view(torch.int32), rl_f.view(torch.int32))
            assert torch.equal(o_d.view(torch.int16), o_f.view(torch.int16))
            assert torch.equal(lse_d.view(torch.int32), lse_f.view(torch.int32))
            assert torch.equal(r_d.view(torch.int16), r_f.view(torch.int16))
            assert torch.equal(rl_d.view(torch.int32), rl_f.view(torch.int32))
        assert torch.equal(out["o"].view(torch.int16), r_f.view(torch.int16))
        if max(w.tiles_per_head()) * w.heads * w.B < 1024:
            queue_bytes = queue.clone()
            V.sparse_attn_fwd(*args, work_queue=queue)
            torch.cuda.synchronize()
            assert torch.equal(queue, queue_bytes)


@pytest.mark.parametrize("grid,tiles,d,r", [
    ((5, 6, 20), [(2, 4, 16)], 64, 64),
    ((3, 9, 17), [(1, 8, 16), (8, 4, 4)], 128, 32),
    ((2, 8, 8), [(2, 8, 8)], 128, 64),
])
def test_dense_when_every_tile_is_kept(grid, tiles, d, r):
    """k = all tiles: the sparse layer is plain softmax attention."""
    w = _random_workload(grid, tiles, d, r, heads=len(tiles), seed=21)
    say(f"[dense] grid {grid} tiles {tiles} d {d} r {r}")
    data = datagen.generate(w)
    ks = w.tiles_per_head()
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    for hd in range(w.heads):
        q, k, v = (O.bf16_bits_to_float(data[n][0, :, hd, :]) for n in ("q", "k", "v"))
        od, lsed = O.dense_attention(q, k, v, 1.0 / math.sqrt(d))
        compare_o(f32_of_bf16(out["o"][0, :, hd, :]), od, f"dense head {hd}")
        pos = O.tiled_position(grid, tiles[hd % len(tiles)])
        compare_lse(out["lse"][0, hd].cpu().numpy().reshape(-1)[pos], lsed, f"dense head {hd}")
        check_head(w, data, out, hd, ks, list(range(ks[hd])))


@pytest.mark.parametrize("grid,tiles,d,r,B", [
    ((5, 6, 20), [(2, 4, 16)], 64, 64, 1),
    ((3, 9, 17), [(1, 8, 16), (8, 4, 4)], 128, 32, 1),
    ((9, 27, 33), [(2, 4, 16), (1, 8, 16)], 128, 64, 4),     # 1,600 work items: through the work queue
])
def test_dense_kernel(grid, tiles, d, r, B):
    """The dedicated dense forward (no index list): raster O and LSE against
    the oracle's dense attention, and the same bytes as the tile-sparse
    kernel with every tile kept (tiled O, raster O, LSE)."""
    V = _lib()
    w = dataclasses.replace(_random_workload(grid, tiles, d, r, heads=len(tiles), seed=31), B=B)
    say(f"[dense kernel] grid {grid} tiles {tiles} d {d} B {B}")
    data = datagen.generate(w)
    geom = geometry(w)
    q, k, v = (to_dev_bf16(data[n]) for n in ("q", "k", "v"))
    q_t, k_t = V.tile_permute(q, geom), V.tile_permute(k, geom)
    v_t = V.tile_permute(v, geom, layout=V.CHANNEL_MAJOR)
    o_t, lse = V.dense_attn_fwd(q_t, k_t, v_t, geom)
    o_r, lse_r = V.dense_attn_fwd_raster(q_t, k_t, v_t, geom)
    idx, ks = V.dense_index(geom, q.device)
    o_s, lse_s = V.sparse_attn_fwd(q_t, k_t, v_t, idx, geom, ks)
    o_sr, _ = V.sparse_attn_fwd_raster(q_t, k_t, v_t, idx, geom, ks)
    torch.cuda.synchronize()
    assert torch.equal(o_t.view(torch.int16), o_s.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_s.view(torch.int32))
    assert torch.equal(o_r.view(torch.int16), o_sr.view(torch.int16))
    for b in range(B):
        for hd in range(w.heads):
            qh, kh, vh = (O.bf16_bits_to_float(data[n][b, :, hd, :]) for n in ("q", "k", "v"))
            od, lsed = O.dense_attention(qh, kh, vh, 1.0 / math.sqrt(d))
            compare_o(f32_of_bf16(o_r[b, :, hd, :]), od, f"dense kernel b {b} head {hd}")
            pos = O.tiled_position(grid, tiles[hd])
            compare_lse(lse[b, hd].cpu().numpy().reshape(-1)[pos], lsed, f"dense kernel b {b} head {hd}")
            real = lse_r[b, hd].cpu().numpy().reshape(-1)[pos]
            assert np.array_equal(real.view(np.uint32), lse[b, hd].cpu().numpy().reshape(-1)[pos].view(np.uint32))


def test_dense_kernel_long_sampled():
    """Dense forward on one head of the 245,760-token workload (1920 x 1920
    tile pairs), sampled query tiles against the oracle (every key tile
    kept, raster order)."""
    V = _lib()
    w = W["long"].with_heads(1)
    say("[dense kernel] long, 1 head")
    data = datagen.generate(w)
    geom = geometry(w)
    q, k, v = (to_dev_bf16(data[n]) for n in ("q", "k", "v"))
    q_t, k_t = V.tile_permute(q, geom), V.tile_permute(k, geom)
    v_t = V.tile_permute(v, geom, layout=V.CHANNEL_MAJOR)
    o_r, lse = V.dense_attn_fwd_raster(q_t, k_t, v_t, geom)
    torch.cuda.synchronize()
    tile = w.head_tiles()[0]
    nT = geom.num_tiles(0)
    tiles = [0, 777, nT - 1]
    qh, kh, vh = (O.bf16_bits_to_float(data[n][0, :, 0, :]) for n in ("q", "k", "v"))
    sel = np.tile(np.arange(nT), (nT, 1))
    od, lsed = O.sparse_attention(qh, kh, vh, w.grid, tile, sel, 1.0 / math.sqrt(w.d), query_tiles=tiles)
    rows = np.flatnonzero(np.isfinite(lsed))
    assert len(rows) == 128 * len(tiles)
    compare_o(f32_of_bf16(o_r[0, :, 0, :])[rows], od[rows], "dense kernel long")
    pos = O.tiled_position(w.grid, tile)
    compare_lse(lse[0, 0].cpu().numpy().reshape(-1)[pos[rows]], lsed[rows], "dense kernel long")


def test_single_tile_kept():
    w = _random_workload((4, 16, 16), [(2, 8, 8)], 64, 32, heads=2, seed=5)
    data = datagen.generate(w)
    ks = [1, 1]
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    for hd in range(2):
        check_head(w, data, out, hd, ks, list(range(8)))


@pytest.mark.parametrize("grid,tiles,d,r", [
    ((1, 1, 1), [(1, 8, 16), (8, 4, 4)], 64, 32),      # one real token: one box of 127 pad slots
    ((1, 1, 3), [(1, 8, 16), (2, 8, 8)], 128, 64),     # three real tokens in one box
    ((3, 1, 2), [(2, 8, 8), (8, 4, 4)], 64, 64),       # boxes with 4 and 2 real tokens
])
def test_grids_smaller_than_a_tile(grid, tiles, d, r):
    """Degenerate grids: every box is mostly pad slots; the attention of a
    query covers only the few real keys of its head."""
    w = _random_workload(grid, tiles, d, r, heads=2, seed=13)
    data = datagen.generate(w)
    ks = [w.tiles_per_head()[hd] for hd in range(2)]
    say(f"[degenerate] grid {grid} tiles {tiles} -> {w.tiles_per_head()} boxes")
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    for hd in range(2):
        check_head(w, data, out, hd, ks, list(range(w.tiles_per_head()[hd])))


def test_largest_tile_count():
    """A head at the library's limit of 8192 tiles (1,048,576 tokens) through
    the whole layer; the oracle checks sampled query tiles."""
    V = _lib()
    w = _random_workload((64, 128, 128), [(4, 4, 8)], 64, 32, heads=1, seed=17, k=16)
    assert w.tiles_per_head() == [8192] == [V._lib.VEDA_MAX_TILES]
    say("[max] 8192 tiles, 1,048,576 tokens")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data)
    check_head(w, data, out, 0, w.k_per_head(), _sample_tiles(8192, 6, 1))


def test_largest_head_count():
    """The library's limit of 128 heads (three tile shapes in turn, so the
    last head's geometry differs from the first's) through the whole layer;
    the oracle checks every query tile of four heads, the last among them."""
    V = _lib()
    w = _random_workload((3, 9, 17), [(1, 8, 16), (8, 4, 4), (2, 8, 8)], 64, 32, heads=128, seed=23, k=2)
    assert w.heads == V._lib.VEDA_MAX_HEADS
    say(f"[max] {w.heads} heads, tiles per head {sorted(set(w.tiles_per_head()))}")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data)
    ks = w.k_per_head()
    for hd in (0, 1, 65, 127):
        check_head(w, data, out, hd, ks, list(range(w.tiles_per_head()[hd])))


def test_extreme_k_mixed_across_heads():
    """One call with k = 1 on one head, k = every tile on the next and a
    middle k on the third (three tile shapes, ragged boxes, B = 2): the
    per-head k reaches Top-k, the masks and the attention loop unchanged."""
    w = dataclasses.replace(_random_workload((3, 9, 17), [(1, 8, 16), (8, 4, 4), (2, 8, 8)], 128, 64, heads=3,
                                             seed=29, k=2), B=2)
    nT = w.tiles_per_head()
    ks = [1, nT[1], nT[2] // 2]
    say(f"[k] tiles per head {nT}, k {ks}")
    data = datagen.generate(w)
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    for b in range(w.B):
        for hd in range(w.heads):
            check_head(w, data, out, hd, ks, list(range(nT[hd])), b=b)


@pytest.mark.parametrize("scale", [0.35, 0.02])
def test_explicit_softmax_scale(scale):
    """A caller's softmax scale in place of 1/sqrt(d): 0.35 makes the
    softmax sharp, 0.02 nearly uniform. O and the LSE (of the scaled
    logits) against the oracle run with the same scale."""
    V = _lib()
    w = _random_workload((3, 9, 17), [(1, 8, 16), (8, 4, 4)], 128, 64, heads=2, seed=31, k=3)
    data = datagen.generate(w)
    geom, out, (q, _, _, _, _) = run_layer(w, data)
    ks = w.k_per_head()
    o, lse = V.sparse_attn_fwd_raster_io(q, out["k_t"], out["v_t"], out["idx"], geom, ks, scale=scale)
    torch.cuda.synchronize()
    for hd in range(w.heads):
        nT = w.tiles_per_head()[hd]
        r = oracle_head(data, w, 0, hd, ks[hd], query_tiles=list(range(nT)), scale=scale)
        assert np.array_equal(out["idx"][0, hd].cpu().numpy()[:nT, :ks[hd]], r["idx"]), ("idx", hd)
        rows = np.flatnonzero(np.isfinite(r["lse"]))
        compare_o(f32_of_bf16(o[0, :, hd, :])[rows], r["o"][rows], f"scale {scale} head {hd} O")
        pos = O.tiled_position(w.grid, w.head_tiles()[hd])
        compare_lse(lse[0, hd].cpu().numpy().reshape(-1)[pos[rows]], r["lse"][rows], f"scale {scale} head {hd}")


def test_running_max_rescales():
    """Logits that climb with the key tile's index: channel 0 of every query
    is 8 and of every key 2 x its tile's index, which adds about 2 (base 2)
    per tile at d = 128. The ascending key loop then meets a row max more
    than 8 above the running one every few tiles, so the online softmax
    rescales O, l and m many times per row; O and the LSE against the oracle."""
    w = _random_workload((3, 9, 17), [(1, 8, 16), (8, 4, 4)], 128, 64, heads=2, seed=37, k=2)
    data = datagen.generate(w)
    nT = w.tiles_per_head()
    ks = [t // 2 + 1 for t in nT]
    for hd in range(w.heads):
        tile_of = O.tiled_position(w.grid, w.head_tiles()[hd]) // 128
        data["q"][0, :, hd, 0] = O.float_to_bf16_bits(np.full(w.tokens, 8.0, np.float32))
        data["k"][0, :, hd, 0] = O.float_to_bf16_bits((2.0 * tile_of).astype(np.float32))
    say(f"[rescale] tiles per head {nT}, k {ks}")
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    for hd in range(w.heads):
        r = check_head(w, data, out, hd, ks, list(range(nT[hd])))
        sel = r["idx"]
        assert (sel[:, -1] - sel[:, 0]).max() >= 8, "the selections must span enough tiles to force rescales"


def test_equal_scores_keep_the_lower_tile():
    """Duplicate key tiles give exactly equal scores: the lower index must win
    end to end, and the lists must match the oracle's."""
    w = _random_workload((4, 16, 16), [(2, 8, 8)], 64, 32, heads=2, seed=9)
    data = datagen.generate(w)
    # copy key box 0 into boxes 3, 5 and 6 (raster positions of each box)
    pos = O.tiled_position(w.grid, (2, 8, 8))
    box = pos // 128
    for hd in range(2):
        src = data["k"][0, box == 0, hd, :]
        order0 = np.argsort(pos[box == 0])
        for dst in (3, 5, 6):
            sel = np.flatnonzero(box == dst)
            data["k"][0, sel[np.argsort(pos[sel])], hd, :] = src[order0]
    ks = [2, 2]
    geom, out, _ = run_layer(w, data, k_per_head=ks)
    S = _layer_scores(out, data, geom).cpu().numpy()
    assert np.array_equal(S[0, 0, :, 0], S[0, 0, :, 3]) and np.array_equal(S[0, 0, :, 0], S[0, 0, :, 6])
    for hd in range(2):
        check_head(w, data, out, hd, ks, list(range(8)))


def test_topk_on_crafted_scores():
    """Given scores full of exact ties and signed zeros, the GPU lists equal a
    brute-force stable sort's, at several row lengths including the largest."""
    V = _lib()
    rng = np.random.default_rng(3)
    for grid, tile, k in (((4, 16, 16), (2, 8, 8), 3), ((21, 30, 52), (4, 4, 8), 34),
                          ((64, 64, 256), (4, 4, 8), 200)):
        g = V.Geometry(1, 1, 128, grid, [tile])
        nT = g.max_tiles()
        say(f"[topk] {nT} key tiles, k {k}")
        rows = min(nT, 256)
        S = rng.integers(-4, 5, size=(rows, nT)).astype(np.float32) * np.float32(0.25)
        S[S == 0] = np.where(rng.random((S == 0).sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
        S[::7] = rng.standard_normal((len(S[::7]), nT)).astype(np.float32)
        full = np.full((nT, nT), np.float32(1.0))
        full[:rows] = S
        dev = torch.from_numpy(full).reshape(1, 1, nT, nT).cuda()
        idx, bm = V.topk_mask(dev, g, [k])
        torch.cuda.synchronize()
        got = idx[0, 0, :rows].cpu().numpy()
        assert np.array_equal(got, O.topk(S, k))
        for rr in range(0, rows, 37):
            assert got[rr].tolist() == O.topk_row_bruteforce(S[rr], k)
        assert np.array_equal(bits_of(bm[0, 0, :rows]), O.bitmask(got, nT))
        # the constant rows keep the first k tiles
        assert np.all(idx[0, 0, rows:].cpu().numpy() == np.arange(k))


@pytest.mark.parametrize("grid,tile,n_tiles,k", [((60, 40, 80), (4, 4, 8), 1500, 75),
                                                  ((7, 48, 40), (1, 16, 8), 105, 10)])
def test_topk_on_narrow_and_skewed_rows(grid, tile, n_tiles, k):
    """Rows whose scores share long leading bits (a band of width 2^-12
    around 1, or around -3), two-valued rows, rows with one outlier above a
    constant, values spanning the whole float range, constant rows and
    rows whose threshold lies many octaves below the maximum: the lists equal
    the oracle's. Both row lengths leave pad slots in the last 64-wide chunk
    of every row; with 105 tiles the rows start at every 4-byte offset modulo
    16 bytes, so the kernel's rows staged through LDS and its rows read
    directly are both exercised."""
    V = _lib()
    rng = np.random.default_rng(43)
    g = V.Geometry(1, 1, 128, grid, [tile])
    nT = g.max_tiles()
    assert nT == n_tiles and nT % 64
    S = np.empty((nT, nT), np.float32)
    for i in range(nT):
        kind = i % 8
        if kind == 0:
            S[i] = 1.0 + rng.integers(0, 64, nT) * np.float32(2.0 ** -18)
        elif kind == 1:
            S[i] = -3.0 - rng.integers(0, 64, nT) * np.float32(2.0 ** -17)
        elif kind == 2:
            S[i] = np.where(rng.random(nT) < 0.3, np.float32(2.5), np.float32(-2.5))
        elif kind == 3:
            S[i] = 7.0
            S[i, rng.integers(0, nT)] = 7.0 + 2.0 ** -20
        elif kind == 4:
            S[i] = (rng.standard_normal(nT) * 10.0 ** rng.uniform(-30, 30, nT)).astype(np.float32)
        elif kind == 5:
            S[i] = -rng.uniform(0, 1, nT).astype(np.float32) ** 8
        elif kind == 6:
            S[i] = 0.5
        else:   # one huge value, the rest spread far below it
            S[i] = np.exp(rng.standard_normal(nT) * 3).astype(np.float32)
            S[i, rng.integers(0, nT)] = 1e30
    idx, bm = V.topk_mask(torch.from_numpy(S).reshape(1, 1, nT, nT).cuda(), g, [k])
    torch.cuda.synchronize()
    got = idx[0, 0].cpu().numpy()
    assert np.array_equal(got, O.topk(S, k))
    assert np.array_equal(bits_of(bm[0, 0]), O.bitmask(got, nT))


def test_topk_orders_nan_scores_by_bit_pattern():
    """Three +NaN and five -NaN scores in every row (no infinities): +NaN
    ranks above every finite score and -NaN below, so the lists equal the
    oracle's with +NaN read as +inf and -NaN as -inf, every +NaN tile is
    kept and no -NaN tile is."""
    V = _lib()
    rng = np.random.default_rng(41)
    g = V.Geometry(1, 1, 128, (21, 30, 52), [(4, 4, 8)])
    nT, k = g.max_tiles(), 34
    S = rng.standard_normal((nT, nT)).astype(np.float32)
    pos_nan = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    neg_nan = np.array([0xFFC00000], np.uint32).view(np.float32)[0]
    for i in range(nT):
        c = rng.choice(nT, size=8, replace=False)
        S[i, c[:3]] = pos_nan
        S[i, c[3:]] = neg_nan
    as_inf = np.where(np.isnan(S), np.where(np.signbit(S), np.float32(-np.inf), np.float32(np.inf)), S)
    idx, _ = V.topk_mask(torch.from_numpy(S).reshape(1, 1, nT, nT).cuda(), g, [k])
    torch.cuda.synchronize()
    got = idx[0, 0].cpu().numpy()
    assert np.array_equal(got, O.topk(as_inf.astype(np.float32), k))
    for i in range(nT):
        kept = set(got[i].tolist())
        assert set(np.flatnonzero(np.isposinf(as_inf[i])).tolist()) <= kept
        assert not set(np.flatnonzero(np.isneginf(as_inf[i])).tolist()) & kept


@pytest.mark.parametrize("tiled_q", [False, True])
def test_every_output_byte_is_written(tiled_q):
    """Outputs pre-filled with garbage end up fully defined."""
    w = W["hc"].with_heads(6)
    data = datagen.generate(w)
    geom = geometry(w)
    nT = geom.max_tiles()
    B, Hh, d = w.B, w.heads, w.d
    g = lambda shape, dt: torch.full(shape, 0x7FC0 if dt == torch.bfloat16 else -1, dtype=torch.int16 if dt == torch.bfloat16 else torch.int32, device="cuda").view(dt)
    bufs = {
        "q_t": g((B, Hh, nT, 128, d), torch.bfloat16), "k_t": g((B, Hh, nT, 128, d), torch.bfloat16),
        "v_t": g((B, Hh, nT, d, 128), torch.bfloat16),
        "stats_q": g((B, Hh, nT, 3 * d), torch.bfloat16), "stats_k": g((B, Hh, nT, 3 * d), torch.bfloat16),
        "feat_q": g((B, Hh, nT, w.r), torch.bfloat16), "feat_k": g((B, Hh, nT, w.r), torch.bfloat16),
        "scores": g((B, Hh, nT, nT), torch.float32), "idx": g((B, Hh, nT, max(w.k_per_head())), torch.int32),
        "bitmask": g((B, Hh, nT, (nT + 31) // 32), torch.int32).view(torch.uint32),
        "lse": g((B, Hh, nT, 128), torch.float32), "o": g((B, w.tokens, Hh, d), torch.bfloat16),
    }
    if not tiled_q:
        del bufs["q_t"]
    geom, out, _ = run_layer(w, data, buffers=bufs, tiled_q=tiled_q)
    ks = w.k_per_head()
    for hd in (0, 1, 2):
        check_head(w, data, out, hd, ks, _sample_tiles(w.tiles_per_head()[hd], 6, hd))
    assert not torch.isnan(out["o"].float()).any()


def test_invalid_call_raises_and_writes_nothing():
    V = _lib()
    w = W["tiny"]
    geom = geometry(w)
    s = torch.zeros((1, 2, 8, 8), dtype=torch.float32, device="cuda")
    idx = torch.full((1, 2, 8, 4), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(V.VedaError):
        V.topk_mask(s, geom, [9, 4], k_max=4, idx=idx, with_bitmask=False)
    torch.cuda.synchronize()
    assert torch.all(idx == 7)


def test_layer_is_deterministic():
    """Three runs of the whole layer give the same bytes in every output
    (the work-queue workspace is scratch: its counts vary with timing)."""
    V = _lib()
    w = W["480p"]
    data = datagen.generate(w)
    geom, first, (q, k, v, wq, wk) = run_layer(w, data)
    for _ in range(2):
        again = V.layer_forward(q, k, v, wq, wk, geom, w.k_per_head())
        torch.cuda.synchronize()
        for name, t in first.items():
            if name == "queue":
                continue
            a, b = t.contiguous().view(torch.uint8), again[name].contiguous().view(torch.uint8)
            assert torch.equal(a, b), name


_GUARD_BYTES = 4096


def _guarded(shape, dtype):
    """A tensor of `shape` inside a larger buffer whose first and last 4 KiB
    hold a known pattern; returns (tensor, buffer)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((n + 2 * _GUARD_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    return buf[_GUARD_BYTES:_GUARD_BYTES + n].view(dtype).view(shape), buf


def _guards_intact(buf):
    return bool(torch.all(buf[:_GUARD_BYTES] == 0xA5)) and bool(torch.all(buf[-_GUARD_BYTES:] == 0xA5))


@pytest.mark.parametrize("tiled_q", [False, True])
def test_outputs_stay_in_their_buffers(tiled_q):
    """Every call writes inside its outputs and the attention's work-queue
    workspace: 4 KiB before and after each one stay untouched (ragged boxes,
    three tile shapes, B = 2; the layer with and without tiled Q)."""
    V = _lib()
    w = dataclasses.replace(W["hc"].with_heads(6), B=2)
    data = datagen.generate(w)
    geom = geometry(w)
    nT, B, Hh, d, r = geom.max_tiles(), w.B, w.heads, w.d, w.r
    kmax = max(w.k_per_head())
    shapes = {
        "q_t": ((B, Hh, nT, 128, d), torch.bfloat16), "k_t": ((B, Hh, nT, 128, d), torch.bfloat16),
        "v_t": ((B, Hh, nT, d, 128), torch.bfloat16),
        "stats_q": ((B, Hh, nT, 3 * d), torch.bfloat16), "stats_k": ((B, Hh, nT, 3 * d), torch.bfloat16),
        "feat_q": ((B, Hh, nT, r), torch.bfloat16), "feat_k": ((B, Hh, nT, r), torch.bfloat16),
        "scores": ((B, Hh, nT, nT), torch.float32), "idx": ((B, Hh, nT, kmax), torch.int32),
        "bitmask": ((B, Hh, nT, (nT + 31) // 32), torch.int32), "lse": ((B, Hh, nT, 128), torch.float32),
        "o": ((B, w.tokens, Hh, d), torch.bfloat16), "queue": ((V.ATTN_QUEUE_BYTES // 4,), torch.int32),
    }
    bufs, raw = {}, {}
    for name, (shape, dt) in shapes.items():
        if name != "q_t" or tiled_q:
            bufs[name], raw[name] = _guarded(shape, dt)
    bufs["bitmask"] = bufs["bitmask"].view(torch.uint32)
    geom, out, (q, k, v, wq, wk) = run_layer(w, data, buffers=bufs, tiled_q=tiled_q)
    for name, buf in raw.items():
        assert _guards_intact(buf), ("fused layer", name)
    q_t = _tiled_q(out, data, geom)
    # the unfused route and the measurement calls, into guarded outputs too
    checks = []
    xt, b1 = _guarded(shapes["q_t"][0], torch.bfloat16)
    V.tile_permute(q, geom, xt); checks.append(("tile_permute", b1))
    xc, b2 = _guarded(shapes["v_t"][0], torch.bfloat16)
    V.tile_permute(v, geom, xc, layout=V.CHANNEL_MAJOR); checks.append(("tile_permute channel-major", b2))
    est = {}
    for name in ("stats_q", "stats_k", "feat_q", "feat_k", "scores"):
        est[name], b3 = _guarded(*shapes[name]); checks.append(("trippool_score " + name, b3))
    V.trippool_score(q_t, out["k_t"], wq, wk, geom, est)
    o_t, b4 = _guarded(shapes["q_t"][0], torch.bfloat16)
    V.sparse_attn_fwd(q_t, out["k_t"], out["v_t"], out["idx"], geom, w.k_per_head(), o_t=o_t)
    checks.append(("sparse_attn_fwd", b4))
    o, b5 = _guarded(shapes["o"][0], torch.bfloat16)
    V.tile_unpermute(o_t, geom, o); checks.append(("tile_unpermute", b5))
    teacher, b6 = _guarded(shapes["scores"][0], torch.float32)
    V.teacher_tile_max(q_t, out["k_t"], out["lse"], geom, out=teacher); checks.append(("teacher", b6))
    st, b7 = _guarded(shapes["stats_q"][0], torch.bfloat16)
    V.tile_stats(q, geom, st); checks.append(("tile_stats", b7))
    i2, b8 = _guarded(*shapes["idx"])
    m2, b9 = _guarded(*shapes["bitmask"])
    V.topk_mask(est["scores"], geom, w.k_per_head(), idx=i2, bitmask=m2.view(torch.uint32))
    checks += [("topk_mask idx", b8), ("topk_mask bitmask", b9)]
    torch.cuda.synchronize()
    for name, buf in checks:
        assert _guards_intact(buf), name
    assert torch.equal(o.view(torch.int16), out["o"].view(torch.int16))
    assert torch.equal(i2, out["idx"]) and torch.equal(m2.view(torch.int32), out["bitmask"].view(torch.int32))


def test_layer_replays_in_a_graph():
    """The layer captured in a HIP graph: its kernels only (the work-queue
    counters are cleared by a kernel, not a memset). Between replays eager
    work fills every output and the workspace with garbage; each replay must
    give the eager layer's bytes again."""
    V = _lib()
    w = W["480p"].with_heads(4)
    data = datagen.generate(w)
    geom = geometry(w)
    ks = w.k_per_head()
    q, k, v = (to_dev_bf16(data[n]) for n in ("q", "k", "v"))
    wq, wk = to_dev_bf16(data["wq"]), to_dev_bf16(data["wk"])
    bufs = V.layer_forward(q, k, v, wq, wk, geom, ks)
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in bufs.items() if n != "queue"}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        V.layer_forward(q, k, v, wq, wk, geom, ks, buffers=bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        V.layer_forward(q, k, v, wq, wk, geom, ks, buffers=bufs)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"[graph] replay {rep}")
        for t in bufs.values():
            t.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(bufs[n].contiguous().view(torch.uint8), t.contiguous().view(torch.uint8)), (rep, n)


def test_concurrent_calls_with_separate_workspaces():
    """Two attention calls in flight at once on two streams, each with its
    own work-queue workspace (two different workloads), give the bytes the
    same calls give one after the other."""
    V = _lib()
    runs = []
    for w in (W["480p"].with_heads(6), dataclasses.replace(W["hc"].with_heads(3), B=1)):
        data = datagen.generate(w)
        geom, out, (q, _, _, _, _) = run_layer(w, data)
        runs.append((geom, w.k_per_head(), q, out))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = []
    for rep in range(3):
        say(f"[streams] round {rep}")
        outs = []
        for (geom, ks, q, out), st in zip(runs, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                o = torch.full_like(out["o"], 7)
                lse = torch.full_like(out["lse"], 7.0)
                V.sparse_attn_fwd_raster_io(q, out["k_t"], out["v_t"], out["idx"], geom, ks, out=o, lse=lse,
                                            work_queue=V.attn_queue(q.device))
                outs.append((o, lse))
        torch.cuda.synchronize()
        results.append(outs)
    for outs in results:
        for (o, lse), (_, _, _, out) in zip(outs, runs):
            assert torch.equal(o.view(torch.int16), out["o"].view(torch.int16))
            assert torch.equal(lse.view(torch.int32), out["lse"].view(torch.int32))
