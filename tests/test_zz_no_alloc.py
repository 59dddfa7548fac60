"""The allocation-free attention call (static work queue) against the same
call with a caller's workspace, through the C ABI: two calls in a row on
different workloads, the second smaller, and one too small for the queue.
Both run the same kernels on the same inputs, so O and LSE must be the same
bytes."""

import ctypes

import numpy as np
import pytest
import torch

import datagen
from gpu_harness import say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _prepared(name, heads):
    import block_sparse_attention_13_amd as V
    w = datagen.WORKLOADS[name].with_heads(heads)
    data = datagen.generate(w)
    q, k, v, wq, wk = (to_dev_bf16(data[n]) for n in ("q", "k", "v", "wq", "wk"))
    geom = V.Geometry(w.B, w.heads, w.d, w.grid, w.head_tiles())
    ks = w.k_per_head()
    out = V.layer_forward(q, k, v, wq, wk, geom, ks)
    torch.cuda.synchronize()
    return w, geom, ks, q, out


def _call(fn, geom, ks, q, out, o, lse, *queue):
    import block_sparse_attention_13_amd as V
    from block_sparse_attention_13_amd import _lib
    sq = V._raster_strides(q, geom, "q")
    so = V._raster_strides(o, geom, "o")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return fn(geom.c, q.data_ptr(), sq, out["k_t"].data_ptr(), out["v_t"].data_ptr(), out["idx"].data_ptr(),
              _lib.int_array(ks), int(out["idx"].shape[3]), 0.0, o.data_ptr(), so, lse.data_ptr(), *queue, stream)


def test_noalloc_attention_matches_workspace_call():
    from block_sparse_attention_13_amd import _lib
    lib = _lib.lib
    cases = [("720p", 8), ("480p", 6), ("tiny", 2)]          # items 5760, 2016 (queue), 16 (no queue)
    for name, heads in cases:
        w, geom, ks, q, out = _prepared(name, heads)
        items = w.B * w.heads * geom.max_tiles()
        say(f"[no-alloc] {name} heads {heads}: {items} work items")
        ref_o = torch.full_like(out["o"], float("nan"))
        ref_lse = torch.full_like(out["lse"], float("nan"))
        ws = torch.full((16,), -7, dtype=torch.int32, device=q.device)
        rc = _call(lib.veda_sparse_attn_fwd_raster_io, geom, ks, q, out, ref_o, ref_lse, ws.data_ptr())
        assert rc == 0, _lib.STATUS.get(rc, rc)
        o = torch.full_like(out["o"], float("nan"))
        lse = torch.full_like(out["lse"], float("nan"))
        rc = _call(lib.veda_sparse_attn_fwd_raster_io_noalloc, geom, ks, q, out, o, lse)
        assert rc == 0, _lib.STATUS.get(rc, rc)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"{name}: O bytes differ"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), f"{name}: LSE bytes differ"
        # and both equal the layer's own attention output (workspace of its own)
        assert torch.equal(o.view(torch.int16), out["o"].view(torch.int16)), f"{name}: O differs from the layer's"
        # the Python binding of the same call, writing into caller buffers
        import block_sparse_attention_13_amd as V
        o2 = torch.full_like(out["o"], float("nan"))
        lse2 = torch.full_like(out["lse"], float("nan"))
        V.sparse_attn_fwd_raster_io_noalloc(q, out["k_t"], out["v_t"], out["idx"], geom, ks, o2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), ref_o.view(torch.int16)), f"{name}: binding O bytes differ"
        assert torch.equal(lse2.view(torch.int32), ref_lse.view(torch.int32)), f"{name}: binding LSE bytes differ"


def test_noalloc_rejects_bad_arguments_without_writing():
    from block_sparse_attention_13_amd import _lib
    w, geom, ks, q, out = _prepared("tiny", 2)
    o = torch.full_like(out["o"], 3.0)
    lse = torch.full_like(out["lse"], 3.0)
    bad_k = list(ks)
    bad_k[0] = geom.num_tiles(0) + 1
    rc = _call(_lib.lib.veda_sparse_attn_fwd_raster_io_noalloc, geom, bad_k, q, out, o, lse)
    assert rc == -4  # VEDA_ERR_K
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 3.0).all())
