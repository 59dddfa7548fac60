"""Host-side logic of the HIP library, checked on the CPU: the box geometry
helpers (slot masks, box decoding) are compiled for the host from the same
header the kernels use and checked exhaustively."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_box_slot_masks_match_definition(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = tmp_path / "host_geometry_check"
    src = os.path.join(HERE, "host_geometry_check.cpp")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_k_from_keep_is_the_exact_ceiling():
    """veda_k_from_keep: k_hd = ceil(keep * nT_hd) in exact rational arithmetic,
    clamped to [1, nT_hd]; a fraction outside (0, 1] is an error."""
    import fractions
    import math
    import datagen
    import block_sparse_attention_13_amd as V
    for w in datagen.WORKLOADS.values():
        if w.keep is None:
            continue
        g = V.Geometry(w.B, w.heads, w.d, w.grid, w.head_tiles())
        assert V.k_from_keep(g, w.keep) == w.k_per_head(), w.name
    g = V.Geometry(1, 3, 128, (21, 45, 80), [(4, 4, 8), (1, 8, 16), (8, 4, 4)])
    for keep in ("0.05", "0.1", "1/3", "1", "1e-9", "0.999"):
        f = fractions.Fraction(keep)
        want = [max(1, min(n, math.ceil(f * n))) for n in (720, 630, 720)]
        assert V.k_from_keep(g, f) == want, keep
    from block_sparse_attention_13_amd import _lib
    for num, den in ((0, 1), (-1, 2), (3, 2), (1, 0)):
        assert _lib.lib.veda_k_from_keep(g.c, 0, num, den) == -4, (num, den)
    assert _lib.lib.veda_k_from_keep(g.c, 3, 1, 2) == -2


def test_candidate_tiles_enumerate_the_budget():
    """veda_candidate_tiles: every power-of-two (pt, ph, pw) with product 128
    that fits the grid and stays within the tile limit, enumerated here by
    brute force over all divisor triples of 128."""
    import block_sparse_attention_13_amd as V
    from block_sparse_attention_13_amd import _lib
    for grid in ((21, 45, 80), (64, 48, 80), (4, 16, 16), (1, 1, 1), (2, 300, 300), (128, 1, 1)):
        want = []
        for pt in range(1, 129):
            for ph in range(1, 129):
                if 128 % (pt * ph):
                    continue
                pw = 128 // (pt * ph)
                if pt <= grid[0] and ph <= grid[1] and pw <= grid[2]:
                    n = -(-grid[0] // pt) * -(-grid[1] // ph) * -(-grid[2] // pw)
                    if n <= 8192:
                        want.append((pt, ph, pw))
        assert V.candidate_tiles(grid) == sorted(want), grid
    small = (_lib.VedaTile * 2)()
    assert _lib.lib.veda_candidate_tiles(_lib.VedaGrid(21, 45, 80), small, 2) == -2


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it exits with status 2 and a
    message, before it touches a device."""
    import sys
    root = os.path.dirname(HERE)
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=root)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_attention_target_is_half_the_peak_at_the_long_layer():
    """The bench line's attention target: half the bf16 peak over the long
    layer's 7,372,800 tile pairs, i.e. 49.48 ms."""
    import sys
    sys.path.insert(0, os.path.dirname(HERE))
    import bench
    import datagen
    w = datagen.WORKLOADS["long"]
    assert bench.attention_flops(w) == 4.0 * 128 * 128 * 128 * 1920 * 96 * 40
    ms = bench.attention_flops(w) / (bench.ATTN_TARGET_FRAC * bench.PEAK_BF16_TFLOPS * 1e12) * 1e3
    assert abs(ms - 49.48) < 0.01
