"""ctypes view of libveda.so (the C ABI declared in include/veda.h).

Argument marshalling only: every computation runs in the library's HIP
kernels. Importing this module fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libveda.so")

VEDA_TILE_TOKENS = 128
VEDA_MAX_HEADS = 128
VEDA_MAX_TILES = 8192
VEDA_TILED_TOKEN_MAJOR = 0
VEDA_TILED_CHANNEL_MAJOR = 1

STATUS = {
    0: "VEDA_OK", -1: "VEDA_ERR_NULL", -2: "VEDA_ERR_SHAPE", -3: "VEDA_ERR_TILE", -4: "VEDA_ERR_K",
    -5: "VEDA_ERR_ALIGN", -6: "VEDA_ERR_DEVICE", -7: "VEDA_ERR_LAUNCH",
}

EXPORTS = ["veda_status_str", "veda_num_tiles", "veda_max_tiles", "veda_tile_permute", "veda_trippool_score",
           "veda_topk_mask", "veda_sparse_attn_fwd", "veda_tile_unpermute", "veda_teacher_tile_max",
           "veda_mask_overlap", "veda_head_sq_error", "veda_distill_kl", "veda_distill_grad",
           "veda_adam_step", "veda_tile_permute_stats", "veda_trippool_project_score",
           "veda_sparse_attn_fwd_raster", "veda_sparse_attn_fwd_raster_io", "veda_sparse_attn_fwd_raster_io_noalloc",
           "veda_avgpool_score", "veda_tile_recall", "veda_tile_search_select", "veda_k_from_keep",
           "veda_distill_mean_kl", "veda_candidate_tiles", "veda_dense_attn_fwd", "veda_dense_attn_fwd_raster",
           "veda_tile_scores_mfma", "veda_score_topk"]


class VedaGrid(ctypes.Structure):
    _fields_ = [("T", c_int32), ("H", c_int32), ("W", c_int32)]


class VedaTile(ctypes.Structure):
    _fields_ = [("pt", c_int32), ("ph", c_int32), ("pw", c_int32)]


class VedaGeom(ctypes.Structure):
    _fields_ = [("B", c_int32), ("n_heads", c_int32), ("head_dim", c_int32), ("grid", VedaGrid),
                ("head_tile", POINTER(VedaTile))]


class VedaRasterStrides(ctypes.Structure):
    _fields_ = [("b", c_int64), ("n", c_int64), ("h", c_int64)]


class VedaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({_text(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_sparse_attention_13_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.veda_status_str.argtypes = [ctypes.c_int]
    lib.veda_status_str.restype = ctypes.c_char_p
    lib.veda_num_tiles.argtypes = [POINTER(VedaGeom), c_int32]
    lib.veda_num_tiles.restype = ctypes.c_int
    lib.veda_max_tiles.argtypes = [POINTER(VedaGeom)]
    lib.veda_max_tiles.restype = ctypes.c_int
    lib.veda_tile_permute.argtypes = [POINTER(VedaGeom), c_void_p, VedaRasterStrides, c_void_p, c_int32, c_void_p]
    lib.veda_tile_permute.restype = ctypes.c_int
    lib.veda_tile_permute_stats.argtypes = [POINTER(VedaGeom), c_void_p, VedaRasterStrides, c_void_p, c_void_p,
                                            c_void_p]
    lib.veda_tile_permute_stats.restype = ctypes.c_int
    lib.veda_trippool_project_score.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                                c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_trippool_project_score.restype = ctypes.c_int
    lib.veda_tile_unpermute.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, VedaRasterStrides, c_void_p]
    lib.veda_tile_unpermute.restype = ctypes.c_int
    lib.veda_trippool_score.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_trippool_score.restype = ctypes.c_int
    lib.veda_avgpool_score.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_avgpool_score.restype = ctypes.c_int
    lib.veda_tile_scores_mfma.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
    lib.veda_tile_scores_mfma.restype = ctypes.c_int
    lib.veda_score_topk.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32,
                                    c_void_p, c_void_p, c_void_p]
    lib.veda_score_topk.restype = ctypes.c_int
    lib.veda_topk_mask.argtypes = [POINTER(VedaGeom), c_void_p, POINTER(c_int32), c_int32, c_void_p, c_void_p,
                                   c_void_p]
    lib.veda_topk_mask.restype = ctypes.c_int
    lib.veda_sparse_attn_fwd.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p,
                                         POINTER(c_int32), c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                         c_void_p]
    lib.veda_sparse_attn_fwd.restype = ctypes.c_int
    lib.veda_sparse_attn_fwd_raster.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p,
                                                POINTER(c_int32), c_int32, c_float, c_void_p, VedaRasterStrides,
                                                c_void_p, c_void_p, c_void_p]
    lib.veda_sparse_attn_fwd_raster.restype = ctypes.c_int
    lib.veda_sparse_attn_fwd_raster_io.argtypes = [POINTER(VedaGeom), c_void_p, VedaRasterStrides, c_void_p, c_void_p,
                                                   c_void_p, POINTER(c_int32), c_int32, c_float, c_void_p,
                                                   VedaRasterStrides, c_void_p, c_void_p, c_void_p]
    lib.veda_sparse_attn_fwd_raster_io.restype = ctypes.c_int
    lib.veda_sparse_attn_fwd_raster_io_noalloc.argtypes = [POINTER(VedaGeom), c_void_p, VedaRasterStrides, c_void_p,
                                                           c_void_p, c_void_p, POINTER(c_int32), c_int32, c_float,
                                                           c_void_p, VedaRasterStrides, c_void_p, c_void_p]
    lib.veda_sparse_attn_fwd_raster_io_noalloc.restype = ctypes.c_int
    lib.veda_dense_attn_fwd.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                        c_void_p, c_void_p]
    lib.veda_dense_attn_fwd.restype = ctypes.c_int
    lib.veda_dense_attn_fwd_raster.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                                               VedaRasterStrides, c_void_p, c_void_p, c_void_p]
    lib.veda_dense_attn_fwd_raster.restype = ctypes.c_int
    lib.veda_teacher_tile_max.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                          c_void_p]
    lib.veda_teacher_tile_max.restype = ctypes.c_int
    lib.veda_mask_overlap.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_mask_overlap.restype = ctypes.c_int
    lib.veda_tile_recall.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, POINTER(c_int32), c_void_p, c_void_p,
                                     c_void_p]
    lib.veda_tile_recall.restype = ctypes.c_int
    lib.veda_tile_search_select.argtypes = [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_tile_search_select.restype = ctypes.c_int
    lib.veda_candidate_tiles.argtypes = [VedaGrid, POINTER(VedaTile), c_int32]
    lib.veda_candidate_tiles.restype = ctypes.c_int
    lib.veda_k_from_keep.argtypes = [POINTER(VedaGeom), c_int32, c_int64, c_int64]
    lib.veda_k_from_keep.restype = ctypes.c_int
    lib.veda_distill_mean_kl.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_void_p]
    lib.veda_distill_mean_kl.restype = ctypes.c_int
    lib.veda_head_sq_error.argtypes = [POINTER(VedaGeom), c_void_p, VedaRasterStrides, c_void_p, VedaRasterStrides,
                                       c_void_p, c_void_p]
    lib.veda_head_sq_error.restype = ctypes.c_int
    lib.veda_distill_kl.argtypes = [POINTER(VedaGeom), c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p]
    lib.veda_distill_kl.restype = ctypes.c_int
    lib.veda_distill_grad.argtypes = [POINTER(VedaGeom), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.veda_distill_grad.restype = ctypes.c_int
    lib.veda_adam_step.argtypes = [c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_float, c_float,
                                   c_float, c_void_p, c_void_p]
    lib.veda_adam_step.restype = ctypes.c_int
    return lib


lib = _load()


def _text(status: int) -> str:
    return lib.veda_status_str(status).decode()


def check(status: int, call: str) -> int:
    if status < 0:
        raise VedaError(status, call)
    return status


def int_array(values):
    arr = (c_int32 * len(values))(*[int(v) for v in values])
    return arr


__all__ = ["lib", "VedaGeom", "VedaGrid", "VedaTile", "VedaRasterStrides", "VedaError", "check", "int_array",
           "EXPORTS", "STATUS", "VEDA_TILE_TOKENS", "VEDA_MAX_HEADS", "VEDA_MAX_TILES",
           "VEDA_TILED_TOKEN_MAJOR", "VEDA_TILED_CHANNEL_MAJOR", "c_uint32"]
