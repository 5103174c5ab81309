"""ctypes loader of liboasis.so (the C ABI declared in include/oasis.h).

The HIP library is the only implementation of the path: if it is not built,
loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboasis.so")

OASIS_OK = 0
OASIS_EINVAL = -1
OASIS_EUNSUPPORTED = -2
OASIS_EWORKSPACE = -3
OASIS_EHIP = -4

OASIS_F32 = 0
OASIS_BF16 = 1

OASIS_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/oasis.h

IMPL_AUTO = 0
IMPL_VALU = 1
IMPL_MFMA = 2

# Every symbol include/oasis.h declares.
EXPORTS = (
    "oasis_status_string",
    "oasis_version",
    "oasis_build_summaries",
    "oasis_score_topk_workspace",
    "oasis_score_topk",
    "oasis_select_plan",
    "oasis_append_kv",
    "oasis_copy_blocks",
    "oasis_copy_blocks_mapped",
    "oasis_host_tier_create",
    "oasis_host_tier_destroy",
    "oasis_host_tier_set_workers",
    "oasis_host_tier_fetch",
    "oasis_host_tier_submit",
    "oasis_host_tier_wait_issued",
    "oasis_host_tier_add_generated",
    "oasis_host_tier_trim",
    "oasis_host_tier_state",
    "oasis_sparse_attn_workspace",
    "oasis_sparse_attn",
    "oasis_sparse_attn_impl",
    "oasis_lookahead_step_workspace",
    "oasis_lookahead_step",
    "oasis_lookahead_step_append",
    "oasis_lookahead_step_noalloc",
)


class OasisShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("tile_stride", ctypes.c_int64),
    ]


class OasisStepOpts(ctypes.Structure):
    _fields_ = [
        ("scan_chunks", ctypes.c_int32),
        ("attn_splits", ctypes.c_int32),
        ("attn_impl", ctypes.c_int32),
        ("use_alpha", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("draft_avg", ctypes.c_int32),
    ]


class OasisError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_shp = ctypes.POINTER(OasisShape)


def load() -> ctypes.CDLL:
    """Load liboasis.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950).  There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    lib.oasis_status_string.argtypes = [ctypes.c_int]
    lib.oasis_status_string.restype = ctypes.c_char_p
    lib.oasis_version.argtypes = []
    lib.oasis_version.restype = ctypes.c_int
    lib.oasis_build_summaries.argtypes = [_shp, _vp, _i32, _vp, _i32, _i32, _vp, _vp]
    _opts = ctypes.POINTER(OasisStepOpts)
    lib.oasis_score_topk_workspace.argtypes = [_shp, _i32, _i32, _opts]
    lib.oasis_score_topk_workspace.restype = _sz
    lib.oasis_score_topk.argtypes = [_shp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _opts, _vp,
                                     _sz, _vp]
    lib.oasis_select_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                      _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.oasis_copy_blocks.argtypes = [_shp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
    lib.oasis_append_kv.argtypes = [_shp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]
    lib.oasis_copy_blocks_mapped.argtypes = [_shp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32,
                                             _vp, _vp, _vp, _vp]
    lib.oasis_host_tier_create.argtypes = [_i32, _i32, _i32, _i32, _vp, _i32, _sz, _vp, _vp, _vp]
    lib.oasis_host_tier_create.restype = _vp
    lib.oasis_host_tier_destroy.argtypes = [_vp]
    lib.oasis_host_tier_destroy.restype = None
    lib.oasis_host_tier_set_workers.argtypes = [_vp, _i32]
    lib.oasis_host_tier_fetch.argtypes = [_vp, ctypes.c_int64, _vp, _vp, _vp]
    lib.oasis_host_tier_submit.argtypes = [_vp, _shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp]
    lib.oasis_host_tier_wait_issued.argtypes = [_vp]
    lib.oasis_host_tier_add_generated.argtypes = [_vp, _i32, _i32, ctypes.c_int64, _vp]
    lib.oasis_host_tier_trim.argtypes = [_vp, _vp, _vp]
    lib.oasis_host_tier_state.argtypes = [_vp, _vp, _vp, _vp]
    lib.oasis_sparse_attn_workspace.argtypes = [_shp, _i32]
    lib.oasis_sparse_attn_workspace.restype = _sz
    lib.oasis_sparse_attn.argtypes = [_shp, _vp, _vp, _vp, _vp, _i32, ctypes.c_int64, _vp, _vp,
                                      ctypes.c_float, _vp, _vp, _vp, _sz, _vp]
    lib.oasis_sparse_attn_impl.argtypes = [_shp, _vp, _vp, _vp, _vp, _i32, ctypes.c_int64, _vp,
                                           _vp, ctypes.c_float, _vp, _vp, _vp, _sz, _i32, _vp]
    lib.oasis_lookahead_step_workspace.argtypes = [_shp, _i32, _i32, _i32, _opts]
    lib.oasis_lookahead_step_workspace.restype = _sz
    lib.oasis_lookahead_step.argtypes = (
        [_shp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp,          # q .. scores
         _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,  # slots .. plan
         _vp, _vp, _vp, _i32, ctypes.c_int64, _vp, _vp, ctypes.c_float, _vp, _vp,  # attention
         _opts, _vp, _sz, _vp])
    lib.oasis_lookahead_step_noalloc.argtypes = (
        [_shp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp,          # q .. scores
         _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,  # slots .. plan
         _vp, _vp, _vp, _i32, ctypes.c_int64, _vp, _vp, ctypes.c_float, _vp, _vp,  # attention
         _opts, _vp])
    lib.oasis_lookahead_step_append.argtypes = (
        [_shp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp,          # q .. scores
         _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,  # slots .. plan
         _vp, _vp, _vp, _i32, ctypes.c_int64, _vp, _vp, _vp,      # store, table, new token
         ctypes.c_float, _vp, _vp, _opts, _vp, _sz, _vp])
    for name in ("oasis_copy_blocks_mapped", "oasis_host_tier_fetch", "oasis_host_tier_set_workers",
                 "oasis_host_tier_submit", "oasis_host_tier_wait_issued",
                 "oasis_host_tier_add_generated",
                 "oasis_host_tier_trim", "oasis_host_tier_state"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("oasis_build_summaries", "oasis_score_topk", "oasis_select_plan", "oasis_append_kv",
                 "oasis_copy_blocks", "oasis_sparse_attn", "oasis_sparse_attn_impl",
                 "oasis_lookahead_step", "oasis_lookahead_step_append",
                 "oasis_lookahead_step_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != OASIS_OK:
        text = load().oasis_status_string(status).decode()
        raise OasisError(fn, status, text)
