"""CPU oracle of the lookahead sparse-KV decode path (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library: the arithmetic lives in ``oracle.c`` (plain loops, double
precision); this module only marshals numpy arrays into it.

Every function takes float64 arrays holding the exact values of the caller's
fp32/bf16 tensors and returns fresh arrays.  Layouts are documented in
``oracle.h``.  Pages cited there: the paperpeel.com text of the OasisKV paper
(arXiv v2), the signal-papers reader text (earlier version) and the metallab.ai
summary page.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .host_tier import HostTierModel  # noqa: F401  (decode-host cache reference)

_HERE = os.path.dirname(os.path.abspath(__file__))
# OASIS_ORACLE_LIB names another build of oracle.c (the sanitizer test loads an
# address/undefined-behaviour instrumented one); by default the plain build.
_LIB_PATH = os.environ.get("OASIS_ORACLE_LIB") or os.path.join(_HERE, "liboasis_oracle.so")
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: F401  (plain gcc build of oracle.c)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oro_build_summaries.argtypes = [ctypes.c_int] * 5 + [_f64p, _i32p, ctypes.c_int,
                                                               ctypes.c_int, _f64p]
    lib.oro_append_kv.argtypes = [ctypes.c_int] * 5 + [_f64p, _f64p, _f64p, _f64p, _i32p, _f64p]
    lib.oro_block_scores.argtypes = [ctypes.c_int] * 6 + [_f64p, _f64p, _i32p, _f64p]
    lib.oro_block_scores_variant.argtypes = ([ctypes.c_int] * 6 + [_f64p, _f64p, _i32p,
                                                                  ctypes.c_double, ctypes.c_int,
                                                                  _f64p])
    lib.oro_topk.argtypes = [ctypes.c_int] * 4 + [_f64p, _i32p, ctypes.c_int, _i32p, _f64p]
    lib.oro_select_plan.argtypes = [ctypes.c_int] * 5 + [_i32p, _i32p, _i32p, ctypes.c_int,
                                                           ctypes.c_int, _i32p, _i32p, _i32p,
                                                           _i32p, _i32p]
    lib.oro_copy_blocks.argtypes = [ctypes.c_int] * 4 + [ctypes.c_long, _u8p, _u8p, _u8p,
                                                           _u8p, _i32p, _i32p, _i32p]
    lib.oro_sparse_attn.argtypes = ([ctypes.c_int] * 6 + [_f64p, _f64p, _f64p, ctypes.c_long,
                                                          _i32p, ctypes.c_int, ctypes.c_long,
                                                          _i32p, _i32p, ctypes.c_double,
                                                          _f64p, _f64p])
    lib.oro_num_threads.argtypes = []
    lib.oro_set_threads.argtypes = [ctypes.c_int]
    for name in ("oro_build_summaries", "oro_append_kv", "oro_block_scores",
                 "oro_block_scores_variant", "oro_topk",
                 "oro_select_plan",
                 "oro_copy_blocks", "oro_sparse_attn", "oro_num_threads", "oro_set_threads"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS honoured)."""
    return int(_load().oro_num_threads())


def set_threads(n: int) -> int:
    """Threads of the following oracle calls; returns the count now in use."""
    return int(_load().oro_set_threads(int(n)))


def build_summaries(keys, block_size: int, seq_len=None, blk_begin: int = 0,
                    blk_end: int | None = None, out=None) -> np.ndarray:
    """keys [R][H][L_max][D] -> summaries [R][H][n_blk_max][2][D] (0 = min, 1 = max).

    Blocks outside [blk_begin, min(blk_end, full blocks)) keep the values of
    ``out`` (zeros when ``out`` is None).
    """
    keys = _f64(keys)
    R, H, Lmax, D = keys.shape
    B = int(block_size)
    if Lmax % B:
        raise ValueError("L_max must be a multiple of the block size")
    nb = Lmax // B
    summ = np.zeros((R, H, nb, 2, D)) if out is None else _f64(out).copy()
    sl = None if seq_len is None else _i32(seq_len)
    end = nb if blk_end is None else int(blk_end)
    _check(_load().oro_build_summaries(R, H, D, B, nb, _p(keys, _f64p), _p(sl, _i32p),
                                       int(blk_begin), end, _p(summ, _f64p)),
           "build_summaries")
    return summ


def append_kv(keys, values, k_new, v_new, pos, block_size: int, summ=None):
    """Write each request's new token (position pos[r], -1 = none) for every KV
    head; rebuild the summary of a block the token completes.

    keys / values [R][H][L_max][D] token-major, k_new / v_new [R][H][D],
    summ [R][H][L_max/B][2][D] or None.  Returns new (keys, values, summ).
    """
    keys, values = _f64(keys).copy(), _f64(values).copy()
    R, H, Lmax, D = keys.shape
    B = int(block_size)
    if Lmax % B or values.shape != keys.shape:
        raise ValueError("keys / values must be [R][H][L_max][D] with L_max a multiple of B")
    s = None if summ is None else _f64(summ).copy()
    _check(_load().oro_append_kv(R, H, D, B, Lmax // B, _p(keys, _f64p), _p(values, _f64p),
                                 _p(_f64(k_new), _f64p), _p(_f64(v_new), _f64p),
                                 _p(_i32(pos), _i32p), _p(s, _f64p)), "append_kv")
    return keys, values, s


def block_scores(q, summ, n_blk=None, alpha: float = 1.0, draft_avg: bool = False) -> np.ndarray:
    """q [R][n_q][Hq][D], summaries [R][H][n_blk_max][2][D] -> scores [R][n_s][H][n_blk_max].

    alpha: the s_b(alpha) weight of the radius term (1 = the exact bound).
    draft_avg: q has 3 rows (normal, draft a, draft b); the two drafts are
    averaged before scoring, so n_s = 2.  Otherwise n_s = n_q.
    """
    q = _f64(q)
    summ = _f64(summ)
    R, nq, Hq, D = q.shape
    _, H, nb, two, D2 = summ.shape
    assert two == 2 and D2 == D and summ.shape[0] == R
    nbk = None if n_blk is None else _i32(n_blk)
    if alpha == 1.0 and not draft_avg:
        out = np.empty((R, nq, H, nb))
        _check(_load().oro_block_scores(R, nq, Hq, H, D, nb, _p(q, _f64p), _p(summ, _f64p),
                                        _p(nbk, _i32p), _p(out, _f64p)), "block_scores")
        return out
    out = np.empty((R, 2 if draft_avg else nq, H, nb))
    _check(_load().oro_block_scores_variant(R, nq, Hq, H, D, nb, _p(q, _f64p), _p(summ, _f64p),
                                            _p(nbk, _i32p), float(alpha), int(bool(draft_avg)),
                                            _p(out, _f64p)), "block_scores")
    return out


def topk(scores, k: int, n_blk=None):
    """scores [R][n_q][H][n_blk_max] -> (idx int32, score f64), each [R][n_q][H][k], ranked."""
    s = _f64(scores)
    R, nq, H, nb = s.shape
    nbk = None if n_blk is None else _i32(n_blk)
    idx = np.empty((R, nq, H, k), dtype=np.int32)
    val = np.empty((R, nq, H, k))
    _check(_load().oro_topk(R, nq, H, nb, _p(s, _f64p), _p(nbk, _i32p), int(k),
                            _p(idx, _i32p), _p(val, _f64p)), "topk")
    return idx, val


def select_plan(topk_idx, slot_block, slot_stamp, step: int, cap: int, pred_row: int = 1,
                ins_blk=None):
    """Capped least-recently-selected plan, plus the optional insertion of each
    request's newly completed block (ins_blk [R], -1 = none).

    topk_idx [R][n_q][H][K]; slot_block / slot_stamp [R][H][K] (not modified).
    Returns dict with new slot_block, slot_stamp and plan_count [R][H],
    plan_src / plan_dst / plan_evicted [R][H][K].
    """
    t = _i32(topk_idx)
    R, nq, H, K = t.shape
    blk = _i32(slot_block).copy()
    stp = _i32(slot_stamp).copy()
    assert blk.shape == (R, H, K) and stp.shape == (R, H, K)
    ins = None if ins_blk is None else _i32(ins_blk)
    assert ins is None or ins.shape == (R,)
    cnt = np.empty((R, H), dtype=np.int32)
    src = np.empty((R, H, K), dtype=np.int32)
    dst = np.empty((R, H, K), dtype=np.int32)
    ev = np.empty((R, H, K), dtype=np.int32)
    _check(_load().oro_select_plan(R, H, nq, int(pred_row), K, _p(t, _i32p), _p(blk, _i32p),
                                   _p(stp, _i32p), int(step), int(cap),
                                   None if ins is None else _p(ins, _i32p), _p(cnt, _i32p),
                                   _p(src, _i32p), _p(dst, _i32p), _p(ev, _i32p)),
           "select_plan")
    return {"slot_block": blk, "slot_stamp": stp, "plan_count": cnt, "plan_src": src,
            "plan_dst": dst, "plan_evicted": ev}


def copy_blocks(host_k, host_v, res_k, res_v, plan_count, plan_src, plan_dst):
    """Byte copy of planned tiles.

    host_k/host_v [R][H][n_blk_max][tile bytes] uint8; res_k/res_v [R][H][K][tile bytes]
    uint8 (copied, then updated).  Returns (res_k, res_v).
    """
    hk = np.ascontiguousarray(host_k, dtype=np.uint8)
    hv = np.ascontiguousarray(host_v, dtype=np.uint8)
    rk = np.ascontiguousarray(res_k, dtype=np.uint8).copy()
    rv = np.ascontiguousarray(res_v, dtype=np.uint8).copy()
    R, H, nb, tb = hk.shape
    K = rk.shape[2]
    cnt, src, dst = _i32(plan_count), _i32(plan_src), _i32(plan_dst)
    _check(_load().oro_copy_blocks(R, H, nb, K, tb, _p(hk, _u8p), _p(hv, _u8p), _p(rk, _u8p),
                                   _p(rv, _u8p), _p(cnt, _i32p), _p(src, _i32p),
                                   _p(dst, _i32p)), "copy_blocks")
    return rk, rv


def sparse_attn(q, k_tiles, v_tiles, tile_table, unit_stride: int, tail_tile=None,
                tail_len=None, scale: float = 0.0):
    """q [R][n_q][Hq][D]; k/v tiles [n_tiles][B][D]; tile_table [R][H][n_sel].

    Returns (out [R][n_q][Hq][D], lse [R][n_q][Hq]).
    """
    q = _f64(q)
    kt = _f64(k_tiles)
    vt = _f64(v_tiles)
    R, nq, Hq, D = q.shape
    n_tiles, B, D2 = kt.shape
    assert D2 == D and vt.shape == kt.shape
    tbl = _i32(tile_table)
    H, n_sel = tbl.shape[1], tbl.shape[2]
    assert tbl.shape[0] == R
    tt = None if tail_tile is None else _i32(tail_tile)
    tl = None if tail_len is None else _i32(tail_len)
    out = np.empty((R, nq, Hq, D))
    lse = np.empty((R, nq, Hq))
    _check(_load().oro_sparse_attn(R, nq, Hq, H, D, B, _p(q, _f64p), _p(kt, _f64p),
                                   _p(vt, _f64p), n_tiles, _p(tbl, _i32p), n_sel,
                                   int(unit_stride), _p(tt, _i32p), _p(tl, _i32p),
                                   float(scale), _p(out, _f64p), _p(lse, _f64p)),
           "sparse_attn")
    return out, lse
