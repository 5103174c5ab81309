"""The C ABI: every symbol include/oasis.h declares is exported by liboasis.so,
and host-side argument checks reject bad calls before any kernel is launched
(these calls never touch a GPU)."""
import ctypes
import os
import re

import pytest

from sparse_kv_block_quest_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "oasis.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("liboasis.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert lib.oasis_status_string(code)
    assert lib.oasis_version() >= 100


def _shape(**kw):
    d = dict(batch=1, n_q=2, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=16, dtype=1)
    d.update(kw)
    return _lib.OasisShape(**d)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), _lib.OASIS_EINVAL),
    (dict(n_q=4), _lib.OASIS_EINVAL),
    (dict(n_q_heads=5), _lib.OASIS_EINVAL),
    (dict(dtype=7), _lib.OASIS_EUNSUPPORTED),
    (dict(head_dim=96), _lib.OASIS_EUNSUPPORTED),
    (dict(block_size=12), _lib.OASIS_EUNSUPPORTED),
    (dict(block_size=128), _lib.OASIS_EUNSUPPORTED),
    (dict(tile_stride=2047), _lib.OASIS_EINVAL),       # below one tile (B*D = 2048)
    (dict(tile_stride=-4096), _lib.OASIS_EINVAL),
    (dict(tile_stride=2052), _lib.OASIS_EINVAL),       # 4104 bytes: not 16-byte aligned
])
def test_shape_validation(lib, kw, code):
    s = _shape(**kw)
    assert lib.oasis_build_summaries(ctypes.byref(s), FAKE, 4, None, 0, 4, FAKE, None) == code
    assert lib.oasis_score_topk(ctypes.byref(s), FAKE, FAKE, 4, None, 2, FAKE, None, FAKE, None,
                                None, 0, None) == code
    assert lib.oasis_sparse_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 2, 4, None, None, 0.0,
                                 FAKE, None, FAKE, 1 << 20, None) == code
    assert lib.oasis_score_topk_workspace(ctypes.byref(s), 4, 2, None) == 0
    assert lib.oasis_sparse_attn_workspace(ctypes.byref(s), 2) == 0


def test_argument_validation(lib):
    s = _shape()
    E = _lib.OASIS_EINVAL
    assert lib.oasis_build_summaries(None, FAKE, 4, None, 0, 4, FAKE, None) == E
    assert lib.oasis_build_summaries(ctypes.byref(s), None, 4, None, 0, 4, FAKE, None) == E
    assert lib.oasis_build_summaries(ctypes.byref(s), FAKE, 4, None, 3, 2, FAKE, None) == E
    assert lib.oasis_build_summaries(ctypes.byref(s), FAKE, 4, None, 2, 2, FAKE, None) == 0  # empty
    assert lib.oasis_score_topk(ctypes.byref(s), FAKE, FAKE, 4, None, 0, FAKE, None, FAKE, None,
                                None, 0, None) == E
    assert lib.oasis_score_topk(ctypes.byref(s), FAKE, FAKE, 4, None, 1025, FAKE, None, FAKE, None,
                                None, 0, None) == E
    assert lib.oasis_score_topk(ctypes.byref(s), FAKE, FAKE, 40000, None, 8, FAKE, None, FAKE,
                                None, None, 0, None) == _lib.OASIS_EUNSUPPORTED
    # scores NULL and no workspace, at a shape whose units are split (needs scratch)
    assert lib.oasis_score_topk_workspace(ctypes.byref(s), 4096, 2, None) > 0
    assert lib.oasis_score_topk(ctypes.byref(s), FAKE, FAKE, 4096, None, 2, FAKE, None, None, None,
                                None, 0, None) == _lib.OASIS_EWORKSPACE
    # plan: pred_row out of range, negative cap, K too large
    args = [FAKE] * 5
    assert lib.oasis_select_plan(1, 2, 2, 2, 8, *args, 0, 1, None, FAKE, FAKE, FAKE, None,
                                 None) == E
    assert lib.oasis_select_plan(1, 2, 2, 1, 8, *args, 0, -1, None, FAKE, FAKE, FAKE, None,
                                 None) == E
    assert lib.oasis_select_plan(1, 2, 2, 1, 2048, *args, 0, 1, None, FAKE, FAKE, FAKE, None,
                                 None) == E
    assert lib.oasis_select_plan(1, 2, 2, 1, 8, None, *args[1:], 0, 1, None, FAKE, FAKE, FAKE,
                                 None, None) == E
    # attention: workspace too small (split units), group too large, MFMA forced on fp32
    assert lib.oasis_sparse_attn_workspace(ctypes.byref(s), 64) > 0
    assert lib.oasis_sparse_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 64, 64, None, None, 0.0,
                                 FAKE, None, FAKE, 0, None) == _lib.OASIS_EWORKSPACE
    big = _shape(n_q_heads=34, n_kv_heads=1)
    assert lib.oasis_sparse_attn(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 2, 4, None, None, 0.0,
                                 FAKE, None, FAKE, 1 << 30, None) == _lib.OASIS_EUNSUPPORTED
    f32 = _shape(dtype=0)
    assert lib.oasis_sparse_attn_impl(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, 2, 4, None, None,
                                      0.0, FAKE, None, FAKE, 1 << 30, 2, None) == \
        _lib.OASIS_EUNSUPPORTED
    assert lib.oasis_copy_blocks(ctypes.byref(s), None, FAKE, 4, FAKE, FAKE, 8, FAKE, FAKE, FAKE,
                                 None) == E


def test_workspace_queries(lib):
    # 256 units: one workgroup per unit and role, scores in LDS, no scratch
    s = _shape(batch=32, n_q_heads=32, n_kv_heads=8)
    assert lib.oasis_score_topk_workspace(ctypes.byref(s), 2048, 128, None) == 0
    assert lib.oasis_sparse_attn_workspace(ctypes.byref(s), 128) == 0
    assert lib.oasis_lookahead_step_workspace(ctypes.byref(s), 2048, 128, 128, None) == 0
    # split units: global scores and attention partials
    small = _shape(batch=1, n_q_heads=32, n_kv_heads=8)
    assert lib.oasis_score_topk_workspace(ctypes.byref(small), 2048, 128, None) >= 2 * 8 * 2048 * 4
    assert lib.oasis_sparse_attn_workspace(ctypes.byref(small), 128) >= 8 * 2 * 8 * 2 * 128 * 4
    # forced splits at 256 units need scratch too
    o = _lib.OasisStepOpts(2, 2, 0, 0, 1.0, 0)
    assert lib.oasis_lookahead_step_workspace(ctypes.byref(s), 2048, 128, 128,
                                              ctypes.byref(o)) >= 32 * 2 * 8 * 2048 * 4


def test_workspace_split_layout_qwen3_235b(lib):
    """Qwen3-235B-A22B shape (batch 8, 4 KV heads, G = 16, 8,192 blocks, K = 128):
    32 units, 16 items each.  Fused step: 3 attention splits (x 2 query-row
    items on the MFMA path, or 1 item each on VALU), the scan the rest; the
    scratch is both rows' global scores plus (max, sum, acc) partials of every
    split and row, the same for either path.  Attention alone: 8 splits with row
    groups, 16 without; the query answers the larger layout."""
    s = _shape(batch=8, n_q_heads=64, n_kv_heads=4)
    U, NR, D, nb, S = 32, 32, 128, 8192, 3
    scores = 2 * U * nb * 4
    partials = U * S * NR * 2 * 4 + U * S * NR * D * 4
    assert lib.oasis_lookahead_step_workspace(ctypes.byref(s), nb, 128, 128, None) == \
        scores + partials
    assert lib.oasis_sparse_attn_workspace(ctypes.byref(s), 128) == U * 16 * NR * (2 + D) * 4


def _step(lib, s, **kw):
    """oasis_lookahead_step with every pointer FAKE unless overridden."""
    a = dict(q=FAKE, summ=FAKE, nb=8, n_blk=None, K=4, idx=FAKE, tsc=None, sc=None,
             bi=FAKE, si=FAKE, bo=ctypes.c_void_p(0x9000), so=ctypes.c_void_p(0xA000), step=1,
             cap=2, pred=1, ins=None, cnt=FAKE, src=FAKE, dst=FAKE, ev=None, kt=FAKE, vt=FAKE,
             tbl=ctypes.c_void_p(0x100000), n_sel=4, stride=8, tt=None, tl=None, scale=0.0,
             out=FAKE, lse=None, opts=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.oasis_lookahead_step(
        ctypes.byref(s), a["q"], a["summ"], a["nb"], a["n_blk"], a["K"], a["idx"], a["tsc"],
        a["sc"], a["bi"], a["si"], a["bo"], a["so"], a["step"], a["cap"], a["pred"], a["ins"],
        a["cnt"],
        a["src"], a["dst"], a["ev"], a["kt"], a["vt"], a["tbl"], a["n_sel"], a["stride"],
        a["tt"], a["tl"], a["scale"], a["out"], a["lse"], a["opts"], a["ws"], a["wsb"], None)


def test_lookahead_step_validation(lib):
    s = _shape()
    E = _lib.OASIS_EINVAL
    assert _step(lib, s, q=None) == E
    assert _step(lib, s, pred=2) == E
    assert _step(lib, s, cap=-1) == E
    assert _step(lib, s, K=0) == E
    assert _step(lib, s, K=1025) == E
    assert _step(lib, s, n_sel=-1) == E
    assert _step(lib, s, stride=-1) == E
    assert _step(lib, s, tbl=None) == E
    # new slot table overlapping the tile table the attention reads
    assert _step(lib, s, bo=ctypes.c_void_p(0x100000 + 8)) == E
    assert _step(lib, s, so=ctypes.c_void_p(0x100000 - 8)) == E
    bad = _lib.OasisStepOpts(-1, 0, 0, 0, 1.0, 0)
    assert _step(lib, s, opts=ctypes.byref(bad)) == E
    mf = _lib.OasisStepOpts(0, 0, 2, 0, 1.0, 0)
    assert _step(lib, _shape(dtype=0), opts=ctypes.byref(mf)) == _lib.OASIS_EUNSUPPORTED
    assert _step(lib, _shape(head_dim=96)) == _lib.OASIS_EUNSUPPORTED
    big = dict(nb=2048, K=64, n_sel=64)  # one request: split units need scratch
    assert lib.oasis_lookahead_step_workspace(ctypes.byref(s), 2048, 64, 64, None) > 0
    assert _step(lib, s, wsb=0, **big) == _lib.OASIS_EWORKSPACE
    assert _step(lib, s, ws=None, **big) == _lib.OASIS_EWORKSPACE
    assert lib.oasis_lookahead_step_workspace(ctypes.byref(_shape(batch=0)), 8, 4, 4, None) == 0


def test_append_kv_validation(lib):
    s = _shape()
    E = _lib.OASIS_EINVAL
    assert lib.oasis_append_kv(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None) == E
    assert lib.oasis_append_kv(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, 4, None, None) == E
    assert lib.oasis_append_kv(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, 4, None, None) == E
    assert lib.oasis_append_kv(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, None) == E
    bad = _shape(head_dim=96)
    assert lib.oasis_append_kv(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None,
                               None) == _lib.OASIS_EUNSUPPORTED


def test_scoring_variant_validation(lib):
    """Three query rows only with draft averaging, averaging only with three rows,
    and alpha finite and non-negative (all rejected before any launch)."""
    E = _lib.OASIS_EINVAL
    three = _shape(n_q=3)
    avg = _lib.OasisStepOpts(0, 0, 0, 0, 1.0, 1)
    assert lib.oasis_score_topk(ctypes.byref(three), FAKE, FAKE, 4, None, 2, FAKE, None, FAKE,
                                None, None, 0, None) == E
    assert lib.oasis_score_topk(ctypes.byref(_shape()), FAKE, FAKE, 4, None, 2, FAKE, None, FAKE,
                                ctypes.byref(avg), None, 0, None) == E
    assert lib.oasis_score_topk_workspace(ctypes.byref(three), 4, 2, None) == 0
    for alpha in (-0.5, float("inf"), float("nan")):
        bad = _lib.OasisStepOpts(0, 0, 0, 1, alpha, 0)
        assert lib.oasis_score_topk(ctypes.byref(_shape()), FAKE, FAKE, 4, None, 2, FAKE, None,
                                    FAKE, ctypes.byref(bad), None, 0, None) == E
    # the fused step: pred_row must be a scored row (2 rows with averaging)
    assert _step(lib, three, pred=2, opts=ctypes.byref(avg)) == E
    assert _step(lib, three, opts=None) == E


def test_host_tier_submit_validation(lib):
    """oasis_host_tier_submit rejects bad calls before any HIP call; a tier with
    nothing submitted reports every job issued."""
    import numpy as np
    R, H, K, n_blk, B, D = 1, 2, 4, 8, 16, 128
    rec = 2 * B * D * 2                        # interleaved bf16 record
    remote = np.zeros((R, n_blk, H * rec), np.uint8)
    cache = np.zeros((R, 4, H * rec), np.uint8)
    map_ = np.zeros((R, n_blk), np.int32)
    cap = np.array([4], np.int32)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    t = lib.oasis_host_tier_create(R, H, K, n_blk, ptr(cap), 4, H * rec, ptr(remote), ptr(cache),
                                   ptr(map_))
    assert t
    t = ctypes.c_void_p(t)
    E = _lib.OASIS_EINVAL
    try:
        good = _shape(batch=R, n_q=1, n_q_heads=H, n_kv_heads=H, tile_stride=2 * B * D)
        args = [FAKE] * 8 + [FAKE, None, FAKE]     # caches, res, plan x3, slots, after, stream, done
        assert lib.oasis_host_tier_submit(None, ctypes.byref(good), *args) == E
        assert lib.oasis_host_tier_submit(t, None, *args) == E
        wrong_r = _shape(batch=2, n_q=1, n_q_heads=H, n_kv_heads=H, tile_stride=2 * B * D)
        assert lib.oasis_host_tier_submit(t, ctypes.byref(wrong_r), *args) == E
        # records of B*D elements: two per block do not fill block_bytes
        narrow = _shape(batch=R, n_q=1, n_q_heads=H, n_kv_heads=H)
        assert lib.oasis_host_tier_submit(t, ctypes.byref(narrow), *args) == E
        no_after = [FAKE] * 8 + [None, None, FAKE]
        assert lib.oasis_host_tier_submit(t, ctypes.byref(good), *no_after) == E
        no_done = [FAKE] * 8 + [FAKE, None, None]
        assert lib.oasis_host_tier_submit(t, ctypes.byref(good), *no_done) == E
        assert lib.oasis_host_tier_wait_issued(t) == 0
        assert lib.oasis_host_tier_wait_issued(None) == E
        assert lib.oasis_host_tier_set_workers(t, 0) == E
        assert lib.oasis_host_tier_set_workers(None, 2) == E
    finally:
        lib.oasis_host_tier_destroy(t)


def test_lookahead_step_append_validation(lib):
    """The append form needs the new token and the full-cache store."""
    s = _shape()
    E = _lib.OASIS_EINVAL
    head = [ctypes.byref(s), FAKE, FAKE, 64, None, 4, FAKE, None, None,
            FAKE, FAKE, FAKE, FAKE, 1, 2, 1, None, FAKE, FAKE, FAKE, None,
            FAKE, FAKE, FAKE, 4]
    tail = [0.0, FAKE, None, None, None, 0, None]
    # unit_stride other than n_blk_max
    assert lib.oasis_lookahead_step_append(*head, 4, FAKE, FAKE, FAKE, *tail) == E
    # missing k_new / v_new / pos
    assert lib.oasis_lookahead_step_append(*head, 64, None, FAKE, FAKE, *tail) == E
    assert lib.oasis_lookahead_step_append(*head, 64, FAKE, None, FAKE, *tail) == E
    assert lib.oasis_lookahead_step_append(*head, 64, FAKE, FAKE, None, *tail) == E
