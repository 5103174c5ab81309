"""oasis_lookahead_step_noalloc (the fused layer-step for callers that cannot
allocate device memory) against oasis_lookahead_step with a caller workspace.

Both calls get the same inputs and the same kernels run, so every output must
be bit-identical: attention out and lse, scores, top-K, the plan and the new
slot tables.  The shapes are split units (fewer than 256 (request, KV head)
units), so the library's per-GPU scratch array really carries block scores and
attention partials.  Two calls in a row, the second with a smaller input,
check that the scratch left by the first call does not leak into the second.
"""
import ctypes

import pytest
import torch

from sparse_kv_block_quest_amd import _lib, ops, synth


def say(msg):
    print(msg, flush=True)


def _case(dev, wl, seed_shift):
    """Inputs of one fused step after a seeding plan (resident set of K slots)."""
    wl = synth.replace(wl, seed=wl.seed + seed_shift)
    qf = synth.queries(wl, dev)
    keys = synth.keys(wl, qf[:, 0], dev)
    vt = synth.v_tiles(synth.values(wl, dev), wl.B)
    summ = ops.build_summaries(keys, wl.B)
    kt = keys.view(wl.R, wl.H, wl.n_blk, wl.B, wl.D)
    q = qf.to(wl.dtype)
    idx, _, _ = ops.score_topk(q, summ, wl.K)
    blk = torch.full((wl.R, wl.H, wl.K), -1, dtype=torch.int32, device=dev)
    stamp = torch.full_like(blk, -1)
    ops.select_plan(idx, blk, stamp, 0, wl.cap, pred_row=0)
    # the next step's queries
    q1 = synth.drift(qf[:, 0], wl.rho, synth.generator(wl.seed, synth.S_DRIFT, dev)).to(wl.dtype)
    return wl, q1, summ, kt, vt, blk, stamp


def _run(wl, q, summ, kt, vt, blk, stamp, no_alloc):
    blk_out = torch.empty_like(blk)
    stamp_out = torch.empty_like(stamp)
    res = ops.lookahead_step(q, summ, wl.K, blk, stamp, blk_out, stamp_out, 1, wl.cap, kt, vt,
                             blk, wl.n_blk, wl.B, pred_row=1, want_scores=True,
                             no_alloc=no_alloc)
    torch.cuda.synchronize()
    out = {k: v.clone() for k, v in res.items() if v is not None}
    out["slot_block_out"] = blk_out
    out["slot_stamp_out"] = stamp_out
    return out


def _workspace(wl):
    return ops.lookahead_step_workspace_bytes((wl.R, wl.n_q, wl.Hq, wl.D), wl.H, wl.B, wl.n_blk,
                                              wl.K, wl.K, wl.dtype)


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice(cuda):
    big = synth.workload("qwen3-235b-1layer", R=2, L=16384, K=64, cap=8)
    small = synth.workload("qwen3-8b-1layer", R=1, H=2, Hq=8, L=4096, K=32, cap=4)
    for i, wl0 in enumerate((big, small)):  # the second call's input is smaller
        need = _workspace(wl0)
        say(f"no-alloc call {i}: R={wl0.R} Hq={wl0.Hq} H={wl0.H} L={wl0.L} K={wl0.K}, "
            f"scratch {need} B")
        assert 0 < need <= _lib.OASIS_NOALLOC_SCRATCH_BYTES
        wl, q, summ, kt, vt, blk, stamp = _case(cuda, wl0, i)
        ref = _run(wl, q, summ, kt, vt, blk, stamp, no_alloc=False)
        got = _run(wl, q, summ, kt, vt, blk, stamp, no_alloc=True)
        assert set(ref) == set(got)
        for k in ref:
            assert torch.equal(ref[k], got[k]), f"call {i}: {k} differs"
        assert int(got["plan_count"].sum()) > 0


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose scratch exceeds the array is refused on the host (no GPU
    touched): 32 requests x 8 KV heads at 16,384 blocks per head keep their
    block scores outside LDS, 64 MiB of them."""
    lib = _lib.load()
    s = ops._shape(32, 2, 32, 8, 128, 16, _lib.OASIS_BF16)
    nb, K = 16384, 128
    need = lib.oasis_lookahead_step_workspace(ctypes.byref(s), nb, K, K, None)
    assert need > _lib.OASIS_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    st = lib.oasis_lookahead_step_noalloc(
        ctypes.byref(s), fake, fake, nb, None, K, fake, None, None,
        fake, fake, fake, fake, 1, 16, 1, None, fake, fake, fake, None,
        fake, fake, fake, K, nb, None, None, 0.0, fake, None, None, None)
    assert st == _lib.OASIS_EWORKSPACE
