"""GPU parity of decode with growing contexts: one token per request per step.

Each step appends a synthetic key/value row to every request's active block
(the model's KV write), builds the summaries of blocks that have become full,
and runs the fused step with n_blk = full blocks before the active one, the
active block as the always-attended tail, and ins_blk = the block the new token
completed (it joins every KV head's resident set through the plan for the next
step).  Lengths are staggered so requests complete blocks on different steps.
Every step is checked against the oracle: scores, top-K, plan with the
insertion, slot tables, and attention over resident blocks plus the tail.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_block_quest_amd import ops, synth
from test_gpu_step import check_step, small

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def np64(t):
    return t.detach().float().cpu().double().numpy()




def run_grow(cuda, wl, L0, steps, opts=None, units=None, kv_write="append"):
    dev = cuda
    R, H, K, B, D = wl.R, wl.H, wl.K, wl.B, wl.D
    nb = wl.n_blk  # store capacity in blocks
    qf = synth.queries(wl, dev)
    keys = synth.keys(wl, qf[:, 0], dev)
    vt = synth.v_tiles(synth.values(wl, dev), B)
    kt = keys.view(R, H, nb, B, D)
    _, kt, vt = synth.interleave_kv(kt, vt)  # the interleaved store the bench uses
    del keys
    L = torch.tensor(L0, dtype=torch.int64, device=dev)
    assert int(L.max()) + steps <= nb * B
    summ = torch.zeros((R, H, nb, 2, D), dtype=wl.dtype, device=dev)
    n_blk = (L // B).to(torch.int32)  # L0 tokens; the next token opens/extends a block
    ops.build_summaries(kt, B, seq_len=(n_blk * B).to(torch.int32), out=summ)
    q = qf.to(wl.dtype)
    # seed from the prompt: full blocks only
    idx, _, _ = ops.score_topk(q, summ, K, n_blk=n_blk)
    blk = [torch.full((R, H, K), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    stamp = [torch.full((R, H, K), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    ops.select_plan(idx, blk[0], stamp[0], 0, wl.cap, pred_row=0)
    gen = synth.generator(wl.seed + 7, synth.S_MISC, dev)
    gq = synth.generator(wl.seed + 8, synth.S_DRIFT, dev)
    cur = qf
    bufs = {}
    ar = torch.arange(R, device=dev)
    if units is None:
        units = [(r, g) for r in range(R) for g in range(H)]
    inserted = 0
    for t in range(steps):
        a, b = t % 2, 1 - t % 2
        # the model's KV write: one token per request at position L
        pos = L
        bi, ti = (pos // B), (pos % B)
        knew = torch.randn((R, H, D), generator=gen, device=dev).to(wl.dtype)
        vnew = torch.randn((R, H, D), generator=gen, device=dev).to(wl.dtype)
        if kv_write == "append":  # the library's append (summary of a completed block included)
            ops.append_kv(knew, vnew, pos.to(torch.int32), kt, vt, B, summaries=summ)
        elif kv_write == "fused":  # appended by the step itself (oasis_lookahead_step_append)
            pass
        else:
            kt[ar, :, bi, ti, :] = knew
            vt[ar, :, bi, :, ti] = vnew
        L = L + 1
        act = ((L - 1) // B).to(torch.int32)
        tail_len = (L - act.long() * B).to(torch.int32)
        n_blk = act.clone()
        ins = torch.where(tail_len == B, act, torch.full_like(act, -1))
        inserted += int((ins >= 0).sum())
        if kv_write == "torch":  # summaries of blocks that became full since the last build
            lo = max(int(n_blk.min()) - 1, 0)
            ops.build_summaries(kt, B, seq_len=(n_blk * B).to(torch.int32), blk_begin=lo,
                                blk_end=int(n_blk.max()), out=summ)
        tt = act[:, None].expand(R, H).contiguous()
        qs = cur.to(wl.dtype)
        say(f"  grow step {t}: L={L.tolist()} ins={ins.tolist()}")
        if kv_write == "fused":
            res = ops.lookahead_step(qs, summ, K, blk[a], stamp[a], blk[b], stamp[b], t + 1,
                                     wl.cap, kt, vt, blk[a], nb, B, pred_row=1, n_blk=n_blk,
                                     ins_blk=ins, want_scores=True, opts=opts, bufs=bufs,
                                     new_token=(knew, vnew, pos.to(torch.int32)))
        else:
            res = ops.lookahead_step(qs, summ, K, blk[a], stamp[a], blk[b], stamp[b], t + 1,
                                     wl.cap, kt, vt, blk[a], nb, B, pred_row=1, n_blk=n_blk,
                                     ins_blk=ins, tail_tile=tt, tail_len=tail_len,
                                     want_scores=True, opts=opts, bufs=bufs)
        torch.cuda.synchronize()
        check_step(wl, qs, summ, kt, vt, blk[a], stamp[a], blk[b], stamp[b], res, t + 1,
                   n_blk.cpu().numpy(), tt, tail_len, units, ins=ins)
        # the completed block is resident for every head of its request
        for r in range(R):
            if int(ins[r]) >= 0:
                assert bool((blk[b][r] == ins[r]).any(dim=1).all())
        if kv_write == "fused":  # the token landed in its row and column
            torch.testing.assert_close(kt[ar, :, bi, ti, :], knew, rtol=0, atol=0)
            torch.testing.assert_close(vt[ar, :, bi, :, ti], vnew, rtol=0, atol=0)
        cur = synth.drift(cur[:, 0], wl.rho, gq)
    assert inserted > 0, "the run completed no block"
    if kv_write == "torch":  # summaries there trail the writes by a step
        return
    # every complete block's summary equals the oracle's over the final keys
    full = (L // B).cpu().numpy().astype(np.int32)
    for r, g in units:
        keys64 = np64(kt[r:r + 1, g:g + 1]).reshape(1, 1, nb * B, D)
        ref = oracle.build_summaries(keys64, B, seq_len=full[r:r + 1] * B)
        got = np64(summ[r, g, :full[r]])
        np.testing.assert_array_equal(got, ref[0, 0, :full[r]])


@pytest.mark.parametrize("case", [
    dict(wl=dict(R=3, H=2, Hq=8, L=1024, K=16, cap=4), L0=[700, 713, 725], steps=24, opts=None,
         kv_write="append"),
    dict(wl=dict(R=3, H=2, Hq=8, L=1024, K=16, cap=4), L0=[704, 719, 735], steps=18,
         opts=(2, 2, 0), kv_write="torch"),
    dict(wl=dict(R=3, H=2, Hq=8, L=1024, K=16, cap=4), L0=[700, 713, 725], steps=24, opts=None,
         kv_write="fused"),
    dict(wl=dict(R=3, H=2, Hq=8, L=1024, K=16, cap=4), L0=[704, 719, 735], steps=18,
         opts=(2, 2, 0), kv_write="fused"),
    dict(wl=dict(R=2, H=2, Hq=8, L=512, K=8, cap=2, dtype=torch.float32), L0=[300, 317],
         steps=20, opts=None, kv_write="fused"),
])
def test_grow_chain(cuda, case):
    wl = small("qwen3-8b-1layer", **case["wl"])
    say(f"growing contexts {case}")
    o = None if case["opts"] is None else ops.step_opts(*case["opts"])
    run_grow(cuda, wl, case["L0"], case["steps"], opts=o, kv_write=case["kv_write"])


def test_grow_full_size(cuda):
    """The growing-context benchmark's shape and launch configuration (batch 32,
    32K store, K = 128, cap 16, interleaved store, automatic splits), the token
    appended inside the fused step; sampled units checked every step."""
    wl = synth.workload("llama3.1-8b-32layer", layers=1)
    L0 = [wl.L - 64 + (5 * r) % wl.B for r in range(wl.R)]
    say("growing contexts full size, fused append")
    run_grow(cuda, wl, L0, 18, units=[(0, 0), (3, 1), (13, 5), (31, 7)], kv_write="fused")


@pytest.mark.parametrize("dtype,D,B,interleaved", [(torch.float32, 64, 16, False),
                                                   (torch.bfloat16, 128, 16, True),
                                                   (torch.bfloat16, 128, 8, False),
                                                   (torch.float32, 128, 4, True)])
def test_append_kv_bitwise(cuda, dtype, D, B, interleaved):
    """oasis_append_kv against the oracle, token by token: the tiles hold every
    token, and a block's summary is rebuilt exactly when its last token lands."""
    say(f"append_kv dtype={dtype} D={D} B={B} interleaved={interleaved}")
    R, H, nb = 3, 2, 6
    gen = synth.generator(5, synth.S_MISC, cuda)
    kt = synth.normal((R, H, nb, B, D), gen, cuda, dtype)
    vt = synth.normal((R, H, nb, D, B), gen, cuda, dtype)
    if interleaved:
        _, kt, vt = synth.interleave_kv(kt, vt)
    summ = synth.normal((R, H, nb, 2, D), gen, cuda, dtype)
    keys64 = np64(kt).reshape(R, H, nb * B, D)
    vals64 = np64(synth.v_tiles_to_tokens(vt))
    summ64 = np64(summ)
    pos = np.array([B - 3, 2 * B - 1, -1], np.int32)
    for step in range(2 * B + 2):
        kn = synth.normal((R, H, D), gen, cuda, dtype)
        vn = synth.normal((R, H, D), gen, cuda, dtype)
        p = pos.copy()
        if step % 5 == 4:
            p[0] = -1  # request 0 skips this step
        ops.append_kv(kn, vn, torch.from_numpy(p).to(cuda), kt, vt, B, summaries=summ)
        torch.cuda.synchronize()
        keys64, vals64, summ64 = oracle.append_kv(keys64, vals64, np64(kn), np64(vn), p, B, summ64)
        np.testing.assert_array_equal(np64(kt).reshape(R, H, nb * B, D), keys64)
        np.testing.assert_array_equal(np64(synth.v_tiles_to_tokens(vt)), vals64)
        np.testing.assert_array_equal(np64(summ), summ64)
        pos = np.where(p >= 0, p + 1, pos)
        pos[2] = -1 if step < 3 else (pos[2] + 1 if pos[2] >= 0 else 0)
        pos = np.minimum(pos, nb * B - 1)
