"""GPU parity of the fused layer-step (oasis_lookahead_step) against the CPU
oracle, over chains of decode steps with double-buffered slot tables.

Per step the fused call must give
  - attention of both rows over the current resident set: within 1e-5 (fp32)
    / 2e-2 (bf16) max-abs of the oracle;
  - block scores within 1e-5 relative of the oracle's, and bitwise equal to
    the standalone oasis_score_topk;
  - top-K exactly the oracle's selection on the kernel's own fp32 scores;
  - the plan and new slot tables bit-exact against the oracle's plan on the
    kernel's top-K.
Workgroup splits (scan chunks, attention splits) are swept through the
options, so the split-unit path (per-chunk partial results merged by the
second launch, finish_kernel) is exercised next to the one-launch path.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_block_quest_amd import ops, synth

pytestmark = pytest.mark.gpu

ATTN_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
SCORE_RTOL = 1e-5


def np64(t):
    return t.detach().float().cpu().double().numpy()


def say(msg):
    print(msg, flush=True)


def score_scale(q64, summ64, G):
    R, nq, Hq, D = q64.shape
    H = Hq // G
    amax = np.maximum(np.abs(summ64[:, :, :, 0]), np.abs(summ64[:, :, :, 1]))
    qa = np.abs(q64).reshape(R, nq, H, G, D).sum(axis=3)
    return np.einsum("rjhd,rhbd->rjhb", qa, amax)


def three_rows(cur, gen):
    """[normal, draft a, draft b]: a second draft beside synth's [normal, draft]."""
    extra = 0.98 * cur[:, 0] + 0.2 * torch.randn(cur[:, 0].shape, generator=gen,
                                                 device=cur.device)
    return torch.cat([cur, extra[:, None]], dim=1)


def run_chain(cuda, wl, steps, opts=None, tail=0, n_blk=None, units=None, seed=0,
              interleaved=False):
    """Seed the resident set, then run `steps` fused steps, checking each.  With
    `interleaved` the K and V tiles live in one interleaved store (tile stride
    2*B*D) and the summaries are built from its K half."""
    qf = synth.queries(wl, cuda)
    keys = synth.keys(wl, qf[:, 0], cuda)
    vals = synth.values(wl, cuda)
    vt = synth.v_tiles(vals, wl.B)
    del vals
    summ = ops.build_summaries(keys, wl.B)
    kt = keys.view(wl.R, wl.H, wl.n_blk, wl.B, wl.D)
    if interleaved:
        _, kt, vt = synth.interleave_kv(kt, vt)
        del keys
        assert torch.equal(ops.build_summaries(kt, wl.B), summ)
    R, H, K = wl.R, wl.H, wl.K
    dev = cuda
    if tail and n_blk is None:
        n_blk = [wl.n_blk - 1] * wl.R  # the active block is not scored
    nbk = None if n_blk is None else torch.tensor(n_blk, dtype=torch.int32, device=dev)
    n_valid = np.full(R, wl.n_blk, np.int32) if n_blk is None else np.array(n_blk, np.int32)
    tt = tl = None
    if tail:
        # the active block: the last block of the store, `tail` valid tokens
        tt = torch.full((R, H), wl.n_blk - 1, dtype=torch.int32, device=dev)
        tl = torch.tensor([max(1, tail - (r % 3)) for r in range(R)], dtype=torch.int32, device=dev)
    alpha = opts.alpha if (opts is not None and opts.use_alpha) else None
    avg = bool(opts is not None and opts.draft_avg)
    g3 = synth.generator(wl.seed + 5, synth.S_MISC, dev)
    if avg:
        qf = three_rows(qf, g3)
    # seeding from row 0 of the first queries
    q = qf.to(wl.dtype)
    idx, _, _ = ops.score_topk(q, summ, K, n_blk=nbk, opts=opts)
    slots = [torch.full((R, H, K), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    stamps = [torch.full((R, H, K), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    ops.select_plan(idx, slots[0], stamps[0], 0, wl.cap, pred_row=0)
    gen = synth.generator(wl.seed + seed, synth.S_DRIFT, dev)
    cur = qf
    bufs = {}
    if units is None:
        units = [(r, g) for r in range(R) for g in range(H)]
    for t in range(steps):
        a, b = t % 2, 1 - t % 2
        q = cur.to(wl.dtype)
        say(f"  step {t}: opts={None if opts is None else (opts.scan_chunks, opts.attn_splits, opts.attn_impl)}")
        res = ops.lookahead_step(q, summ, K, slots[a], stamps[a], slots[b], stamps[b], t + 1,
                                 wl.cap, kt, vt, slots[a], wl.n_blk, wl.B, pred_row=1,
                                 n_blk=nbk, tail_tile=tt, tail_len=tl, want_scores=True,
                                 opts=opts, bufs=bufs)
        torch.cuda.synchronize()
        # standalone scan + top-K: identical fp32 scores and selection
        i2, v2, s2 = ops.score_topk(q, summ, K, n_blk=nbk, want_scores=True, opts=opts)
        torch.cuda.synchronize()
        assert torch.equal(res["scores"], s2)
        assert torch.equal(res["topk_idx"], i2)
        assert torch.equal(res["topk_score"], v2)
        check_step(wl, q, summ, kt, vt, slots[a], stamps[a], slots[b], stamps[b], res, t + 1,
                   n_valid, tt, tl, units, alpha=alpha, draft_avg=avg)
        cur = synth.drift(cur[:, 0], wl.rho, gen)
        if avg:
            cur = three_rows(cur, g3)
    return res


def check_step(wl, q, summ, kt, vt, blk_in, stamp_in, blk_out, stamp_out, res, step, n_valid,
               tt, tl, units, ins=None, alpha=None, draft_avg=False):
    R, H, K, G = wl.R, wl.H, wl.K, wl.G
    q64 = np64(q)
    # the rows that are scored: [normal, mean of the drafts] when averaging
    qsc = np.stack([q64[:, 0], (q64[:, 1] + q64[:, 2]) / 2], axis=1) if draft_avg else q64
    blk_in_np = blk_in.cpu().numpy()
    # scores against the fp64 oracle, on the sampled units
    sc = res["scores"].cpu().double().numpy()
    for r, g in units:
        s_sub = np64(summ[r:r + 1, g:g + 1])
        qs = q64[r:r + 1, :, g * G:(g + 1) * G]
        ref = oracle.block_scores(qs, s_sub, n_blk=n_valid[r:r + 1],
                                  alpha=1.0 if alpha is None else alpha, draft_avg=draft_avg)
        got = sc[r:r + 1, :, g:g + 1]
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(got), fin)
        scale = score_scale(qsc[r:r + 1, :, g * G:(g + 1) * G], s_sub, G)
        scale = scale * max(1.0, 1.0 if alpha is None else alpha)
        err = np.abs(got[fin] - ref[fin])
        assert np.all(err <= SCORE_RTOL * np.maximum(np.abs(ref[fin]), scale[fin]))
    # top-K: the oracle's selection on the kernel's scores
    i_ref, v_ref = oracle.topk(sc, K, n_blk=n_valid)
    np.testing.assert_array_equal(res["topk_idx"].cpu().numpy(), i_ref)
    np.testing.assert_array_equal(res["topk_score"].cpu().double().numpy(), v_ref)
    # plan on the kernel's top-K
    p_ref = oracle.select_plan(res["topk_idx"].cpu().numpy(), blk_in_np, stamp_in.cpu().numpy(),
                               step, wl.cap, pred_row=1,
                               ins_blk=None if ins is None else ins.cpu().numpy())
    np.testing.assert_array_equal(blk_out.cpu().numpy(), p_ref["slot_block"])
    np.testing.assert_array_equal(stamp_out.cpu().numpy(), p_ref["slot_stamp"])
    for key in ("plan_count", "plan_src", "plan_dst", "plan_evicted"):
        if res[key] is not None:  # plan_evicted is optional
            np.testing.assert_array_equal(res[key].cpu().numpy(), p_ref[key], err_msg=key)
    # attention over the input resident set (sampled units)
    D, B = wl.D, wl.B
    for r, g in units:
        sl = slice(g * G, (g + 1) * G)
        k_u = np64(kt[r, g]).reshape(-1, B, D)
        v_u = np64(synth.v_tiles_to_tokens(vt[r, g].reshape(-1, 1, D, B))).reshape(-1, B, D)
        o_ref, l_ref = oracle.sparse_attn(
            q64[r:r + 1, :, sl], k_u, v_u, blk_in_np[r:r + 1, g:g + 1], wl.n_blk,
            None if tt is None else tt[r:r + 1, g:g + 1].cpu().numpy(),
            None if tl is None else tl[r:r + 1].cpu().numpy())
        out = np64(res["out"][r:r + 1, :, sl])
        err = np.max(np.abs(out - o_ref))
        assert err <= ATTN_TOL[wl.dtype], f"unit {(r, g)} attention err {err}"
        lse = res["lse"][r:r + 1, :, sl].cpu().double().numpy()
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - l_ref[fin]), initial=0.0) <= max(ATTN_TOL[wl.dtype], 1e-5)


def small(name="tiny-fp32", **kw):
    return synth.replace(synth.workload(name), **kw)


@pytest.mark.parametrize("case", [
    dict(wl=dict(), opts=None),
    dict(wl=dict(), opts=(3, 2, 0)),
    dict(wl=dict(L=1040), opts=(1, 1, 0), tail=7),
])
def test_step_tiny_fp32(cuda, case):
    wl = small(**case["wl"])
    o = None if case["opts"] is None else ops.step_opts(*case["opts"])
    say(f"fused step tiny fp32 {case}")
    run_chain(cuda, wl, 4, opts=o, tail=case.get("tail", 0))


@pytest.mark.parametrize("G,D,B,K,opts", [
    (4, 128, 16, 32, dict(alpha=0.5)),
    (4, 128, 16, 32, dict(alpha=2.0, scan_chunks=2, attn_splits=2)),
    (4, 128, 16, 32, dict(draft_avg=True)),
    (4, 128, 16, 24, dict(draft_avg=True, alpha=0.25, scan_chunks=3, attn_splits=2)),
    (8, 64, 16, 16, dict(draft_avg=True, impl=1)),  # 24 rows, VALU attention
    (8, 128, 16, 16, dict(draft_avg=True)),          # 24 rows: three MFMA row groups
    (8, 128, 16, 16, dict(draft_avg=True, scan_chunks=2, attn_splits=3)),
])
def test_step_scoring_variants(cuda, G, D, B, K, opts):
    """s_b(alpha) and two drafts averaged before scoring (three query rows)."""
    wl = small("qwen3-8b-1layer", R=3, H=2, Hq=2 * G, D=D, B=B, L=2064, K=K, cap=5)
    say(f"fused step variants G={G} D={D} K={K} {opts}")
    run_chain(cuda, wl, 3, opts=ops.step_opts(**opts), tail=7)


@pytest.mark.parametrize("G,D,B,L,K,nq_opts", [
    (4, 128, 16, 4096, 32, (1, 1, 0)),
    (4, 128, 16, 4096, 32, (4, 3, 0)),
    (4, 128, 16, 4112, 32, (0, 0, 1)),   # VALU attention in the fused kernel
    (16, 128, 16, 2048, 24, (2, 2, 0)),  # 32 rows: two MFMA row groups
    (16, 128, 16, 2064, 24, (3, 1, 0)),  # row groups of one split each (no merge), tail
    (8, 64, 32, 2048, 16, (0, 0, 0)),
    (4, 128, 8, 1024, 20, (2, 3, 0)),    # B < 16: VALU
])
def test_step_bf16(cuda, G, D, B, L, K, nq_opts):
    wl = small("qwen3-8b-1layer", R=3, H=2, Hq=2 * G, D=D, B=B, L=L, K=K, cap=5)
    say(f"fused step bf16 G={G} D={D} B={B} L={L} K={K} opts={nq_opts}")
    run_chain(cuda, wl, 3, opts=ops.step_opts(*nq_opts), tail=5 if L % 64 else 0)


@pytest.mark.parametrize("name,G,D,B,L,K,opts", [
    ("tiny-fp32", None, None, None, 1040, None, (1, 1, 0)),
    ("qwen3-8b-1layer", 4, 128, 16, 4112, 32, (2, 2, 0)),
    ("qwen3-8b-1layer", 4, 128, 16, 4096, 32, (0, 0, 1)),  # VALU attention
    ("qwen3-8b-1layer", 4, 128, 8, 1024, 20, (2, 3, 0)),   # B < 16: VALU
])
def test_step_interleaved_store(cuda, name, G, D, B, L, K, opts):
    """K and V tiles interleaved in one store (tile stride 2*B*D)."""
    kw = dict(L=L) if G is None else dict(R=3, H=2, Hq=2 * G, D=D, B=B, L=L, K=K, cap=5)
    wl = small(name, **kw)
    say(f"fused step interleaved store {name} {kw} opts={opts}")
    run_chain(cuda, wl, 3, opts=ops.step_opts(*opts), tail=5 if L % 64 else 0,
              interleaved=True)


@pytest.mark.parametrize("L,K,cap,opts", [
    (16 * 1024, 258, 40, (4, 2, 0)),   # K > 256: the plan's block-scan branch, K not a multiple of 4
    (16 * 1024, 18, 6, (3, 2, 0)),     # K < 64, not a multiple of 4: the one-wave branch
    (16 * 9000, 64, 16, (2, 2, 0)),    # rows over 8,192 blocks: 256-thread selection and plan
])
def test_step_split_plan_branches(cuda, L, K, cap, opts):
    """The second launch's plan on each of its branches, over a chain of steps
    with forced scan chunks (so the selection and plan run in finish_kernel)."""
    wl = small("qwen3-8b-1layer", R=2, H=2, Hq=8, L=L, K=K, cap=cap)
    say(f"fused step split plan L={L} K={K} cap={cap} opts={opts}")
    run_chain(cuda, wl, 3, opts=ops.step_opts(*opts))


def test_step_merge_weights_from_memory(cuda):
    """More (split, row) pairs than the merge keeps in LDS (160 splits x 32 rows
    of the VALU attention at G = 16): the merge reads its weights' inputs from
    memory instead."""
    wl = small("qwen3-8b-1layer", R=1, H=1, Hq=16, L=16 * 2048, K=160, cap=8)
    say("fused step, 160 attention splits x 32 rows")
    run_chain(cuda, wl, 2, opts=ops.step_opts(2, 160, 1))


def test_step_short_contexts(cuda):
    """Requests with fewer full blocks than K, and an empty one."""
    wl = small("qwen3-8b-1layer", R=3, H=2, Hq=8, L=1024, K=32, cap=4)
    say("fused step short contexts")
    run_chain(cuda, wl, 3, opts=ops.step_opts(2, 2, 0), n_blk=[64, 20, 0])


@pytest.mark.parametrize("name,steps,units,interleaved", [
    ("qwen3-8b-1layer", 3, None, False),
    ("llama3.1-8b-32layer", 2, [(0, 0), (13, 5), (31, 7)], True),
    ("llama3.1-8b-32layer", 2, [(3, 2), (30, 1)], False),
    ("qwen3-235b-1layer", 2, [(0, 1), (7, 3)], True),
])
def test_step_full_size(cuda, name, steps, units, interleaved):
    """The benchmark's launch configuration (automatic splits) at full shape."""
    wl = synth.workload(name, layers=1)
    say(f"fused step full size {name} interleaved={interleaved}")
    run_chain(cuda, wl, steps, units=units, interleaved=interleaved)


def test_step_resident_layout(cuda):
    """Resident store of K slots per head (unit_stride = K) read through an
    identity tile table, the layout the pinned-host pipeline uses."""
    wl = small("qwen3-8b-1layer", R=2, H=2, Hq=8, L=2048, K=16, cap=4)
    say("fused step resident layout")
    dev = cuda
    qf = synth.queries(wl, dev)
    keys = synth.keys(wl, qf[:, 0], dev)
    vt_full = synth.v_tiles(synth.values(wl, dev), wl.B)
    summ = ops.build_summaries(keys, wl.B)
    kt_full = keys.view(wl.R, wl.H, wl.n_blk, wl.B, wl.D)
    q = qf.to(wl.dtype)
    R, H, K = wl.R, wl.H, wl.K
    blk = torch.stack([torch.stack([torch.randperm(wl.n_blk, device=dev)[:K] for _ in range(H)])
                       for _ in range(R)]).to(torch.int32)
    stamp = torch.zeros_like(blk)
    res_k = kt_full[torch.arange(R, device=dev)[:, None, None],
                    torch.arange(H, device=dev)[None, :, None], blk.long()].contiguous()
    res_v = vt_full[torch.arange(R, device=dev)[:, None, None],
                    torch.arange(H, device=dev)[None, :, None], blk.long()].contiguous()
    ident = torch.arange(K, dtype=torch.int32, device=dev).repeat(R, H, 1).contiguous()
    bo, so = torch.empty_like(blk), torch.empty_like(stamp)
    res = ops.lookahead_step(q, summ, K, blk, stamp, bo, so, 1, wl.cap, res_k, res_v, ident, K,
                             wl.B, want_scores=True, opts=ops.step_opts(2, 2, 0))
    torch.cuda.synchronize()
    check_step(wl, q, summ, kt_full, vt_full, blk, stamp, bo, so, res, 1,
               np.full(R, wl.n_blk, np.int32), None, None, [(r, g) for r in range(R) for g in range(H)])


def test_step_rejects_aliased_slots(cuda):
    wl = small("qwen3-8b-1layer", R=1, H=2, Hq=8, L=512, K=8)
    dev = cuda
    q = torch.zeros((1, 2, 8, wl.D), dtype=wl.dtype, device=dev)
    summ = torch.zeros((1, 2, wl.n_blk, 2, wl.D), dtype=wl.dtype, device=dev)
    kt = torch.zeros((1, 2, wl.n_blk, wl.B, wl.D), dtype=wl.dtype, device=dev)
    blk = torch.zeros((1, 2, 8), dtype=torch.int32, device=dev)
    st = torch.zeros_like(blk)
    with pytest.raises(ops._lib.OasisError):
        ops.lookahead_step(q, summ, 8, blk, st, blk, st, 1, 2, kt, kt, blk, wl.n_blk, wl.B)
