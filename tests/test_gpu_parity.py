"""GPU parity: every HIP kernel, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bars: summaries, top-K (on the kernel's own fp32 scores), plans and copies
bit-exact; scores within 1e-5 relative of max(|s|, sum of |terms|); top-K sets
against the fp64 oracle equal up to blocks within that band of the K-th score;
attention within 1e-5 max-abs (fp32 inputs) / 2e-2 max-abs (bf16 inputs, fp32
accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_block_quest_amd import ops, synth

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-5
ATTN_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype != torch.float64 else t.cpu().numpy()


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ helpers
def make_layer(wl, dev, layer=0, L=None):
    """Keys [R][H][L][D], dim-major V tiles, stacked queries [R][2][Hq][D] (wl.dtype)."""
    if L is not None:
        wl = synth.replace(wl, L=L)
    qf = synth.queries(wl, dev, layer=layer)
    k = synth.keys(wl, qf[:, 0], dev, layer=layer)
    v = synth.values(wl, dev, layer=layer)
    return wl, k, synth.v_tiles(v, wl.B), qf.to(wl.dtype)


def score_scale(q64, summ64, G):
    """sum_h sum_d |q_hd| * max(|max_d|, |min_d|) per block: the size of the terms."""
    R, nq, Hq, D = q64.shape
    H = Hq // G
    amax = np.maximum(np.abs(summ64[:, :, :, 0]), np.abs(summ64[:, :, :, 1]))
    qa = np.abs(q64).reshape(R, nq, H, G, D).sum(axis=3)
    return np.einsum("rjhd,rhbd->rjhb", qa, amax)


def check_scores(sc_gpu, sc_ref, scale):
    fin = np.isfinite(sc_ref)
    assert np.array_equal(np.isfinite(sc_gpu), fin)
    err = np.abs(sc_gpu[fin] - sc_ref[fin])
    bound = SCORE_RTOL * np.maximum(np.abs(sc_ref[fin]), scale[fin])
    assert np.all(err <= bound), f"max score err ratio {np.max(err / bound):.3g}"


def check_topk_band(idx_gpu, idx_ref, sc_ref, scale, n_blk):
    """GPU set may differ from the fp64 set only by blocks within the band of the K-th score."""
    R, nq, H, K = idx_gpu.shape
    for r in range(R):
        for j in range(nq):
            for h in range(H):
                kp = min(K, int(n_blk[r]))
                a = set(idx_gpu[r, j, h, :kp].tolist())
                b = set(idx_ref[r, j, h, :kp].tolist())
                assert -1 not in a
                if a == b:
                    continue
                s = sc_ref[r, j, h]
                sk = s[idx_ref[r, j, h, kp - 1]]
                for blk in a ^ b:
                    band = SCORE_RTOL * max(abs(sk), scale[r, j, h, blk])
                    assert abs(s[blk] - sk) <= band, (r, j, h, blk)
                assert np.all(idx_gpu[r, j, h, kp:] == -1)


# ------------------------------------------------------------------ summaries
@pytest.mark.parametrize("dtype,D,B,L", [
    (torch.float32, 64, 16, 1024), (torch.float32, 128, 4, 256), (torch.bfloat16, 128, 16, 4096),
    (torch.bfloat16, 64, 1, 64), (torch.bfloat16, 128, 64, 2048), (torch.float32, 64, 2, 100)])
def test_summaries_bitwise(cuda, dtype, D, B, L):
    say(f"summaries dtype={dtype} D={D} B={B} L={L}")
    R, H = 3, 2
    Lmax = (L + B - 1) // B * B
    gen = synth.generator(11, synth.S_KEYS, cuda)
    keys = synth.normal((R, H, Lmax, D), gen, cuda, dtype)
    seq = torch.tensor([L, max(0, L - B - 3), Lmax], dtype=torch.int32, device=cuda)
    out = ops.build_summaries(keys, B, seq_len=seq)
    torch.cuda.synchronize()
    ref = oracle.build_summaries(np64(keys), B, seq_len=seq.cpu().numpy())
    np.testing.assert_array_equal(np64(out), ref)
    # incremental range update leaves the rest untouched
    nb = Lmax // B
    sentinel = torch.full_like(out, 7.0)
    part = ops.build_summaries(keys, B, seq_len=seq, blk_begin=nb // 3, blk_end=nb // 3 + 2,
                               out=sentinel)
    ref2 = oracle.build_summaries(np64(keys), B, seq_len=seq.cpu().numpy(), blk_begin=nb // 3,
                                  blk_end=nb // 3 + 2, out=np.full(ref.shape, 7.0))
    np.testing.assert_array_equal(np64(part), ref2)


@pytest.mark.parametrize("dtype,D,B", [(torch.float32, 64, 16), (torch.bfloat16, 128, 16),
                                        (torch.bfloat16, 64, 8)])
def test_summaries_interleaved_store(cuda, dtype, D, B):
    """Summaries read from the K half of an interleaved K|V store (tile stride
    2*B*D) equal those of the dense key store, bit for bit."""
    say(f"summaries interleaved dtype={dtype} D={D} B={B}")
    R, H, nb = 2, 3, 37
    gen = synth.generator(12, synth.S_KEYS, cuda)
    kt = synth.normal((R, H, nb, B, D), gen, cuda, dtype)
    vt = synth.normal((R, H, nb, D, B), gen, cuda, dtype)
    _, k2, _ = synth.interleave_kv(kt, vt)
    seq = torch.tensor([nb * B, nb * B - 2 * B - 1], dtype=torch.int32, device=cuda)
    out = ops.build_summaries(k2, B, seq_len=seq)
    torch.cuda.synchronize()
    ref = oracle.build_summaries(np64(kt.reshape(R, H, nb * B, D)), B, seq_len=seq.cpu().numpy())
    np.testing.assert_array_equal(np64(out), ref)


def test_summaries_full_size_qwen3_8b(cuda):
    say("summaries qwen3-8b-1layer full size")
    wl, k, _, _ = make_layer(synth.workload("qwen3-8b-1layer"), cuda)
    out = ops.build_summaries(k, wl.B)
    torch.cuda.synchronize()
    ref = oracle.build_summaries(np64(k), wl.B)
    np.testing.assert_array_equal(np64(out), ref)
    again = ops.build_summaries(k, wl.B)
    assert torch.equal(again, out)


# ------------------------------------------------------------------ score + top-K
def run_score_topk(wl, k, q, n_blk=None, K=None):
    summ = ops.build_summaries(k, wl.B)
    idx, val, sc = ops.score_topk(q, summ, K or wl.K, n_blk=n_blk, want_scores=True)
    torch.cuda.synchronize()
    return summ, idx, val, sc


def check_score_topk_against_oracle(wl, summ, q, idx, val, sc, n_blk_np, K):
    summ64, q64 = np64(summ), np64(q)
    sc_ref = oracle.block_scores(q64, summ64, n_blk=n_blk_np)
    scale = score_scale(q64, summ64, wl.G)
    sc_gpu = sc.cpu().double().numpy()
    check_scores(sc_gpu, sc_ref, scale)
    # the kernel's selection on its own fp32 scores: exact
    i2, v2 = oracle.topk(sc_gpu, K, n_blk=n_blk_np)
    np.testing.assert_array_equal(idx.cpu().numpy(), i2)
    np.testing.assert_array_equal(val.cpu().double().numpy(), v2)
    # against the fp64 scores: equal sets up to the tolerance band
    iref, _ = oracle.topk(sc_ref, K, n_blk=n_blk_np)
    check_topk_band(idx.cpu().numpy(), iref, sc_ref, scale, n_blk_np)


@pytest.mark.parametrize("name,L,K,G", [("tiny-fp32", 1024, 8, None), ("tiny-fp32", 1031, 8, None),
                                        ("tiny-fp32", 256, 20, 4), ("qwen3-8b-1layer", 4096, 64, None),
                                        # split selection: staged row beyond the keys held in
                                        # registers, and a row too long to stage (global reads)
                                        ("tiny-fp32", 16 * 9000 + 5, 64, None),
                                        ("tiny-fp32", 16 * 20000 + 3, 64, None)])
def test_score_topk_small(cuda, name, L, K, G):
    say(f"score_topk {name} L={L} K={K} G={G}")
    wl = synth.workload(name)
    if G:
        wl = synth.replace(wl, Hq=G * 2, H=2)
    Lmax = (L + wl.B - 1) // wl.B * wl.B
    wl, k, _, q = make_layer(wl, cuda, L=Lmax)
    n_blk = torch.tensor([L // wl.B] * wl.R, dtype=torch.int32, device=cuda)
    summ, idx, val, sc = run_score_topk(wl, k, q, n_blk=n_blk, K=K)
    check_score_topk_against_oracle(wl, summ, q, idx, val, sc, n_blk.cpu().numpy(), K)


def test_score_topk_ties_and_short_contexts(cuda):
    say("score_topk ties / n_blk < K / empty")
    R, H, G, D, B, nb = 3, 2, 2, 64, 4, 50
    gen = synth.generator(5, synth.S_KEYS, cuda)
    base = synth.normal((R, H, 5, B, D), gen, cuda)
    keys = base.repeat(1, 1, nb // 5, 1, 1).reshape(R, H, nb * B, D)  # 10 copies of each block
    q = synth.normal((R, 2, H * G, D), gen, cuda)
    wl = synth.replace(synth.workload("tiny-fp32"), R=R, H=H, Hq=H * G, D=D, B=B, L=nb * B, K=16)
    n_blk = torch.tensor([nb, 7, 0], dtype=torch.int32, device=cuda)
    summ, idx, val, sc = run_score_topk(wl, keys, q, n_blk=n_blk, K=16)
    check_score_topk_against_oracle(wl, summ, q, idx, val, sc, n_blk.cpu().numpy(), 16)
    assert torch.all(idx[2] == -1)


def edge_summaries(case, R, H, nb, D, gen, dev):
    """Summaries whose scores stress the selection: all equal, a few distinct
    values (radix passes run into the block-index bits), or random."""
    x = synth.normal((R, H, nb, D), gen, dev).abs()
    if case == "equal":
        x = torch.zeros_like(x)
    elif case in ("two_values", "few"):
        n_pat = 2 if case == "two_values" else 5
        pats = synth.normal((R, H, n_pat, D), gen, dev).abs()
        pick = torch.randint(0, n_pat, (R, H, nb), generator=gen, device=dev)
        x = torch.gather(pats, 2, pick[..., None].expand(R, H, nb, D))
    return torch.stack([-x, x], dim=3).contiguous()  # [R][H][nb][2][D]: min, max


@pytest.mark.parametrize("case,nb,K,n_blk", [
    ("random", 8192, 128, None), ("equal", 8192, 128, None), ("two_values", 8192, 128, None),
    ("few", 3000, 64, None), ("random", 8192, 1024, None), ("random", 8192, 1, None),
    ("two_values", 8192, 1024, None), ("random", 2048, 128, [2048, 100, 7, 0]),
    ("equal", 1500, 16, [1500, 1499, 16, 15]),
])
def test_score_topk_split_selection_edges(cuda, case, nb, K, n_blk):
    """The second launch's selection of split units (scan chunks forced), on
    rows held in registers: ties everywhere, a few distinct scores (several
    radix passes, the last ones into the block-index bits), K up to 1024 (more
    candidates than four lanes each can rank), K = 1, rows no longer than the
    candidate bound (no pass), shorter than K, and empty."""
    say(f"split selection {case} nb={nb} K={K} n_blk={n_blk}")
    R, H, G, D = 4, 2, 2, 64
    gen = synth.generator(11, synth.S_MISC, cuda)
    summ = edge_summaries(case, R, H, nb, D, gen, cuda)
    q = synth.normal((R, 2, H * G, D), gen, cuda)
    wl = synth.replace(synth.workload("tiny-fp32"), R=R, H=H, Hq=H * G, D=D, B=16, L=nb * 16, K=K)
    nbt = None if n_blk is None else torch.tensor(n_blk, dtype=torch.int32, device=cuda)
    for chunks in (2, 5):
        idx, val, sc = ops.score_topk(q, summ, K, n_blk=nbt, want_scores=True,
                                      opts=ops.step_opts(scan_chunks=chunks))
        torch.cuda.synchronize()
        nbn = np.full(R, nb, dtype=np.int32) if n_blk is None else np.array(n_blk, dtype=np.int32)
        check_score_topk_against_oracle(wl, summ, q, idx, val, sc, nbn, K)


@pytest.mark.parametrize("name,units", [("qwen3-8b-1layer", None), ("qwen3-235b-1layer", [(0, 1), (7, 3)]),
                                        ("llama3.1-8b-32layer", [(0, 0), (13, 5), (31, 7)])])
def test_score_topk_full_size(cuda, name, units):
    say(f"score_topk full size {name}")
    wl, k, _, q = make_layer(synth.workload(name), cuda)
    summ, idx, val, sc = run_score_topk(wl, k, q)
    nbk = np.full(wl.R, wl.n_blk, dtype=np.int32)
    if units is None:
        check_score_topk_against_oracle(wl, summ, q, idx, val, sc, nbk, wl.K)
        return
    for r, g in units:
        sl = slice(g * wl.G, (g + 1) * wl.G)
        sub = synth.replace(wl, R=1, H=1, Hq=wl.G)
        check_score_topk_against_oracle(sub, summ[r:r + 1, g:g + 1], q[r:r + 1, :, sl].contiguous(),
                                        idx[r:r + 1, :, g:g + 1], val[r:r + 1, :, g:g + 1],
                                        sc[r:r + 1, :, g:g + 1], nbk[:1], wl.K)


# ------------------------------------------------------------------ plan
@pytest.mark.parametrize("insert", [False, True])
def test_plan_bitwise_over_history(cuda, insert):
    say(f"select_plan 12-step history, R=4 H=8 K=32 cap=4, insertion={insert}")
    R, H, K, nb, cap = 4, 8, 32, 300, 4
    rng = np.random.default_rng(17)
    blk = torch.full((R, H, K), -1, dtype=torch.int32, device=cuda)
    stamp = torch.full((R, H, K), -1, dtype=torch.int32, device=cuda)
    blk_ref, stamp_ref = blk.cpu().numpy(), stamp.cpu().numpy()
    cur = np.stack([[rng.permutation(nb)[:K] for _ in range(H)] for _ in range(R)])
    for step in range(12):
        mask = rng.random(cur.shape) < 0.25
        cur = np.where(mask, rng.integers(0, nb, cur.shape), cur)
        topk = np.full((R, 2, H, K), -1, dtype=np.int32)
        for r in range(R):
            for h in range(H):
                row = list(dict.fromkeys(cur[r, h].tolist()))  # distinct, in rank order
                if (r + h + step) % 5 == 0:
                    row = row[: K // 2]
                topk[r, 0, h, :len(row)] = row
                topk[r, 1, h, :len(row)] = row[::-1]
        pred_row = 0 if step == 0 else 1
        t = torch.from_numpy(topk).to(cuda)
        ins = None
        if insert:  # a fresh block for most requests; now and then one already resident
            ins = np.where(rng.random(R) < 0.7, nb + step * R + np.arange(R), -1).astype(np.int32)
            if step % 4 == 3:
                ins[1] = blk_ref[1, 0, 0]
        plan = ops.select_plan(t, blk, stamp, step, cap, pred_row=pred_row,
                               ins_blk=None if ins is None else torch.from_numpy(ins).to(cuda))
        torch.cuda.synchronize()
        ref = oracle.select_plan(topk, blk_ref, stamp_ref, step, cap, pred_row=pred_row,
                                 ins_blk=ins)
        for key in ("plan_count", "plan_src", "plan_dst", "plan_evicted"):
            np.testing.assert_array_equal(plan[key].cpu().numpy(), ref[key], err_msg=key)
        np.testing.assert_array_equal(blk.cpu().numpy(), ref["slot_block"])
        np.testing.assert_array_equal(stamp.cpu().numpy(), ref["slot_stamp"])
        blk_ref, stamp_ref = ref["slot_block"], ref["slot_stamp"]


def test_plan_separate_outputs_and_large_k(cuda):
    say("select_plan out-of-place, K=1024")
    R, H, K = 2, 3, 1024
    rng = np.random.default_rng(3)
    topk = np.stack([[[rng.permutation(5000)[:K] for _ in range(H)] for _ in range(1)]
                     for _ in range(R)]).astype(np.int32)
    blk = np.stack([[rng.permutation(5000)[:K] for _ in range(H)] for _ in range(R)]).astype(np.int32)
    stamp = rng.integers(0, 50, (R, H, K)).astype(np.int32)
    tb, ts = torch.from_numpy(blk).to(cuda), torch.from_numpy(stamp).to(cuda)
    ob, os_ = torch.empty_like(tb), torch.empty_like(ts)
    plan = ops.select_plan(torch.from_numpy(topk).to(cuda), tb, ts, 77, 100, pred_row=0,
                           slot_block_out=ob, slot_stamp_out=os_)
    torch.cuda.synchronize()
    ref = oracle.select_plan(topk, blk, stamp, 77, 100, pred_row=0)
    np.testing.assert_array_equal(ob.cpu().numpy(), ref["slot_block"])
    np.testing.assert_array_equal(os_.cpu().numpy(), ref["slot_stamp"])
    np.testing.assert_array_equal(plan["plan_src"].cpu().numpy(), ref["plan_src"])
    assert torch.equal(tb.cpu(), torch.from_numpy(blk))  # inputs untouched


# ------------------------------------------------------------------ copy
@pytest.mark.parametrize("pinned,interleaved", [(False, False), (True, False), (False, True),
                                                (True, True)])
def test_copy_blocks_bitwise(cuda, pinned, interleaved):
    say(f"copy_blocks pinned={pinned} interleaved={interleaved}")
    R, H, nb, K, B, D = 2, 4, 40, 16, 16, 128
    gen = synth.generator(23, synth.S_MISC, cuda)
    sk = synth.normal((R, H, nb, B, D), gen, cuda, torch.bfloat16)
    sv = synth.normal((R, H, nb, D, B), gen, cuda, torch.bfloat16)
    if pinned:
        sk, sv = sk.cpu().pin_memory(), sv.cpu().pin_memory()
    rk = synth.normal((R, H, K, B, D), gen, cuda, torch.bfloat16)
    rv = synth.normal((R, H, K, D, B), gen, cuda, torch.bfloat16)
    if interleaved:
        buf = torch.empty((R, H, nb, 2, B, D), dtype=torch.bfloat16, pin_memory=pinned,
                          device="cpu" if pinned else cuda)
        _, sk, sv = synth.interleave_kv(sk, sv, out=buf)
        _, rk, rv = synth.interleave_kv(rk, rv)
    rng = np.random.default_rng(8)
    cnt = rng.integers(0, K + 1, (R, H)).astype(np.int32)
    src = np.stack([[rng.permutation(nb)[:K] for _ in range(H)] for _ in range(R)]).astype(np.int32)
    dst = np.stack([[rng.permutation(K) for _ in range(H)] for _ in range(R)]).astype(np.int32)
    plan = {"plan_count": torch.from_numpy(cnt).to(cuda), "plan_src": torch.from_numpy(src).to(cuda),
            "plan_dst": torch.from_numpy(dst).to(cuda)}
    u8 = lambda t: t.cpu().contiguous().view(torch.uint8).numpy().reshape(R, H, t.shape[2], -1)
    ek, ev = oracle.copy_blocks(u8(sk), u8(sv), u8(rk), u8(rv), cnt, src, dst)
    ops.copy_blocks(sk, sv, rk, rv, plan, B)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u8(rk), ek)
    np.testing.assert_array_equal(u8(rv), ev)


@pytest.mark.parametrize("workers", [1, 3])
def test_copy_blocks_mapped_bitwise(cuda, workers):
    """Host fetch into the decode-host cache (oasis_host_tier_fetch), then the
    gather through the union map (oasis_copy_blocks_mapped): the planned slots
    hold the remote blocks' records, entries whose block is absent are skipped
    (their slots keep what they held), over three rounds with evictions."""
    say(f"copy_blocks_mapped workers={workers}")
    R, H, nb, K, B, D, cap = 3, 4, 96, 8, 16, 128, 40
    gen = synth.generator(29, synth.S_MISC, cuda)
    rec = synth.normal((R, nb, H, 2, B, D), gen, cuda, torch.bfloat16)
    remote = torch.empty(rec.shape, dtype=rec.dtype, pin_memory=True)
    remote.copy_(rec.cpu())
    cache = torch.empty((R, cap, H, 2, B, D), dtype=rec.dtype, pin_memory=True)
    map_ = torch.empty((R, nb), dtype=torch.int32, pin_memory=True)
    tier = ops.HostTier(R, H, K, nb, [cap] * R, remote, cache, map_, H * 2 * B * D * 2,
                        workers=workers)
    res = synth.normal((R, H, K, 2, B, D), gen, cuda, torch.bfloat16)
    rk, rv = ops.interleaved_kv(res)
    rng = np.random.default_rng(12)
    u8 = lambda t: t.cpu().contiguous().view(torch.uint8).numpy().reshape(R, H, t.shape[2], -1)
    src_store = remote.permute(0, 2, 1, 3, 4, 5).contiguous()     # [R][H][nb][2][B][D]
    for step in range(1, 4):
        cnt = rng.integers(1, K + 1, (R, H)).astype(np.int32)
        src = np.stack([[rng.permutation(nb)[:K] for _ in range(H)] for _ in range(R)]).astype(np.int32)
        dst = np.stack([[rng.permutation(K) for _ in range(H)] for _ in range(R)]).astype(np.int32)
        # unit (r, 0)'s last planned block is left out of the fetch: absent unless cached
        fcnt = cnt.copy()
        fcnt[:, 0] -= 1
        assert tier.fetch(step, fcnt, src, None) == 0
        plan = {"plan_count": torch.from_numpy(cnt).to(cuda),
                "plan_src": torch.from_numpy(src).to(cuda),
                "plan_dst": torch.from_numpy(dst).to(cuda)}
        present = map_.numpy()[np.arange(R)[:, None, None], src] >= 0      # [R][H][K]
        ecnt = cnt.copy()
        esrc, edst = src.copy(), dst.copy()
        for r in range(R):       # the oracle copies exactly the present entries, in order
            for g in range(H):
                keep = [i for i in range(cnt[r, g]) if present[r, g, i]]
                ecnt[r, g] = len(keep)
                esrc[r, g, :len(keep)] = src[r, g, keep]
                edst[r, g, :len(keep)] = dst[r, g, keep]
        assert (ecnt <= cnt).all() and ecnt.sum() >= cnt.sum() - R
        before = u8(res)
        both = lambda t: t.reshape(R, H, t.shape[2], 2, -1)
        ek, ev = oracle.copy_blocks(both(u8(src_store))[..., 0, :].copy(),
                                    both(u8(src_store))[..., 1, :].copy(),
                                    both(before)[..., 0, :].copy(), both(before)[..., 1, :].copy(),
                                    ecnt, esrc, edst)
        ops.prepare_copy_blocks_mapped(cache, map_, rk, rv, plan, B)(torch.cuda.current_stream())
        torch.cuda.synchronize()
        got = both(u8(res))
        np.testing.assert_array_equal(got[..., 0, :], ek)
        np.testing.assert_array_equal(got[..., 1, :], ev)
    assert tier.state()[2]["evicted"] > 0
    tier.close()


# ------------------------------------------------------------------ attention
def attn_reference(q, k, vt, table, unit_stride, B, tail_tile=None, tail_len=None, scale=0.0):
    D = q.shape[-1]
    kt = np64(k).reshape(-1, B, D)
    vtok = np64(synth.v_tiles_to_tokens(vt.reshape(-1, 1, D, B))).reshape(-1, B, D)
    return oracle.sparse_attn(np64(q), kt, vtok, table.cpu().numpy(), unit_stride,
                              None if tail_tile is None else tail_tile.cpu().numpy(),
                              None if tail_len is None else tail_len.cpu().numpy(), scale)


def check_attn(out, lse, ref, dtype):
    o_ref, l_ref = ref
    err = np.max(np.abs(np64(out) - o_ref))
    assert err <= ATTN_TOL[dtype], f"max abs err {err}"
    fin = np.isfinite(l_ref)
    l = lse.cpu().double().numpy()
    assert np.array_equal(np.isfinite(l), fin)
    assert np.max(np.abs(l[fin] - l_ref[fin]), initial=0.0) <= max(ATTN_TOL[dtype], 1e-5)


IMPLS = {torch.float32: [ops.IMPL_VALU], torch.bfloat16: [ops.IMPL_VALU, ops.IMPL_MFMA]}


@pytest.mark.parametrize("dtype,G,B,nb,n_sel,tail", [
    (torch.float32, 2, 16, 64, 8, 0),        # tiny config
    (torch.float32, 2, 16, 65, 64, 7),       # all blocks + ragged active block
    (torch.float32, 4, 4, 40, 13, 3),
    (torch.bfloat16, 4, 16, 96, 37, 0),
    (torch.bfloat16, 4, 16, 97, 96, 11),
    (torch.bfloat16, 16, 16, 48, 20, 16),
    (torch.bfloat16, 8, 32, 24, 9, 19),
    (torch.bfloat16, 2, 64, 12, 5, 63),
    (torch.bfloat16, 4, 8, 30, 7, 5),
])
def test_attn_parity(cuda, dtype, G, B, nb, n_sel, tail):
    R, H, D = 2, 2, 128 if dtype == torch.bfloat16 else 64
    gen = synth.generator(31 + G + B, synth.S_MISC, cuda)
    q = synth.normal((R, 2, H * G, D), gen, cuda, dtype)
    k = synth.normal((R, H, nb, B, D), gen, cuda, dtype)
    vt = synth.normal((R, H, nb, D, B), gen, cuda, dtype)
    table = synth.random_tile_table(R, H, n_sel, nb - 1, gen, cuda)
    if n_sel > 3:
        table[0, 1, 2] = -1
    tt = tl = None
    if tail:
        tt = torch.full((R, H), nb - 1, dtype=torch.int32, device=cuda)
        tl = torch.tensor([tail, max(1, tail // 2)], dtype=torch.int32, device=cuda)
    ref = attn_reference(q, k, vt, table, nb, B, tt, tl)
    _, ki, vi = synth.interleave_kv(k, vt)
    for impl in IMPLS[dtype]:
        if impl == ops.IMPL_MFMA and B % 16:
            continue
        say(f"attn dtype={dtype} G={G} B={B} n_sel={n_sel} tail={tail} impl={impl}")
        out, lse = ops.sparse_attn(q, k, vt, table, nb, B, tail_tile=tt, tail_len=tl, impl=impl)
        torch.cuda.synchronize()
        check_attn(out, lse, ref, dtype)
        out2, lse2 = ops.sparse_attn(q, k, vt, table, nb, B, tail_tile=tt, tail_len=tl, impl=impl)
        assert torch.equal(out, out2) and torch.equal(lse, lse2)  # deterministic
        # the same tiles in an interleaved K|V store: identical results
        o3, l3 = ops.sparse_attn(q, ki, vi, table, nb, B, tail_tile=tt, tail_len=tl, impl=impl)
        assert torch.equal(out, o3) and torch.equal(lse, l3)
        # stacked rows == two single-row calls, bitwise
        for j in range(2):
            o1, l1 = ops.sparse_attn(q[:, j:j + 1].contiguous(), k, vt, table, nb, B, tail_tile=tt,
                                     tail_len=tl, impl=impl)
            assert torch.equal(o1, out[:, j:j + 1]) and torch.equal(l1, lse[:, j:j + 1])


@pytest.mark.parametrize("G,impl", [(4, None), (8, None), (10, None), (4, "valu")])
def test_attn_three_rows(cuda, G, impl):
    """Three stacked rows (normal + two drafts) attend the same tiles; each row
    equals its own single-row call bit for bit."""
    say(f"attn three rows G={G} impl={impl}")
    R, H, D, B, nb, n_sel = 2, 2, 128, 16, 40, 13
    dtype = torch.bfloat16
    gen = synth.generator(41 + G, synth.S_MISC, cuda)
    q = synth.normal((R, 3, H * G, D), gen, cuda, dtype)
    k = synth.normal((R, H, nb, B, D), gen, cuda, dtype)
    vt = synth.normal((R, H, nb, D, B), gen, cuda, dtype)
    table = synth.random_tile_table(R, H, n_sel, nb - 1, gen, cuda)
    tt = torch.full((R, H), nb - 1, dtype=torch.int32, device=cuda)
    tl = torch.tensor([9, 16], dtype=torch.int32, device=cuda)
    im = ops.IMPL_VALU if impl == "valu" else ops.IMPL_AUTO
    out, lse = ops.sparse_attn(q, k, vt, table, nb, B, tail_tile=tt, tail_len=tl, impl=im)
    torch.cuda.synchronize()
    check_attn(out, lse, attn_reference(q, k, vt, table, nb, B, tt, tl), dtype)
    for j in range(3):
        o1, l1 = ops.sparse_attn(q[:, j:j + 1].contiguous(), k, vt, table, nb, B, tail_tile=tt,
                                 tail_len=tl, impl=im)
        assert torch.equal(o1, out[:, j:j + 1]) and torch.equal(l1, lse[:, j:j + 1])


def test_attn_empty_and_custom_scale(cuda):
    say("attn empty units + explicit scale")
    R, H, G, D, B, nb = 2, 2, 4, 128, 16, 10
    gen = synth.generator(77, synth.S_MISC, cuda)
    q = synth.normal((R, 2, H * G, D), gen, cuda, torch.bfloat16)
    k = synth.normal((R, H, nb, B, D), gen, cuda, torch.bfloat16)
    vt = synth.normal((R, H, nb, D, B), gen, cuda, torch.bfloat16)
    table = synth.random_tile_table(R, H, 6, nb, gen, cuda)
    table[1, 0] = -1  # unit (1, 0) attends nothing
    for impl in (ops.IMPL_VALU, ops.IMPL_MFMA):
        out, lse = ops.sparse_attn(q, k, vt, table, nb, B, scale=0.05, impl=impl)
        torch.cuda.synchronize()
        ref = attn_reference(q, k, vt, table, nb, B, scale=0.05)
        check_attn(out, lse, ref, torch.bfloat16)
        assert torch.all(out[1, :, :G] == 0) and torch.all(torch.isneginf(lse[1, :, :G]))
    # n_sel = 0 with only the active block
    e = torch.empty((R, H, 0), dtype=torch.int32, device=cuda)
    tt = torch.full((R, H), 3, dtype=torch.int32, device=cuda)
    tl = torch.tensor([5, 16], dtype=torch.int32, device=cuda)
    out, lse = ops.sparse_attn(q, k, vt, e, nb, B, tail_tile=tt, tail_len=tl)
    torch.cuda.synchronize()
    check_attn(out, lse, attn_reference(q, k, vt, e, nb, B, tt, tl), torch.bfloat16)


@pytest.mark.parametrize("name,units", [("qwen3-8b-1layer", None),
                                        ("llama3.1-8b-32layer", [(0, 0), (17, 3), (31, 7)]),
                                        ("qwen3-235b-1layer", [(2, 1), (7, 3)])])
def test_attn_full_size_on_topk_selection(cuda, name, units):
    """The benchmark's launch configuration: full shape, tiles chosen by the
    kernel's own top-K (row 0), full-cache store (unit_stride = n_blk)."""
    say(f"attn full size {name}")
    wl, k, vt, q = make_layer(synth.workload(name), cuda)
    summ = ops.build_summaries(k, wl.B)
    idx, _, _ = ops.score_topk(q, summ, wl.K)
    table = idx[:, 0].contiguous()
    kt = k.view(wl.R, wl.H, wl.n_blk, wl.B, wl.D)
    out, lse = ops.sparse_attn(q, kt, vt, table, wl.n_blk, wl.B)
    torch.cuda.synchronize()
    if units is None:
        units = [(r, g) for r in range(wl.R) for g in range(wl.H)]
    for r, g in units:
        sl = slice(g * wl.G, (g + 1) * wl.G)
        ref = attn_reference(q[r:r + 1, :, sl].contiguous(), kt[r:r + 1, g:g + 1], vt[r:r + 1, g:g + 1],
                             table[r:r + 1, g:g + 1], wl.n_blk, wl.B)
        check_attn(out[r:r + 1, :, sl], lse[r:r + 1, :, sl], ref, wl.dtype)
