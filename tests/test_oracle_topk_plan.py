"""Pins of the oracle's top-K, capped least-recently-selected plan and block
copy.

Top-K: OasisKV paperpeel v2 text, §3.3.1; signal-papers reader text (per-KV-head
ranking of all logical blocks).  Plan: reader text, capped-eviction paragraph;
v2 §3.3.2 (cap applies after seeding; exactly K resident blocks per head).
Worked example: v2 §3.2.2 and Fig. 7 (head-wise block mapping).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _f(x):
    return -np.inf if x == "-inf" else float(x)


# ---------------------------------------------------------------- top-K
def test_topk_hand_example():
    ex = GOLD["topk"]
    s = np.array(ex["scores"], dtype=np.float64)[None, None, None]
    for case in ex["cases"]:
        idx, val = oracle.topk(s, case["k"])
        assert idx[0, 0, 0].tolist() == case["expected_idx"]
        np.testing.assert_array_equal(val[0, 0, 0], [_f(x) for x in case["expected_score"]])


@pytest.mark.parametrize("n,k,levels", [(64, 8, 0), (100, 16, 5), (37, 50, 3), (2048, 128, 40)])
def test_topk_equals_full_sort(n, k, levels):
    rng = np.random.default_rng(n + k)
    R, nq, H = 2, 2, 3
    s = rng.standard_normal((R, nq, H, n))
    if levels:  # heavy ties
        s = np.round(s * levels) / levels
    n_blk = np.array([n, max(1, n // 2)], dtype=np.int32)
    idx, val = oracle.topk(s, k, n_blk=n_blk)
    for r in range(R):
        for j in range(nq):
            for h in range(H):
                nr = int(n_blk[r])
                order = sorted(range(nr), key=lambda b: (-s[r, j, h, b], b))[:k]
                want = order + [-1] * (k - len(order))
                assert idx[r, j, h].tolist() == want
                wv = [s[r, j, h, b] for b in order] + [-np.inf] * (k - len(order))
                np.testing.assert_array_equal(val[r, j, h], wv)


# ---------------------------------------------------------------- plan
def _plan_one(P, blk, stamp, step, cap, ins=None):
    R, H, K = 1, 1, len(blk)
    t = np.array(P, dtype=np.int32).reshape(1, 1, 1, K)
    return oracle.select_plan(t, np.array(blk, dtype=np.int32).reshape(R, H, K),
                              np.array(stamp, dtype=np.int32).reshape(R, H, K), step, cap,
                              pred_row=0,
                              ins_blk=None if ins is None else np.array([ins], np.int32))


def test_plan_hand_sequence():
    ex = GOLD["plan_sequence"]
    K, cap = ex["K"], ex["cap"]
    blk, stamp = [-1] * K, [-1] * K
    for st in ex["steps"]:
        out = _plan_one(st["P"], blk, stamp, st["step"], cap)
        assert int(out["plan_count"][0, 0]) == st["count"], st["derivation"]
        assert out["plan_src"][0, 0].tolist() == st["src"]
        assert out["plan_dst"][0, 0].tolist() == st["dst"]
        assert out["plan_evicted"][0, 0].tolist() == st["evicted"]
        assert out["slot_block"][0, 0].tolist() == st["slot_block"]
        assert out["slot_stamp"][0, 0].tolist() == st["slot_stamp"]
        blk, stamp = st["slot_block"], st["slot_stamp"]


@pytest.mark.parametrize("name", ["plan_partial_seed", "plan_short_prediction"])
def test_plan_hand_cases(name):
    ex = GOLD[name]
    out = _plan_one(ex["P"], ex["slot_block"], ex["slot_stamp"], ex["step"], ex["cap"])
    assert int(out["plan_count"][0, 0]) == ex["count"]
    if "src" in ex:
        assert out["plan_src"][0, 0].tolist() == ex["src"]
        assert out["plan_dst"][0, 0].tolist() == ex["dst"]
    assert out["slot_block"][0, 0].tolist() == ex["expected_block"]
    assert out["slot_stamp"][0, 0].tolist() == ex["expected_stamp"]


@pytest.mark.parametrize("name", ["plan_insert_basic", "plan_insert_resident",
                                  "plan_insert_over_admission"])
def test_plan_insert_hand_cases(name):
    ex = GOLD[name]
    out = _plan_one(ex["P"], ex["slot_block"], ex["slot_stamp"], ex["step"], ex["cap"], ex["ins"])
    assert int(out["plan_count"][0, 0]) == ex["count"], ex["derivation"]
    assert out["plan_src"][0, 0].tolist() == ex["src"]
    assert out["plan_dst"][0, 0].tolist() == ex["dst"]
    assert out["plan_evicted"][0, 0].tolist() == ex["evicted"]
    assert out["slot_block"][0, 0].tolist() == ex["expected_block"]
    assert out["slot_stamp"][0, 0].tolist() == ex["expected_stamp"]


def test_plan_insert_none_is_the_plain_plan():
    for step, topk, blk, stamp in _random_history(9, 8, 30, 2, steps=6, churn=0.3):
        pr = 0 if step == 0 else 1
        a = oracle.select_plan(topk, blk, stamp, step, 2, pred_row=pr)
        b = oracle.select_plan(topk, blk, stamp, step, 2, pred_row=pr,
                               ins_blk=-np.ones(topk.shape[0], np.int32))
        for k in a:
            np.testing.assert_array_equal(a[k], b[k])


def _set_based_insert(pairs, blk, stamp, step, ins):
    """The new block after the plan, written with lists: refresh if resident,
    else take the oldest (stamp, slot); an entry that admitted into that slot
    is taken over."""
    blk, stamp, pairs = list(blk), list(stamp), list(pairs)
    if ins in blk:
        stamp[blk.index(ins)] = step
        return pairs, blk, stamp
    v = min(range(len(blk)), key=lambda s: (stamp[s], s))
    hit = [i for i, p in enumerate(pairs) if p[1] == v]
    if hit:
        i = hit[0]
        pairs[i] = (ins, v, pairs[i][2])
    else:
        pairs.append((ins, v, blk[v]))
    blk[v] = ins
    stamp[v] = step
    return pairs, blk, stamp


@pytest.mark.parametrize("seed,K,n_blocks,cap", [(11, 8, 20, 2), (12, 16, 64, 4), (13, 4, 6, 1),
                                                  (14, 32, 200, 16), (15, 4, 50, 0)])
def test_plan_insert_matches_set_formulation_and_invariants(seed, K, n_blocks, cap):
    rng = np.random.default_rng(seed)
    for step, topk, blk, stamp in _random_history(seed, K, n_blocks, cap, steps=10, churn=0.3):
        pred_row = 0 if step == 0 else 1
        R, _, H, _ = topk.shape
        # a fresh block id per request (beyond every scored block), some requests without
        ins = np.where(rng.random(R) < 0.7, n_blocks + step * R + np.arange(R), -1).astype(np.int32)
        if step % 3 == 2:  # an already resident block now and then
            ins[0] = blk[0, 0, 0]
        out = oracle.select_plan(topk, blk, stamp, step, cap, pred_row=pred_row, ins_blk=ins)
        for r in range(R):
            for h in range(H):
                P = topk[r, pred_row, h].tolist()
                b0, s0 = blk[r, h].tolist(), stamp[r, h].tolist()
                pairs, nb, ns = _set_based_plan(P, b0, s0, step, cap)
                if ins[r] >= 0:
                    pairs, nb, ns = _set_based_insert(pairs, nb, ns, step, int(ins[r]))
                n = int(out["plan_count"][r, h])
                got = list(zip(out["plan_src"][r, h, :n].tolist(), out["plan_dst"][r, h, :n].tolist(),
                               out["plan_evicted"][r, h, :n].tolist()))
                assert got == pairs
                assert out["slot_block"][r, h].tolist() == nb
                assert out["slot_stamp"][r, h].tolist() == ns
                new = nb
                live = [b for b in new if b >= 0]
                assert len(live) == len(set(live)), "duplicate resident block"
                if ins[r] >= 0:
                    assert int(ins[r]) in new
                    seeding = any(b == -1 for b in b0)
                    if not seeding:
                        assert n <= cap + 1
                assert all(x == -1 for x in out["plan_src"][r, h, n:].tolist())


def _set_based_plan(P, blk, stamp, step, cap):
    """Independent formulation with Python sets: which blocks stay, which go."""
    pred = [p for p in P if p >= 0]
    pset = set(pred)
    resident = {b: s for s, b in enumerate(blk) if b >= 0}
    seeding = any(b == -1 for b in blk)
    new_stamp = list(stamp)
    for b, s in resident.items():
        if b in pset:
            new_stamp[s] = step
    need = [p for p in pred if p not in resident]
    free = sorted((stamp[s], s) for s in range(len(blk)) if blk[s] not in pset)
    n = min(len(need), len(free))
    if not seeding:
        n = min(n, cap)
    new_blk = list(blk)
    pairs = []
    for i in range(n):
        s = free[i][1]
        pairs.append((need[i], s, blk[s]))
        new_blk[s] = need[i]
        new_stamp[s] = step
    return pairs, new_blk, new_stamp


def _random_history(seed, K, n_blocks, cap, steps, churn):
    rng = np.random.default_rng(seed)
    R, H = 2, 3
    blk = -np.ones((R, H, K), dtype=np.int32)
    stamp = -np.ones((R, H, K), dtype=np.int32)
    base = [[list(rng.permutation(n_blocks)[:K]) for _ in range(H)] for _ in range(R)]
    for step in range(steps):
        topk = -np.ones((R, 2, H, K), dtype=np.int32)
        for r in range(R):
            for h in range(H):
                cur = base[r][h]
                for i in range(len(cur)):  # drift: replace some entries
                    if rng.random() < churn:
                        cand = int(rng.integers(n_blocks))
                        if cand not in cur:
                            cur[i] = cand
                kk = min(K, n_blocks) if rng.random() > 0.1 else max(1, K // 2)
                row = list(rng.permutation(cur)[:kk])
                topk[r, 1, h, :len(row)] = row
                topk[r, 0, h, :len(row)] = row
        yield step, topk, blk, stamp
        out = oracle.select_plan(topk, blk, stamp, step, cap, pred_row=0 if step == 0 else 1)
        blk, stamp = out["slot_block"], out["slot_stamp"]


@pytest.mark.parametrize("seed,K,n_blocks,cap", [(1, 8, 20, 2), (2, 16, 64, 4), (3, 8, 8, 1),
                                                  (4, 32, 200, 16), (5, 4, 50, 0)])
def test_plan_matches_set_formulation_and_invariants(seed, K, n_blocks, cap):
    for step, topk, blk, stamp in _random_history(seed, K, n_blocks, cap, steps=12, churn=0.3):
        pred_row = 0 if step == 0 else 1
        out = oracle.select_plan(topk, blk, stamp, step, cap, pred_row=pred_row)
        R, _, H, _ = topk.shape
        for r in range(R):
            for h in range(H):
                P = topk[r, pred_row, h].tolist()
                b0, s0 = blk[r, h].tolist(), stamp[r, h].tolist()
                pairs, nb, ns = _set_based_plan(P, b0, s0, step, cap)
                n = int(out["plan_count"][r, h])
                assert n == len(pairs)
                got = list(zip(out["plan_src"][r, h, :n].tolist(), out["plan_dst"][r, h, :n].tolist(),
                               out["plan_evicted"][r, h, :n].tolist()))
                assert got == pairs
                assert out["slot_block"][r, h].tolist() == nb
                assert out["slot_stamp"][r, h].tolist() == ns
                # invariants
                new = out["slot_block"][r, h].tolist()
                live = [b for b in new if b >= 0]
                assert len(live) == len(set(live)), "duplicate resident block"
                pset = {p for p in P if p >= 0}
                seeding = any(b == -1 for b in b0)
                if not seeding:
                    assert n <= cap
                if pset <= set(b0):
                    assert n == 0
                assert len(pset & set(new)) >= len(pset & set(b0))
                for e in out["plan_evicted"][r, h, :n].tolist():
                    assert e not in pset
                if cap >= K or seeding:
                    assert pset <= set(new)
                assert all(x == -1 for x in out["plan_src"][r, h, n:].tolist())


def test_plan_fig7_headwise_mapping_and_copy():
    # v2 §3.2.2 / Fig. 7: tokens A..H in blocks of B = 2 -> (A,B)=0, (C,D)=1,
    # (E,F)=2, (G,H)=3.  Head 0 selects (A,B), head 1 selects (G,H); GPU logical
    # block 0 then holds a different source block for each head, and the gather
    # places (A,B) under head 0 and (G,H) under head 1.
    R, H, K, nb, B, D = 1, 2, 1, 4, 2, 1
    topk = np.array([[[[0], [3]]]], dtype=np.int32)  # [R][n_q=1][H][K]
    out = oracle.select_plan(topk, -np.ones((R, H, K), np.int32), -np.ones((R, H, K), np.int32),
                             0, 0, pred_row=0)
    assert out["plan_count"].tolist() == [[1, 1]]
    assert out["plan_src"][0, :, 0].tolist() == [0, 3]
    assert out["plan_dst"][0, :, 0].tolist() == [0, 0]
    letters = np.frombuffer(b"ABCDEFGH", dtype=np.uint8)
    # per-head stores hold the same tokens; head 1's entries are lowercase
    host_k = np.stack([letters, letters + 32]).reshape(R, H, nb, B * D)
    host_v = host_k.copy()
    res_k = np.zeros((R, H, K, B * D), np.uint8)
    rk, rv = oracle.copy_blocks(host_k, host_v, res_k, res_k, out["plan_count"], out["plan_src"],
                                out["plan_dst"])
    assert bytes(rk[0, 0, 0]) == b"AB" and bytes(rk[0, 1, 0]) == b"gh"
    assert bytes(rv[0, 0, 0]) == b"AB" and bytes(rv[0, 1, 0]) == b"gh"


def test_copy_moves_exactly_the_planned_tiles():
    rng = np.random.default_rng(21)
    R, H, nb, K, tb = 2, 3, 10, 4, 12
    host_k = rng.integers(0, 255, (R, H, nb, tb), dtype=np.uint8)
    host_v = rng.integers(0, 255, (R, H, nb, tb), dtype=np.uint8)
    res_k = rng.integers(0, 255, (R, H, K, tb), dtype=np.uint8)
    res_v = rng.integers(0, 255, (R, H, K, tb), dtype=np.uint8)
    cnt = rng.integers(0, K + 1, (R, H)).astype(np.int32)
    src = np.stack([[rng.permutation(nb)[:K] for _ in range(H)] for _ in range(R)]).astype(np.int32)
    dst = np.stack([[rng.permutation(K) for _ in range(H)] for _ in range(R)]).astype(np.int32)
    rk, rv = oracle.copy_blocks(host_k, host_v, res_k, res_v, cnt, src, dst)
    ek, ev = res_k.copy(), res_v.copy()
    for r in range(R):
        for h in range(H):
            n = cnt[r, h]
            ek[r, h, dst[r, h, :n]] = host_k[r, h, src[r, h, :n]]
            ev[r, h, dst[r, h, :n]] = host_v[r, h, src[r, h, :n]]
    np.testing.assert_array_equal(rk, ek)
    np.testing.assert_array_equal(rv, ev)
