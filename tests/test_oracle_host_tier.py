"""Pins of the decode-host block cache reference model (oracle.HostTierModel):
a hand-derived sequence and invariants over random histories."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def test_host_tier_hand_sequence():
    ex = GOLD["host_tier_sequence"]
    m = oracle.HostTierModel([ex["capacity"]], ex["n_blk"])
    for st in ex["steps"]:
        sb = np.array([st["slot_block"]], np.int32)
        if st["op"] == "fetch":
            got = m.fetch(st["step"], np.array([st["plan_count"]], np.int32),
                          np.array([st["plan_src"]], np.int32), sb)
            assert [[b, s] for _, b, s in got] == st["fetched"], st["derivation"]
            assert m.last[0] == st["last"]
        else:
            m.trim([st["target"]], sb)
        assert m.slot_blk[0] == st["slot_blk"], st["derivation"]
        for s, b in enumerate(m.slot_blk[0]):
            if b >= 0:
                assert m.map[0, b] == s
        assert int((m.map[0] >= 0).sum()) == sum(1 for b in m.slot_blk[0] if b >= 0)


def _history(seed, R, H, K, n_blk, steps):
    rng = np.random.default_rng(seed)
    work = np.stack([[rng.permutation(n_blk)[:K] for _ in range(H)] for _ in range(R)])
    for step in range(1, steps + 1):
        cnt = rng.integers(0, min(3, K) + 1, (R, H)).astype(np.int32)
        src = -np.ones((R, H, K), np.int32)
        for r in range(R):
            for g in range(H):
                for i in range(cnt[r, g]):
                    nb = int(rng.integers(n_blk))
                    while nb in work[r, g]:
                        nb = int(rng.integers(n_blk))
                    src[r, g, i] = nb
                    work[r, g, rng.integers(K)] = nb
        yield step, cnt, src, work.astype(np.int32).copy()


@pytest.mark.parametrize("seed,R,H,K,n_blk,cap", [(1, 2, 2, 4, 40, 14), (2, 3, 4, 3, 30, 16),
                                                  (3, 1, 8, 2, 64, 20)])
def test_host_tier_invariants(seed, R, H, K, n_blk, cap):
    rng = np.random.default_rng(seed + 100)
    remote = rng.integers(0, 255, (R, n_blk, 32), dtype=np.uint8)
    m = oracle.HostTierModel([cap] * R, n_blk, remote)
    for step, cnt, src, work in _history(seed, R, H, K, n_blk, 30):
        absent = {}
        for r in range(R):
            union = []
            for g in range(H):
                for i in range(cnt[r, g]):
                    if src[r, g, i] not in union:
                        union.append(int(src[r, g, i]))
            absent[r] = [b for b in union if m.map[r, b] < 0]
        before = [list(x) for x in m.slot_blk]
        last_before = [list(x) for x in m.last]
        got = m.fetch(step, cnt, src, work)
        for r in range(R):
            # least recently used first: every evicted block was used no later
            # than every evictable block that stayed
            union_r = {int(src[r, g, i]) for g in range(H) for i in range(cnt[r, g])}
            keep = {int(x) for x in work[r].ravel()} | union_r | m.generated[r]
            after = set(m.slot_blk[r])
            ev_last = [last_before[r][s] for s, b in enumerate(before[r])
                       if b >= 0 and b not in after]
            stay_last = [last_before[r][s] for s, b in enumerate(before[r])
                         if b >= 0 and b in after and b not in keep]
            if ev_last and stay_last:
                assert max(ev_last) <= min(stay_last)
            # exactly the absent blocks are fetched, in union order
            assert [b for rr, b, _ in got if rr == r] == absent[r]
            protected = {int(x) for x in work[r].ravel()}
            for s, b in enumerate(before[r]):
                if b >= 0 and b in protected:
                    assert m.slot_blk[r][s] == b, "a protected block was evicted"
            assert sum(1 for b in m.slot_blk[r] if b >= 0) <= cap
            for g in range(H):
                for i in range(cnt[r, g]):
                    b = int(src[r, g, i])
                    assert m.map[r, b] >= 0 and m.last[r][m.map[r, b]] == step
            for s, b in enumerate(m.slot_blk[r]):
                if b >= 0:
                    assert m.map[r, b] == s
                    np.testing.assert_array_equal(m.cache[r][s], remote[r, b])
            assert int((m.map[r] >= 0).sum()) == sum(1 for b in m.slot_blk[r] if b >= 0)
        if step % 7 == 0:
            m.trim([cap // 2] * R, work)
            for r in range(R):
                protected = {int(x) for x in work[r].ravel()}
                live = [b for b in m.slot_blk[r] if b >= 0]
                assert len(live) <= max(cap // 2, len(protected & set(live)))


def test_host_tier_generated_blocks_are_never_evicted():
    m = oracle.HostTierModel([3], 20)
    empty = -np.ones((1, 1, 1), np.int32)
    m.add_generated(0, 19, 1, empty)
    for step, b in enumerate([1, 2, 3, 4, 5], start=2):
        m.fetch(step, np.array([[1]], np.int32), np.array([[[b]]], np.int32), empty)
        assert 19 in m.slot_blk[0]
    assert m.slot_blk[0].count(-1) == 0


def test_host_tier_budget_too_small_fails():
    m = oracle.HostTierModel([2], 10)
    work = np.array([[[1, 2]]], np.int32)
    m.fetch(1, np.array([[2]], np.int32), np.array([[[1, 2]]], np.int32), work)
    with pytest.raises(RuntimeError):
        m.fetch(2, np.array([[1]], np.int32), np.array([[[3, -1]]], np.int32),
                np.array([[[1, 2]]], np.int32))
