"""The native decode-host block cache (oasis_host_tier_*, CPU code) against the
reference model oracle.HostTierModel over random histories: same fetches,
evictions, slot contents, union map, last-use stamps and cache bytes."""
import numpy as np
import pytest

import oracle
from sparse_kv_block_quest_amd import ops
from test_oracle_host_tier import _history


def _tier(R, H, K, n_blk, cap, nbytes, seed, workers=1):
    rng = np.random.default_rng(seed)
    remote = rng.integers(0, 255, (R, n_blk, nbytes), dtype=np.uint8)
    cache = np.full((R, max(cap), nbytes), 0xA5, np.uint8)
    map_ = np.zeros((R, n_blk), np.int32)
    tier = ops.HostTier(R, H, K, n_blk, cap, remote, cache, map_, nbytes, workers=workers)
    assert not cache.any()  # create zeroes the cache
    model = oracle.HostTierModel(cap, n_blk, remote)
    return tier, model, remote, cache, map_


def _same(tier, model, cache, map_):
    sb, last, stats = tier.state()
    for r in range(model.R):
        c = model.cap[r]
        assert sb[r, :c].tolist() == model.slot_blk[r]
        assert last[r, :c].tolist() == model.last[r]
        for s, b in enumerate(model.slot_blk[r]):
            if b >= 0:
                np.testing.assert_array_equal(cache[r, s], model.cache[r][s])
    np.testing.assert_array_equal(map_, model.map)
    assert stats["fetched"] == model.fetched and stats["evicted"] == model.evicted
    assert stats["failed"] == 0


@pytest.mark.parametrize("workers", [1, 2, 5])
@pytest.mark.parametrize("seed,R,H,K,n_blk,cap", [(1, 2, 2, 4, 40, [14, 11]), (2, 3, 4, 3, 30, [16, 16, 14]),
                                                  (3, 1, 8, 2, 64, [20]),
                                                  (4, 5, 2, 3, 24, [12, 13, 14, 12, 12])])
def test_native_tier_matches_model(seed, R, H, K, n_blk, cap, workers):
    """Requests split over `workers` host threads (more threads than requests
    included) give the single-threaded model's state exactly."""
    tier, model, remote, cache, map_ = _tier(R, H, K, n_blk, cap, 48, seed, workers)
    _same(tier, model, cache, map_)  # empty
    for step, cnt, src, work in _history(seed, R, H, K, n_blk, 30):
        got = model.fetch(step, cnt, src, work)
        assert tier.fetch(step, cnt, src, work) == 0
        _same(tier, model, cache, map_)
        if step == 5:
            for r in range(R):
                nb = n_blk - 1 - r
                if model.map[r, nb] < 0:
                    model.add_generated(r, nb, step, work)
                    assert tier.add_generated(r, nb, step, work) == 0
            _same(tier, model, cache, map_)
        if step % 9 == 0:
            target = [c // 2 for c in cap]
            model.trim(target, work)
            tier.trim(target, work)
            _same(tier, model, cache, map_)
        assert got is not None
    tier.close()


def test_native_tier_budget_too_small_reports_failure():
    tier, model, remote, cache, map_ = _tier(1, 1, 2, 10, [2], 16, 7)
    work = np.array([[[1, 2]]], np.int32)
    assert tier.fetch(1, np.array([[2]], np.int32), np.array([[[1, 2]]], np.int32), work) == 0
    rc = tier.fetch(2, np.array([[1]], np.int32), np.array([[[3, -1]]], np.int32), work)
    assert rc == -1
    assert tier.state()[2]["failed"] == 1
    assert map_[0, 3] == -1  # nothing half-done


def test_native_tier_worker_count_change_keeps_state_and_counts():
    R, H, K, n_blk, cap = 4, 2, 3, 24, [12, 13, 14, 12]
    tier, model, remote, cache, map_ = _tier(R, H, K, n_blk, cap, 32, 11)
    for i, (step, cnt, src, work) in enumerate(_history(11, R, H, K, n_blk, 24)):
        if i in (6, 13, 19):
            tier.set_workers({6: 3, 13: 1, 19: 4}[i])
        model.fetch(step, cnt, src, work)
        assert tier.fetch(step, cnt, src, work) == 0
        _same(tier, model, cache, map_)
    st = tier.state()[2]
    assert st["fetch_ns"] > 0
    tier.close()


def test_native_tier_rejects_bad_worker_counts():
    tier, model, remote, cache, map_ = _tier(1, 1, 2, 10, [5], 8, 3)
    for n in (0, -1, 65):
        with pytest.raises(RuntimeError):
            tier.set_workers(n)
    tier.set_workers(64)
    tier.close()


def test_native_tier_rejects_bad_arguments():
    with pytest.raises(ValueError):
        ops.HostTier(1, 1, 2, 10, [5], np.zeros((1, 10, 8), np.uint8), np.zeros((1, 4, 8), np.uint8),
                     np.zeros((1, 10), np.int32), 8)  # capacity above cap_max
