"""Pins of the oracle's summaries and block scores to facts fixed by the pages
and by mathematics (not to the oracle's own formulas).

Summaries: OasisKV signal-papers reader text, paragraph on ranking
non-resident blocks; paperpeel v2 text, §4.1 (two summary rows per block,
1/16 of the KV cache at B = 16).  Scores: paperpeel v2 text, §3.1 equation
s_b(alpha), alpha = 1.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _f(x):
    return -np.inf if x == "-inf" else float(x)


def test_summaries_hand_example():
    ex = GOLD["summaries"]
    keys = np.array(ex["keys"], dtype=np.float64)[None, None]  # [1][1][6][3]
    s = oracle.build_summaries(keys, ex["block_size"], seq_len=[ex["seq_len"]])
    np.testing.assert_array_equal(s[0, 0, :2, 0], np.array(ex["expected_min"]))
    np.testing.assert_array_equal(s[0, 0, :2, 1], np.array(ex["expected_max"]))
    # the partial block (token 4) is not summarised
    np.testing.assert_array_equal(s[0, 0, 2], 0.0)


@pytest.mark.parametrize("B", [1, 2, 4, 16])
def test_summaries_bound_and_attained(B):
    rng = np.random.default_rng(7 + B)
    R, H, nb, D = 2, 3, 9, 8
    keys = rng.standard_normal((R, H, nb * B, D))
    s = oracle.build_summaries(keys, B)
    blocks = keys.reshape(R, H, nb, B, D)
    mn, mx = s[:, :, :, 0], s[:, :, :, 1]
    # every key lies inside [min, max] coordinate-wise ...
    assert np.all(blocks >= mn[:, :, :, None, :])
    assert np.all(blocks <= mx[:, :, :, None, :])
    # ... and both bounds are attained by some key of the block (tightness)
    assert np.all(np.any(blocks == mn[:, :, :, None, :], axis=3))
    assert np.all(np.any(blocks == mx[:, :, :, None, :], axis=3))
    if B == 1:
        np.testing.assert_array_equal(mn, blocks[:, :, :, 0])
        np.testing.assert_array_equal(mx, blocks[:, :, :, 0])


def test_summaries_size_is_one_sixteenth_of_kv():
    # v2 §4.1: two summary rows per 16-token block = 1/16 of the K+V cache.
    R, H, B, nb, D = 1, 2, 16, 4, 8
    keys = np.zeros((R, H, nb * B, D))
    s = oracle.build_summaries(keys, B)
    kv_elems = 2 * keys.size
    assert s.size * 16 == kv_elems


def test_summaries_range_and_seq_len():
    rng = np.random.default_rng(3)
    R, H, B, nb, D = 2, 1, 4, 6, 4
    keys = rng.standard_normal((R, H, nb * B, D))
    full = oracle.build_summaries(keys, B)
    seq = np.array([9, 24], dtype=np.int32)  # request 0: 2 full blocks + 1 token
    part = oracle.build_summaries(keys, B, seq_len=seq, blk_begin=1, blk_end=5)
    # request 0: only block 1 is both in range and full
    np.testing.assert_array_equal(part[0, :, 1], full[0, :, 1])
    assert np.all(part[0, :, [0, 2, 3, 4, 5]] == 0)
    np.testing.assert_array_equal(part[1, :, 1:5], full[1, :, 1:5])
    assert np.all(part[1, :, [0, 5]] == 0)


def test_scores_hand_example():
    ex = GOLD["scores"]
    keys = np.array(GOLD["summaries"]["keys"], dtype=np.float64)[None, None]
    s = oracle.build_summaries(keys, 2, seq_len=[5])
    q = np.array(ex["q"], dtype=np.float64)[None, None]  # [1][1][2][3]
    sc = oracle.block_scores(q, s, n_blk=[ex["n_blk"]])
    np.testing.assert_array_equal(sc[0, 0, 0], np.array([_f(x) for x in ex["expected"]]))


def _center_radius_form(q, summ, G):
    """The paper's written form: sum_h (q_h . c_b + |q_h| . r_b), c = (max+min)/2,
    r = (max-min)/2 (paperpeel v2 §3.1, alpha = 1)."""
    R, nq, Hq, D = q.shape
    H = Hq // G
    c = 0.5 * (summ[:, :, :, 1] + summ[:, :, :, 0])
    rad = 0.5 * (summ[:, :, :, 1] - summ[:, :, :, 0])
    qg = q.reshape(R, nq, H, G, D)
    return (np.einsum("rjhgd,rhbd->rjhb", qg, c) + np.einsum("rjhgd,rhbd->rjhb", np.abs(qg), rad))


@pytest.mark.parametrize("G,B", [(1, 4), (2, 16), (4, 8), (16, 2)])
def test_scores_equal_center_radius_form(G, B):
    rng = np.random.default_rng(100 + G * B)
    R, H, nb, D, nq = 2, 2, 7, 16, 2
    keys = rng.standard_normal((R, H, nb * B, D))
    q = rng.standard_normal((R, nq, H * G, D))
    summ = oracle.build_summaries(keys, B)
    got = oracle.block_scores(q, summ)
    ref = _center_radius_form(q, summ, G)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G,B", [(1, 16), (4, 16), (16, 4)])
def test_scores_upper_bound_brute_force(G, B):
    rng = np.random.default_rng(200 + G)
    R, H, nb, D, nq = 2, 2, 11, 8, 2
    keys = rng.standard_normal((R, H, nb * B, D))
    q = rng.standard_normal((R, nq, H * G, D))
    summ = oracle.build_summaries(keys, B)
    sc = oracle.block_scores(q, summ)
    qsum = q.reshape(R, nq, H, G, D).sum(axis=3)           # sum of the group's queries
    dots = np.einsum("rjhd,rhld->rjhl", qsum, keys)         # every key
    best = dots.reshape(R, nq, H, nb, B).max(axis=-1)
    assert np.all(sc >= best - 1e-12 * (1 + np.abs(best)))


def test_scores_tight_for_single_key_blocks_and_constant_blocks():
    rng = np.random.default_rng(5)
    R, H, G, D, nq = 1, 2, 4, 8, 2
    q = rng.standard_normal((R, nq, H * G, D))
    qsum = q.reshape(R, nq, H, G, D).sum(axis=3)
    # B = 1: the bound is the exact dot product
    keys = rng.standard_normal((R, H, 5, D))
    sc = oracle.block_scores(q, oracle.build_summaries(keys, 1))
    np.testing.assert_allclose(sc, np.einsum("rjhd,rhld->rjhl", qsum, keys), rtol=1e-12, atol=1e-12)
    # every key of a block identical: the bound is that key's dot product
    k1 = rng.standard_normal((R, H, 3, D))
    keys = np.repeat(k1, 4, axis=2)
    sc = oracle.block_scores(q, oracle.build_summaries(keys, 4))
    np.testing.assert_allclose(sc, np.einsum("rjhd,rhld->rjhl", qsum, k1), rtol=1e-12, atol=1e-12)


def test_scores_group_mapping_is_contiguous():
    # query head h reads KV head h // G: zeroing KV head 1's group zeroes only its scores.
    rng = np.random.default_rng(9)
    R, H, G, D, B, nb = 1, 2, 3, 4, 2, 3
    keys = rng.standard_normal((R, H, nb * B, D))
    q = rng.standard_normal((R, 1, H * G, D))
    q[:, :, G:2 * G] = 0.0
    sc = oracle.block_scores(q, oracle.build_summaries(keys, B))
    assert np.all(sc[0, 0, 1] == 0.0)
    assert np.all(sc[0, 0, 0] != 0.0)


def test_scores_past_n_blk_are_minus_inf():
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((2, 1, 40, 4))
    summ = oracle.build_summaries(keys, 4)
    q = rng.standard_normal((2, 2, 1, 4))
    sc = oracle.block_scores(q, summ, n_blk=[3, 10])
    assert np.all(np.isneginf(sc[0, :, :, 3:]))
    assert np.all(np.isfinite(sc[0, :, :, :3]))
    assert np.all(np.isfinite(sc[1]))


# ---------------------------------------------------------------- token append
def test_append_fills_blocks_and_builds_their_summaries():
    """Appending a context token by token writes each token in place, leaves a
    block's summary alone until its last token arrives, then sets it to the
    coordinate-wise min / max of the block's keys (numpy's reductions)."""
    rng = np.random.default_rng(21)
    R, H, D, B, nb = 2, 3, 8, 4, 5
    keys = np.zeros((R, H, nb * B, D))
    vals = np.zeros((R, H, nb * B, D))
    summ = np.full((R, H, nb, 2, D), 7.0)
    L = np.array([3, 9], np.int32)  # tokens already present
    keys[:, :, :12] = rng.standard_normal((R, H, 12, D))
    for _ in range(9):
        kn, vn = rng.standard_normal((R, H, D)), rng.standard_normal((R, H, D))
        pos = L.copy()
        pos[1] = -1 if _ % 4 == 3 else pos[1]  # request 1 skips some steps
        before = summ.copy()
        keys, vals, summ = oracle.append_kv(keys, vals, kn, vn, pos, B, summ)
        for r in range(R):
            if pos[r] < 0:
                np.testing.assert_array_equal(summ[r], before[r])
                continue
            np.testing.assert_array_equal(keys[r, :, pos[r]], kn[r])
            np.testing.assert_array_equal(vals[r, :, pos[r]], vn[r])
            b = pos[r] // B
            if pos[r] % B == B - 1:
                blk = keys[r, :, b * B:(b + 1) * B]
                np.testing.assert_array_equal(summ[r, :, b, 0], blk.min(axis=1))
                np.testing.assert_array_equal(summ[r, :, b, 1], blk.max(axis=1))
            else:
                np.testing.assert_array_equal(summ[r, :, b], before[r, :, b])
            L[r] += 1


def test_append_without_summaries_and_bad_position():
    keys = np.zeros((1, 1, 8, 2))
    k, v, s = oracle.append_kv(keys, keys, np.ones((1, 1, 2)), np.full((1, 1, 2), 2.0),
                               np.array([3], np.int32), 4)
    assert s is None and k[0, 0, 3].tolist() == [1.0, 1.0] and v[0, 0, 3].tolist() == [2.0, 2.0]
    with pytest.raises(ValueError):
        oracle.append_kv(keys, keys, np.ones((1, 1, 2)), np.ones((1, 1, 2)),
                         np.array([8], np.int32), 4)


# ---------------------------------------------------------------- scoring variants
def _variant_inputs(seed, G=4, B=8, nq=2):
    rng = np.random.default_rng(seed)
    R, H, nb, D = 2, 2, 9, 16
    keys = rng.standard_normal((R, H, nb * B, D))
    summ = oracle.build_summaries(keys, B)
    q = rng.standard_normal((R, nq, H * G, D))
    return keys, summ, q, G, B


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.5, 2.0])
def test_scores_alpha_is_affine_between_centre_and_bound(alpha):
    """s(alpha) = s(0) + alpha * (s(1) - s(0)), with s(1) from the max form and
    s(0) = sum_h q_h . c (numpy): OasisKV v2 text, 3.1, equation s_b(alpha)."""
    _, summ, q, G, _ = _variant_inputs(31)
    R, nq, Hq, D = q.shape
    H = summ.shape[1]
    s1 = oracle.block_scores(q, summ)
    centre = (summ[:, :, :, 0] + summ[:, :, :, 1]) / 2
    s0 = np.einsum("rjhd,rhbd->rjhb", q.reshape(R, nq, H, G, D).sum(axis=3), centre)
    np.testing.assert_allclose(oracle.block_scores(q, summ, alpha=0.0), s0, rtol=1e-12, atol=1e-12)
    got = oracle.block_scores(q, summ, alpha=alpha)
    np.testing.assert_allclose(got, s0 + alpha * (s1 - s0), rtol=1e-11, atol=1e-11)


def test_scores_alpha_above_one_still_bounds_every_key():
    keys, summ, q, G, B = _variant_inputs(32)
    R, nq, Hq, D = q.shape
    H, nb = summ.shape[1], summ.shape[2]
    best = np.einsum("rjhd,rhld->rjhl", q.reshape(R, nq, H, G, D).sum(axis=3), keys)
    best = best.reshape(R, nq, H, nb, B).max(axis=-1)
    assert np.all(oracle.block_scores(q, summ, alpha=1.5) >= best - 1e-12 * (1 + np.abs(best)))


@pytest.mark.parametrize("alpha", [1.0, 0.4])
def test_scores_draft_average_equals_scoring_the_mean_query(alpha):
    """Two drafts averaged before scoring (v2 text, 4.2.3) = scoring the row
    [normal, (draft a + draft b) / 2] formed in numpy."""
    _, summ, q3, G, _ = _variant_inputs(33, nq=3)
    got = oracle.block_scores(q3, summ, alpha=alpha, draft_avg=True)
    mean = np.stack([q3[:, 0], (q3[:, 1] + q3[:, 2]) / 2], axis=1)
    ref = oracle.block_scores(mean, summ, alpha=alpha)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert got.shape[1] == 2


def test_scores_centre_form_is_linear_in_the_query():
    """At alpha = 0 the averaged-draft score is the mean of the two drafts' scores."""
    _, summ, q3, _, _ = _variant_inputs(34, nq=3)
    avg = oracle.block_scores(q3, summ, alpha=0.0, draft_avg=True)[:, 1]
    each = oracle.block_scores(q3, summ, alpha=0.0)
    np.testing.assert_allclose(avg, (each[:, 1] + each[:, 2]) / 2, rtol=1e-12, atol=1e-12)
