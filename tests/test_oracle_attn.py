"""Pins of the oracle's sparse decode attention.

OasisKV paperpeel v2 text, §3.1 and Fig. 6 (one call, both stacked queries,
one resident working set) and §4.1 (K selected blocks plus the active local
block).  Checked against textbook dense softmax attention (scipy), closed forms
and identities of softmax attention.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _dense(q, k_tok, v_tok, G, scale):
    """Textbook attention: q [R][nq][Hq][D]; k/v per KV head [R][H][T][D]."""
    R, nq, Hq, D = q.shape
    out = np.empty_like(q)
    lse = np.empty((R, nq, Hq))
    for r in range(R):
        for j in range(nq):
            for h in range(Hq):
                z = scale * (k_tok[r, h // G] @ q[r, j, h])
                out[r, j, h] = softmax(z) @ v_tok[r, h // G]
                lse[r, j, h] = logsumexp(z)
    return out, lse


def _case(seed, R=2, nq=2, H=2, G=3, D=16, B=4, nb=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((R, nq, H * G, D))
    k = rng.standard_normal((R, H, nb, B, D))
    v = rng.standard_normal((R, H, nb, B, D))
    return q, k, v


def test_attention_hand_example():
    ex = GOLD["attention"]
    q = np.array(ex["q"], dtype=np.float64).reshape(1, 1, 1, 2)
    kt = np.array(ex["keys"], dtype=np.float64).reshape(1, 2, 2)
    vt = np.array(ex["values"], dtype=np.float64).reshape(1, 2, 2)
    out, lse = oracle.sparse_attn(q, kt, vt, np.zeros((1, 1, 1), np.int32), 1, scale=ex["scale"])
    np.testing.assert_allclose(out[0, 0, 0], ex["expected_out"], rtol=1e-14, atol=1e-14)
    assert abs(lse[0, 0, 0] - ex["expected_lse"]) < 1e-14


@pytest.mark.parametrize("G,B", [(1, 4), (3, 4), (4, 16), (16, 2)])
def test_all_blocks_selected_equals_dense(G, B):
    q, k, v = _case(10 + G, G=G, B=B)
    R, H, nb = k.shape[:3]
    D = q.shape[-1]
    table = np.tile(np.arange(nb, dtype=np.int32), (R, H, 1))
    out, lse = oracle.sparse_attn(q, k.reshape(-1, B, D), v.reshape(-1, B, D), table, nb)
    ref, rl = _dense(q, k.reshape(R, H, nb * B, D), v.reshape(R, H, nb * B, D), G,
                     1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_subset_and_tail_equal_dense_over_those_tokens():
    q, k, v = _case(31, B=4, nb=8)
    R, H, nb, B, D = k.shape
    G = q.shape[2] // H
    rng = np.random.default_rng(5)
    sel = np.stack([[rng.permutation(nb - 1)[:3] for _ in range(H)] for _ in range(R)]).astype(np.int32)
    sel[0, 1, 2] = -1                                   # skipped entry
    tail_tile = np.full((R, H), nb - 1, dtype=np.int32)
    tail_len = np.array([3, 1], dtype=np.int32)
    out, lse = oracle.sparse_attn(q, k.reshape(-1, B, D), v.reshape(-1, B, D), sel, nb,
                                  tail_tile=tail_tile, tail_len=tail_len, scale=0.37)
    for r in range(R):
        for h in range(H):
            ids = [t for t in sel[r, h] if t >= 0]
            kt = np.concatenate([k[r, h, ids].reshape(-1, D), k[r, h, nb - 1, :tail_len[r]]])
            vt = np.concatenate([v[r, h, ids].reshape(-1, D), v[r, h, nb - 1, :tail_len[r]]])
            for j in range(q.shape[1]):
                for hh in range(h * G, (h + 1) * G):
                    z = 0.37 * (kt @ q[r, j, hh])
                    np.testing.assert_allclose(out[r, j, hh], softmax(z) @ vt, rtol=1e-12, atol=1e-12)
                    assert abs(lse[r, j, hh] - logsumexp(z)) < 1e-12


def test_stacked_equals_two_single_calls():
    q, k, v = _case(41)
    R, H, nb, B, D = k.shape
    table = np.stack([[np.random.default_rng(r * 7 + h).permutation(nb)[:4] for h in range(H)]
                      for r in range(R)]).astype(np.int32)
    kt, vt = k.reshape(-1, B, D), v.reshape(-1, B, D)
    both, lb = oracle.sparse_attn(q, kt, vt, table, nb)
    for j in range(2):
        one, l1 = oracle.sparse_attn(q[:, j:j + 1], kt, vt, table, nb)
        np.testing.assert_array_equal(both[:, j:j + 1], one)
        np.testing.assert_array_equal(lb[:, j:j + 1], l1)


def test_tile_order_does_not_matter():
    q, k, v = _case(51)
    R, H, nb, B, D = k.shape
    table = np.tile(np.arange(nb, dtype=np.int32), (R, H, 1))
    perm = table[:, :, ::-1].copy()
    a, la = oracle.sparse_attn(q, k.reshape(-1, B, D), v.reshape(-1, B, D), table, nb)
    b, lb = oracle.sparse_attn(q, k.reshape(-1, B, D), v.reshape(-1, B, D), perm, nb)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-13)


def test_split_and_lse_merge_equals_whole():
    q, k, v = _case(61, nb=8)
    R, H, nb, B, D = k.shape
    table = np.tile(np.arange(nb, dtype=np.int32), (R, H, 1))
    kt, vt = k.reshape(-1, B, D), v.reshape(-1, B, D)
    whole, lw = oracle.sparse_attn(q, kt, vt, table, nb)
    o1, l1 = oracle.sparse_attn(q, kt, vt, table[:, :, :3].copy(), nb)
    o2, l2 = oracle.sparse_attn(q, kt, vt, table[:, :, 3:].copy(), nb)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m + np.log(w1 + w2), lw, rtol=1e-12, atol=1e-12)


def test_closed_forms_single_token_uniform_and_empty():
    rng = np.random.default_rng(71)
    R, H, G, D, B = 1, 1, 2, 8, 4
    q = rng.standard_normal((R, 2, H * G, D))
    k = rng.standard_normal((2, B, D))
    v = rng.standard_normal((2, B, D))
    # a single attended token returns its value exactly, lse = its logit
    out, lse = oracle.sparse_attn(q, k, v, -np.ones((R, H, 1), np.int32), 1,
                                  tail_tile=np.array([[1]], np.int32),
                                  tail_len=np.array([1], np.int32), scale=0.5)
    for j in range(2):
        for h in range(G):
            np.testing.assert_array_equal(out[0, j, h], v[1, 0])
            assert abs(lse[0, j, h] - 0.5 * (q[0, j, h] @ k[1, 0])) < 1e-13
    # identical keys: uniform weights -> mean of the values, lse = z + log n
    ku = np.repeat(k[:1, :1], B, axis=1)
    out, lse = oracle.sparse_attn(q, ku, v[:1], np.zeros((R, H, 1), np.int32), 1, scale=1.0)
    for j in range(2):
        for h in range(G):
            np.testing.assert_allclose(out[0, j, h], v[0].mean(axis=0), rtol=1e-12, atol=1e-14)
            assert abs(lse[0, j, h] - (q[0, j, h] @ k[0, 0] + math.log(B))) < 1e-12
    # nothing attended: zeros and -inf
    out, lse = oracle.sparse_attn(q, k, v, -np.ones((R, H, 2), np.int32), 1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
