"""Pins of the sparse (top-k) oracle against facts that do not re-type it:
the pinned dense decode (a full in-order list is a dense request, a list cut
at the causal edge is a causal row), brute force, closed forms for repeated
and empty lists, and invariance under reordering and padding."""

import math

import numpy as np
import pytest

import oracle
from oracle.brute import brute_attention
from oracle.sparse import reference_sparse_decode

from helpers import build_paged, random_dense


def _flat_tokens(prob, b):
    """Flat token index (page * page_size + slot) of request b's rows, in order."""
    L = int(prob.seq_lens[b])
    ps = prob.page_size
    t = np.arange(L)
    return prob.block_tables[b, t // ps].astype(np.int64) * ps + t % ps


def _sparse(prob, idx, sinks=None):
    return reference_sparse_decode(prob.q_bits, prob.kv_bits, prob.kv_dtype, idx, prob.bmm1_scale, prob.bmm2_scale,
                                   sinks=sinks)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_full_list_is_the_dense_request(kv_dtype):
    """Listing every row of the request, in order, is the dense decode."""
    rng = np.random.default_rng(40)
    H = 16
    q, ks = random_dense(rng, 2, H, [2, 3], [70, 129], kv_dtype=kv_dtype)
    prob = build_paged(q, ks, 32, rng=rng, q_lens=[2, 3], packed=True, bmm1=0.08, bmm2=1.3, causal=False,
                       kv_dtype=kv_dtype)
    full_o, full_l = oracle.reference_decode(prob)
    K = 160
    idx = np.full((5, K), -1, dtype=np.int32)
    for b, rows in ((0, range(0, 2)), (1, range(2, 5))):
        tok = _flat_tokens(prob, b)
        for r in rows:
            idx[r, :tok.size] = tok
    o, l = _sparse(prob, idx)
    np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, full_l, rtol=1e-12, atol=1e-13)


def test_list_cut_at_the_causal_edge_is_the_causal_row():
    rng = np.random.default_rng(41)
    H = 16
    q, ks = random_dense(rng, 1, H, [4], [45])
    prob = build_paged(q, ks, 16, rng=rng, q_lens=[4], packed=True, bmm1=0.1, causal=True)
    ref_o, ref_l = oracle.reference_decode(prob)
    tok = _flat_tokens(prob, 0)
    idx = np.full((4, 64), -1, dtype=np.int32)
    for i in range(4):
        n = oracle.visible_count(45, 4, i, True)
        idx[i, :n] = tok[:n]
    o, l = _sparse(prob, idx)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, ref_l, rtol=1e-12, atol=1e-13)


def test_order_and_padding_do_not_matter():
    rng = np.random.default_rng(42)
    H = 16
    q, ks = random_dense(rng, 1, H, [2], [300])
    prob = build_paged(q, ks, 64, rng=rng, q_lens=[2], bmm1=0.07, causal=False)
    tok = _flat_tokens(prob, 0)
    pick = np.stack([rng.choice(300, 90, replace=False) for _ in range(2)])
    idx = tok[pick].astype(np.int32)
    o1, l1 = _sparse(prob, idx)
    # shuffle each row and scatter -1 entries among the real ones
    idx2 = np.full((2, 130), -1, dtype=np.int32)
    for r in range(2):
        slots = np.sort(rng.choice(130, 90, replace=False))
        idx2[r, slots] = rng.permutation(idx[r])
    o2, l2 = _sparse(prob, idx2)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


def test_brute_force_on_a_selection():
    """Pure-Python loops over the selected rows (as a dense request of them)."""
    rng = np.random.default_rng(43)
    H = 16
    q, ks = random_dense(rng, 1, H, [1], [50])
    prob = build_paged(q, ks, 16, rng=rng, q_lens=[1], bmm1=0.09, bmm2=0.6, causal=False)
    tok = _flat_tokens(prob, 0)
    sel = np.array([49, 3, 17, 17, 0, 31], dtype=np.int64)  # one row listed twice
    idx = np.concatenate([tok[sel], [-1, -1]]).astype(np.int32)[None, :]
    o, l = _sparse(prob, idx)
    bo, bl = brute_attention([[list(q[0, h]) for h in range(H)]], [list(ks[0][j]) for j in sel], 0.09, 0.6, False)
    np.testing.assert_allclose(o[0], np.array(bo[0]), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l[0], np.array(bl[0]), rtol=1e-11, atol=1e-13)


def test_one_row_listed_m_times():
    """out = bmm2 * V and lse = s + ln m for a single row listed m times."""
    rng = np.random.default_rng(44)
    H = 16
    q, ks = random_dense(rng, 1, H, [1], [20])
    prob = build_paged(q, ks, 16, rng=rng, q_lens=[1], bmm1=0.2, bmm2=1.7, causal=False)
    tok = _flat_tokens(prob, 0)
    for m in (1, 3, 33):
        idx = np.full((1, 40), -1, dtype=np.int32)
        idx[0, :m] = tok[7]
        o, l = _sparse(prob, idx)
        for h in range(H):
            s = 0.2 * float(q[0, h] @ ks[0][7])
            np.testing.assert_allclose(o[0, h], 1.7 * ks[0][7, :512], rtol=1e-12, atol=1e-300)
            assert abs(l[0, h] - (s + math.log(m))) < 1e-12


def test_empty_list():
    rng = np.random.default_rng(45)
    H = 16
    q, ks = random_dense(rng, 1, H, [2], [20])
    prob = build_paged(q, ks, 16, rng=rng, q_lens=[2], bmm1=0.2, causal=False)
    tok = _flat_tokens(prob, 0)
    idx = np.full((2, 8), -1, dtype=np.int32)
    idx[1, 0] = tok[4]
    o, l = _sparse(prob, idx)
    assert np.all(o[0] == 0.0) and np.all(l[0] == -np.inf)
    assert np.all(np.isfinite(l[1]))
    sinks = rng.uniform(-2, 2, H)
    o, l = _sparse(prob, idx, sinks=sinks)
    assert np.all(o[0] == 0.0)
    np.testing.assert_array_equal(l[0], sinks)


def test_sinks_match_the_dense_definition():
    rng = np.random.default_rng(46)
    H = 16
    q, ks = random_dense(rng, 1, H, [2], [77])
    prob = build_paged(q, ks, 32, rng=rng, q_lens=[2], bmm1=0.1, causal=False)
    sinks = rng.uniform(-3, 5, H)
    prob.sinks = sinks
    ref_o, ref_l = oracle.reference_decode(prob)
    tok = _flat_tokens(prob, 0)
    idx = np.tile(tok.astype(np.int32), (2, 1))
    o, l = _sparse(prob, idx, sinks=sinks)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, ref_l, rtol=1e-12, atol=1e-13)
