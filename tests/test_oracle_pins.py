"""Pins of the float64 oracle to facts other than itself (CPU only).

Each test ties the oracle to something it does not share code with: the
formats' bit definitions vs torch's casts, closed forms that follow from the
pages' definition (seq_len 1, equal logits, one-hot values, scale linearity),
brute-force loops on dense un-paged keys, torch's own scaled-dot-product
attention with a bottom-right causal bias, and invariants (page permutation,
split + LSE merge, dense rows = single-row decodes, causal row = truncated
decode, fixed = packed).  test_mutants_are_caught plants plausible mistakes in
the oracle and checks that these pins catch every one.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla as oracle_mla
from oracle.brute import brute_attention
from oracle.formats import bf16_bits_to_f64, e4m3fn_bits_to_f64, e4m3fn_table

from helpers import bf16_round, build_paged, random_dense, e4m3_round

TIGHT = dict(rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- formats

def test_e4m3fn_table_matches_torch_all_codes():
    ours = e4m3fn_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    assert np.array_equal(ours[~np.isnan(ours)], theirs[~np.isnan(theirs)])
    # Format facts: max finite 448, min subnormal 2^-9, NaN only at 0x7F / 0xFF.
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert ours[1] == 2.0 ** -9
    assert set(np.flatnonzero(np.isnan(ours)).tolist()) == {0x7F, 0xFF}


def test_bf16_decode_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(codes)
    theirs = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    m = ~np.isnan(ours)
    assert np.array_equal(ours[m], theirs[m])


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_seq_len_one_gives_scaled_value_row(kv_dtype):
    """L = 1, q = 1: out = bmm2 * V[0] and lse = bmm1 * q.k0, exactly."""
    rng = np.random.default_rng(11)
    H = 16
    q, ks = random_dense(rng, 3, H, [1, 1, 1], [1, 1, 1], kv_dtype=kv_dtype)
    prob = build_paged(q, ks, 32, rng=rng, bmm1=0.37, bmm2=1.75, kv_dtype=kv_dtype)
    out, lse = oracle.reference_decode(prob)
    for b in range(3):
        np.testing.assert_allclose(out[b], np.broadcast_to(1.75 * ks[b][0, :512], (H, 512)), **TIGHT)
        np.testing.assert_allclose(lse[b], 0.37 * (q[b] @ ks[b][0]), **TIGHT)


@pytest.mark.parametrize("causal", [True, False])
def test_equal_logits_give_mean_of_values(causal):
    """Latent query part zero and one shared RoPE key part: every logit is the same
    s, so out = bmm2 * mean of the visible V rows and lse = s + ln(n)."""
    rng = np.random.default_rng(12)
    H, B = 16, 2
    q_lens, L = [3, 2], [45, 70]
    q, ks = random_dense(rng, B, H, q_lens, L)
    q[..., :512] = 0.0
    rope = bf16_round(rng.standard_normal(64).astype(np.float32))
    for k in ks:
        k[:, 512:] = rope
    prob = build_paged(q, ks, 32, rng=rng, q_lens=q_lens, bmm1=0.21, bmm2=0.5, causal=causal)
    out, lse = oracle.reference_decode(prob)
    r = 0
    for b in range(B):
        for i in range(q_lens[b]):
            n = L[b] - q_lens[b] + i + 1 if causal else L[b]
            mean_v = ks[b][:n, :512].mean(axis=0)
            for h in range(H):
                s = 0.21 * float(q[r, h, 512:] @ rope)
                np.testing.assert_allclose(out[r, h], 0.5 * mean_v, rtol=1e-12, atol=1e-14)
                assert abs(lse[r, h] - (s + math.log(n))) < 1e-12
            r += 1


def test_one_hot_values_reveal_visible_rows():
    """V rows one-hot (row j -> e_j) with equal logits: out[i, h, c] = bmm2*[c < n_i]/n_i,
    which spells out exactly which rows row i saw (bottom-right aligned)."""
    rng = np.random.default_rng(13)
    H = 16
    for L, ql in [(5, 5), (37, 4), (100, 8), (64, 1)]:
        q = bf16_round(rng.standard_normal((ql, H, 576)).astype(np.float32))
        q[..., :512] = 0.0
        k = np.zeros((L, 576))
        k[np.arange(L), np.arange(L)] = 1.0
        k[:, 512:] = bf16_round(rng.standard_normal(64).astype(np.float32))
        prob = build_paged(q, [k], 32, rng=rng, q_lens=[ql], bmm1=0.3, bmm2=2.0, causal=True)
        out, lse = oracle.reference_decode(prob)
        for i in range(ql):
            visible = np.flatnonzero(out[i, 0] > 0)
            # row i attends through KV row L - q + i inclusive
            assert visible.tolist() == list(range(L - ql + i + 1))
            np.testing.assert_allclose(out[i, :, :L - ql + i + 1], 2.0 / (L - ql + i + 1), rtol=1e-12)


def test_scale_linearity_and_zero_bmm1():
    rng = np.random.default_rng(14)
    H = 32
    q, ks = random_dense(rng, 2, H, [2, 2], [50, 33])
    p1 = build_paged(q, ks, 32, rng=np.random.default_rng(1), bmm1=0.2, bmm2=1.0)
    p3 = build_paged(q, ks, 32, rng=np.random.default_rng(1), bmm1=0.2, bmm2=3.0)
    o1, l1 = oracle.reference_decode(p1)
    o3, l3 = oracle.reference_decode(p3)
    np.testing.assert_allclose(o3, 3.0 * o1, **TIGHT)
    np.testing.assert_array_equal(l1, l3)  # LSE excludes bmm2
    p0 = build_paged(q, ks, 32, rng=np.random.default_rng(1), bmm1=0.0, bmm2=1.0)
    o0, l0 = oracle.reference_decode(p0)
    for b, (ql, L) in enumerate([(2, 50), (2, 33)]):
        for i in range(ql):
            n = L - ql + i + 1
            np.testing.assert_allclose(o0[2 * b + i], np.broadcast_to(ks[b][:n, :512].mean(0), (H, 512)), **TIGHT)
            np.testing.assert_allclose(l0[2 * b + i], math.log(n), **TIGHT)


# ---------------------------------------------------------------- attention sinks

def _with_sinks(prob, sinks):
    import dataclasses
    return dataclasses.replace(prob, sinks=np.asarray(sinks, dtype=np.float64))


def test_sink_seq_len_one_is_a_logistic_gate():
    """L = 1 with a sink: the one real key competes with the sink alone, so
    out = bmm2 * V[0] * e^s / (e^s + e^sink) and lse = ln(e^s + e^sink)."""
    rng = np.random.default_rng(21)
    H = 16
    q, ks = random_dense(rng, 2, H, [1, 1], [1, 1])
    prob = build_paged(q, ks, 32, rng=rng, bmm1=0.3, bmm2=1.5)
    sinks = rng.normal(0.0, 2.0, size=H)
    sinks[0], sinks[1] = 40.0, -40.0  # a dominating sink and a negligible one
    out, lse = oracle.reference_decode(_with_sinks(prob, sinks))
    for b in range(2):
        for h in range(H):
            s = 0.3 * float(q[b, h] @ ks[b][0])
            gate = 1.0 / (1.0 + math.exp(sinks[h] - s))
            np.testing.assert_allclose(out[b, h], 1.5 * gate * ks[b][0, :512], rtol=1e-12, atol=1e-300)
            assert abs(lse[b, h] - np.logaddexp(s, sinks[h])) < 1e-12


def test_sink_with_equal_logits():
    """Equal logits s over n visible rows plus a sink: out = bmm2 * mean(V) *
    n e^s / (n e^s + e^sink), lse = ln(n e^s + e^sink)."""
    rng = np.random.default_rng(22)
    H = 16
    q_lens, L = [3], [70]
    q, ks = random_dense(rng, 1, H, q_lens, L)
    q[..., :512] = 0.0
    rope = bf16_round(rng.standard_normal(64).astype(np.float32))
    ks[0][:, 512:] = rope
    prob = build_paged(q, ks, 32, rng=rng, q_lens=q_lens, bmm1=0.21, bmm2=0.5, causal=True)
    sinks = rng.normal(1.0, 3.0, size=H)
    out, lse = oracle.reference_decode(_with_sinks(prob, sinks))
    for i in range(3):
        n = 70 - 3 + i + 1
        mean_v = ks[0][:n, :512].mean(axis=0)
        for h in range(H):
            s = 0.21 * float(q[i, h, 512:] @ rope)
            frac = n * math.exp(s) / (n * math.exp(s) + math.exp(sinks[h]))
            np.testing.assert_allclose(out[i, h], 0.5 * frac * mean_v, rtol=1e-12, atol=1e-14)
            assert abs(lse[i, h] - np.logaddexp(s + math.log(n), sinks[h])) < 1e-12


def test_sink_is_a_zero_value_partial():
    """Merging the sink-free decode's (O, lse) with one more partial (O = 0,
    lse = sink) reproduces the decode with the sink; a sink at -inf changes
    nothing, bit for bit."""
    rng = np.random.default_rng(23)
    H = 32
    q, ks = random_dense(rng, 2, H, [2, 2], [90, 41])
    prob = build_paged(q, ks, 32, rng=rng, bmm1=0.09, bmm2=1.25, causal=True)
    sinks = rng.normal(0.0, 2.0, size=H)
    o0, l0 = oracle.reference_decode(prob)
    o1, l1 = oracle.reference_decode(_with_sinks(prob, sinks))
    sink_rows = np.tile(sinks, (4, 1))
    mo, ml = oracle.merge_partials([(o0 / 1.25, l0), (np.zeros_like(o0), sink_rows)], 1.25)
    np.testing.assert_allclose(mo, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, l1, rtol=1e-12, atol=1e-13)
    o2, l2 = oracle.reference_decode(_with_sinks(prob, np.full(H, -np.inf)))
    assert np.array_equal(o2, o0) and np.array_equal(l2, l0)


# ---------------------------------------------------------------- brute force / library

@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    rng = np.random.default_rng(15)
    H = 2
    q_lens, L = [2, 1, 3], [5, 9, 3]
    # Small D would not exercise the 576 layout; loops stay cheap at these sizes.
    q, ks = random_dense(rng, 3, H, q_lens, L)
    prob = build_paged(q, ks, 4, rng=rng, q_lens=q_lens, bmm1=0.05, bmm2=1.3, causal=causal)
    out, lse = oracle.reference_decode(prob)
    r = 0
    for b in range(3):
        bo, bl = brute_attention(q[r:r + q_lens[b]].tolist(), ks[b].tolist(), 0.05, 1.3, causal)
        np.testing.assert_allclose(out[r:r + q_lens[b]], np.array(bo), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[r:r + q_lens[b]], np.array(bl), rtol=1e-12, atol=1e-13)
        r += q_lens[b]


def test_matches_torch_sdpa_lower_right_causal():
    from torch.nn.attention.bias import causal_lower_right
    rng = np.random.default_rng(16)
    H = 16
    q_lens, L = [4, 1, 8, 3], [70, 33, 8, 129]
    q, ks = random_dense(rng, 4, H, q_lens, L)
    prob = build_paged(q, ks, 32, rng=rng, q_lens=q_lens, bmm1=1 / math.sqrt(192), bmm2=0.8, causal=True)
    out, lse = oracle.reference_decode(prob)
    r = 0
    for b in range(4):
        qt = torch.from_numpy(q[r:r + q_lens[b]]).permute(1, 0, 2).unsqueeze(0)  # [1, H, q, 576]
        kt = torch.from_numpy(ks[b]).expand(1, H, L[b], 576)
        vt = torch.from_numpy(np.ascontiguousarray(ks[b][:, :512])).expand(1, H, L[b], 512)
        bias = causal_lower_right(q_lens[b], L[b])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias,
                                                               scale=1 / math.sqrt(192))
        ref = ref[0].permute(1, 0, 2).numpy() * 0.8
        np.testing.assert_allclose(out[r:r + q_lens[b]], ref, rtol=1e-10, atol=1e-12)
        # LSE from the library's logits: logsumexp over the lower-right-causal visible set
        logits = torch.from_numpy(q[r:r + q_lens[b]]).reshape(-1, 576) @ torch.from_numpy(ks[b]).T / math.sqrt(192)
        logits = logits.reshape(q_lens[b], H, L[b])
        mask = bias._materialize("cpu").reshape(q_lens[b], 1, L[b])
        lib_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
        np.testing.assert_allclose(lse[r:r + q_lens[b]], lib_lse, rtol=1e-11, atol=1e-11)
        r += q_lens[b]


# ---------------------------------------------------------------- invariants

def test_page_permutation_invariance_is_bitwise():
    rng = np.random.default_rng(17)
    q, ks = random_dense(rng, 3, 16, [2, 2, 2], [77, 64, 5])
    pa = build_paged(q, ks, 32, rng=np.random.default_rng(100), bmm1=0.1)
    pb = build_paged(q, ks, 32, rng=np.random.default_rng(200), bmm1=0.1)
    assert not np.array_equal(pa.block_tables, pb.block_tables)
    oa, la = oracle.reference_decode(pa)
    ob, lb = oracle.reference_decode(pb)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_split_merge_reproduces_full():
    rng = np.random.default_rng(18)
    H = 16
    for causal, ql in [(False, 3), (True, 1), (True, 4)]:
        q, ks = random_dense(rng, 1, H, [ql], [203])
        prob = build_paged(q, ks, 32, rng=rng, q_lens=[ql], bmm1=0.07, bmm2=1.6, causal=causal)
        full_o, full_l = oracle.reference_decode(prob)
        for cuts in ([0, 64, 203], [0, 1, 203], [0, 37, 101, 150, 203], [0, 200, 203]):
            parts = [oracle.reference_partial(prob, 0, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
            mo, ml = oracle.merge_partials(parts, 1.6)
            np.testing.assert_allclose(mo, full_o[:ql], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(ml, full_l[:ql], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("world", [2, 3, 8])
def test_dcp_partials_merge_to_the_full_decode(world):
    """Round-robin sequence shards: each rank's partial over its own rows,
    merged by LSE weight, reproduces the unsharded decode; ranks that hold
    no visible row of some query row report lse = -inf and out = 0."""
    rng = np.random.default_rng(24)
    H = 16
    for causal, q_lens, L in [(True, [4, 1], [5, 123]), (False, [2, 3], [7, 64]), (True, [3, 3], [3, 40])]:
        q, ks = random_dense(rng, 2, H, q_lens, L)
        prob = build_paged(q, ks, 32, rng=rng, q_lens=q_lens, packed=True, bmm1=0.11, bmm2=1.3, causal=causal)
        full_o, full_l = oracle.reference_decode(prob)
        parts = [oracle.reference_dcp_partial(prob, r, world) for r in range(world)]
        mo, ml = oracle.merge_partials(parts, 1.0)
        np.testing.assert_allclose(mo, full_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ml, full_l, rtol=1e-12, atol=1e-13)
        # a rank with no visible row: the first request's first row sees L - q + 1 global rows
        n0 = L[0] - q_lens[0] + 1 if causal else L[0]
        for r in range(world):
            if r >= n0:
                assert np.all(parts[r][1][0] == -np.inf) and np.all(parts[r][0][0] == 0.0)


@pytest.mark.parametrize("world", [2, 5])
def test_dcp_sinks_ride_on_rank_zero(world):
    """With sinks, rank 0's partial carries them and the merge counts each
    sink once, reproducing the unsharded decode with sinks; a rank-0 row that
    sees none of its own rows reports out = 0 and lse = sink."""
    rng = np.random.default_rng(26)
    H = 16
    sinks = rng.uniform(-3.0, 6.0, H)
    q, ks = random_dense(rng, 2, H, [3, 1], [3, 77])
    prob = build_paged(q, ks, 32, rng=rng, q_lens=[3, 1], packed=True, bmm1=0.09, bmm2=1.2, causal=True)
    prob.sinks = sinks
    full_o, full_l = oracle.reference_decode(prob)
    parts = [oracle.reference_dcp_partial(prob, r, world) for r in range(world)]
    mo, ml = oracle.merge_partials(parts, 1.0)
    np.testing.assert_allclose(mo, full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, full_l, rtol=1e-12, atol=1e-13)
    for r in range(1, world):
        # the other ranks are the sink-free partials
        prob.sinks = None
        o_r, l_r = oracle.reference_dcp_partial(prob, r, world)
        prob.sinks = sinks
        np.testing.assert_array_equal(parts[r][1], l_r)
        np.testing.assert_array_equal(parts[r][0], o_r)


def test_dcp_sink_closed_forms():
    """q = 3, L = 3, causal, two ranks: row i sees global positions 0..i;
    rank 0 holds positions 0 and 2, rank 1 holds position 1.  Rank 0's row 0
    is a logistic gate between position 0 and the sink; rank 1's row 0 has
    nothing (out = 0, lse = -inf); rank 1's row 1 is position 1 alone."""
    rng = np.random.default_rng(27)
    H = 16
    sinks = rng.uniform(-2.0, 2.0, H)
    q, ks = random_dense(rng, 1, H, [3], [3])
    prob = build_paged(q, ks, 32, rng=rng, q_lens=[3], packed=True, bmm1=0.1, bmm2=0.8, causal=True)
    prob.sinks = sinks
    o0, l0 = oracle.reference_dcp_partial(prob, 0, 2)
    o1, l1 = oracle.reference_dcp_partial(prob, 1, 2)
    K = ks[0]
    for h in range(H):
        s00 = 0.1 * float(q[0, h] @ K[0])
        gate = 1.0 / (1.0 + math.exp(sinks[h] - s00))
        np.testing.assert_allclose(o0[0, h], 0.8 * gate * K[0, :512], rtol=1e-12, atol=1e-300)
        assert abs(l0[0, h] - np.logaddexp(s00, sinks[h])) < 1e-12
        assert l1[0, h] == -np.inf and np.all(o1[0, h] == 0.0)
        s11 = 0.1 * float(q[1, h] @ K[1])
        np.testing.assert_allclose(o1[1, h], 0.8 * K[1, :512], rtol=1e-12, atol=1e-300)
        assert abs(l1[1, h] - s11) < 1e-12


def test_dcp_single_rank_is_the_full_decode():
    rng = np.random.default_rng(25)
    q, ks = random_dense(rng, 2, 16, [2, 2], [33, 80])
    prob = build_paged(q, ks, 32, rng=rng, bmm1=0.2, bmm2=0.7, causal=True)
    o, l = oracle.reference_decode(prob)
    o1, l1 = oracle.reference_dcp_partial(prob, 0, 1)
    np.testing.assert_allclose(o1, o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l, rtol=1e-13, atol=1e-15)


def test_dense_rows_equal_single_row_decodes():
    """A dense multi-row request equals each of its rows run as its own q=1 request
    over the same cache (the flattening vLLM uses for non-causal blocks)."""
    rng = np.random.default_rng(19)
    H = 16
    q, ks = random_dense(rng, 2, H, [3, 2], [40, 90])
    packed = build_paged(q, ks, 32, rng=np.random.default_rng(5), q_lens=[3, 2], causal=False, bmm1=0.1)
    flat = build_paged(q, [ks[0]] * 3 + [ks[1]] * 2, 32, rng=np.random.default_rng(6), q_lens=[1] * 5,
                       causal=False, bmm1=0.1)
    o1, l1 = oracle.reference_decode(packed)
    o2, l2 = oracle.reference_decode(flat)
    np.testing.assert_allclose(o1, o2, **TIGHT)
    np.testing.assert_allclose(l1, l2, **TIGHT)


def test_causal_row_equals_truncated_decode():
    rng = np.random.default_rng(20)
    H = 16
    ql, L = 5, 83
    q, ks = random_dense(rng, 1, H, [ql], [L])
    prob = build_paged(q, ks, 32, rng=rng, q_lens=[ql], causal=True, bmm1=0.09)
    o, l = oracle.reference_decode(prob)
    for i in range(ql):
        n = L - ql + i + 1
        single = build_paged(q[i:i + 1], [ks[0][:n]], 32, rng=rng, q_lens=[1], causal=False, bmm1=0.09)
        so, sl = oracle.reference_decode(single)
        np.testing.assert_allclose(o[i], so[0], **TIGHT)
        np.testing.assert_allclose(l[i], sl[0], **TIGHT)


def test_fixed_equals_packed():
    rng = np.random.default_rng(21)
    q, ks = random_dense(rng, 3, 16, [2, 2, 2], [10, 50, 99])
    fixed = build_paged(q, ks, 32, rng=np.random.default_rng(3), q_lens=[2, 2, 2], bmm1=0.1)
    packed = build_paged(q, ks, 32, rng=np.random.default_rng(3), q_lens=[2, 2, 2], packed=True, bmm1=0.1)
    assert fixed.qo_indptr is None and packed.qo_indptr is not None
    o1, l1 = oracle.reference_decode(fixed)
    o2, l2 = oracle.reference_decode(packed)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_nan_in_unread_slots_never_leaks():
    """Tail slots past seq_len and the padding page are NaN; the output is finite."""
    rng = np.random.default_rng(22)
    q, ks = random_dense(rng, 2, 16, [1, 1], [33, 7])
    prob = build_paged(q, ks, 32, rng=rng, bmm1=0.1, extra_width=3)
    o, l = oracle.reference_decode(prob)
    assert np.isfinite(o).all() and np.isfinite(l).all()


# ---------------------------------------------------------------- mutation check

def _pins_catch(monkeypatch, attr, mutant):
    monkeypatch.setattr(oracle_mla, attr, mutant)
    caught = 0
    for t in (test_brute_force_tiny, test_matches_torch_sdpa_lower_right_causal,
              test_seq_len_one_gives_scaled_value_row):
        try:
            if t is test_brute_force_tiny:
                t(True)
            elif t is test_seq_len_one_gives_scaled_value_row:
                t("bf16")
            else:
                t()
        except AssertionError:
            caught += 1
    monkeypatch.undo()
    return caught


def test_mutants_are_caught(monkeypatch):
    """Plant plausible oracle mistakes on the CPU; each must break a pin."""
    real_vis = oracle_mla.visible_count
    assert _pins_catch(monkeypatch, "visible_count", lambda L, q, i, c: real_vis(L, q, i, c) - 1 if c else L) > 0
    assert _pins_catch(monkeypatch, "visible_count", lambda L, q, i, c: (i + 1) if c else L) > 0
    real_decode = oracle_mla.bf16_bits_to_f64

    def drop_rope(bits):  # query loses its RoPE part
        x = real_decode(bits)
        if x.ndim == 3 and x.shape[-1] == 576:
            x = x.copy()
            x[..., 512:] = 0
        return x
    assert _pins_catch(monkeypatch, "bf16_bits_to_f64", drop_rope) > 0
    real_gather = oracle_mla.gather_request_rows

    def reversed_rows(problem, b):  # token order lost in the gather
        return real_gather(problem, b)[::-1]
    assert _pins_catch(monkeypatch, "gather_request_rows", reversed_rows) > 0


# ---------------------------------------------------------------- fp8 query

def test_fp8_query_is_the_same_decode_of_its_values():
    """Every E4M3FN value is exactly a bf16 value, so a problem whose query is
    given as fp8 codes equals the same problem with those values as bf16
    codes (the pinned bf16-query definition), bitwise in float64."""
    import dataclasses
    from helpers import to_bf16_bits, to_e4m3_bits, e4m3_round
    rng = np.random.default_rng(30)
    H = 16
    q, ks = random_dense(rng, 2, H, [2, 1], [60, 9], kv_dtype="fp8_e4m3fn")
    q8 = e4m3_round(q * 3.0)  # spread over the fp8 range, subnormals included
    q8[0, 0, :8] = [448.0, -448.0, 2.0 ** -9, -(2.0 ** -9), 0.0, 1.5, -0.1015625, 240.0]
    prob = build_paged(q8, ks, 32, rng=rng, q_lens=[2, 1], packed=True, bmm1=0.01, bmm2=0.5, causal=True,
                       kv_dtype="fp8_e4m3fn")
    assert np.array_equal(oracle.bf16_bits_to_f64(prob.q_bits), q8)  # bf16 holds the fp8 values exactly
    prob8 = dataclasses.replace(prob, q_bits=to_e4m3_bits(q8), q_dtype="fp8_e4m3fn")
    o, l = oracle.reference_decode(prob)
    o8, l8 = oracle.reference_decode(prob8)
    np.testing.assert_array_equal(o8, o)
    np.testing.assert_array_equal(l8, l)
    # and the codes do reach the logits: a different query gives a different result
    prob8b = dataclasses.replace(prob8, q_bits=to_e4m3_bits(q8 * 0.5))
    assert not np.allclose(oracle.reference_decode(prob8b)[1], l)
