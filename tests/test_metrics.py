"""The roofline's algorithmic work (paged_mla_decode_03_amd/metrics.py)
against a direct count over the visible (row, key) pairs of small inputs."""

import numpy as np

from paged_mla_decode_03_amd.metrics import workload_counts, sparse_counts, mixed_mfma_peak


def _brute(seq_lens, q_lens, H, ps, kv_bytes, causal, lse, packed):
    visible = 0
    for L, q in zip(seq_lens, q_lens):
        for i in range(q):
            visible += (L - q + i + 1) if causal else L
    R = sum(q_lens)
    nbytes = (sum(seq_lens) * 576 * kv_bytes + R * H * 576 * 2 + R * H * 512 * 2 + (R * H * 4 if lse else 0)
              + 4 * sum(-(-L // ps) for L in seq_lens) + 4 * len(seq_lens) + (4 * (len(seq_lens) + 1) if packed else 0))
    return visible, nbytes, 2 * 1088 * H * visible


def test_paged_counts_match_a_direct_count():
    rng = np.random.default_rng(0)
    for _ in range(50):
        B = int(rng.integers(1, 9))
        L = rng.integers(1, 500, B)
        causal = bool(rng.random() < 0.5)
        q = np.minimum(rng.integers(1, 6, B), L) if causal else rng.integers(1, 6, B)
        H, ps = int(rng.choice([16, 128])), int(rng.choice([16, 32, 64]))
        kvb, lse, packed = int(rng.choice([1, 2])), bool(rng.random() < 0.5), bool(rng.random() < 0.5)
        c = workload_counts(L, q, H, ps, kvb, causal, lse, packed)
        vis, nbytes, flops = _brute(L.tolist(), q.tolist(), H, ps, kvb, causal, lse, packed)
        assert c["visible_pairs_per_head"] == vis
        assert c["bytes"] == nbytes and c["flops"] == flops and c["kv_tokens"] == int(L.sum())


def test_sparse_counts_match_a_direct_count():
    lists = np.array([[3, -1, 7, 7], [-1, -1, -1, -1], [0, 1, 2, 9]], dtype=np.int32)
    c = sparse_counts(lists, 3, 16, 2, True)  # only the first 3 entries of each list count
    live = 2 + 0 + 3
    assert c["kv_tokens"] == live
    assert c["flops"] == 2 * 1088 * 16 * live
    assert c["bytes"] == live * 1152 + 3 * 16 * 1152 + 3 * 16 * 1024 + 3 * 16 * 4 + 4 * 3 * 3


def test_mixed_peak_is_the_harmonic_combination():
    # QK^T (576 of 1088 dims) at 5.0 PF/s, P.V at 2.5 PF/s
    t = (576 / 1088) / 5000.0 + (512 / 1088) / 2500.0
    assert abs(mixed_mfma_peak() - 1.0 / t) < 1e-9
    assert 2500.0 < mixed_mfma_peak() < 5000.0
