"""GPU checks at the limits: the largest batch, degenerate lengths, a head
count that leaves a unit partly filled, cache offsets past 4 GiB, and the
sparse layout at its row limit."""

import numpy as np
import pytest
import torch

import oracle
from oracle.sparse import reference_sparse_decode
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, sparse_lists, to_device_tensors, INV_SQRT_192

from gpu_cases import check_close, compare_with_oracle, run_hip

pytestmark = pytest.mark.gpu

MAX_BATCH = 1024  # MLA_MAX_BATCH in include/mla_decode.h


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def test_largest_batch():
    """1024 requests (four per plan thread), short ragged lengths, every request."""
    w = make_workload("maxb", seed=90, batch=MAX_BATCH, seq_len_range=(1, 40), num_heads=16, q_len=1, page_size=16,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    compare_with_oracle(w)


def test_largest_batch_grouped():
    """1024 requests of 2 rows x 128 heads: every request holds two units, so
    the plan groups workgroups in pairs, over the largest batch."""
    w = make_workload("maxb_g", seed=97, batch=MAX_BATCH, seq_len_range=(2, 60), num_heads=128, q_len=2,
                      page_size=16, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    compare_with_oracle(w)


def test_every_request_one_row():
    """seq_len 1 everywhere: out = bmm2 * V[0] and lse = bmm1 * q.k[0] per (row, head)."""
    w = make_workload("len1", seed=91, seq_lens=[1] * 37, num_heads=32, q_len=1, page_size=32,
                      bmm1_scale=0.05, bmm2_scale=1.5, causal=True, want_lse=True)
    compare_with_oracle(w)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_causal_query_as_long_as_the_cache(kv_dtype):
    """q_len = L: the first query row sees exactly one key."""
    w = make_workload("qeqL", seed=92, seq_lens=[3, 8, 17], num_heads=64, q_len=3, page_size=16, kv_dtype=kv_dtype,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    compare_with_oracle(w)
    w2 = make_workload("qeqL8", seed=93, seq_lens=[8, 8], num_heads=16, q_len=8, page_size=32, kv_dtype=kv_dtype,
                       bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    compare_with_oracle(w2)


def test_head_count_leaving_a_unit_partly_filled():
    """H = 192 at q = 1: the second 128-pair unit holds 64 pairs."""
    w = make_workload("h192", seed=94, seq_len_range=(50, 700), batch=5, num_heads=192, q_len=1, page_size=64,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    compare_with_oracle(w)


def test_cache_offsets_past_4_gib():
    """The same pages placed after 4.5 GiB of other cache give bitwise the same
    result: page offsets are 64-bit."""
    w = make_workload("far", seed=95, seq_lens=[300, 1000, 77], num_heads=128, q_len=2, page_size=64,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    o_near, l_near = run_hip(w)
    page_bytes = w.page_size * 576 * 2
    shift = (9 << 29) // page_bytes + 3  # pages before ours: > 4.5 GiB
    P = w.kv_bits.shape[0]
    big = torch.empty((shift + P, w.page_size, 576), dtype=torch.bfloat16, device="cuda")
    big[:shift].fill_(float("nan"))
    big[shift:] = torch.from_numpy(w.kv_bits).view(torch.bfloat16).cuda()
    t = to_device_tensors(w, "cuda")
    bt = (t["block_tables"] + shift).contiguous()
    q = t["q"].view(w.batch, w.q_len_fixed, w.num_heads, 576)
    ws = torch.empty(binding.workspace_bytes_for(q, big, bt, t["seq_lens"], w.max_seq_len, return_lse=True),
                     dtype=torch.uint8, device="cuda")
    o, l = binding.decode(q, big, ws, bt, t["seq_lens"], w.max_seq_len, return_lse=True, bmm1_scale=w.bmm1_scale,
                          causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().reshape(o_near.shape).cpu().numpy(), o_near)
    assert np.array_equal(l.reshape(l_near.shape).cpu().numpy(), l_near)
    del big
    torch.cuda.empty_cache()


def test_sparse_at_the_row_limit():
    """1024 query rows in the sparse layout, top-k 64, sampled rows."""
    w = make_workload("sp_max", seed=96, batch=MAX_BATCH, seq_len_range=(20, 200), num_heads=16, q_len=1,
                      page_size=16, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    idx = sparse_lists(w, 64, seed=97, empty_frac=0.1, empty_rows=(5,))
    kv = torch.from_numpy(w.kv_bits).view(torch.bfloat16).cuda()
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda()
    it = torch.from_numpy(idx).cuda()
    ws = torch.empty(binding.sparse_workspace_bytes_for(q, kv, it, return_lse=True), dtype=torch.uint8, device="cuda")
    o, l = binding.decode_sparse(q, kv, ws, it, return_lse=True, bmm1_scale=w.bmm1_scale)
    torch.cuda.synchronize()
    rows = [0, 5, 511, 1023]
    ref_o, ref_l = reference_sparse_decode(w.q_bits[rows], w.kv_bits, w.kv_dtype, idx[rows], w.bmm1_scale, 1.0)
    got_o, got_l = o.float().cpu().numpy()[rows], l.cpu().numpy()[rows]
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty) and np.all(got_o[empty] == 0.0)
    check_close(got_o[~empty], ref_o[~empty], "sparse max rows out")
    check_close(got_l[~empty], ref_l[~empty], "sparse max rows lse")
