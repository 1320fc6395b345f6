"""GPU parity of the fp8-query path (QK^T on the fp8 matrix cores) against the
float64 oracle given the same E4M3FN query codes: fixed and packed queries,
causal and dense, page sizes 16/32/64, forced splits, LSE, sinks, a query
scale folded into bmm1, and unscaled logits that force reference restarts."""

import numpy as np
import pytest
import torch

import oracle
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, fp8_query_codes, INV_SQRT_192, FP8_K_SCALE

from gpu_cases import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def _run_and_check(w, *, inv_q_scale=1.0, sinks=None, what=""):
    codes = fp8_query_codes(w, inv_q_scale)
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    prob.q_bits = codes
    prob.q_dtype = "fp8_e4m3fn"
    if sinks is not None:
        prob.sinks = sinks.astype(np.float64)
    B, H = w.batch, w.num_heads
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).cuda()
    if w.qo_indptr is None:
        q = q.view(B, w.q_len_fixed, H, 576)
    kv = torch.from_numpy(w.kv_bits).view(torch.float8_e4m3fn).cuda()
    bt = torch.from_numpy(w.block_tables).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    qo = None if w.qo_indptr is None else torch.from_numpy(w.qo_indptr).cuda()
    mq = w.max_q_len if qo is not None else None
    ws = torch.empty(binding.workspace_bytes_for(q, kv, bt, sl, w.max_seq_len, qo_indptr=qo, max_seq_len_q=mq,
                                                 return_lse=True), dtype=torch.uint8, device="cuda")
    s = None if sinks is None else torch.from_numpy(sinks.astype(np.float32)).cuda()
    o, l = binding.decode(q, kv, ws, bt, sl, w.max_seq_len, qo_indptr=qo, max_seq_len_q=mq, return_lse=True,
                          bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, causal=w.causal, sinks=s)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.reference_decode(prob)
    got_o = o.float().reshape(w.total_q, H, 512).cpu().numpy()
    got_l = l.reshape(w.total_q, H).cpu().numpy()
    check_close(got_o, ref_o, f"{what} out")
    check_close(got_l, ref_l, f"{what} lse")


@pytest.mark.parametrize("page_size", [16, 32, 64])
@pytest.mark.parametrize("grid", [0, 5])
def test_fp8_query_fixed_causal(page_size, grid):
    binding.set_grid_override(grid)
    w = make_workload("q8", seed=80, seq_lens=[5, 64, 100, 1000, 3333], num_heads=128, q_len=2,
                      page_size=page_size, kv_dtype="fp8_e4m3fn", kv_value_scale=0.5,
                      bmm1_scale=FP8_K_SCALE * INV_SQRT_192 * 50, bmm2_scale=1.0, causal=True, want_lse=True)
    _run_and_check(w, what=f"ps {page_size} grid {grid}")


def test_fp8_query_packed_dense_small_heads():
    w = make_workload("q8p", seed=81, batch=12, seq_len_range=(1, 900), num_heads=16, q_len_range=(1, 6),
                      page_size=32, kv_dtype="fp8_e4m3fn", bmm1_scale=INV_SQRT_192, causal=False, want_lse=True)
    _run_and_check(w, what="packed dense")


def test_fp8_query_scale_and_sinks():
    """A query stored as q / q_scale (q_scale = 1/4), q_scale folded into bmm1."""
    w = make_workload("q8s", seed=82, seq_lens=[77, 2100], num_heads=64, q_len=3, page_size=64,
                      kv_dtype="fp8_e4m3fn", bmm1_scale=INV_SQRT_192 / 4.0, causal=True, want_lse=True)
    sinks = np.random.default_rng(83).uniform(-2.0, 4.0, 64)
    _run_and_check(w, inv_q_scale=4.0, sinks=sinks, what="q_scale + sinks")


def test_fp8_query_reference_restart():
    """Unscaled logits force segment restarts with a raised reference max."""
    binding.set_grid_override(8)
    w = make_workload("q8r", seed=84, batch=3, seq_len_range=(600, 2000), num_heads=32, q_len=2, page_size=32,
                      kv_dtype="fp8_e4m3fn", bmm1_scale=1.0, causal=True, want_lse=True)
    _run_and_check(w, what="restart")


def test_full_size_benched_workload_all_requests():
    """fp8_long_context with an fp8 query at full size (8 requests of 64K-128K
    rows), in the launch the benchmark times, every request against the
    oracle."""
    from paged_mla_decode_03_amd.inputs import named_workload, to_device_tensors
    w = named_workload("fp8_long_context", poison=True)
    codes = fp8_query_codes(w)
    t = to_device_tensors(w, "cuda")
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).cuda().view(w.batch, w.q_len_fixed, w.num_heads, 576)
    ws = torch.empty(binding.workspace_bytes_for(q, t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                                 return_lse=True), dtype=torch.uint8, device="cuda")
    o, l = binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, return_lse=True,
                          bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, causal=w.causal)
    torch.cuda.synchronize()
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    prob.q_bits = codes
    prob.q_dtype = "fp8_e4m3fn"
    ref_o, ref_l = oracle.reference_decode(prob)
    H = w.num_heads
    got_o = o.float().reshape(w.total_q, H, 512).cpu().numpy()
    got_l = l.reshape(w.total_q, H).cpu().numpy()
    check_close(got_o, ref_o, "q8 full-size out")
    check_close(got_l, ref_l, "q8 full-size lse")
