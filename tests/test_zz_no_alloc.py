"""GPU test of mla_decode_paged_noalloc, the entry point for callers that
cannot allocate: through the C ABI, two calls in a row (the second on a
smaller input), each against mla_decode_paged with a caller-owned workspace on
the same inputs, and against the float64 oracle; plus its size limit."""

import numpy as np
import pytest
import torch

import oracle
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, named_workload, to_device_tensors, INV_SQRT_192

from gpu_cases import check_close

pytestmark = pytest.mark.gpu


def _launch_args(w):
    t = to_device_tensors(w, "cuda")
    B, H = w.batch, w.num_heads
    q = t["q"] if w.qo_indptr is not None else t["q"].view(B, w.q_len_fixed, H, 576)
    max_q = w.max_q_len if w.qo_indptr is not None else None
    dims, max_q_len, _, _ = binding.dims_for(q, t["kv"], t["block_tables"], t["seq_lens"], t["qo_indptr"], max_q)
    return t, q, dims, max_q_len


def _run_both(w):
    """(noalloc out, noalloc lse, workspace out, workspace lse) as float32 numpy."""
    t, q, dims, max_q_len = _launch_args(w)
    R, H = w.total_q, w.num_heads
    outs = []
    for noalloc in (True, False):
        out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda") if w.want_lse else None
        args = (q, t["kv"], t["block_tables"], t["seq_lens"], t["qo_indptr"], w.max_seq_len, max_q_len,
                w.bmm1_scale, w.bmm2_scale, w.causal, out, lse)
        if noalloc:
            rc = binding.mla_decode_paged_noalloc(*args, dims)
        else:
            nbytes = binding.mla_decode_paged_workspace_size(dims, w.max_seq_len, max_q_len, w.want_lse)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            rc = binding.mla_decode_paged(*args, ws, nbytes, dims)
        assert rc == binding.MLA_OK, binding.mla_status_string(rc)
        torch.cuda.synchronize()
        outs.append(out)
        outs.append(lse)
    return outs


def _check(w):
    o_n, l_n, o_w, l_w = _run_both(w)
    # same kernels, same split: bitwise equal to the workspace entry point
    assert torch.equal(o_n, o_w)
    if l_n is not None:
        assert torch.equal(l_n, l_w)
    ref_o, ref_l = oracle.reference_decode(oracle.MlaProblem(**w.oracle_problem_kwargs()))
    check_close(o_n.float().cpu().numpy(), ref_o, f"{w.name} noalloc out")
    if l_n is not None:
        check_close(l_n.cpu().numpy(), ref_l, f"{w.name} noalloc lse")


def test_noalloc_two_calls_second_smaller():
    """A larger launch, then a smaller one reusing the same scratch (which
    still holds the first call's partials)."""
    big = make_workload("noalloc_big", seed=300, batch=12, seq_len_range=(500, 4000), num_heads=128, q_len=2,
                        page_size=64, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    small = make_workload("noalloc_small", seed=301, batch=3, seq_len_range=(20, 300), num_heads=16,
                          q_len_range=(1, 4), page_size=32, bmm1_scale=INV_SQRT_192, causal=True, want_lse=False)
    _check(big)
    _check(small)


def test_noalloc_benchmark_shape():
    """The DeepSeek-V3-shaped decode through the no-allocation entry point."""
    _check(named_workload("dsv3_bf16_decode"))


def test_noalloc_rejects_shapes_beyond_its_scratch():
    w = make_workload("noalloc_tiny", seed=302, batch=2, seq_len_range=(10, 40), num_heads=16, q_len=1,
                      page_size=32, bmm1_scale=INV_SQRT_192, causal=True)
    t, q, dims, max_q_len = _launch_args(w)
    out = torch.empty((w.total_q, 16, 512), dtype=torch.bfloat16, device="cuda")
    # the same launch declared with a huge max_q_len needs far more workspace
    big_q = 1 << 14
    need = binding.mla_decode_paged_workspace_size(
        binding.make_dims(batch=2, num_heads=16, q_len_fixed=1, total_q=2, page_size=32, num_pages=dims.num_pages,
                          block_table_stride=dims.block_table_stride, kv_dtype=0), w.max_seq_len, big_q)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    packed = binding.make_dims(batch=2, num_heads=16, q_len_fixed=1, total_q=2, page_size=32,
                               num_pages=dims.num_pages, block_table_stride=dims.block_table_stride, kv_dtype=0)
    qo = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    rc = binding.mla_decode_paged_noalloc(q, t["kv"], t["block_tables"], t["seq_lens"], qo, w.max_seq_len, big_q,
                                          w.bmm1_scale, w.bmm2_scale, True, out, None, packed)
    assert rc == 13, binding.mla_status_string(rc)
    assert "MLA_NOALLOC_SCRATCH_BYTES" in binding.mla_status_string(rc)
