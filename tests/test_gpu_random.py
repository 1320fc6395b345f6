"""Seeded random sweep over the option space against the float64 oracle:
head counts, page sizes, fixed / packed queries, causal / dense, bf16 / fp8
cache, fp8 query, sinks, LSE, forced grids and split costs, grouped or
unit-by-unit splits, and the sparse top-k layout.  Every case is reproducible
from its index."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle.sparse import reference_sparse_decode
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, sparse_lists, fp8_query_codes

from gpu_cases import check_close

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("MLA_RANDOM_CASES", "96"))
FIRST_CASE = int(os.environ.get("MLA_RANDOM_FIRST", "0"))  # longer sweeps can start past the default cases


@pytest.fixture(autouse=True)
def _reset_hooks():
    yield
    binding.set_grid_override(0)
    binding.set_segment_cost(-1)
    binding.set_work_groups(True)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    c = dict(
        H=int(rng.choice([16, 32, 48, 64, 128, 144, 256])),
        ps=int(rng.choice([16, 32, 64])),
        fp8=bool(rng.random() < 0.4),
        causal=bool(rng.random() < 0.7),
        lse=bool(rng.random() < 0.6),
        grid=int(rng.choice([0, 0, 1, 3, 7, 40])),
        seg=int(rng.choice([-1, 0, 4, 20])),
        sinks=bool(rng.random() < 0.3),
        B=int(rng.integers(1, 9)),
        packed=bool(rng.random() < 0.4),
        q=int(rng.integers(1, 5)),
        Lmax=int(rng.choice([40, 300, 2500])),
        sparse=bool(rng.random() < 0.2),
    )
    c["q8"] = c["fp8"] and not c["sparse"] and bool(rng.random() < 0.5)
    c["bmm1"] = float(rng.choice([0.02, 0.0722, 0.3]))
    c["bmm2"] = float(rng.choice([1.0, 0.5]))
    # grids with whole groups of 2, 4 or 8 workgroups per XCD, and the groups
    # switched off in some cases
    if rng.random() < 0.3:
        c["grid"] = int(rng.choice([16, 32, 64]))
    c["groups"] = bool(rng.random() < 0.8)
    return c


@pytest.mark.parametrize("i", range(FIRST_CASE, FIRST_CASE + N_CASES))
def test_random_case(i):
    c = _case(i)
    kv_dtype = "fp8_e4m3fn" if c["fp8"] else "bf16"
    qlen = dict(q_len_range=(1, c["q"])) if c["packed"] else dict(q_len=c["q"])
    lo = c["q"] if c["causal"] else 1
    w = make_workload(f"rand{i}", seed=2000 + i, batch=c["B"], seq_len_range=(lo, max(lo, c["Lmax"])),
                      num_heads=c["H"], page_size=c["ps"], kv_dtype=kv_dtype, bmm1_scale=c["bmm1"],
                      bmm2_scale=c["bmm2"], causal=c["causal"], want_lse=c["lse"] or c["sparse"], **qlen)
    binding.set_grid_override(c["grid"])
    binding.set_segment_cost(c["seg"])
    binding.set_work_groups(c["groups"])
    sinks = np.random.default_rng(3000 + i).uniform(-3.0, 5.0, c["H"]).astype(np.float32) if c["sinks"] else None
    s_t = None if sinks is None else torch.from_numpy(sinks).cuda()
    kv = torch.from_numpy(w.kv_bits)
    kv = (kv.view(torch.bfloat16) if kv_dtype == "bf16" else kv.view(torch.float8_e4m3fn)).cuda()
    H = c["H"]
    if c["sparse"]:
        K = int(np.random.default_rng(4000 + i).choice([32, 100, 256]))
        idx = sparse_lists(w, K, seed=5000 + i, empty_frac=0.05)
        q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda()
        it = torch.from_numpy(idx).cuda()
        ws = torch.empty(binding.sparse_workspace_bytes_for(q, kv, it, return_lse=True), dtype=torch.uint8,
                         device="cuda")
        o, l = binding.decode_sparse(q, kv, ws, it, return_lse=True, bmm1_scale=w.bmm1_scale,
                                     bmm2_scale=w.bmm2_scale, sinks=s_t)
        torch.cuda.synchronize()
        ref_o, ref_l = reference_sparse_decode(w.q_bits, w.kv_bits, kv_dtype, idx, w.bmm1_scale, w.bmm2_scale,
                                               sinks=None if sinks is None else sinks.astype(np.float64))
        got_o, got_l = o.float().cpu().numpy(), l.cpu().numpy()
        empty = np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(got_l), empty), (i, c)
        assert np.all(got_o[empty] == 0.0), (i, c)
        check_close(got_o[~empty], ref_o[~empty], f"case {i} {c} out")
        check_close(got_l[~empty], ref_l[~empty], f"case {i} {c} lse")
        return
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    if sinks is not None:
        prob.sinks = sinks.astype(np.float64)
    if c["q8"]:
        codes = fp8_query_codes(w)
        prob.q_bits = codes
        prob.q_dtype = "fp8_e4m3fn"
        q = torch.from_numpy(codes).view(torch.float8_e4m3fn).cuda()
    else:
        q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda()
    if w.qo_indptr is None:
        q = q.view(w.batch, w.q_len_fixed, H, 576)
    bt = torch.from_numpy(w.block_tables).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    qo = None if w.qo_indptr is None else torch.from_numpy(w.qo_indptr).cuda()
    mq = w.max_q_len if qo is not None else None
    ws = torch.empty(binding.workspace_bytes_for(q, kv, bt, sl, w.max_seq_len, qo_indptr=qo, max_seq_len_q=mq,
                                                 return_lse=w.want_lse), dtype=torch.uint8, device="cuda")
    res = binding.decode(q, kv, ws, bt, sl, w.max_seq_len, qo_indptr=qo, max_seq_len_q=mq, return_lse=w.want_lse,
                         bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, causal=w.causal, sinks=s_t)
    torch.cuda.synchronize()
    o, l = res if w.want_lse else (res, None)
    ref_o, ref_l = oracle.reference_decode(prob)
    check_close(o.float().reshape(w.total_q, H, 512).cpu().numpy(), ref_o, f"case {i} {c} out")
    if l is not None:
        check_close(l.reshape(w.total_q, H).cpu().numpy(), ref_l, f"case {i} {c} lse")
