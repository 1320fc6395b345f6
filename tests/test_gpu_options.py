"""GPU checks of the device-resident options (mla_decode_paged_ex): per-head
attention sinks against the float64 oracle, device scales against host
scales, and a captured HIP graph that follows scale updates between replays."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, to_device_tensors, INV_SQRT_192

from gpu_cases import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def _setup(w):
    t = to_device_tensors(w, "cuda")
    B, H = w.batch, w.num_heads
    q = t["q"] if w.qo_indptr is not None else t["q"].view(B, w.q_len_fixed, H, 576)
    max_q = w.max_q_len if w.qo_indptr is not None else None
    nbytes = binding.workspace_bytes_for(q, t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=t["qo_indptr"], max_seq_len_q=max_q, return_lse=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    return t, q, max_q, ws


def _run(w, t, q, max_q, ws, **kw):
    o, l = binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, qo_indptr=t["qo_indptr"],
                          max_seq_len_q=max_q, return_lse=True, causal=w.causal, **kw)
    torch.cuda.synchronize()
    return o, l


def _workload(kv_dtype, seed):
    fp8 = kv_dtype != "bf16"
    return make_workload("opts", seed=seed, batch=3, seq_len_range=(60, 900), num_heads=32, q_len=2, page_size=32,
                         kv_dtype=kv_dtype, kv_value_scale=0.5 if fp8 else 1.0,
                         bmm1_scale=INV_SQRT_192 * (0.02 if fp8 else 1.0), bmm2_scale=0.02 if fp8 else 1.0,
                         causal=True, want_lse=True)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("grid", [0, 5])
def test_sinks_match_oracle(kv_dtype, grid):
    binding.set_grid_override(grid)
    w = _workload(kv_dtype, 41)
    H = w.num_heads
    rng = np.random.default_rng(42)
    sinks = rng.normal(0.0, 3.0, size=H).astype(np.float32)
    sinks[0], sinks[1] = 30.0, -30.0  # a sink that takes almost all the mass, and one that takes none
    t, q, max_q, ws = _setup(w)
    o, l = _run(w, t, q, max_q, ws, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                sinks=torch.from_numpy(sinks).cuda())
    prob = dataclasses.replace(oracle.MlaProblem(**w.oracle_problem_kwargs()), sinks=sinks.astype(np.float64))
    ref_o, ref_l = oracle.reference_decode(prob)
    got_o = o.float().reshape(w.total_q, H, 512).cpu().numpy()
    got_l = l.reshape(w.total_q, H).cpu().numpy()
    check_close(got_o, ref_o, "out with sinks")
    check_close(got_l, ref_l, "lse with sinks")
    # the dominating sink: lse sits on the sink
    assert np.abs(got_l[:, 0] - 30.0).max() < 1e-3


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_device_scales_equal_host_scales(kv_dtype):
    w = _workload(kv_dtype, 43)
    t, q, max_q, ws = _setup(w)
    o_h, l_h = _run(w, t, q, max_q, ws, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
    b1 = torch.tensor([w.bmm1_scale], dtype=torch.float32, device="cuda")
    b2 = torch.tensor([w.bmm2_scale], dtype=torch.float32, device="cuda")
    o_d, l_d = _run(w, t, q, max_q, ws, bmm1_scale=b1, bmm2_scale=b2)
    assert torch.equal(o_h, o_d) and torch.equal(l_h, l_d)
    # no-sink options path (all-NaN-free) equals the plain entry point too
    o_s, l_s = _run(w, t, q, max_q, ws, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                    sinks=torch.full((w.num_heads,), float("-inf"), device="cuda"))
    assert torch.equal(o_h, o_s) and torch.equal(l_h, l_s)


def test_graph_replays_follow_device_scales():
    """Capture one decode with device scales and sinks in a graph; between
    replays, eager work rewrites the scales; each replay must equal an eager
    decode with the same values."""
    w = _workload("bf16", 44)
    H = w.num_heads
    t, q, max_q, ws = _setup(w)
    b1 = torch.tensor([w.bmm1_scale], dtype=torch.float32, device="cuda")
    b2 = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    sinks = torch.linspace(-2.0, 2.0, H, device="cuda")
    out = torch.empty((w.batch, w.q_len_fixed, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.q_len_fixed, H), dtype=torch.float32, device="cuda")
    kw = dict(qo_indptr=t["qo_indptr"], max_seq_len_q=max_q, return_lse=True, causal=w.causal, out=out, lse=lse,
              bmm1_scale=b1, bmm2_scale=b2, sinks=sinks)
    # warm up (caches the CU count) outside the capture
    binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, **kw)
    for s1, s2 in ((w.bmm1_scale, 1.0), (w.bmm1_scale * 3.0, 0.5), (w.bmm1_scale * 0.25, 2.0)):
        b1.fill_(s1)
        b2.fill_(s2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = _run(w, t, q, max_q, ws, bmm1_scale=float(np.float32(s1)), bmm2_scale=float(np.float32(s2)),
                            sinks=sinks)
        assert torch.equal(got_o, ref_o.view_as(got_o)) and torch.equal(got_l, ref_l.view_as(got_l)), (s1, s2)


def _compositions(rng, B, total, lo, hi, lens, n):
    """n distinct per-request query-length vectors (each in [lo, hi], at most the
    request's length) with the same sum `total`."""
    out = []
    while len(out) < n:
        q = rng.integers(lo, hi, endpoint=True, size=B)
        q = np.minimum(q, lens)
        d = total - int(q.sum())
        # move the difference onto requests that have room, one row at a time
        order = rng.permutation(B)
        for b in np.concatenate([order] * (hi * B)):
            if d == 0:
                break
            if d > 0 and q[b] < min(hi, lens[b]):
                q[b] += 1
                d -= 1
            elif d < 0 and q[b] > lo:
                q[b] -= 1
                d += 1
        if d == 0 and not any(np.array_equal(q, o) for o in out):
            out.append(q.copy())
    return [np.concatenate([[0], np.cumsum(q)]).astype(np.int32) for q in out]


def test_graph_replays_follow_qo_indptr_updates():
    """A packed launch captured once: between replays, eager work rewrites the
    values of qo_indptr in its stable storage (same total_q and max_q_len, every
    offset vector valid), as the FlashInfer API docs contract paragraph allows.
    Each of 24 replays must equal, bitwise, an eager decode with the same
    offsets, and match the oracle."""
    w = make_workload("gqo", seed=45, batch=7, seq_len_range=(40, 1200), num_heads=32, q_len_range=(1, 6),
                      page_size=32, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    H, R = w.num_heads, w.total_q
    rng = np.random.default_rng(46)
    variants = _compositions(rng, w.batch, R, 1, w.max_q_len, w.seq_lens.astype(np.int64), 6)
    t, q, max_q, ws = _setup(w)
    qo = t["qo_indptr"]
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    kw = dict(qo_indptr=qo, max_seq_len_q=max_q, return_lse=True, causal=True, out=out, lse=lse,
              bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
    binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, **kw)
    eager_out = torch.empty_like(out)
    eager_lse = torch.empty_like(lse)
    for i in range(24):
        v = variants[i % len(variants)]
        qo.copy_(torch.from_numpy(v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, qo_indptr=qo,
                       max_seq_len_q=max_q, return_lse=True, causal=True, out=eager_out, lse=eager_lse,
                       bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
        torch.cuda.synchronize()
        assert torch.equal(got_o, eager_out) and torch.equal(got_l, eager_lse), f"replay {i}"
        if i < len(variants):
            prob = dataclasses.replace(oracle.MlaProblem(**w.oracle_problem_kwargs()), qo_indptr=v)
            ref_o, ref_l = oracle.reference_decode(prob)
            check_close(got_o.float().cpu().numpy(), ref_o, f"replay {i} out")
            check_close(got_l.cpu().numpy(), ref_l, f"replay {i} lse")
