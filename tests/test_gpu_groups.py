"""GPU parity of the grouped work split: fixed-shape launches whose requests
hold U = 2, 4 or 8 units of 128 (row, head) pairs hand each request's tiles to
a group of U workgroups that walk them together, one unit each.

Every case is checked against the float64 oracle on every request, with the
groups on and off, at several grid sizes and segment-start costs.  The plan
words the decode kernel leaves at the head of the workspace ([0] cost per
range, [1] total cost) show which split ran: grouped, a request is one cost
unit of T_b tiles; otherwise it is U units of T_b tiles each.
"""

import numpy as np
import pytest
import torch

from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, to_device_tensors, INV_SQRT_192

from gpu_cases import check_close, oracle_rows

pytestmark = pytest.mark.gpu

TILE, PAIRS = 32, 128


@pytest.fixture(autouse=True)
def _defaults():
    binding.set_grid_override(0)
    binding.set_segment_cost(-1)
    binding.set_work_groups(True)
    yield
    binding.set_grid_override(0)
    binding.set_segment_cost(-1)
    binding.set_work_groups(True)


def _run(w):
    """Decode w; returns (out [R, H, 512], lse [R, H] or None, plan words [C, TC])."""
    t = to_device_tensors(w, "cuda")
    B, H = w.batch, w.num_heads
    q = t["q"].view(B, w.q_len_fixed, H, 576)
    nbytes = binding.workspace_bytes_for(q, t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         return_lse=w.want_lse)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    res = binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, return_lse=w.want_lse,
                         bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, causal=w.causal)
    torch.cuda.synchronize()
    o, l = res if w.want_lse else (res, None)
    plan = ws[:8].view(torch.int32).cpu().numpy()
    o = o.float().reshape(w.total_q, H, 512).cpu().numpy()
    l = None if l is None else l.reshape(w.total_q, H).cpu().numpy()
    return o, l, plan


def _expected_total_cost(w, grouped, seg_cost):
    T = [-(-int(L) // TILE) for L in w.seq_lens]
    U = -(-w.q_len_fixed * w.num_heads // PAIRS)
    if grouped:
        return sum(T) + len(T) * seg_cost
    return U * sum(T) + len(T) * U * seg_cost


CASES = [
    # (H, q_len, page_size, kv_dtype): units per request U = ceil(q_len H / 128)
    (128, 2, 64, "bf16"),        # U = 2
    (64, 3, 32, "bf16"),         # U = 2, the second unit 64 pairs
    (80, 5, 16, "bf16"),         # U = 4, the last unit 16 pairs
    (128, 4, 64, "bf16"),        # U = 4, the speculative 1+3 shape
    (128, 8, 32, "bf16"),        # U = 8
    (16, 16, 64, "bf16"),        # U = 2 from many rows of few heads
    (128, 2, 64, "fp8_e4m3fn"),  # U = 2, the long-context fp8 shape
    (96, 5, 32, "fp8_e4m3fn"),   # U = 4, the last unit 96 pairs
]


def _workload(H, ql, ps, kv_dtype, seed, batch, lens):
    fp8 = kv_dtype != "bf16"
    return make_workload("groups", seed=seed, batch=batch, seq_len_range=lens, num_heads=H, q_len=ql, page_size=ps,
                         kv_dtype=kv_dtype, kv_value_scale=0.5 if fp8 else 1.0,
                         bmm1_scale=INV_SQRT_192 * (0.02 if fp8 else 1.0), bmm2_scale=0.02 if fp8 else 1.0,
                         causal=True, want_lse=True)


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}-q{c[1]}-ps{c[2]}-{c[3]}" for c in CASES])
def test_grouped_split_matches_oracle(case):
    H, ql, ps, kv_dtype = case
    U = -(-ql * H // PAIRS)
    w = _workload(H, ql, ps, kv_dtype, seed=40 + H + ql, batch=6, lens=(ql, 2600))
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    # grids: one group per XCD, three per XCD, one workgroup per CU
    for grid in (8 * U, 24 * U, 0):
        binding.set_grid_override(grid)
        for groups in (True, False):
            binding.set_work_groups(groups)
            o, l, plan = _run(w)
            assert plan[1] == _expected_total_cost(w, groups, 8), (grid, groups, plan)
            check_close(o[rows], ref_o[rows], f"{case} grid {grid} groups {groups} out")
            check_close(l[rows], ref_l[rows], f"{case} grid {grid} groups {groups} lse")


@pytest.mark.parametrize("cost", [0, 1, 40])
def test_grouped_split_segment_costs(cost):
    """Segment-start costs that put range boundaries anywhere, including ranges
    with no tile at all, and short requests of a single tile."""
    binding.set_segment_cost(cost)
    binding.set_grid_override(64)
    w = _workload(128, 4, 32, "bf16", seed=77, batch=9, lens=(4, 900))
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    o, l, plan = _run(w)
    assert plan[1] == _expected_total_cost(w, True, cost)
    check_close(o[rows], ref_o[rows], f"cost {cost} out")
    check_close(l[rows], ref_l[rows], f"cost {cost} lse")


def test_groups_need_whole_groups_per_xcd():
    """A grid whose workgroups per XCD are not a multiple of U falls back to
    the unit-by-unit split (U = 4 here, 8 x 6 workgroups)."""
    binding.set_grid_override(48)
    w = _workload(128, 4, 64, "bf16", seed=78, batch=3, lens=(4, 1500))
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    o, l, plan = _run(w)
    assert plan[1] == _expected_total_cost(w, False, 8)
    check_close(o[rows], ref_o[rows], "fallback out")


def test_packed_launch_is_never_grouped():
    """Packed (qo_indptr) launches keep the unit-by-unit split, whatever their
    row counts."""
    w = make_workload("packed", seed=79, batch=4, seq_len_range=(8, 800), num_heads=128, q_len_range=(2, 2),
                      page_size=64, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    t = to_device_tensors(w, "cuda")
    nbytes = binding.workspace_bytes_for(t["q"], t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=t["qo_indptr"], max_seq_len_q=w.max_q_len, return_lse=True)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    binding.decode(t["q"], t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, qo_indptr=t["qo_indptr"],
                   max_seq_len_q=w.max_q_len, return_lse=True, bmm1_scale=w.bmm1_scale, causal=True)
    torch.cuda.synchronize()
    plan = ws[:8].view(torch.int32).cpu().numpy()
    T = [-(-int(L) // TILE) for L in w.seq_lens]
    assert plan[1] == 2 * sum(T) + 2 * len(T) * 8


def test_graph_replays_follow_length_updates_grouped():
    """A grouped launch captured once: between replays eager work rewrites
    seq_lens in place (within max_seq_len), which moves every range boundary of
    the device-side split; each replay must equal an eager decode bitwise."""
    w = _workload(128, 4, 64, "bf16", seed=81, batch=5, lens=(4, 1800))
    t = to_device_tensors(w, "cuda")
    B, H = w.batch, w.num_heads
    q = t["q"].view(B, w.q_len_fixed, H, 576)
    sl = t["seq_lens"]
    nbytes = binding.workspace_bytes_for(q, t["kv"], t["block_tables"], sl, w.max_seq_len, return_lse=True)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, w.q_len_fixed, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, w.q_len_fixed, H), dtype=torch.float32, device="cuda")
    kw = dict(return_lse=True, bmm1_scale=w.bmm1_scale, causal=True, out=out, lse=lse)
    binding.decode(q, t["kv"], ws, t["block_tables"], sl, w.max_seq_len, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode(q, t["kv"], ws, t["block_tables"], sl, w.max_seq_len, **kw)
    rng = np.random.default_rng(82)
    full = w.seq_lens.astype(np.int64)
    for rep in range(6):
        # shorter lengths use a prefix of each request's pages: still valid
        new = rng.integers(w.q_len_fixed, full, endpoint=True).astype(np.int32)
        sl.copy_(torch.from_numpy(new).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        eo = torch.empty_like(out)
        el = torch.empty_like(lse)
        binding.decode(q, t["kv"], ws, t["block_tables"], sl, w.max_seq_len, return_lse=True,
                       bmm1_scale=w.bmm1_scale, causal=True, out=eo, lse=el)
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo) and torch.equal(got_l, el), rep
        plan = ws[:8].view(torch.int32).cpu().numpy()
        assert plan[1] == sum(-(-int(L) // TILE) for L in new) + B * 8
