"""GPU parity of the grouped work split: launches whose requests all hold the
same U = 2, 4 or 8 units of 128 (row, head) pairs hand each request's tiles to
a group of U workgroups that walk them together, one unit each.  The kernel
decides this on the device, for fixed-shape and packed launches alike.

Every case is checked against the float64 oracle on every request, with the
groups on and off, at several grid sizes and segment-start costs.  The plan
words the decode kernel leaves at the head of the workspace ([0] cost per
range, [1] group size, 1 when not grouped) show which split ran.
"""

import numpy as np
import pytest
import torch

from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, to_device_tensors, INV_SQRT_192

from gpu_cases import check_close, oracle_rows

pytestmark = pytest.mark.gpu

TILE, PAIRS = 32, 128


def _cus():
    """The default grid: one workgroup per compute unit."""
    return torch.cuda.get_device_properties(0).multi_processor_count


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


def _cost_per_range(w, group, grid, seg_cost):
    """The plan's cost per range C: total cost over the ranges (grid / group)."""
    T = [-(-int(L) // TILE) for L in w.seq_lens]
    units = [-(-int(q) * w.num_heads // PAIRS) for q in w.q_lens()]
    if group > 1:
        total = sum(T) + len(T) * seg_cost
    else:
        total = sum(u * t for u, t in zip(units, T)) + sum(units) * seg_cost
    return max(1, -(-total // (grid // group)))


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
            G = grid or _cus()
            gu = U if groups and G % (8 * U) == 0 else 1
            assert plan[1] == gu and plan[0] == _cost_per_range(w, gu, G, 8), (grid, groups, plan)
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
    assert plan[1] == 4 and plan[0] == _cost_per_range(w, 4, 64, cost)
    check_close(o[rows], ref_o[rows], f"cost {cost} out")
    check_close(l[rows], ref_l[rows], f"cost {cost} lse")


def test_groups_need_whole_groups_per_xcd():
    """A grid whose workgroups per XCD are not a multiple of U falls back to
    the unit-by-unit split (U = 4 here, 8 x 6 workgroups)."""
    binding.set_grid_override(48)
    w = _workload(128, 4, 64, "bf16", seed=78, batch=3, lens=(4, 1500))
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    o, l, plan = _run(w)
    assert plan[1] == 1
    check_close(o[rows], ref_o[rows], "fallback out")


def _run_packed(w):
    t = to_device_tensors(w, "cuda")
    nbytes = binding.workspace_bytes_for(t["q"], t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=t["qo_indptr"], max_seq_len_q=w.max_q_len, return_lse=True)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    o, l = binding.decode(t["q"], t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len,
                          qo_indptr=t["qo_indptr"], max_seq_len_q=w.max_q_len, return_lse=True,
                          bmm1_scale=w.bmm1_scale, causal=True)
    torch.cuda.synchronize()
    plan = ws[:8].view(torch.int32).cpu().numpy()
    H = w.num_heads
    return o.float().reshape(w.total_q, H, 512).cpu().numpy(), l.reshape(w.total_q, H).cpu().numpy(), plan


PACKED = [
    # (H, q_b range, grouped): packed launches are grouped exactly when every
    # request holds the same number of units
    (128, (4, 4), 4),    # compact speculative 1+3
    (16, (9, 16), 2),    # two units each, the second of 16..128 pairs
    (128, (1, 3), 1),    # one to three units: not grouped
    (64, (1, 2), 1),     # one unit each: nothing to group
]


@pytest.mark.parametrize("case", PACKED, ids=[f"H{c[0]}-q{c[1][0]}to{c[1][1]}" for c in PACKED])
def test_packed_launches(case):
    H, qr, gu = case
    w = make_workload("packed", seed=79 + H, batch=7, seq_len_range=(qr[1], 1500), num_heads=H, q_len_range=qr,
                      page_size=64, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    units = {-(-int(q) * H // PAIRS) for q in w.q_lens()}
    assert (len(units) == 1) == (gu > 1 or units == {1})
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    for grid in (0, 64):
        binding.set_grid_override(grid)
        o, l, plan = _run_packed(w)
        G = grid or _cus()
        assert plan[1] == (gu if G % (8 * gu) == 0 else 1), (grid, plan)
        check_close(o[rows], ref_o[rows], f"packed {case} grid {grid} out")
        check_close(l[rows], ref_l[rows], f"packed {case} grid {grid} lse")


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
        assert plan[1] == 4 and plan[0] == -(-(sum(-(-int(L) // TILE) for L in new) + B * 8) // (_cus() // 4))


def test_graph_replays_follow_qo_indptr_updates_grouped():
    """A packed launch captured once: between replays eager work rewrites
    qo_indptr in place (same total_q and max_q_len), switching the device-side
    decision between grouped (every request 4 rows of 128 heads: 4 units) and
    unit by unit (mixed unit counts); each replay equals an eager decode
    bitwise."""
    B, H, R, MQ = 6, 128, 24, 8
    w = make_workload("gqo", seed=83, batch=B, seq_len_range=(MQ, 1400), num_heads=H, q_len_range=(4, 4),
                      page_size=64, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    assert w.total_q == R
    t = to_device_tensors(w, "cuda")
    qo = t["qo_indptr"]
    nbytes = binding.workspace_bytes_for(t["q"], t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=qo, max_seq_len_q=MQ, return_lse=True)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    kw = dict(qo_indptr=qo, max_seq_len_q=MQ, return_lse=True, bmm1_scale=w.bmm1_scale, causal=True)
    binding.decode(t["q"], t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode(t["q"], t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, out=out, lse=lse, **kw)
    variants = [([4] * 6, 4), ([2, 6, 4, 4, 5, 3], 1), ([8, 8, 2, 2, 2, 2], 1), ([3, 5, 3, 5, 3, 5], 1), ([4] * 6, 4)]
    for qb, gu in variants:
        assert sum(qb) == R and max(qb) <= MQ
        qo.copy_(torch.tensor(np.concatenate([[0], np.cumsum(qb)]), dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        plan = ws[:8].view(torch.int32).cpu().numpy()
        assert plan[1] == gu, (qb, plan)
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        binding.decode(t["q"], t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, out=eo, lse=el, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo) and torch.equal(got_l, el), qb
