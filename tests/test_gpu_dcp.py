"""GPU checks of the sequence-sharded (DCP) partial mode and of
mla_merge_partials: each virtual rank decodes its round-robin share of every
request's cached rows with causal limits from the global lengths, against the
float64 oracle's partial, and the merged ranks against the full decode."""

import numpy as np
import pytest
import torch

import oracle
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, INV_SQRT_192, BF16_NAN, E4M3FN_NAN

from gpu_cases import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def _rank_cache(w, rank, world):
    """Rank `rank`'s share of every request: global rows rank, rank + world, ...
    re-paged into a pool of its own (unused slots NaN) with its block table."""
    ps = w.page_size
    nan = BF16_NAN if w.kv_dtype == "bf16" else E4M3FN_NAN
    rows, lens = [], []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        t = np.arange(rank, L, world)
        pages = w.block_tables[b, t // ps].astype(np.int64)
        rows.append(w.kv_bits[pages, t % ps, :])
        lens.append(len(t))
    npg = [max(1, (n + ps - 1) // ps) for n in lens]
    pool = np.full((sum(npg) + 1, ps, 576), nan, dtype=w.kv_bits.dtype)
    W = max(npg)
    bt = np.full((w.batch, W), sum(npg), dtype=np.int32)
    off = 0
    for b in range(w.batch):
        n = lens[b]
        for k in range(npg[b]):
            seg = rows[b][k * ps:(k + 1) * ps]
            pool[off + k, :len(seg)] = seg
            bt[b, k] = off + k
        off += npg[b]
    return pool, bt, np.asarray(lens, dtype=np.int32)


def _to_kv(pool, kv_dtype):
    t = torch.from_numpy(pool)
    t = t.view(torch.bfloat16) if kv_dtype == "bf16" else t.view(torch.float8_e4m3fn)
    return t.cuda()


def _check_partial(got_o, got_l, ref_o, ref_l, what):
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty), f"{what}: empty rows differ"
    assert np.all(got_o[empty] == 0.0), f"{what}: empty rows must be zero"
    if (~empty).any():
        check_close(got_o[~empty], ref_o[~empty], f"{what} out")
        check_close(got_l[~empty], ref_l[~empty], f"{what} lse")


def _run_shards(kv_dtype, world, with_sinks, num_heads=32, q_len=3):
    fp8 = kv_dtype != "bf16"
    # short requests too, so that some ranks hold no visible row (or no row) of them
    w = make_workload("dcp", seed=50 + world, seq_lens=[3, 5, 40, 333, 1200], num_heads=num_heads, q_len=q_len,
                      page_size=32, kv_dtype=kv_dtype, kv_value_scale=0.5 if fp8 else 1.0,
                      bmm1_scale=INV_SQRT_192 * (0.02 if fp8 else 1.0), bmm2_scale=0.02 if fp8 else 1.0,
                      causal=True, want_lse=True)
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    B, H, R = w.batch, w.num_heads, w.total_q
    sinks = None
    if with_sinks:
        # logits around the scale of the scores, some dominating
        sv = np.random.default_rng(70 + world).uniform(-4.0, 8.0, H).astype(np.float32)
        prob.sinks = sv.astype(np.float64)
        sinks = torch.from_numpy(sv).cuda()
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda().view(B, w.q_len_fixed, H, 576)
    lens_g = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    outs, lses = [], []
    for r in range(world):
        pool, bt, lens = _rank_cache(w, r, world)
        kv = _to_kv(pool, kv_dtype)
        bt_t, lens_t = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
        max_len = max(1, int(lens.max()))
        ws = torch.empty(binding.workspace_bytes_for(q, kv, bt_t, lens_t, max_len, return_lse=True),
                         dtype=torch.uint8, device="cuda")
        o, l = binding.decode(q, kv, ws, bt_t, lens_t, max_len, return_lse=True, bmm1_scale=w.bmm1_scale,
                              bmm2_scale=w.bmm2_scale, causal=True, dcp=(lens_g, world, r), sinks=sinks)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.reference_dcp_partial(prob, r, world)
        _check_partial(o.float().reshape(R, H, 512).cpu().numpy(), l.reshape(R, H).cpu().numpy(), ref_o, ref_l,
                       f"rank {r}/{world}")
        outs.append(o)
        lses.append(l)
    mo, ml = binding.merge_partials(torch.stack(outs), torch.stack(lses))
    torch.cuda.synchronize()
    full_o, full_l = oracle.reference_decode(prob)
    check_close(mo.float().reshape(R, H, 512).cpu().numpy(), full_o, "merged out")
    check_close(ml.reshape(R, H).cpu().numpy(), full_l, "merged lse")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("world", [2, 3, 8])
def test_sequence_shards_match_oracle_and_merge_to_full(kv_dtype, world):
    _run_shards(kv_dtype, world, with_sinks=False)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_sequence_shards_with_sinks(kv_dtype):
    """Rank 0 carries the sinks; the merged ranks equal the full decode with sinks."""
    _run_shards(kv_dtype, 3, with_sinks=True)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_sequence_shards_grouped_split(kv_dtype):
    """128 heads x 2 rows: two units per request, so each rank's launch walks
    every request with a pair of workgroups (the grouped split), including
    ranks that hold no row of the short requests."""
    _run_shards(kv_dtype, 8, with_sinks=True, num_heads=128, q_len=2)


def test_single_rank_partial_equals_plain_decode():
    w = make_workload("dcp1", seed=60, seq_len_range=(50, 700), batch=3, num_heads=32, q_len=2, page_size=32,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    B, H = w.batch, w.num_heads
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda().view(B, w.q_len_fixed, H, 576)
    kv = _to_kv(w.kv_bits, "bf16")
    bt, lens = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    ws = torch.empty(binding.workspace_bytes_for(q, kv, bt, lens, w.max_seq_len, return_lse=True),
                     dtype=torch.uint8, device="cuda")
    o1, l1 = binding.decode(q, kv, ws, bt, lens, w.max_seq_len, return_lse=True, bmm1_scale=w.bmm1_scale)
    o2, l2 = binding.decode(q, kv, ws, bt, lens, w.max_seq_len, return_lse=True, bmm1_scale=w.bmm1_scale,
                            dcp=(lens, 1, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
