"""GPU parity of the sparse top-k layout against the float64 oracle
(oracle/sparse.py): every head of query row r attends to the cache rows its
list names.  Lists come from inputs.sparse_lists (random selections of each
row's request, -1 padding, empties and repeats), on NaN-poisoned caches whose
unlisted slots must never leak."""

import numpy as np
import pytest
import torch

from oracle.sparse import reference_sparse_decode
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, sparse_lists, INV_SQRT_192

from gpu_cases import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def _run(w, idx, *, top_k=None, sinks=None, return_lse=True):
    kv = torch.from_numpy(w.kv_bits)
    kv = (kv.view(torch.bfloat16) if w.kv_dtype == "bf16" else kv.view(torch.float8_e4m3fn)).cuda()
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda()
    it = torch.from_numpy(idx).cuda()
    ws = torch.empty(binding.sparse_workspace_bytes_for(q, kv, it, top_k=top_k, return_lse=return_lse),
                     dtype=torch.uint8, device="cuda")
    s = None if sinks is None else torch.from_numpy(sinks.astype(np.float32)).cuda()
    res = binding.decode_sparse(q, kv, ws, it, top_k=top_k, return_lse=return_lse, bmm1_scale=w.bmm1_scale,
                                bmm2_scale=w.bmm2_scale, sinks=s)
    torch.cuda.synchronize()
    return res


def _check(w, idx, *, top_k=None, sinks=None, what=""):
    k = idx.shape[1] if top_k is None else top_k
    o, l = _run(w, idx, top_k=top_k, sinks=sinks)
    ref_o, ref_l = reference_sparse_decode(w.q_bits, w.kv_bits, w.kv_dtype, idx[:, :k], w.bmm1_scale, w.bmm2_scale,
                                           sinks=sinks)
    got_o = o.float().cpu().numpy()
    got_l = l.cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty), f"{what}: empty (row, head) pairs differ"
    assert np.all(got_o[empty] == 0.0), f"{what}: empty pairs must give zeros"
    check_close(got_o[~empty], ref_o[~empty], f"{what} out")
    check_close(got_l[~empty], ref_l[~empty], f"{what} lse")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("grid", [0, 7])
def test_sparse_matches_oracle(kv_dtype, grid):
    fp8 = kv_dtype != "bf16"
    binding.set_grid_override(grid)
    # requests shorter and longer than top-k; 2 rows each (8 query rows)
    w = make_workload("sparse", seed=70, seq_lens=[90, 700, 3000, 5000], num_heads=128, q_len=2, page_size=64,
                      kv_dtype=kv_dtype, kv_value_scale=0.5 if fp8 else 1.0,
                      bmm1_scale=INV_SQRT_192 * (0.02 if fp8 else 1.0), bmm2_scale=0.02 if fp8 else 1.0,
                      causal=True, want_lse=True)
    idx = sparse_lists(w, 2048, seed=71, empty_frac=0.05, repeat_frac=0.02, empty_rows=(3,))
    _check(w, idx, what=f"{kv_dtype} grid {grid}")


@pytest.mark.parametrize("top_k", [1, 33, 100, 515])
def test_ragged_top_k_and_row_width(top_k):
    """top-k not a multiple of the 32-row tile, and lists narrower than their
    rows (only the first top_k entries count: the rest hold NaN-page ids)."""
    w = make_workload("sparse_k", seed=72, seq_lens=[600, 40], num_heads=32, q_len=3, page_size=32,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    idx = sparse_lists(w, top_k, seed=73, empty_frac=0.1)
    wide = np.concatenate([idx, np.full((idx.shape[0], 9), w.poison_page * w.page_size, dtype=np.int32)], axis=1)
    _check(w, wide, top_k=top_k, what=f"top_k {top_k}")


def test_sparse_with_sinks_and_small_head_count():
    w = make_workload("sparse_s", seed=74, seq_lens=[300, 2500], num_heads=16, q_len=4, page_size=16,
                      bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    idx = sparse_lists(w, 256, seed=75, empty_frac=0.02, empty_rows=(1, 6))
    sinks = np.random.default_rng(76).uniform(-2.0, 6.0, 16)
    _check(w, idx, sinks=sinks, what="sinks")


def test_full_in_order_lists_equal_the_dense_path():
    """A row listing its whole request in order is a dense (mask_type 'dense')
    decode of that request: the sparse and paged layouts agree to the parity
    bar on the same inputs."""
    w = make_workload("sparse_d", seed=77, seq_lens=[777, 1500], num_heads=128, q_len=1, page_size=64,
                      bmm1_scale=INV_SQRT_192, causal=False, want_lse=True)
    ps = w.page_size
    K = int(w.seq_lens.max())
    idx = np.full((2, K), -1, dtype=np.int32)
    for b in range(2):
        L = int(w.seq_lens[b])
        t = np.arange(L)
        idx[b, :L] = w.block_tables[b, t // ps] * ps + t % ps
    o_s, l_s = _run(w, idx)
    kv = torch.from_numpy(w.kv_bits).view(torch.bfloat16).cuda()
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda().view(2, 1, 128, 576)
    bt = torch.from_numpy(w.block_tables).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    ws = torch.empty(binding.workspace_bytes_for(q, kv, bt, sl, w.max_seq_len, return_lse=True), dtype=torch.uint8,
                     device="cuda")
    o_d, l_d = binding.decode(q, kv, ws, bt, sl, w.max_seq_len, return_lse=True, bmm1_scale=w.bmm1_scale,
                              causal=False)
    torch.cuda.synchronize()
    check_close(o_s.float().cpu().numpy(), o_d.float().reshape(2, 128, 512).cpu().numpy().astype(np.float64),
                "sparse vs dense out")
    check_close(l_s.cpu().numpy(), l_d.reshape(2, 128).cpu().numpy().astype(np.float64), "sparse vs dense lse")


def test_full_size_benched_workload_all_rows():
    """The benched sparse workload at full size (64 rows, top-k 2048, 128
    heads), in the launch the benchmark times, every row against the oracle."""
    from paged_mla_decode_03_amd.inputs import named_sparse_workload
    w, lists = named_sparse_workload("sparse_topk_decode", poison=True)
    o, l = _run(w, lists)
    ref_o, ref_l = reference_sparse_decode(w.q_bits, w.kv_bits, w.kv_dtype, lists, w.bmm1_scale, w.bmm2_scale)
    check_close(o.float().cpu().numpy(), ref_o, "sparse full-size out")
    check_close(l.cpu().numpy(), ref_l, "sparse full-size lse")
