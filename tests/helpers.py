"""Test-side helpers: build small paged problems from dense per-request rows.

The paging here (scatter rows into a shuffled page pool, write block tables)
is written independently of the oracle's gather so the oracle's paging is
checked, not reused.
"""

import numpy as np
import torch

from oracle import MlaProblem


def to_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()


def bf16_round(x):
    """Values rounded to bf16, returned as float64 (via torch's own cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def to_e4m3_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def build_paged(q_rows, k_per_req, page_size, *, rng, q_lens=None, packed=False, bmm1=0.1, bmm2=1.0,
                causal=True, kv_dtype="bf16", extra_width=1, fill_tail=np.nan):
    """Assemble an MlaProblem.

    q_rows     float [R, H, 576] (already representable in bf16)
    k_per_req  list of float [L_b, 576] (already representable in the KV type)
    q_lens     per-request query lengths (sum = R); fixed when all equal and not packed
    """
    B = len(k_per_req)
    L = np.array([k.shape[0] for k in k_per_req], dtype=np.int64)
    if q_lens is None:
        q_lens = [q_rows.shape[0] // B] * B
    q_lens = np.asarray(q_lens, dtype=np.int64)
    assert q_lens.sum() == q_rows.shape[0]
    ps = page_size
    npages = [(int(l) + ps - 1) // ps for l in L]
    total = sum(npages)
    perm = rng.permutation(total)
    W = max(npages) + extra_width
    pad_id = total
    bt = np.full((B, W), pad_id, dtype=np.int32)
    if kv_dtype == "bf16":
        pool = np.zeros((total + 1, ps, 576), dtype=np.uint16)
        enc = to_bf16_bits
        nan_code = np.uint16(0x7FC0)
    else:
        pool = np.zeros((total + 1, ps, 576), dtype=np.uint8)
        enc = to_e4m3_bits
        nan_code = np.uint8(0x7F)
    off = 0
    for b in range(B):
        for p in range(npages[b]):
            pid = int(perm[off + p])
            bt[b, p] = pid
            rows = k_per_req[b][p * ps:(p + 1) * ps]
            pool[pid, :rows.shape[0]] = enc(rows)
            if rows.shape[0] < ps and fill_tail is not None:
                pool[pid, rows.shape[0]:] = nan_code
        off += npages[b]
    pool[pad_id] = nan_code
    qo = None
    if packed or len(set(q_lens.tolist())) > 1:
        qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return MlaProblem(q_bits=to_bf16_bits(q_rows), kv_bits=pool, kv_dtype=kv_dtype, block_tables=bt,
                      seq_lens=L.astype(np.int32), qo_indptr=qo, q_len_fixed=int(q_lens[0]),
                      bmm1_scale=bmm1, bmm2_scale=bmm2, causal=causal)


def random_dense(rng, B, H, q_lens, seq_lens, scale=1.0, kv_dtype="bf16"):
    R = int(sum(q_lens))
    q = bf16_round(rng.standard_normal((R, H, 576)).astype(np.float32) * scale)
    rnd = bf16_round if kv_dtype == "bf16" else e4m3_round
    ks = [rnd(rng.standard_normal((int(L), 576)).astype(np.float32) * scale) for L in seq_lens]
    return q, ks
