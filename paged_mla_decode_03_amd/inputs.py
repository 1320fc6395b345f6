"""Seeded synthetic workloads for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of the
decode arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle
consume what it produces: raw storage bits (bf16 codes as uint16, fp8 E4M3FN
codes as uint8) plus int32 metadata, so neither side depends on the other.

Workload shapes follow the pages' uses of the method (DeepSeek-style MLA
decode: 128 query heads, 512 latent + 64 RoPE dims, page sizes 32/64,
uniform multi-token spec decode, ragged packed queries through qo_indptr, an
fp8 KV cache with a per-tensor scale folded into bmm1/bmm2).  No dataset is
involved; every value is drawn here.

Draw order for a seed (numpy default_rng): seq_lens, then per-request query
lengths (ragged workloads only), then the page permutation, then Q, then KV.
Normals are drawn in float32 and rounded to bf16 / fp8 E4M3FN by torch
(round-to-nearest-even).
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_QK = 576
BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)


@dataclass
class Workload:
    name: str
    q_bits: np.ndarray            # uint16 [R, H, 576]
    kv_bits: np.ndarray           # uint16 / uint8 [num_pages, page_size, 576]
    kv_dtype: str                 # "bf16" | "fp8_e4m3fn"
    block_tables: np.ndarray      # int32 [B, W]
    seq_lens: np.ndarray          # int32 [B]
    qo_indptr: Optional[np.ndarray]  # int32 [B+1] or None
    q_len_fixed: int              # SQ for fixed launches (max_q_len otherwise)
    max_seq_len: int
    max_q_len: int
    bmm1_scale: float
    bmm2_scale: float
    causal: bool
    want_lse: bool
    poison_page: int              # id of the all-NaN padding page
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_heads(self):
        return int(self.q_bits.shape[1])

    @property
    def page_size(self):
        return int(self.kv_bits.shape[1])

    @property
    def total_q(self):
        return int(self.q_bits.shape[0])

    def q_lens(self):
        if self.qo_indptr is None:
            return np.full(self.batch, self.q_len_fixed, dtype=np.int64)
        return np.diff(self.qo_indptr.astype(np.int64))

    def oracle_problem_kwargs(self):
        """Keyword arguments for the oracle's problem container."""
        return dict(q_bits=self.q_bits, kv_bits=self.kv_bits, kv_dtype=self.kv_dtype,
                    block_tables=self.block_tables, seq_lens=self.seq_lens,
                    qo_indptr=self.qo_indptr, q_len_fixed=self.q_len_fixed,
                    bmm1_scale=self.bmm1_scale, bmm2_scale=self.bmm2_scale,
                    causal=self.causal)


def _round_bf16(x32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.uint16).numpy()


def _round_e4m3fn(x32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _normal_bits(rng, shape, kv_dtype, scale=1.0, chunk_rows=1 << 14):
    """Draw N(0,1)*scale in float32 row-chunks and round to the storage type."""
    rows = shape[0]
    inner = tuple(shape[1:])
    dt = np.uint16 if kv_dtype == "bf16" else np.uint8
    out = np.empty(shape, dtype=dt)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0,) + inner, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[r0:r1] = _round_bf16(x) if kv_dtype == "bf16" else _round_e4m3fn(x)
    return out


def make_workload(name, *, seed, seq_lens=None, seq_len_range=None, seq_len_loguniform=None,
                  batch=None, num_heads, q_len=1, q_len_range=None, page_size,
                  kv_dtype="bf16", kv_value_scale=1.0, bmm1_scale, bmm2_scale=1.0,
                  causal=True, want_lse=False, max_seq_len=None, poison=True,
                  block_table_width=None):
    """Build one seeded workload.

    Exactly one of seq_lens (explicit list), seq_len_range (inclusive uniform
    integers) or seq_len_loguniform ((lo, hi): floor(exp(U(ln lo, ln hi)))) gives
    the KV lengths.  q_len_range (inclusive) makes a ragged packed launch with
    qo_indptr; otherwise every request has q_len rows (fixed layout).

    poison=True writes NaN into every cache slot no request may read: the tail
    slots of each request's last page and one extra padding page that unused
    block-table entries point at.  poison=False leaves them as drawn (finite).
    """
    rng = np.random.default_rng(seed)
    if seq_lens is not None:
        L = np.asarray(seq_lens, dtype=np.int64)
        B = len(L)
    elif seq_len_range is not None:
        B = batch
        L = rng.integers(seq_len_range[0], seq_len_range[1], endpoint=True, size=B).astype(np.int64)
    elif seq_len_loguniform is not None:
        B = batch
        lo, hi = seq_len_loguniform
        L = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
    else:
        raise ValueError("no seq_len spec")

    if q_len_range is not None:
        qb = rng.integers(q_len_range[0], q_len_range[1], endpoint=True, size=B).astype(np.int64)
        if seq_len_loguniform is not None:
            L = np.clip(L, np.maximum(seq_len_loguniform[0], qb), seq_len_loguniform[1])
        qo_indptr = np.concatenate([[0], np.cumsum(qb)]).astype(np.int32)
        max_q_len = int(q_len_range[1])
        q_len_fixed = max_q_len
    else:
        qb = np.full(B, q_len, dtype=np.int64)
        qo_indptr = None
        max_q_len = int(q_len)
        q_len_fixed = int(q_len)
    if causal:
        assert np.all(qb <= L), "causal launches need q_len <= seq_len"
    if max_seq_len is None:
        if seq_len_range is not None:
            max_seq_len = int(seq_len_range[1])
        elif seq_len_loguniform is not None:
            max_seq_len = int(seq_len_loguniform[1])
        else:
            max_seq_len = int(L.max())
    assert L.max() <= max_seq_len

    ps = int(page_size)
    pages_per_req = (L + ps - 1) // ps
    n_live = int(pages_per_req.sum())
    perm = rng.permutation(n_live).astype(np.int64)
    poison_id = n_live
    W = block_table_width or (max_seq_len + ps - 1) // ps
    bt = np.full((B, W), poison_id, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_req[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    R = int(qb.sum())
    H = int(num_heads)
    q_bits = _normal_bits(rng, (R, H, D_QK), "bf16")
    kv_bits = _normal_bits(rng, (n_live + 1, ps, D_QK), kv_dtype, scale=kv_value_scale)

    if poison:
        nan = BF16_NAN if kv_dtype == "bf16" else E4M3FN_NAN
        kv_bits[poison_id] = nan
        for b in range(B):
            tail = int(L[b]) % ps
            if tail:
                last_page = bt[b, int(pages_per_req[b]) - 1]
                kv_bits[last_page, tail:, :] = nan

    return Workload(name=name, q_bits=q_bits, kv_bits=kv_bits, kv_dtype=kv_dtype,
                    block_tables=bt, seq_lens=L.astype(np.int32), qo_indptr=qo_indptr,
                    q_len_fixed=q_len_fixed, max_seq_len=int(max_seq_len), max_q_len=max_q_len,
                    bmm1_scale=float(np.float32(bmm1_scale)), bmm2_scale=float(np.float32(bmm2_scale)),
                    causal=bool(causal), want_lse=bool(want_lse), poison_page=poison_id,
                    meta=dict(seed=seed))


INV_SQRT_192 = 1.0 / math.sqrt(192.0)
FP8_K_SCALE = 0.02

# The five workloads, in order: tiny bf16; DeepSeek-V3-shaped bf16 decode;
# uniform speculative 1+3 causal; ragged packed causal through qo_indptr;
# long-context fp8 KV.
WORKLOADS = {
    "tiny_bf16": dict(seed=1, seq_lens=[37, 100], num_heads=16, q_len=1, page_size=32,
                      bmm1_scale=INV_SQRT_192, bmm2_scale=1.0, causal=True, want_lse=True,
                      max_seq_len=100),
    "dsv3_bf16_decode": dict(seed=2, batch=64, seq_len_range=(1024, 8192), num_heads=128, q_len=1,
                             page_size=64, bmm1_scale=INV_SQRT_192, bmm2_scale=1.0, causal=True,
                             want_lse=False),
    "spec_1p3_causal": dict(seed=3, batch=32, seq_len_range=(2048, 6144), num_heads=128, q_len=4,
                            page_size=64, bmm1_scale=INV_SQRT_192, bmm2_scale=1.0, causal=True,
                            want_lse=False),
    "ragged_packed_causal": dict(seed=4, batch=128, seq_len_loguniform=(128, 32768), num_heads=16,
                                 q_len_range=(1, 8), page_size=32, bmm1_scale=INV_SQRT_192,
                                 bmm2_scale=1.0, causal=True, want_lse=False),
    "fp8_long_context": dict(seed=5, batch=8, seq_len_range=(65536, 131072), num_heads=128, q_len=2,
                             page_size=64, kv_dtype="fp8_e4m3fn", kv_value_scale=0.5,
                             bmm1_scale=FP8_K_SCALE * 1.0 * INV_SQRT_192, bmm2_scale=FP8_K_SCALE,
                             causal=True, want_lse=True),
}

WORKLOAD_ORDER = list(WORKLOADS)

# fp8-query variants (mla_decode_options_t.q_fp8): the named workload with its
# query rounded to E4M3FN (q_scale 1, so bmm1 is unchanged).
Q8_WORKLOADS = {"fp8_long_context_q8": "fp8_long_context"}

# Sparse top-k decode (the layout of mla_decode_options_t.sparse_top_k): a
# DeepSeek-shaped batch whose every query row attends to a top-k selection of
# its request.  The pages give no sparse configuration; this one takes the
# decode shape above (128 heads, page size 64, bf16 cache) with top-k 2048
# from requests longer than the list.
SPARSE_WORKLOADS = {
    "sparse_topk_decode": dict(seed=6, batch=64, seq_len_range=(4096, 16384), num_heads=128, q_len=1,
                               page_size=64, bmm1_scale=INV_SQRT_192, bmm2_scale=1.0, causal=False,
                               want_lse=False, top_k=2048, list_seed=7),
}


def named_sparse_workload(name, poison=True):
    """(workload, int32 lists [total_q, top_k]) of a named sparse workload."""
    spec = dict(SPARSE_WORKLOADS[name])
    top_k, list_seed = spec.pop("top_k"), spec.pop("list_seed")
    w = make_workload(name, poison=poison, **spec)
    return w, sparse_lists(w, top_k, list_seed)


def named_workload(name, poison=True, **overrides):
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    return make_workload(name, poison=poison, **spec)


def fp8_query_codes(w, inv_q_scale=1.0):
    """uint8 OCP E4M3FN codes of the workload's query times inv_q_scale, rounded
    by torch (RNE): the fp8 query a caller with per-tensor q_scale =
    1 / inv_q_scale would pass (that q_scale then belongs in bmm1_scale)."""
    import torch
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).to(torch.float32) * float(inv_q_scale)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def sparse_lists(w, top_k, seed, *, empty_frac=0.0, repeat_frac=0.0, empty_rows=()):
    """Seeded top-k lists for a workload's query rows: int32 [total_q, top_k]
    of flat cache-row ids (page * page_size + slot).

    Row r draws min(top_k, L_b) distinct positions of its request b uniformly
    (the selection an indexer would hand over; no trained indexer here), in
    random order, then fills the rest of the row with -1.  empty_frac of the
    listed entries are then overwritten with -1 and repeat_frac with a copy of
    another listed entry; rows in empty_rows are all -1.  Draw order: per row,
    the positions, then the empties, then the repeats.
    """
    rng = np.random.default_rng(seed)
    ps = w.page_size
    out = np.full((w.total_q, top_k), -1, dtype=np.int32)
    q_lens = w.q_lens()
    r = 0
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for _ in range(int(q_lens[b])):
            n = min(top_k, L)
            pos = rng.choice(L, size=n, replace=False)
            ids = w.block_tables[b, pos // ps].astype(np.int64) * ps + pos % ps
            out[r, :n] = ids
            if empty_frac > 0:
                out[r, np.flatnonzero(rng.random(n) < empty_frac)] = -1
            if repeat_frac > 0 and n > 1:
                dst = np.flatnonzero(rng.random(n) < repeat_frac)
                out[r, dst] = out[r, rng.integers(0, n, size=dst.size)]
            if r in empty_rows:
                out[r] = -1
            r += 1
    return out


def to_device_tensors(w, device="cuda"):
    """torch tensors for the binding: q bf16, kv bf16/fp8, int32 metadata."""
    import torch
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16)
    if w.kv_dtype == "bf16":
        kv = torch.from_numpy(w.kv_bits).view(torch.bfloat16)
    else:
        kv = torch.from_numpy(w.kv_bits).view(torch.float8_e4m3fn)
    t = dict(q=q, kv=kv, block_tables=torch.from_numpy(w.block_tables),
             seq_lens=torch.from_numpy(w.seq_lens),
             qo_indptr=None if w.qo_indptr is None else torch.from_numpy(w.qo_indptr))
    return {k: (None if v is None else v.to(device)) for k, v in t.items()}
