"""Plain float64 definition of batched paged MLA decode (oracle; test infrastructure).

What is computed, restated from the pages:

* FlashInfer docs, "prims_ts_batch_decode_with_kv_cache_mla", layout and mask
  paragraph: a query row is 576 wide (512 latent dims followed by 64 RoPE
  dims); the cache is a stack of pages of page_size rows of 576; request b owns
  the pages listed, in order, in row b of block_tables and its live length is
  seq_lens[b]; the query is either fixed [B, SQ, H, 576] or packed
  [total_q, H, 576] with B+1 cumulative offsets qo_indptr; the causal mask is
  aligned to the bottom-right, so query row i of request b sees KV rows up to
  and including seq_lens[b] - q_len[b] + i.  mask_type 'dense' lets every row
  see all seq_lens[b] rows.
* FlashInfer issue #3131, launcher and run_func excerpts: the same cache tensor
  is passed as K and as V (one latent head shared by all query heads), so V is
  the first kv_lora_rank = 512 dims of the very rows used as K.
* FlashInfer PR #1248 (Highlights) and vLLM "FlashInferMLAImpl.forward_mqa":
  bmm1_scale is the whole multiplier applied to q.k (softmax scale times the
  q and k quantisation scales), bmm2_scale multiplies the attention output
  (the k/v quantisation scale).  The kernel re-derives nothing from them.
* vLLM "FlashInferMLAImpl" class attributes: the returned LSE uses the
  natural logarithm.  It is taken over the bmm1-scaled logits and does not
  include bmm2_scale.

Readings where the pages are silent (each also listed in the design notes):
positions past seq_lens[b] and block-table entries past ceil(L/page_size) are
never read; an LSE is also produced for packed launches; the static maxima
(max_seq_len, max_seq_len_q) bound sizes only and never change the result.

The computation is one request at a time: gather the request's rows in token
order, one matrix product for the logits, an explicit mask, a max-subtracted
softmax, one matrix product for P.V.  No blocking, no online softmax, no
reordering beyond what those library products do internally.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_bits_to_f64

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE


@dataclass
class MlaProblem:
    """Raw inputs of one decode launch, as storage bits and int32 metadata.

    q_bits        uint16 [R, H, 576]  bf16 codes (fixed [B, SQ, H, 576] flattened)
    kv_bits       uint16 (bf16) or uint8 (fp8 e4m3fn) [num_pages, page_size, 576]
    kv_dtype      "bf16" or "fp8_e4m3fn"
    block_tables  int32 [B, W]
    seq_lens      int32 [B]
    qo_indptr     int32 [B+1] or None (then every request has q_len_fixed rows)
    sinks         float [H] or None: per-head sink logits (natural-log units, on
                  the scale of bmm1_scale * q.k), one more term of every softmax
                  denominator with no value row
    q_dtype       "bf16" (q_bits uint16 codes) or "fp8_e4m3fn" (q_bits uint8
                  codes: a query quantised to fp8 with its q_scale folded into
                  bmm1_scale, FlashInfer PR #1248 / vLLM forward_mqa)
    """

    q_bits: np.ndarray
    kv_bits: np.ndarray
    kv_dtype: str
    block_tables: np.ndarray
    seq_lens: np.ndarray
    qo_indptr: Optional[np.ndarray]
    q_len_fixed: int
    bmm1_scale: float
    bmm2_scale: float
    causal: bool
    sinks: Optional[np.ndarray] = None
    q_dtype: str = "bf16"

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_heads(self):
        return int(self.q_bits.shape[1])

    @property
    def page_size(self):
        return int(self.kv_bits.shape[1])

    def request_rows(self, b):
        """(first query row r_b, query length q_b) of request b."""
        if self.qo_indptr is None:
            return b * self.q_len_fixed, self.q_len_fixed
        lo = int(self.qo_indptr[b])
        hi = int(self.qo_indptr[b + 1])
        return lo, hi - lo


def _decode_kv(problem, bits):
    if problem.kv_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if problem.kv_dtype == "fp8_e4m3fn":
        return e4m3fn_bits_to_f64(bits)
    raise ValueError(f"unknown kv dtype {problem.kv_dtype!r}")


def _decode_q(problem, bits):
    if problem.q_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if problem.q_dtype == "fp8_e4m3fn":
        return e4m3fn_bits_to_f64(bits)
    raise ValueError(f"unknown query dtype {problem.q_dtype!r}")


def visible_count(L, q_b, i, causal):
    """Number of KV rows query row i of a request sees (rows 0 .. n-1).

    Bottom-right causal alignment: the last query row sees all L rows and each
    earlier row one fewer; dense: every row sees L.
    """
    return (L - q_b + i + 1) if causal else L


def gather_request_rows(problem, b):
    """float64 [L, 576]: request b's cached rows in token order.

    Token t lives in page block_tables[b, t // page_size], slot t % page_size.
    Only the first ceil(L / page_size) block-table entries are touched.
    """
    L = int(problem.seq_lens[b])
    ps = problem.page_size
    t = np.arange(L)
    pages = problem.block_tables[b, t // ps].astype(np.int64)
    rows = problem.kv_bits[pages, t % ps, :]
    return _decode_kv(problem, rows)


def _check_request(problem, b):
    r_b, q_b = problem.request_rows(b)
    L = int(problem.seq_lens[b])
    assert L >= 1, f"request {b}: seq_len must be positive"
    assert q_b >= 1, f"request {b}: query length must be positive"
    if problem.causal:
        assert q_b <= L, f"request {b}: causal query length exceeds seq_len"
    return r_b, q_b, L


def _masked_logits(problem, b, Kb, lo=0, hi=None):
    """Scaled logits [q_b*H, L] of request b with invisible entries at -inf."""
    r_b, q_b, L = _check_request(problem, b)
    H = problem.num_heads
    if hi is None:
        hi = L
    Q = _decode_q(problem, problem.q_bits[r_b:r_b + q_b]).reshape(q_b * H, D_QK)
    S = (Q @ Kb.T) * float(problem.bmm1_scale)
    n = np.array([visible_count(L, q_b, i, problem.causal) for i in range(q_b)])
    n_rows = np.repeat(n, H)  # row index = i*H + h
    j = np.arange(L)
    visible = (j[None, :] < n_rows[:, None]) & (j[None, :] >= lo) & (j[None, :] < hi)
    return np.where(visible, S, -np.inf), visible


def reference_decode(problem, requests=None):
    """Full decode.  Returns (out float64 [R, H, 512], lse float64 [R, H]).

    With sinks, each (row, head) softmax has one more term exp(sink_h) in its
    denominator and none in the numerator; lse is then ln of that whole
    denominator (FlashInfer issue #3131, launcher excerpt: attention_sinks;
    the pages give no formula, this is the plain reading).

    Rows of requests not listed in `requests` are left NaN (lets tests sample
    a few requests of a large launch).
    """
    H = problem.num_heads
    R = problem.q_bits.shape[0]
    out = np.full((R, H, D_LATENT), np.nan)
    lse = np.full((R, H), np.nan)
    reqs = range(problem.batch) if requests is None else requests
    for b in reqs:
        r_b, q_b, L = _check_request(problem, b)
        Kb = gather_request_rows(problem, b)
        S, _ = _masked_logits(problem, b, Kb)
        m = S.max(axis=1, keepdims=True)
        if problem.sinks is not None:
            # the sink is one more logit of the softmax, attached to a zero value row
            sink = np.tile(np.asarray(problem.sinks, dtype=np.float64), q_b)[:, None]  # row index = i*H + h
            m = np.maximum(m, sink)
        e = np.exp(S - m)
        Z = e.sum(axis=1, keepdims=True)
        if problem.sinks is not None:
            Z = Z + np.exp(sink - m)
        P = e / Z
        O = (P @ Kb[:, :D_LATENT]) * float(problem.bmm2_scale)
        out[r_b:r_b + q_b] = O.reshape(q_b, H, D_LATENT)
        lse[r_b:r_b + q_b] = (m[:, 0] + np.log(Z[:, 0])).reshape(q_b, H)
    return out, lse


def reference_partial(problem, b, lo, hi):
    """Attention of request b restricted to KV positions [lo, hi).

    Returns (O float64 [q_b, H, 512], lse float64 [q_b, H]): O is the softmax-
    normalised P.V over the visible positions inside the range, without
    bmm2_scale; rows with nothing visible in the range get O = 0, lse = -inf.
    """
    r_b, q_b, L = _check_request(problem, b)
    H = problem.num_heads
    Kb = gather_request_rows(problem, b)
    S, visible = _masked_logits(problem, b, Kb, lo, hi)
    any_vis = visible.any(axis=1)
    m = np.where(any_vis, S.max(axis=1), 0.0)
    e = np.where(visible, np.exp(S - m[:, None]), 0.0)
    Z = e.sum(axis=1)
    Zs = np.where(any_vis, Z, 1.0)
    O = (e / Zs[:, None]) @ Kb[:, :D_LATENT]
    lse = np.where(any_vis, m + np.log(Zs), -np.inf)
    return O.reshape(q_b, H, D_LATENT), lse.reshape(q_b, H)


def merge_partials(parts, bmm2_scale):
    """Combine range partials [(O_s, lse_s), ...] of the same rows.

    With M = max_s lse_s and w_s = exp(lse_s - M): lse = M + ln(sum_s w_s) and
    out = bmm2_scale * sum_s w_s O_s / sum_s w_s.  This is the identity that
    lets a long KV range be cut into pieces (the multi-CTA-KV split of vLLM's
    "FlashInferMLAImpl" and the per-rank partials of its DCP path).
    """
    lses = np.stack([p[1] for p in parts])  # [S, ...]
    Os = np.stack([p[0] for p in parts])    # [S, ..., 512]
    M = lses.max(axis=0)
    w = np.exp(lses - M[None])
    W = w.sum(axis=0)
    out = float(bmm2_scale) * (w[..., None] * Os).sum(axis=0) / W[..., None]
    return out, M + np.log(W)


def reference_dcp_partial(problem, rank, world):
    """Sequence-sharded partial of every request: the share of rank `rank` of
    `world` ranks, which hold the cached rows round-robin (global position t on
    rank t mod world, in order).  Causal limits come from the global positions:
    query row i of request b sees global positions t < L - q_b + i + 1.

    Returns (out float64 [R, H, 512], lse float64 [R, H]) over the rank's rows:
    out = bmm2 * softmax-normalised P.V and lse = ln sum exp(s) over the
    visible rows the rank holds; a row that sees none of them gets out = 0 and
    lse = -inf.  Merging every rank's partial with merge_partials (bmm2 = 1,
    since each partial already carries it) gives the full decode (vLLM docs,
    "FlashInferMLAImpl", forward_mqa: DCP passes cp_world, cp_rank and the
    global causal lengths and consumes the natural-log LSE).

    Sinks, if any, belong to rank 0's partial alone: a sink is one softmax
    term per (row, head), so the merged result counts it once.  A rank-0 row
    that sees no rows then has out = 0 and lse = sink.
    """
    H = problem.num_heads
    R = problem.q_bits.shape[0]
    out = np.zeros((R, H, D_LATENT))
    lse = np.full((R, H), -np.inf)
    for b in range(problem.batch):
        r_b, q_b, L = _check_request(problem, b)
        Kb = gather_request_rows(problem, b)
        S, visible = _masked_logits(problem, b, Kb)
        mine = (np.arange(L) % world) == rank
        visible = visible & mine[None, :]
        S = np.where(visible, S, -np.inf)
        if problem.sinks is not None and rank == 0:
            # the sink as one more logit, attached to a zero value row
            sink = np.tile(np.asarray(problem.sinks, dtype=np.float64), q_b)  # row index = i*H + h
        else:
            sink = np.full(S.shape[0], -np.inf)
        any_term = visible.any(axis=1) | (sink > -np.inf)
        m = np.where(any_term, np.maximum(S.max(axis=1), sink), 0.0)
        e = np.where(visible, np.exp(S - m[:, None]), 0.0)
        Z = e.sum(axis=1) + np.where(sink > -np.inf, np.exp(sink - m), 0.0)
        Zs = np.where(any_term, Z, 1.0)
        O = (e / Zs[:, None]) @ Kb[:, :D_LATENT] * float(problem.bmm2_scale)
        out[r_b:r_b + q_b] = O.reshape(q_b, H, D_LATENT)
        lse[r_b:r_b + q_b] = np.where(any_term, m + np.log(Zs), -np.inf).reshape(q_b, H)
    return out, lse
