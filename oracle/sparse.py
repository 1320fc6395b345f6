"""Plain float64 definition of sparse (top-k) MLA decode (oracle; test infrastructure).

FlashInfer's MLA decode entry points take a `sparse_mla_top_k` count next to
`block_tables` (FlashInfer issue #3131: the `trtllm_batch_decode_with_kv_cache_mla`
Python signature and the `trtllm_paged_attention_decode` launcher signature).
The pages give no index layout; the reading taken here (also listed in the
design notes):

* with top-k K > 0, `block_tables` holds K int32 entries per query row
  (row-major [R, K], R = rows of the query);
* an entry is a flat token index t into the cache seen as
  [num_pages * page_size, 576] rows (page t // page_size, slot t % page_size);
  a negative entry is an empty slot;
* query row r attends, for every head, to exactly the rows its entries list:
  no causal or length mask (the list is the visible set); an entry listed
  twice is two softmax terms;
* everything else is the dense definition: logits bmm1_scale * q.k over all
  576 dims, max-subtracted softmax, P.V over the first 512 dims times
  bmm2_scale, natural-log LSE without bmm2; a sink, if given, is one more
  denominator term per (row, head);
* a (row, head) with no term at all gets out = 0 and lse = -inf.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_bits_to_f64

D_LATENT = 512
D_QK = 576


def _decode(kv_dtype, bits):
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if kv_dtype == "fp8_e4m3fn":
        return e4m3fn_bits_to_f64(bits)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def reference_sparse_decode(q_bits, kv_bits, kv_dtype, indices, bmm1_scale, bmm2_scale, sinks=None):
    """Sparse decode.  Returns (out float64 [R, H, 512], lse float64 [R, H]).

    q_bits   uint16 [R, H, 576] bf16 codes
    kv_bits  [num_pages, page_size, 576] storage codes
    indices  int32 [R, K] flat token indices, negative = empty
    sinks    float [H] or None
    """
    R, H, _ = q_bits.shape
    ps = kv_bits.shape[1]
    indices = np.asarray(indices)
    assert indices.ndim == 2 and indices.shape[0] == R
    out = np.zeros((R, H, D_LATENT))
    lse = np.full((R, H), -np.inf)
    for r in range(R):
        tok = indices[r][indices[r] >= 0].astype(np.int64)
        K = _decode(kv_dtype, kv_bits[tok // ps, tok % ps, :])          # [n, 576], listing order
        Q = bf16_bits_to_f64(q_bits[r])                                 # [H, 576]
        S = (Q @ K.T) * float(bmm1_scale)                               # [H, n]
        sink = (np.asarray(sinks, dtype=np.float64) if sinks is not None
                else np.full(H, -np.inf))
        if tok.size == 0 and sinks is None:
            continue
        m = np.maximum(S.max(axis=1) if tok.size else np.full(H, -np.inf), sink)
        e = np.exp(S - m[:, None])
        Z = e.sum(axis=1) + np.where(sink > -np.inf, np.exp(sink - m), 0.0)
        live = Z > 0
        Zs = np.where(live, Z, 1.0)
        out[r] = (e / Zs[:, None]) @ K[:, :D_LATENT] * float(bmm2_scale)
        lse[r] = np.where(live, m + np.log(Zs), -np.inf)
    return out, lse
