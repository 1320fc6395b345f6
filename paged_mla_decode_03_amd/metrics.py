"""Algorithmic work of one paged MLA decode launch (for throughput and roofline).

Counts only what the method must move or compute, independent of how the
kernels split the work:
  bytes = sum_b L_b*576*e_kv (cache rows read once) + R*H*576*2 (q)
          + R*H*512*2 (out) + R*H*4 (lse, if returned)
          + 4*sum_b ceil(L_b/ps) (block-table entries) + 4*B (seq_lens)
          + 4*(B+1) (qo_indptr, if packed)
  flops = 2*(576+512)*H * sum_b sum_i n_{b,i}, where n_{b,i} is the number of
          KV rows query row i of request b sees (L_b - q_b + i + 1 when
          causal, L_b when dense); softmax work is not counted.
KV-tokens = sum_b L_b (each cached row once per request).

Sparse top-k layout: every query row r gathers its n_r live list entries, so
  bytes = sum_r n_r*576*e_kv + R*H*576*2 + R*H*512*2 (+ R*H*4 lse)
          + 4*R*K (the lists)
  flops = 2*(576+512)*H * sum_r n_r
  KV-tokens = sum_r n_r (a cache row once per query row that lists it).
"""

import numpy as np

D_QK = 576
D_V = 512

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}

# Share of the decode flops in QK^T (576 of the 1088 dims per visible pair):
# with an fp8 query that part runs at the fp8 peak and P.V at the bf16 one.
QK_SHARE = 576.0 / 1088.0


def mixed_mfma_peak():
    """TFLOP/s of the whole decode at the matrix-core peaks when QK^T is fp8 and
    P.V bf16: F / (F_qk / P_fp8 + F_pv / P_bf16)."""
    return 1.0 / (QK_SHARE / PEAK_MFMA_TFLOPS["fp8"] + (1.0 - QK_SHARE) / PEAK_MFMA_TFLOPS["bf16"])


def workload_counts(seq_lens, q_lens, num_heads, page_size, kv_bytes, causal, want_lse, packed):
    L = np.asarray(seq_lens, dtype=np.int64)
    q = np.asarray(q_lens, dtype=np.int64)
    B = L.size
    R = int(q.sum())
    H = int(num_heads)
    if causal:
        visible = int((q * L - q * (q - 1) // 2).sum())  # sum_i (L - q + i + 1)
    else:
        visible = int((q * L).sum())
    nbytes = (int(L.sum()) * D_QK * kv_bytes + R * H * D_QK * 2 + R * H * D_V * 2 + (R * H * 4 if want_lse else 0)
              + 4 * int(((L + page_size - 1) // page_size).sum()) + 4 * B + (4 * (B + 1) if packed else 0))
    flops = 2 * (D_QK + D_V) * H * visible
    return dict(kv_tokens=int(L.sum()), bytes=int(nbytes), flops=int(flops), rows=R, visible_pairs_per_head=visible)


def counts_for_workload(w):
    return workload_counts(w.seq_lens, w.q_lens(), w.num_heads, w.page_size, 2 if w.kv_dtype == "bf16" else 1,
                           w.causal, w.want_lse, w.qo_indptr is not None)


def sparse_counts(lists, top_k, num_heads, kv_bytes, want_lse):
    lists = np.asarray(lists)[:, :top_k]
    R = int(lists.shape[0])
    H = int(num_heads)
    live = int((lists >= 0).sum())
    nbytes = live * D_QK * kv_bytes + R * H * D_QK * 2 + R * H * D_V * 2 + (R * H * 4 if want_lse else 0) + 4 * R * top_k
    return dict(kv_tokens=live, bytes=int(nbytes), flops=int(2 * (D_QK + D_V) * H * live), rows=R)
