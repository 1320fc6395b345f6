"""Brute-force attention for tiny inputs (oracle self-check; test infrastructure).

Pure-Python loops over (query row, head, key, dim) on a dense, un-paged key
matrix per request.  It shares nothing with oracle.mla beyond the meaning of
the inputs: no paging, no NumPy products, its own mask and softmax.  Used only
to pin the oracle on inputs small enough for loops.
"""

import math


def brute_attention(q_rows, k_rows, bmm1_scale, bmm2_scale, causal, d_v=512):
    """One request.

    q_rows  list over query rows i of list over heads h of a list of floats (len D)
    k_rows  list over KV positions j of a list of floats (len D); V row j is k_rows[j][:d_v]
    Returns (out[i][h][c], lse[i][h]) as nested lists.
    """
    q_len = len(q_rows)
    L = len(k_rows)
    out, lse = [], []
    for i in range(q_len):
        n = L - q_len + i + 1 if causal else L
        out_i, lse_i = [], []
        for qh in q_rows[i]:
            logits = []
            for j in range(n):
                acc = 0.0
                for d in range(len(qh)):
                    acc += qh[d] * k_rows[j][d]
                logits.append(acc * bmm1_scale)
            mx = max(logits)
            ws = [math.exp(x - mx) for x in logits]
            z = sum(ws)
            o = [0.0] * d_v
            for j in range(n):
                p = ws[j] / z
                row = k_rows[j]
                for c in range(d_v):
                    o[c] += p * row[c]
            out_i.append([v * bmm2_scale for v in o])
            lse_i.append(mx + math.log(z))
        out.append(out_i)
        lse.append(lse_i)
    return out, lse
