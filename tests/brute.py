"""Pure-Python brute force of the GDA core on tiny inputs (no numpy in the arithmetic).

Every score, exponential and weighted sum is a Python float operation over
explicitly enumerated (query, key) pairs. It is used only on inputs of a few
thousand elements.

Head maps are passed in explicitly, so a test can state them from the workload
descriptions rather than from a formula.
"""
from __future__ import annotations

import math


def attention_row(q, keys, vals):
    """softmax(q.k / sqrt(len(q))) weighted mean of vals, over the given (key, value) rows."""
    if not keys:
        return [0.0] * len(vals[0]) if vals else []
    scale = 1.0 / math.sqrt(len(q))
    z = [scale * sum(qd * kd for qd, kd in zip(q, k)) for k in keys]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    tot = sum(w)
    dv = len(vals[0])
    return [sum(w[s] * vals[s][e] for s in range(len(vals))) / tot for e in range(dv)]


def gda_fwd(q_sig, q_noise, k, v, lam, gate, window, kv_sig, kv_noise, group):
    """Nested lists: q_sig[b][t][i][d], q_noise[b][t][j][d], k[b][s][h][d], v[b][s][h][e],
    lam[b][t][i], gate[b][t][i][e]. Returns out[b][t][i][e]."""
    out = []
    for b in range(len(q_sig)):
        L = len(q_sig[b])
        rows = []
        for t in range(L):
            vis = [s for s in range(L) if s <= t and (window == 0 or t - s <= window - 1)]
            heads = []
            S = len(q_sig[b][t])
            for i in range(S):
                hs = kv_sig(i)
                j = group(i)
                hn = kv_noise(j)
                HS = attention_row(q_sig[b][t][i], [k[b][s][hs] for s in vis],
                                   [v[b][s][hs] for s in vis])
                HN = attention_row(q_noise[b][t][j], [k[b][s][hn] for s in vis],
                                   [v[b][s][hn] for s in vis])
                li = lam[b][t][i]
                heads.append([gate[b][t][i][e] * (HS[e] - li * HN[e]) for e in range(len(HS))])
            rows.append(heads)
        out.append(rows)
    return out
