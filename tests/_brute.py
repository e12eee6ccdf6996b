"""Brute-force attention with pure-Python loops, for tiny inputs only.

An independent restatement of the definition used to pin the numpy oracle: no
numpy, no vectorisation, no shared helper. Per query row i of a head it forms
every logit s_ij = scale * sum_c q_ic k_jc, optionally soft-caps it, keeps the
keys inside the bottom-right-aligned window, and returns
O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij) and LSE_i = log sum_j exp(s_ij),
with O_i = 0 and LSE_i = -inf when no key is visible.
"""

import math


def brute_head(q, k, v, scale, softcap=0.0, wl=-1, wr=-1, dv=None):
    lq, lk = len(q), len(k)
    if dv is None:
        dv = len(v[0]) if lk else len(q[0])
    out, lse = [], []
    for i in range(lq):
        logits = []
        for j in range(lk):
            lo_ok = wl < 0 or j >= i + (lk - lq) - wl
            hi_ok = wr < 0 or j <= i + (lk - lq) + wr
            if not (lo_ok and hi_ok):
                continue
            s = 0.0
            for c in range(len(q[i])):
                s += q[i][c] * k[j][c]
            s *= scale
            if softcap > 0:
                s = softcap * math.tanh(s / softcap)
            logits.append((j, s))
        if not logits:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        big = max(s for _, s in logits)
        w = [(j, math.exp(s - big)) for j, s in logits]
        tot = sum(x for _, x in w)
        row = [0.0] * dv
        for j, x in w:
            for c in range(dv):
                row[c] += x * v[j][c]
        out.append([r / tot for r in row])
        lse.append(big + math.log(tot))
    return out, lse
