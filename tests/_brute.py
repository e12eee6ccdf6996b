"""Brute-force attention with pure-Python loops, for tiny inputs only.

An independent restatement of the definition used to pin the numpy oracle: no
numpy, no vectorisation, no shared helper. Per query row i of a head it forms
every logit s_ij = scale * sum_c q_ic k_jc, optionally soft-caps it, adds an
optional bias b_ij, keeps the
keys inside the bottom-right-aligned window (plus the first ``sink_size`` keys
when the right bound reaches them), and returns
O_i = sum_j exp(s_ij) v_j / D_i and LSE_i = log D_i with
D_i = sum_j exp(s_ij) + exp(sink) (the sink term only when ``sink`` is given),
with O_i = 0 and LSE_i = log(exp(sink)) or -inf when no key is visible.
"""

import math


def brute_head(q, k, v, scale, softcap=0.0, wl=-1, wr=-1, dv=None, sink_size=0, sink=None, bias=None):
    lq, lk = len(q), len(k)
    if dv is None:
        dv = len(v[0]) if lk else len(q[0])
    out, lse = [], []
    for i in range(lq):
        logits = []
        for j in range(lk):
            lo_ok = wl < 0 or j >= i + (lk - lq) - wl or j < sink_size
            hi_ok = wr < 0 or j <= i + (lk - lq) + wr
            if not (lo_ok and hi_ok):
                continue
            s = 0.0
            for c in range(len(q[i])):
                s += q[i][c] * k[j][c]
            s *= scale
            if softcap > 0:
                s = softcap * math.tanh(s / softcap)
            if bias is not None:
                s += bias[i][j]
            logits.append((j, s))
        if not logits:
            out.append([0.0] * dv)
            lse.append(-math.inf if sink is None else sink)
            continue
        big = max(s for _, s in logits)
        if sink is not None:
            big = max(big, sink)
        w = [(j, math.exp(s - big)) for j, s in logits]
        tot = sum(x for _, x in w)
        if sink is not None:
            tot += math.exp(sink - big)
        row = [0.0] * dv
        for j, x in w:
            for c in range(dv):
                row[c] += x * v[j][c]
        out.append([r / tot for r in row])
        lse.append(big + math.log(tot))
    return out, lse
