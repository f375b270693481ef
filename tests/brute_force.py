"""Scalar pure-Python attention for tiny shapes: an independent check of the oracle.

Every score, exponential and sum is a Python float operation in explicit loops
(math.exp / math.log); no NumPy arithmetic is used.  The definition followed is
"Deep Dive - FlashAttention", "Exact attention without an n x n workspace" and
"Causal 2.1 is the decode gotcha": softmax(scale * q.k) over allowed keys,
bottom-right causal alignment, consecutive GQA groups.  Unlike the oracle it
normalises by the plain sum of exp(score - rowmax) accumulated key by key and
writes lse as log(sum exp(score)) computed directly when scores are small.
"""
import math


def _row(qrow, keys, vals, allowed, scale, dv):
    scores = []
    for j in allowed:
        s = 0.0
        for a, b in zip(qrow, keys[j]):
            s += a * b
        scores.append(scale * s)
    if not scores:
        return [0.0] * dv, -math.inf
    top = scores[0]
    for s in scores:
        if s > top:
            top = s
    weights = [math.exp(s - top) for s in scores]
    total = 0.0
    for w in weights:
        total += w
    out = []
    for c in range(dv):
        acc = 0.0
        for w, j in zip(weights, allowed):
            acc += w * vals[j][c]
        out.append(acc / total)
    lse = top + math.log(total)
    return out, lse


def brute_attention(q, k, v, *, causal, scale, cu_q=None, cu_k=None, window=(-1, -1)):
    """q, k, v as nested Python lists in the dense [B,N,H,d] or packed [T,H,d] layout.

    window (left, right): key j is allowed for row i when i + nk - nq - left
    <= j <= i + nk - nq + right, a side of -1 being unbounded ("Deep Dive -
    FlashAttention", "Causal 2.1 is the decode gotcha").
    """
    if cu_q is None:
        seqs = [(b, 0, len(q[b]), 0, len(k[b])) for b in range(len(q))]
        getq = lambda b, i, h: q[b][i][h]
        getk = lambda b, j, h: k[b][j][h]
        getv = lambda b, j, h: v[b][j][h]
        hq_n = len(q[0][0])
        hkv_n = len(k[0][0])
        dv = len(v[0][0][0])
    else:
        seqs = [(s, cu_q[s], cu_q[s + 1] - cu_q[s], cu_k[s], cu_k[s + 1] - cu_k[s])
                for s in range(len(cu_q) - 1)]
        getq = lambda b, i, h: q[i][h]
        getk = lambda b, j, h: k[j][h]
        getv = lambda b, j, h: v[j][h]
        hq_n = len(q[0])
        hkv_n = len(k[0])
        dv = len(v[0][0])
    group = hq_n // hkv_n
    out = {}
    lse = {}
    for b, qo, nq, ko, nk in seqs:
        for h in range(hq_n):
            kvh = h // group
            keys = [getk(b, ko + j, kvh) for j in range(nk)]
            vals = [getv(b, ko + j, kvh) for j in range(nk)]
            for i in range(nq):
                c = i + nk - nq
                allowed = [j for j in range(nk)
                           if ((not causal) or j <= c)
                           and (window[0] < 0 or j >= c - window[0])
                           and (window[1] < 0 or j <= c + window[1])]
                o, s = _row(getq(b, qo + i, h), keys, vals, allowed, scale, dv)
                out[(b, i, h)] = o
                lse[(b, i, h)] = s
    return out, lse
