"""A test-only float64 tiled forward, written from the online-softmax recurrence.

"Flash Attention: A Complete Architectural Autopsy", "The Online Softmax
Recurrence": per key block t, m_t = max(m_{t-1}, rowmax S_t),
P_t = exp(S_t - m_t), l_t = exp(m_{t-1} - m_t) l_{t-1} + rowsum P_t,
O_t = exp(m_{t-1} - m_t) O_{t-1} + P_t V_t, and finally O = O / l.
"Deep Dive - FlashAttention", "Online softmax is what makes the tiles exact":
start from m = -inf, l = 0, u = 0 and skip a block with no allowed key before
any exponential; an entirely masked row returns zeros.

This is separate code from the oracle (it never calls it); tests compare the
two to pin the oracle's two-pass softmax to the streaming identity.
"""
import math

import numpy as np


def tiled_row(scores, values, tile, trace=None):
    """One query row: scores [n] (finite or -inf), values [n, dv]."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m, l = -math.inf, 0.0
    u = np.zeros(values.shape[1])
    for start in range(0, len(scores), tile):
        s = scores[start:start + tile]
        if not np.any(np.isfinite(s)):
            continue
        m_new = max(m, float(s.max()))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        w = np.exp(s - m_new)
        l = alpha * l + float(w.sum())
        u = alpha * u + w @ values[start:start + tile]
        if trace is not None:
            trace.append(dict(m=m_new, l=l, u=u.copy(), alpha=alpha))
        m = m_new
    if l == 0.0:
        return np.zeros(values.shape[1]), -math.inf
    return u / l, m + math.log(l)


def tiled_attention(Q, K, V, scale, tile, keep=None):
    """All rows of one head, each through tiled_row."""
    S = scale * (np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    outs, lses = [], []
    for i in range(S.shape[0]):
        o, s = tiled_row(S[i], V, tile)
        outs.append(o)
        lses.append(s)
    return np.array(outs), np.array(lses)


def combine_partials(outs, lses):
    """Merge normalised partial outputs with their lse (float64, test-only).

    "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
    "Why decode starves the GPU": each partial output is weighted by
    exp(lse_i - lse_total), lse_total being the log of the summed exp(lse_i).
    Partials with lse = -inf carry no weight.
    """
    lses = np.asarray(lses, dtype=np.float64)
    finite = np.isfinite(lses)
    if not finite.any():
        return np.zeros_like(np.asarray(outs[0], dtype=np.float64)), -math.inf
    top = lses[finite].max()
    total = top + math.log(sum(math.exp(x - top) for x in lses[finite]))
    out = np.zeros_like(np.asarray(outs[0], dtype=np.float64))
    for o, x in zip(outs, lses):
        if np.isfinite(x):
            out = out + math.exp(x - total) * np.asarray(o, dtype=np.float64)
    return out, total
