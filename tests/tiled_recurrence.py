"""A test-only float64 tiled forward, built on the state merge of online softmax.

Each key block on its own has a state (m, l, u): its largest score m, the sum
l of exp(s - m) and the sum u of exp(s - m) v.  Two states combine exactly
into the state of their union by bringing both to the larger maximum
("Flash Attention: A Complete Architectural Autopsy", "The Online Softmax
Recurrence": the factor exp(m_old - m_new) applied to the running sums;
"Deep Dive - FlashAttention", "Online softmax is what makes the tiles
exact").  A block with no allowed key has the empty state, which changes
nothing; a row whose blocks are all empty returns zeros.

This is separate code from the oracle (it never calls it); tests compare the
two to pin the oracle's two-pass softmax to the streaming identity.
"""
import math

import numpy as np

EMPTY = (-math.inf, 0.0, None)


def block_state(scores, values):
    """(m, l, u) of one key block; EMPTY when no score is finite."""
    ok = np.isfinite(scores)
    if not ok.any():
        return EMPTY
    top = float(scores[ok].max())
    weights = np.zeros(len(scores))
    weights[ok] = np.exp(scores[ok] - top)
    return top, float(weights.sum()), weights @ values


def merge_states(run, blk):
    """The state of two blocks taken together, and the factor the running
    state was multiplied by (0 when it was empty)."""
    m_run, l_run, u_run = run
    m_blk, l_blk, u_blk = blk
    if m_blk == -math.inf:
        return run, 1.0
    if m_run == -math.inf:
        return (m_blk, l_blk, u_blk.copy()), 0.0
    top = max(m_run, m_blk)
    f_run, f_blk = math.exp(m_run - top), math.exp(m_blk - top)
    return (top, f_run * l_run + f_blk * l_blk, f_run * u_run + f_blk * u_blk), f_run


def tiled_row(scores, values, tile, trace=None):
    """One query row: scores [n] (finite or -inf), values [n, dv].  Returns
    (out, lse); `trace` collects the running state after each non-empty block."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    state = EMPTY
    for start in range(0, len(scores), tile):
        blk = block_state(scores[start:start + tile], values[start:start + tile])
        if blk is EMPTY:
            continue
        state, factor = merge_states(state, blk)
        if trace is not None:
            trace.append(dict(m=state[0], l=state[1], u=state[2].copy(), alpha=factor))
    m, l, u = state
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
