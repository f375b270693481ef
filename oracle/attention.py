"""Plain fp64 attention: the definition, materialised, on the CPU.

Test infrastructure only (see the package docstring).  Nothing here is blocked,
fused or reordered beyond the definition: for one query head h and its key/value
head, S = scale * Q K^T, masked entries set to -inf, P = softmax over each row,
out = P V and lse = log of the row's sum of exp(S).  Rows are processed in
blocks of at most ROW_BLOCK rows only to bound memory; softmax is row-wise, so
blocking rows leaves every row's result unchanged.
"""
import numpy as np

ROW_BLOCK = 2048


def kv_head_for_queries(num_heads_q, num_heads_kv):
    """K/V head of each query head, as a list.

    "Deep Dive - FlashAttention", "The public interface is several kernels":
    query heads are shared out in consecutive equal groups (six query heads
    over two K/V heads give 0,0,0,1,1,1), so query head h reads K/V head
    floor(h * Hkv / Hq); "FlashAttention: Part 1", section 4.1: Hkv must
    divide Hq.  Non-integer or non-positive counts are refused.
    """
    counts = (num_heads_q, num_heads_kv)
    if not all(isinstance(c, (int, np.integer)) and not isinstance(c, bool) and c >= 1 for c in counts):
        raise ValueError(f"need integer head counts >= 1, got {counts}")
    if num_heads_q % num_heads_kv != 0:
        raise ValueError(f"{num_heads_kv} K/V heads do not split {num_heads_q} query heads into equal groups")
    return [int(x) for x in (np.arange(num_heads_q) * num_heads_kv) // num_heads_q]


def causal_keep(seqlen_q, seqlen_k):
    """Bottom-right aligned causal keep-mask, shape [seqlen_q, seqlen_k].

    "Deep Dive - FlashAttention", "Causal 2.1 is the decode gotcha": from
    FlashAttention 2.1 on, query row i may see key j exactly when
    j <= i + seqlen_k - seqlen_q.  Rows with no allowed key exist when
    seqlen_q > seqlen_k.
    """
    i = np.arange(seqlen_q)[:, None]
    j = np.arange(seqlen_k)[None, :]
    return j <= i + (seqlen_k - seqlen_q)


def window_keep(seqlen_q, seqlen_k, left, right):
    """Local-window keep-mask, shape [seqlen_q, seqlen_k].

    "Deep Dive - FlashAttention", "Causal 2.1 is the decode gotcha": a finite
    window (left, right) lets query row i see key j when
    i + seqlen_k - seqlen_q - left <= j <= i + seqlen_k - seqlen_q + right
    (clipped to the real keys); a side given as -1 is unbounded.
    """
    i = np.arange(seqlen_q)[:, None]
    j = np.arange(seqlen_k)[None, :]
    c = i + (seqlen_k - seqlen_q)
    keep = np.ones((seqlen_q, seqlen_k), dtype=bool)
    if left >= 0:
        keep &= j >= c - left
    if right >= 0:
        keep &= j <= c + right
    return keep


def _keep(seqlen_q, seqlen_k, causal, window):
    """Combined keep-mask (None when everything is kept): causal masking
    further restricts a window's set (same section)."""
    left, right = window
    keep = None
    if causal:
        keep = causal_keep(seqlen_q, seqlen_k)
    if left >= 0 or right >= 0:
        w = window_keep(seqlen_q, seqlen_k, left, right)
        keep = w if keep is None else keep & w
    return keep


def _attend_rows(Q, K, V, scale, keep):
    """Attention for a block of query rows against one key/value head.

    Q [n, d], K [m, d], V [m, dv] float64; keep [n, m] bool or None.
    Returns out [n, dv] and lse [n] (natural log).

    Softmax is taken in its numerically safe form, exp(x - max) / sum exp(x - max)
    ("FlashAttention: Part 1", section 2.2; "Flash Attention: A Complete
    Architectural Autopsy", "The Online Softmax Recurrence").  lse_i = m_i +
    log(l_i) ("Deep Dive - FlashAttention", "Exact attention without an n x n
    workspace").  A row with no allowed key returns out = 0 ("Deep Dive -
    FlashAttention", "Online softmax is what makes the tiles exact") and
    lse = -inf, the log of an empty sum (a reading: the pages define lse only
    for non-empty rows).
    """
    n, m = Q.shape[0], K.shape[0]
    dv = V.shape[1]
    if m == 0:
        return np.zeros((n, dv)), np.full(n, -np.inf)
    S = scale * (Q @ K.T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    row_max = S.max(axis=1)
    nonempty = np.isfinite(row_max)
    shift = np.where(nonempty, row_max, 0.0)
    E = np.exp(S - shift[:, None])
    l = E.sum(axis=1)
    P = E / np.where(nonempty, l, 1.0)[:, None]
    out = P @ V
    out[~nonempty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(nonempty, row_max + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return out, lse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _sequences(cu_seqlens_q, cu_seqlens_k, batch, nq, nk):
    """Yield (seq index, q row offset, Nq, k row offset, Nk)."""
    if cu_seqlens_q is None:
        for b in range(batch):
            yield b, 0, nq, 0, nk
    else:
        cq = [int(x) for x in np.asarray(cu_seqlens_q)]
        ck = [int(x) for x in np.asarray(cu_seqlens_k)]
        for b in range(len(cq) - 1):
            yield b, cq[b], cq[b + 1] - cq[b], ck[b], ck[b + 1] - ck[b]


def attention_ref(q, k, v, *, causal, softmax_scale, cu_seqlens_q=None, cu_seqlens_k=None,
                  window=(-1, -1)):
    """Full forward: (out, lse) in float64.

    Dense layout ("Deep Dive - FlashAttention", "The public interface is
    several kernels"): q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d];
    returns out [B, Nq, Hq, d] and lse [B, Hq, Nq].

    Packed variable-length layout (same page, "Paged KV is a lookup, not a
    cache manager"): q [total_q, Hq, d], k and v [total_k, Hkv, d] with int32
    cumulative offsets cu_seqlens_q / cu_seqlens_k of batch + 1 entries;
    returns out [total_q, Hq, d] and lse [Hq, total_q].  Causal masking is
    bottom-right aligned per sequence, with that sequence's own lengths, and
    so is the optional local window (left, right) (window_keep).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    varlen = cu_seqlens_q is not None
    if varlen != (cu_seqlens_k is not None):
        raise ValueError("give both cu_seqlens arrays or neither")
    if varlen:
        q4, k4, v4 = q[None], k[None], v[None]
    else:
        q4, k4, v4 = q, k, v
    hq_n, hkv_n = q4.shape[2], k4.shape[2]
    kvmap = kv_head_for_queries(hq_n, hkv_n)
    out = np.zeros(q4.shape[:3] + (v4.shape[3],))
    lse = np.full((q4.shape[0], hq_n, q4.shape[1]), -np.inf)
    for b, qo, nq, ko, nk in _sequences(cu_seqlens_q, cu_seqlens_k, q4.shape[0], q4.shape[1], k4.shape[1]):
        bb = 0 if varlen else b
        for h in range(hq_n):
            K = k4[bb, ko:ko + nk, kvmap[h], :]
            V = v4[bb, ko:ko + nk, kvmap[h], :]
            full = _keep(nq, nk, causal, window)
            for r0 in range(0, nq, ROW_BLOCK):
                r1 = min(nq, r0 + ROW_BLOCK)
                keep = None if full is None else full[r0:r1]
                o, s = _attend_rows(q4[bb, qo + r0:qo + r1, h, :], K, V, softmax_scale, keep)
                out[bb, qo + r0:qo + r1, h, :] = o
                lse[bb, h, qo + r0:qo + r1] = s
    if varlen:
        return out[0], lse[0]
    return out, lse


def attention_rows(q, k, v, rows, *, causal, softmax_scale, cu_seqlens_q=None, cu_seqlens_k=None,
                   window=(-1, -1)):
    """The same definition evaluated for selected outputs only.

    rows: iterable of (seq, q_head, i) with i the row index inside the
    sequence.  Returns out [len(rows), d] and lse [len(rows)].  Used to check
    full-size launches on a sample of rows; each row is computed on its own.
    """
    varlen = cu_seqlens_q is not None
    kvmap = kv_head_for_queries(q.shape[-2], k.shape[-2])
    seqs = {s[0]: s for s in _sequences(cu_seqlens_q, cu_seqlens_k,
                                         1 if varlen else q.shape[0],
                                         None if varlen else q.shape[1],
                                         None if varlen else k.shape[1])}
    outs, lses = [], []
    for b, h, i in rows:
        _, qo, nq, ko, nk = seqs[b]
        if varlen:
            Q = _as64(q[qo + i, h, :])[None]
            K = _as64(k[ko:ko + nk, kvmap[h], :])
            V = _as64(v[ko:ko + nk, kvmap[h], :])
        else:
            Q = _as64(q[b, i, h, :])[None]
            K = _as64(k[b, :, kvmap[h], :])
            V = _as64(v[b, :, kvmap[h], :])
        full = _keep(nq, nk, causal, window)
        keep = None if full is None else full[i:i + 1]
        o, s = _attend_rows(Q, K, V, softmax_scale, keep)
        outs.append(o[0])
        lses.append(s[0])
    return np.array(outs), np.array(lses)


def paged_gather(cache, table_row, length):
    """Logical rows 0..length-1 of one request from a paged cache.

    "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
    "Block tables and what the kernel does" and "Runnable Example": logical
    token t lives in physical page table_row[t // page_size] at offset
    t % page_size; the pages are concatenated in table order and cut to the
    used length.  cache has shape [num_pages, page_size, ...].
    """
    page = cache.shape[1]
    n_pages = -(-length // page)
    if n_pages == 0:
        return cache[:0, 0]
    rows = np.concatenate([np.asarray(cache[int(p)]) for p in table_row[:n_pages]], axis=0)
    return rows[:length]


def decode_ref(q, k_cache, v_cache, block_table, seqlens_k, *, softmax_scale, requests=None):
    """One-token decode over a paged cache, computed unsplit.

    q [B, Hq, d]; k_cache and v_cache [num_pages, page_size, Hkv, d];
    block_table int [B, max_pages]; seqlens_k int [B].  Returns out [B, Hq, d]
    and lse [B, Hq] (or only the listed requests, in order).  With one query
    row a bottom-right causal mask keeps every cached key ("Deep Dive -
    FlashAttention", "Review questions"), so no mask is applied.  The split
    into chunks and their combination is deliberately not modelled here.
    """
    hq_n, hkv_n = q.shape[1], k_cache.shape[2]
    kvmap = kv_head_for_queries(hq_n, hkv_n)
    req = range(q.shape[0]) if requests is None else list(requests)
    out = np.zeros((len(req), hq_n, v_cache.shape[3]))
    lse = np.full((len(req), hq_n), -np.inf)
    for n, b in enumerate(req):
        length = int(seqlens_k[b])
        table = [int(x) for x in np.asarray(block_table[b])]
        for kvh in range(hkv_n):
            K = _as64(paged_gather(k_cache[:, :, kvh, :], table, length))
            V = _as64(paged_gather(v_cache[:, :, kvh, :], table, length))
            heads = [h for h in range(hq_n) if kvmap[h] == kvh]
            Q = _as64(np.stack([np.asarray(q[b, h]) for h in heads]))
            o, s = _attend_rows(Q, K, V, softmax_scale, None)
            out[n, heads] = o
            lse[n, heads] = s
    return out, lse


def _attend_rows_bwd(Q, K, V, G, scale, keep):
    """Gradients for a block of query rows against one key/value head.

    Q [n, d], K [m, d], V [m, dv], G = dL/d(out) [n, dv] float64; keep
    [n, m] bool or None.  Returns dQ [n, d], and this block's contribution to
    dK [m, d] and dV [m, dv].

    "Deep Dive - FlashAttention", "Backward recomputes tiles on purpose": with
    S = scale * Q K^T and P = softmax(S) row by row, dV = P^T G, dP = G V^T,
    and dS = P * (dP - rowsum(P * dP)) (the softmax Jacobian applied row by
    row; the row sum is broadcast over keys).  Masked probabilities, and with
    them their gradients, are zero; a row with no allowed key has P = 0 and
    contributes nothing.  The chain rule through S = scale * Q K^T gives
    dQ = scale * dS K and dK = scale * dS^T Q.
    """
    n, m = Q.shape[0], K.shape[0]
    if m == 0:
        return np.zeros_like(Q), np.zeros_like(K), np.zeros((0, V.shape[1]))
    S = scale * (Q @ K.T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    row_max = S.max(axis=1)
    nonempty = np.isfinite(row_max)
    E = np.exp(S - np.where(nonempty, row_max, 0.0)[:, None])
    P = E / np.where(nonempty, E.sum(axis=1), 1.0)[:, None]
    P[~nonempty] = 0.0
    dV = P.T @ G
    dP = G @ V.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    return dQ, dK, dV


def paged_prefill_ref(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, *, causal,
                      softmax_scale, window=(-1, -1), sequences=None):
    """Prefill of new query rows against a paged cache that already holds them.

    q [total_q, Hq, d] packed with cu_seqlens_q; k_cache, v_cache
    [num_pages, page_size, Hkv, d]; block_table [B, max_pages]; seqlens_k [B]
    cached keys per sequence, the last of which belong to that sequence's new
    rows (so masks align bottom-right).  Each sequence's keys are gathered
    through its table row ("Deep Dive - FlashAttention", "Paged KV is a
    lookup, not a cache manager"; "FlashAttention-3 and PagedAttention:
    IO-Aware Attention Kernels (2026)", "Block tables and what the kernel
    does") and attended as in attention_ref.  Returns out [total_q, Hq, d] and
    lse [Hq, total_q]; `sequences` restricts the work (other rows stay 0 /
    -inf).
    """
    hq_n, hkv_n = q.shape[1], k_cache.shape[2]
    kvmap = kv_head_for_queries(hq_n, hkv_n)
    cq = [int(x) for x in np.asarray(cu_seqlens_q)]
    out = np.zeros((q.shape[0], hq_n, v_cache.shape[3]))
    lse = np.full((hq_n, q.shape[0]), -np.inf)
    seqs = range(len(cq) - 1) if sequences is None else sequences
    for b in seqs:
        nq, nk = cq[b + 1] - cq[b], int(seqlens_k[b])
        table = [int(x) for x in np.asarray(block_table[b])]
        full = _keep(nq, nk, causal, window)
        for kvh in range(hkv_n):
            K = _as64(paged_gather(k_cache[:, :, kvh, :], table, nk))
            V = _as64(paged_gather(v_cache[:, :, kvh, :], table, nk))
            for h in [h for h in range(hq_n) if kvmap[h] == kvh]:
                o, s = _attend_rows(_as64(q[cq[b]:cq[b + 1], h, :]), K, V, softmax_scale, full)
                out[cq[b]:cq[b + 1], h] = o
                lse[h, cq[b]:cq[b + 1]] = s
    return out, lse


def attention_bwd_ref(q, k, v, dout, *, causal, softmax_scale, cu_seqlens_q=None,
                      cu_seqlens_k=None, kv_heads=None):
    """Gradients of the forward of attention_ref: (dq, dk, dv) in float64.

    Same layouts as attention_ref; dout has the layout of out.  A K/V head
    shared by a group of query heads receives the sum of its group's
    gradients (the chain rule over the consecutive-group map of "Deep Dive -
    FlashAttention", "The public interface is several kernels").  kv_heads,
    if given, restricts the work to those K/V heads and their query heads;
    the other entries of dq, dk and dv are left at zero.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    varlen = cu_seqlens_q is not None
    if varlen != (cu_seqlens_k is not None):
        raise ValueError("give both cu_seqlens arrays or neither")
    if varlen:
        q4, k4, v4, g4 = q[None], k[None], v[None], dout[None]
    else:
        q4, k4, v4, g4 = q, k, v, dout
    hq_n, hkv_n = q4.shape[2], k4.shape[2]
    kvmap = kv_head_for_queries(hq_n, hkv_n)
    wanted = set(range(hkv_n)) if kv_heads is None else {int(h) for h in kv_heads}
    dq = np.zeros_like(q4)
    dk = np.zeros_like(k4)
    dv = np.zeros_like(v4)
    for b, qo, nq, ko, nk in _sequences(cu_seqlens_q, cu_seqlens_k, q4.shape[0], q4.shape[1], k4.shape[1]):
        bb = 0 if varlen else b
        for h in range(hq_n):
            kvh = kvmap[h]
            if kvh not in wanted:
                continue
            K = k4[bb, ko:ko + nk, kvh, :]
            V = v4[bb, ko:ko + nk, kvh, :]
            for r0 in range(0, nq, ROW_BLOCK):
                r1 = min(nq, r0 + ROW_BLOCK)
                keep = causal_keep(nq, nk)[r0:r1] if causal else None
                gq, gk, gv = _attend_rows_bwd(q4[bb, qo + r0:qo + r1, h, :], K, V,
                                              g4[bb, qo + r0:qo + r1, h, :], softmax_scale, keep)
                dq[bb, qo + r0:qo + r1, h, :] = gq
                dk[bb, ko:ko + nk, kvh, :] += gk
                dv[bb, ko:ko + nk, kvh, :] += gv
    if varlen:
        return dq[0], dk[0], dv[0]
    return dq, dk, dv


__all__ = [
    "kv_head_for_queries", "causal_keep", "attention_ref", "attention_rows",
    "paged_gather", "decode_ref", "attention_bwd_ref", "window_keep", "paged_prefill_ref",
    "ROW_BLOCK",
]
