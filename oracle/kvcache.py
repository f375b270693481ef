"""Decode with an in-place cache append and rotary embeddings, in fp64 on the CPU.

Test infrastructure only (see the package docstring).

"Deep Dive - FlashAttention", "Paged KV is a lookup, not a cache manager": the
cached-decode call of FA2 can write the new token's key and value into the
paged cache itself and apply rotary embeddings first, into space the caller has
already reserved.  "FlashAttention: Part 1", sections 4.1 and 4.2: rotary
embedding (RoPE) is a position-dependent transform of Q and K applied before
attention, which leaves the attention itself unchanged, and cached decoding
with optional RoPE is one of the features production kernels carry.

The pages give no formula, so the plain textbook one is taken: features are
grouped in pairs, and the pair (a, b) of pair index i at position p is turned
by the angle whose cosine and sine are cos[p, i] and sin[p, i] into
(a cos - b sin, a sin + b cos).  Pairs are either the two halves of the rotated
features (feature i with feature i + rotary_dim / 2) or neighbours (2i, 2i + 1);
features from rotary_dim on are left alone.  The caller supplies the cos/sin
tables, so the frequencies are the caller's choice.

Precision (the pages fix none): the cache holds bf16, so the stored key is the
rotated key rounded to bf16 (round to nearest, ties to even); the rotated query
is rounded the same way before attention, as any bf16 query input would be.
Rounding to bf16 picks a stored code, so it is decided in the precision the
kernel computes the turn in: each product rounded to float32, then the
difference (or sum) rounded to float32, then that value rounded to bf16
(rotary_f32).  rotary_ref is the same turn in float64, the mathematical
definition the float32 one is pinned against.  The attention itself is fp64.
"""
import numpy as np

from . import attention as _A


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  With
    x = m * 2**e and 0.5 <= |m| < 1, the value is rint(m * 256) / 256 * 2**e;
    np.rint rounds halves to even.  Zeros, infinities and NaN pass through.
    Values are taken to lie in the normal float32 range (true of everything
    this package rounds).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    return np.where(np.isfinite(x), r, x)


def rotary_ref(x, cos, sin, positions, *, rotary_dim, interleaved):
    """Rotate the first rotary_dim features of every row of x.

    x [n, H, d]; positions [n] integer positions (one per row, shared by its
    H heads); cos, sin [max_pos, rotary_dim / 2].  Returns float64 [n, H, d].
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if rotary_dim == 0:
        return out
    if rotary_dim % 2 or rotary_dim > x.shape[-1]:
        raise ValueError("rotary_dim must be even and at most the head dimension")
    half = rotary_dim // 2
    for n, p in enumerate(positions):
        c = np.asarray(cos[int(p)], dtype=np.float64)
        s = np.asarray(sin[int(p)], dtype=np.float64)
        for i in range(half):
            ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
            a, b = x[n, :, ia], x[n, :, ib]
            out[n, :, ia] = a * c[i] - b * s[i]
            out[n, :, ib] = a * s[i] + b * c[i]
    return out


def rotary_f32(x, cos, sin, positions, *, rotary_dim, interleaved):
    """rotary_ref's turn in float32 arithmetic, as float64 values.

    Each product a*cos, b*sin, a*sin, b*cos is rounded to float32, then
    a*cos - b*sin and a*sin + b*cos are rounded to float32 (no fused
    multiply-add).  x must hold float32-exact values (bf16 inputs do).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if rotary_dim == 0:
        return out
    if rotary_dim % 2 or rotary_dim > x.shape[-1]:
        raise ValueError("rotary_dim must be even and at most the head dimension")
    half = rotary_dim // 2
    x32 = x.astype(np.float32)
    for n, p in enumerate(positions):
        c = np.asarray(cos[int(p)], dtype=np.float32)
        s = np.asarray(sin[int(p)], dtype=np.float32)
        for i in range(half):
            ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
            a, b = x32[n, :, ia], x32[n, :, ib]
            out[n, :, ia] = (a * c[i] - b * s[i]).astype(np.float64)
            out[n, :, ib] = (a * s[i] + b * c[i]).astype(np.float64)
    return out


def _new_rows(q, k_new, rotary_cos, rotary_sin, positions, rotary_dim, interleaved):
    """The rotated, bf16-rounded query and key of the new tokens."""
    kw = dict(rotary_dim=rotary_dim, interleaved=interleaved)
    q_rot = round_bf16(rotary_f32(q, rotary_cos, rotary_sin, positions, **kw))
    k_rot = round_bf16(rotary_f32(k_new, rotary_cos, rotary_sin, positions, **kw))
    return q_rot, k_rot


def append_ref(k_new, v_new, k_cache, v_cache, block_table, seqlens_k, *, rotary_cos=None,
               rotary_sin=None, rotary_dim=0, interleaved=False):
    """The caches after the append, as float64 copies (inputs unchanged).

    k_new, v_new [B, Hkv, d]; caches [num_pages, page_size, Hkv, d];
    block_table [B, max_pages]; seqlens_k [B] keys cached before the call.
    Request b's new token sits at position p_b = seqlens_k[b]: its key, rotated
    at p_b (rotary_f32) and rounded to bf16, and its value go to row
    p_b % page_size of page
    block_table[b][p_b // page_size].  Requests must not share a target row.
    """
    page = k_cache.shape[1]
    pos = [int(x) for x in np.asarray(seqlens_k)]
    _, k_rot = _new_rows(np.zeros((len(pos), 1, k_new.shape[-1])), k_new, rotary_cos, rotary_sin,
                         pos, rotary_dim, interleaved)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    for b, p in enumerate(pos):
        phys = int(block_table[b][p // page])
        kc[phys, p % page] = k_rot[b]
        vc[phys, p % page] = np.asarray(v_new[b], dtype=np.float64)
    return kc, vc


def decode_append_ref(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, *, softmax_scale,
                      rotary_cos=None, rotary_sin=None, rotary_dim=0, interleaved=False,
                      requests=None):
    """One-token decode after the append of append_ref, request by request.

    q [B, Hq, d].  Request b attends with its query rotated at p_b =
    seqlens_k[b] (rounded to bf16) over p_b + 1 keys: its p_b cached keys,
    gathered through its table row from the caches as given, followed by its
    own new key and value.  (This equals decode_ref over append_ref's caches
    with lengths p_b + 1 whenever no request reads a row another request
    writes, which the caller guarantees.)

    Returns out [len(req), Hq, d], lse [len(req), Hq] and q_rot [B, Hq, d],
    float64; `requests` (default: all) lists the requests to attend, in order.
    """
    pos = [int(x) for x in np.asarray(seqlens_k)]
    q_rot, k_rot = _new_rows(q, k_new, rotary_cos, rotary_sin, pos, rotary_dim, interleaved)
    hq_n, hkv_n = q.shape[1], k_cache.shape[2]
    kvmap = _A.kv_head_for_queries(hq_n, hkv_n)
    req = range(q.shape[0]) if requests is None else list(requests)
    out = np.zeros((len(req), hq_n, v_cache.shape[3]))
    lse = np.full((len(req), hq_n), -np.inf)
    for n, b in enumerate(req):
        table = [int(x) for x in np.asarray(block_table[b])]
        for kvh in range(hkv_n):
            K = np.concatenate([_A.paged_gather(k_cache[:, :, kvh, :], table, pos[b]).astype(np.float64),
                                k_rot[b, kvh][None]])
            V = np.concatenate([_A.paged_gather(v_cache[:, :, kvh, :], table, pos[b]).astype(np.float64),
                                np.asarray(v_new[b, kvh], dtype=np.float64)[None]])
            heads = [h for h in range(hq_n) if kvmap[h] == kvh]
            o, s = _A._attend_rows(q_rot[b, heads], K, V, softmax_scale, None)
            out[n, heads] = o
            lse[n, heads] = s
    return out, lse, q_rot
