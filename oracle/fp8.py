"""FP8 attention forward: block quantisation with incoherent processing, in NumPy.

Test infrastructure only (see the package docstring).

"FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
"FlashAttention-3" (the three techniques): FP8 with block quantisation (one
scale per block) and incoherent processing, a random orthogonal transform that
spreads outliers over the vector before quantisation.  "Flash Attention: A
Complete Architectural Autopsy", "FP8 Path and Quantization": each tile gets a
scale from its absolute maximum; scores are formed from the FP8 operands and
dequantised to fp32 for the softmax; V tiles are quantised the same way.

Readings (the pages fix none of these details):
  * Format: E4M3 as defined by the OCP 8-bit floating point specification
    ("fn": bias 7, no infinities, largest finite value 448, NaN = S.1111.111),
    round to nearest, ties to even.
  * Blocks: 64 consecutive rows (sequence positions) of one (sequence, head),
    for Q, K and V alike; the last block of a sequence may be short.
  * Scale: amax = max |x| over the block (after the transform for Q and K);
    inv = 448 / amax and scale = amax / 448, both float32 divisions; the code
    is E4M3(x * inv) with the product rounded to float32 first.  A block of
    zeros gets scale 0 and codes 0.  The dequantised value is code * scale.
  * Incoherent processing: x -> H (s * x) along the head dimension, with s a
    +-1 sign vector and H the Sylvester-ordered Walsh-Hadamard matrix,
    unnormalised; the same s for Q and K, so Q' K'^T = d * Q K^T and the
    softmax scale is divided by d.  V is not transformed.  The transform is
    computed in float32 by butterflies, stage h = 1, 2, 4, ..., d/2, each
    pair (x[i], x[i + h]) with i & h == 0 becoming (x[i] + x[i+h], x[i] -
    x[i+h]); the float32 result decides the codes, so it is taken in the
    precision and order the GPU uses.

Attention on the quantised operands (attention_fp8_ref) is the exact fp64
definition on the dequantised Q, K, V; the kernel also rounds the
probabilities to E4M3 before the P V product (scaled by P_SCALE and the V tile
scales; its shift trails the running maximum by at most RESCALE_LOG2, the
conditional rescaling of "Deep Dive - FlashAttention", "FA1 through FA4 retune
the same IO idea"), an approximation whose error is bounded by fp8_out_bound.
"""
import numpy as np

from . import attention as _A

E4M3_MAX = 448.0
BLOCK = 64
P_SCALE = 64.0      # probabilities are multiplied by this (and s_v / max s_v) before rounding
RESCALE_LOG2 = 2.0  # the kernel's shift may trail the running maximum by up to this (log2 units)


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8) as float64: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal (m / 8 * 2^-6); code
    S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x):
    """E4M3 codes (uint8) of float64 values, round to nearest, ties to even.

    Magnitudes that round above 448 give NaN (0x7F, sign bit kept), as does
    NaN.  Each finite magnitude is mapped onto the grid of its binade
    (spacing 2^(e-3) for normals, 2^-9 below 2^-6) with np.rint, which rounds
    halves to even; a carry into the next binade is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)                      # below 2^-6 the grid is the subnormal one
    step = 2.0 ** (e - 3)
    q = np.rint(a / step) * step               # nearest grid value, ties to even
    out = np.zeros(x.shape, dtype=np.int64)
    ok = np.isfinite(x) & (q <= E4M3_MAX)
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = ok & (q >= 2.0 ** -6)
    sub = ok & (q > 0) & (q < 2.0 ** -6)
    mant_n = np.rint(q / 2.0 ** qe * 8.0).astype(np.int64) - 8
    out = np.where(normal, ((qe.astype(np.int64) + 7) << 3) | mant_n, out)
    out = np.where(sub, np.rint(q / 2.0 ** -9).astype(np.int64), out)
    out = np.where(ok, out, 0x7F)
    return (out | sign).astype(np.uint8)


def fwht_f32(x):
    """Unnormalised Walsh-Hadamard transform along the last axis in float32,
    butterflies in the stage order of the module docstring; float64 result."""
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("the length must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y.astype(np.float64)


def quantize_blocks(x, signs=None, block=BLOCK):
    """Block quantisation of x [B, N, H, d] (values exact in float32).

    Returns codes uint8 [B, N, H, d] and scales float64 [B, H, ceil(N /
    block)] (each a float32 value).  With `signs` (+-1, length d) the rows are
    first turned by fwht_f32(signs * x).
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, H, d = x.shape
    if signs is not None:
        x = fwht_f32(x * np.asarray(signs, dtype=np.float64))
    nblk = -(-N // block)
    codes = np.zeros((B, N, H, d), dtype=np.uint8)
    scales = np.zeros((B, H, nblk))
    for b in range(B):
        for h in range(H):
            for k in range(nblk):
                blk = x[b, k * block:(k + 1) * block, h, :]
                amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0.0)
                if amax == 0:
                    scales[b, h, k] = 0.0
                    continue
                inv = np.float32(E4M3_MAX) / amax
                scales[b, h, k] = float(amax / np.float32(E4M3_MAX))
                codes[b, k * block:(k + 1) * block, h, :] = e4m3_encode(
                    (blk.astype(np.float32) * inv).astype(np.float64))
    return codes, scales


def dequantize(codes, scales, block=BLOCK):
    """code * scale of its block, float64 [B, N, H, d]."""
    vals = e4m3_decode(codes)
    B, N, H, d = vals.shape
    rows = np.arange(N) // block
    s = np.asarray(scales, dtype=np.float64)[:, :, rows]          # [B, H, N]
    return vals * s.transpose(0, 2, 1)[..., None]


def vt_key_of_position(p):
    """Key (0..63) stored at byte position p (0..63) of a 64-key block of a
    V^T row: p = 32 h + 16 kb + 4 g + e holds key 32 kb + 8 g + 4 h + e.  This
    is the order in which a score tile's registers hold keys, so a lane's 32
    probabilities meet 32 contiguous V^T bytes."""
    h, j = p // 32, p % 32
    kb, g, e = j // 16, (j % 16) // 4, j % 4
    return 32 * kb + 8 * g + 4 * h + e


def vt_layout(codes, block=BLOCK):
    """V codes [B, N, H, d] -> [B, H, d, Np] (Np = N rounded up to 64), keys
    permuted inside every 64-key block by vt_key_of_position, padding zero."""
    B, N, H, d = codes.shape
    Np = -(-N // block) * block
    out = np.zeros((B, H, d, Np), dtype=np.uint8)
    perm = np.array([vt_key_of_position(p) for p in range(block)])
    for k0 in range(0, Np, block):
        keys = k0 + perm
        valid = keys < N
        src = np.zeros((B, block, H, d), dtype=np.uint8)
        src[:, valid] = codes[:, keys[valid]]
        out[:, :, :, k0:k0 + block] = src.transpose(0, 2, 3, 1)
    return out


def attention_fp8_ref(q_codes, k_codes, v_codes, q_scales, k_scales, v_scales, *, causal, softmax_scale,
                      incoherent):
    """Exact fp64 attention on the dequantised operands (dense [B, N, H, d]).

    With incoherent processing the scores of the turned operands are d times
    the original ones, so softmax_scale / d is used.
    """
    q = dequantize(q_codes, q_scales)
    k = dequantize(k_codes, k_scales)
    v = dequantize(v_codes, v_scales)
    scale = softmax_scale / q.shape[-1] if incoherent else softmax_scale
    return _A.attention_ref(q, k, v, causal=causal, softmax_scale=scale)


def _bound_block(Q, K, V, Vcode, vs_row, scale, keep):
    """Bound of fp8_out_bound for query rows Q [n, d] against one K/V head
    (K, V, Vcode [Nk, d]; vs_row the head's V block scales; keep [n, Nk])."""
    smax = float(np.max(vs_row)) if len(vs_row) else 0.0
    g = np.where((vs_row > 0) & (smax > 0), vs_row / (smax if smax > 0 else 1.0), 1.0)
    g_key = g[np.arange(K.shape[0]) // BLOCK]
    vref = smax if smax > 0 else 1.0
    S = np.where(keep, scale * (Q @ K.T), -np.inf)
    m = np.max(S, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(keep, np.exp(S - m), 0.0)
    L = np.sum(p, axis=1, keepdims=True)
    Ls = np.where(L > 0, L, 1.0)
    sub = keep & (P_SCALE * g_key[None, :] * p < 2.0 ** -6)
    return 2.0 ** -4 * ((p / Ls) @ np.abs(V)) + 2.0 ** -10 * vref / P_SCALE / Ls * (sub @ np.abs(Vcode))


def fp8_out_bound(q_codes, k_codes, v_codes, q_scales, k_scales, v_scales, *, causal, softmax_scale,
                  incoherent, rows=None):
    """Per-element bound on |out_gpu - out_ref| from rounding the
    probabilities to E4M3: [B, Nq, Hq, d], or [len(rows), d] for `rows`, a
    list of (seq, q_head, i).

    The kernel rounds P'_j = exp(s_j - c) * 64 * g_t to E4M3, where c is its
    shift (never above the running maximum, and at most RESCALE_LOG2 below
    it, so exp(s_j - c) <= 4) and g_t = s_v(t) / max_t s_v(t) folds the V tile
    scales into P (g_t = 1 where a scale is 0).  Each rounding is within 2^-4
    of P'_j when P'_j >= 2^-6 and within 2^-10 absolutely below.  With the
    exact weights w_j = p_j / L, p_j = exp(s_j - m) at the row's final maximum
    m (c <= m, so the kernel's values and row sum are at least p_j and L):
        |err_c| <= 2^-4 sum_j w_j |v_jc| + 2^-10 * vmax / 64 / L
                   * sum_{j: 64 g_t p_j < 2^-6} |code(v_jc)|
    """
    q = dequantize(q_codes, q_scales)
    k = dequantize(k_codes, k_scales)
    vcode = e4m3_decode(v_codes)
    v = dequantize(v_codes, v_scales)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = softmax_scale / d if incoherent else softmax_scale
    kvmap = _A.kv_head_for_queries(Hq, Hkv)
    vs = np.asarray(v_scales, dtype=np.float64)
    full_keep = _A.causal_keep(Nq, Nk) if causal else np.ones((Nq, Nk), dtype=bool)
    if rows is not None:
        out = np.zeros((len(rows), d))
        for n, (b, h, i) in enumerate(rows):
            kvh = kvmap[h]
            out[n] = _bound_block(q[b, i:i + 1, h, :], k[b, :, kvh, :], v[b, :, kvh, :], vcode[b, :, kvh, :],
                                  vs[b, kvh], scale, full_keep[i:i + 1])[0]
        return out
    bound = np.zeros((B, Nq, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kvh = kvmap[h]
            bound[b, :, h, :] = _bound_block(q[b, :, h, :], k[b, :, kvh, :], v[b, :, kvh, :], vcode[b, :, kvh, :],
                                             vs[b, kvh], scale, full_keep)
    return bound
