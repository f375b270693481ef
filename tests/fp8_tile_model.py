"""A slow model of the FP8 kernel's probability rounding, for pinning the error bound.

It walks the keys of each row in 64-key tiles, raising its shift c to a
tile's maximum when that exceeds c by more than 2 (log2 units), rounds
P'_j = exp(s_j - c) * 64 * g_t to E4M3 before multiplying by the V codes, and
keeps the row sum from the unrounded values; everything else is float64.  ("Flash Attention: A Complete Architectural Autopsy", "The Online
Softmax Recurrence" for the tiling; "FP8 Path and Quantization" for the FP8
operands.)  Independent of the oracle's attention code.
"""
import math

import numpy as np

import oracle.fp8 as F


def fp8_tiled_attention(q_codes, k_codes, v_codes, q_scales, k_scales, v_scales, *, causal, softmax_scale,
                        incoherent, rows=None):
    q = F.dequantize(q_codes, q_scales)
    k = F.dequantize(k_codes, k_scales)
    vcode = F.e4m3_decode(v_codes)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = softmax_scale / d if incoherent else softmax_scale
    vs = np.asarray(v_scales, dtype=np.float64)
    out = np.zeros((B, Nq, Hq, d))
    group = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            smax = float(np.max(vs[b, kvh])) if vs.shape[2] else 0.0
            for i in (range(Nq) if rows is None else rows):
                hi = i + Nk - Nq if causal else Nk - 1
                m = -math.inf
                ell = 0.0
                acc = np.zeros(d)
                for t0 in range(0, Nk, 64):
                    keys = [j for j in range(t0, min(Nk, t0 + 64)) if j <= hi]
                    if not keys:
                        continue
                    s = np.array([scale * float(q[b, i, h] @ k[b, j, kvh]) for j in keys])
                    m_new = float(np.max(s))
                    if m_new * math.log2(math.e) > m * math.log2(math.e) + 2.0:
                        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
                        acc *= alpha
                        ell *= alpha
                        m = m_new
                    g = vs[b, kvh, t0 // 64] / smax if (vs[b, kvh, t0 // 64] > 0 and smax > 0) else 1.0
                    p = np.exp(s - m)
                    pq = F.e4m3_decode(F.e4m3_encode(p * 64.0 * g))
                    ell += float(np.sum(p))
                    acc += pq @ vcode[b, keys, kvh, :]
                vref = smax if smax > 0 else 1.0
                out[b, i, h] = acc * vref / 64.0 / ell if ell > 0 else 0.0
    return out
