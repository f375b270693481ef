"""Plant plausible mistakes in the CPU oracle and confirm that the pins catch each.

Every mutant below is applied to the oracle module with monkeypatch (on the CPU
only); the test passes when at least one pin check in tests/pins.py fails
under the mutant, i.e. the pins would have exposed that mistake.
"""
import math

import numpy as np
import pytest

import oracle.attention as OA
import oracle.kvcache as OK
import oracle.fp8 as OF
import pins

_orig_attend = OA._attend_rows
_orig_keep = OA.causal_keep
_orig_seqs = OA._sequences
_orig_gather = OA.paged_gather


def _attend_no_normalise(Q, K, V, scale, keep):
    S = scale * (Q @ K.T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    mx = S.max(axis=1) if K.shape[0] else np.full(Q.shape[0], -np.inf)
    ok = np.isfinite(mx)
    E = np.exp(S - np.where(ok, mx, 0.0)[:, None])
    out = E @ V
    with np.errstate(divide="ignore"):
        lse = np.where(ok, mx + np.log(np.where(ok, E.sum(1), 1.0)), -np.inf)
    return out, lse


def _attend_no_max_in_lse(Q, K, V, scale, keep):
    out, lse = _orig_attend(Q, K, V, scale, keep)
    S = scale * (Q @ K.T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    mx = S.max(axis=1) if K.shape[0] else np.zeros(Q.shape[0])
    return out, np.where(np.isfinite(lse), lse - np.where(np.isfinite(mx), mx, 0.0), lse)


def _attend_empty_rows_nan(Q, K, V, scale, keep):
    out, lse = _orig_attend(Q, K, V, scale, keep)
    out = out.copy()
    out[np.isneginf(lse)] = np.nan
    return out, lse


def _gather_off_by_one(cache, table_row, length):
    rows = _orig_gather(cache, table_row, length + 1)
    return rows[1:length + 1] if len(rows) > length else rows[:length]


def _seqs_shared_k_offset(cu_q, cu_k, batch, nq, nk):
    for b, qo, n_q, ko, n_k in _orig_seqs(cu_q, cu_k, batch, nq, nk):
        yield b, qo, n_q, 0, n_k


_orig_bwd_rows = OA._attend_rows_bwd
_orig_bwd = OA.attention_bwd_ref


def _bwd_parts(Q, K, V, G, scale, keep):
    S = scale * (Q @ K.T)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    mx = S.max(axis=1) if K.shape[0] else np.full(Q.shape[0], -np.inf)
    ok = np.isfinite(mx)
    E = np.exp(S - np.where(ok, mx, 0.0)[:, None])
    P = E / np.where(ok, E.sum(axis=1), 1.0)[:, None]
    P[~ok] = 0.0
    return P, E, G @ V.T


def _bwd_no_rowsum(Q, K, V, G, scale, keep):
    P, _, dP = _bwd_parts(Q, K, V, G, scale, keep)
    dS = P * dP
    return scale * dS @ K, scale * dS.T @ Q, P.T @ G


def _bwd_rowsum_of_dp(Q, K, V, G, scale, keep):
    P, _, dP = _bwd_parts(Q, K, V, G, scale, keep)
    dS = P * (dP - dP.sum(axis=1)[:, None])
    return scale * dS @ K, scale * dS.T @ Q, P.T @ G


def _bwd_dv_unnormalised(Q, K, V, G, scale, keep):
    dq, dk, _ = _orig_bwd_rows(Q, K, V, G, scale, keep)
    _, E, _ = _bwd_parts(Q, K, V, G, scale, keep)
    return dq, dk, E.T @ G


def _bwd_dq_transposed(Q, K, V, G, scale, keep):
    P, _, dP = _bwd_parts(Q, K, V, G, scale, keep)
    dS = P * (dP - (P * dP).sum(axis=1)[:, None])
    _, dk, dv = _orig_bwd_rows(Q, K, V, G, scale, keep)
    return scale * dS.T @ K, dk, dv


def _bwd_group_not_summed(q, k, v, dout, **kw):
    """K/V gradients from the last query head of each group only (overwrite, not sum)."""
    dq, _, _ = _orig_bwd(q, k, v, dout, **kw)
    hq, hkv = q.shape[-2], k.shape[-2]
    g = np.array(dout, dtype=np.float64, copy=True)
    for h in range(hq):
        if (h + 1) % (hq // hkv):
            g[..., h, :] = 0.0
    _, dk, dv = _orig_bwd(q, k, v, g, **kw)
    return dq, dk, dv


_orig_window = OA.window_keep


def _window_left_off_by_one(nq, nk, left, right):
    keep = _orig_window(nq, nk, left, right)
    if left >= 0:
        i = np.arange(nq)[:, None]
        j = np.arange(nk)[None, :]
        keep &= j > i + (nk - nq) - left
    return keep


def _window_top_left(nq, nk, left, right):
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    keep = np.ones((nq, nk), dtype=bool)
    if left >= 0:
        keep &= j >= i - left
    if right >= 0:
        keep &= j <= i + right
    return keep


MUTANTS = {
    "window_left_off_by_one": ("window_keep", _window_left_off_by_one),
    "window_sides_swapped": ("window_keep", lambda nq, nk, l, r: _orig_window(nq, nk, r, l)),
    "window_top_left": ("window_keep", _window_top_left),
    "bwd_no_rowsum_term": ("_attend_rows_bwd", _bwd_no_rowsum),
    "bwd_rowsum_of_dp": ("_attend_rows_bwd", _bwd_rowsum_of_dp),
    "bwd_dq_scale_dropped": ("_attend_rows_bwd", lambda Q, K, V, G, s, keep: (lambda a, b, c: (a / s, b, c))(*_orig_bwd_rows(Q, K, V, G, s, keep))),
    "bwd_dk_scale_squared": ("_attend_rows_bwd", lambda Q, K, V, G, s, keep: (lambda a, b, c: (a, b * s, c))(*_orig_bwd_rows(Q, K, V, G, s, keep))),
    "bwd_dv_unnormalised": ("_attend_rows_bwd", _bwd_dv_unnormalised),
    "bwd_dq_transposed": ("_attend_rows_bwd", _bwd_dq_transposed),
    "bwd_group_not_summed": ("attention_bwd_ref", _bwd_group_not_summed),
    "top_left_causal": ("causal_keep", lambda nq, nk: np.arange(nk)[None, :] <= np.arange(nq)[:, None]),
    "bottom_right_off_by_one": ("causal_keep", lambda nq, nk: np.arange(nk)[None, :] < np.arange(nq)[:, None] + nk - nq),
    "alternating_gqa": ("kv_head_for_queries", lambda hq, hkv: [h % hkv for h in range(hq)]),
    "scale_dropped": ("_attend_rows", lambda Q, K, V, s, keep: _orig_attend(Q, K, V, 1.0, keep)),
    "scale_squared": ("_attend_rows", lambda Q, K, V, s, keep: _orig_attend(Q, K, V, s * s, keep)),
    "values_reversed": ("_attend_rows", lambda Q, K, V, s, keep: _orig_attend(Q, K, V[::-1], s, keep)),
    "keys_reversed": ("_attend_rows", lambda Q, K, V, s, keep: _orig_attend(Q, K[::-1], V, s, keep)),
    "lse_base2": ("_attend_rows", lambda Q, K, V, s, keep: (lambda o, l: (o, l / math.log(2)))(*_orig_attend(Q, K, V, s, keep))),
    "no_normalisation": ("_attend_rows", _attend_no_normalise),
    "lse_without_max": ("_attend_rows", _attend_no_max_in_lse),
    "empty_rows_nan": ("_attend_rows", _attend_empty_rows_nan),
    "paged_gather_off_by_one": ("paged_gather", _gather_off_by_one),
    "varlen_k_offset_ignored": ("_sequences", _seqs_shared_k_offset),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"


# ---- cache append and rotary (planted in oracle.kvcache) -------------------------

_orig_rotary = OK.rotary_ref
_orig_round = OK.round_bf16
_orig_new_rows = OK._new_rows


def _rotary_sign_flipped(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_rotary(x, cos, None if sin is None else -np.asarray(sin), positions,
                        rotary_dim=rotary_dim, interleaved=interleaved)


def _rotary_pairs_swapped(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_rotary(x, cos, sin, positions, rotary_dim=rotary_dim, interleaved=not interleaved)


def _rotary_position_plus_one(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_rotary(x, cos, sin, [int(p) + 1 for p in positions], rotary_dim=rotary_dim,
                        interleaved=interleaved)


def _round_truncates(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.where(np.isfinite(x), np.ldexp(np.trunc(m * 256.0) / 256.0, e), x)


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5)
    return np.where(np.isfinite(x), np.ldexp(r / 256.0, e), x)


def _query_not_rotated(q, k_new, cos, sin, positions, rotary_dim, interleaved):
    _, k_rot = _orig_new_rows(q, k_new, cos, sin, positions, rotary_dim, interleaved)
    return OK.round_bf16(q), k_rot


def _append_previous_row(k_new, v_new, k_cache, v_cache, block_table, seqlens_k, **kw):
    kc, vc = np.array(k_cache, dtype=np.float64), np.array(v_cache, dtype=np.float64)
    page = kc.shape[1]
    pos = [int(x) for x in seqlens_k]
    _, k_rot = OK._new_rows(np.zeros((len(pos), 1, kc.shape[-1])), k_new, kw.get("rotary_cos"),
                            kw.get("rotary_sin"), pos, kw.get("rotary_dim", 0), kw.get("interleaved", False))
    for b, p in enumerate(pos):
        t = max(p - 1, 0)
        kc[int(block_table[b][t // page]), t % page] = k_rot[b]
        vc[int(block_table[b][t // page]), t % page] = v_new[b]
    return kc, vc


def _value_not_appended(k_new, v_new, k_cache, v_cache, block_table, seqlens_k, **kw):
    kc, _ = _orig_append(k_new, v_new, k_cache, v_cache, block_table, seqlens_k, **kw)
    return kc, np.array(v_cache, dtype=np.float64)


_orig_append = OK.append_ref
_orig_f32 = OK.rotary_f32


def _f32_fused(x, cos, sin, positions, *, rotary_dim, interleaved):
    """One rounding per output (as a fused multiply-add chain would give)."""
    r = OK.rotary_ref(x, cos, sin, positions, rotary_dim=rotary_dim, interleaved=interleaved)
    return r.astype(np.float32).astype(np.float64)


def _f32_sign_flipped(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_f32(x, cos, None if sin is None else -np.asarray(sin), positions, rotary_dim=rotary_dim,
                     interleaved=interleaved)


def _f32_pairs_swapped(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_f32(x, cos, sin, positions, rotary_dim=rotary_dim, interleaved=not interleaved)


def _f32_position_plus_one(x, cos, sin, positions, *, rotary_dim, interleaved):
    return _orig_f32(x, cos, sin, [int(p) + 1 for p in positions], rotary_dim=rotary_dim,
                     interleaved=interleaved)

KV_MUTANTS = {
    "rotary_sign_flipped": ("rotary_ref", _rotary_sign_flipped),
    "rotary_pairs_swapped": ("rotary_ref", _rotary_pairs_swapped),
    "rotary_position_plus_one": ("rotary_ref", _rotary_position_plus_one),
    "round_truncates": ("round_bf16", _round_truncates),
    "round_ties_away": ("round_bf16", _round_ties_away),
    "query_not_rotated": ("_new_rows", _query_not_rotated),
    "append_previous_row": ("append_ref", _append_previous_row),
    "value_not_appended": ("append_ref", _value_not_appended),
    "rotary_f32_fused": ("rotary_f32", _f32_fused),
    "rotary_f32_sign_flipped": ("rotary_f32", _f32_sign_flipped),
    "rotary_f32_pairs_swapped": ("rotary_f32", _f32_pairs_swapped),
    "rotary_f32_position_plus_one": ("rotary_f32", _f32_position_plus_one),
}


@pytest.mark.parametrize("name", sorted(KV_MUTANTS))
def test_pins_catch_kvcache_mutant(name, monkeypatch):
    attr, fn = KV_MUTANTS[name]
    monkeypatch.setattr(OK, attr, fn)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"


# ---- FP8 forward (planted in oracle.fp8) ------------------------------------------

_orig_encode = OF.e4m3_encode
_orig_fwht = OF.fwht_f32
_orig_quant = OF.quantize_blocks
_orig_vtkey = OF.vt_key_of_position
_orig_dequant = OF.dequantize
_orig_fp8_attn = OF.attention_fp8_ref
_orig_fp8_bound = OF.fp8_out_bound


def _encode_rounding(fn):
    def enc(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
        step = 2.0 ** (e - 3)
        return _orig_encode(np.sign(x) * fn(a / step) * step)
    return enc


def _fwht_sign_swapped(x):
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, b - a
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y.astype(np.float64)


def _fwht_missing_stage(x):
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    h = 2
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y.astype(np.float64)


def _quant_scale_256(x, signs=None, block=64):
    codes, scales = _orig_quant(np.asarray(x, dtype=np.float64) * (256.0 / 448.0), signs, block)
    return codes, scales * (448.0 / 256.0)


def _quant_ignores_signs(x, signs=None, block=64):
    return _orig_quant(x, None, block)


def _dequant_off_by_one_row(codes, scales, block=64):
    vals = OF.e4m3_decode(codes)
    n = vals.shape[1]
    sc = np.asarray(scales, dtype=np.float64)
    rows = np.minimum((np.arange(n) + 1) // block, sc.shape[2] - 1)
    return vals * sc[:, :, rows].transpose(0, 2, 1)[..., None]


FP8_MUTANTS = {
    "e4m3_truncates": ("e4m3_encode", _encode_rounding(np.trunc)),
    "e4m3_ties_away": ("e4m3_encode", _encode_rounding(lambda t: np.floor(t + 0.5))),
    "fwht_sign_swapped": ("fwht_f32", _fwht_sign_swapped),
    "fwht_missing_stage": ("fwht_f32", _fwht_missing_stage),
    "quantize_scale_256": ("quantize_blocks", _quant_scale_256),
    "quantize_ignores_signs": ("quantize_blocks", _quant_ignores_signs),
    "vt_halves_and_blocks_swapped": ("vt_key_of_position",
                                     lambda p: 32 * (p // 32) + 8 * ((p % 16) // 4) + 4 * ((p % 32) // 16) + p % 4),
    "dequantize_block_off_by_one_row": ("dequantize", _dequant_off_by_one_row),
    "fp8_attention_scale_not_divided": ("attention_fp8_ref",
                                        lambda *a, **kw: _orig_fp8_attn(*a, **dict(kw, incoherent=False))),
    # A bound that is too loose must be caught as well as one that is too tight.
    "fp8_bound_four_times_looser": ("fp8_out_bound", lambda *a, **kw: 4.0 * _orig_fp8_bound(*a, **kw)),
    "fp8_bound_probability_scale_16": ("P_SCALE", 16.0),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_pins_catch_fp8_mutant(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(OF, attr, fn)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
