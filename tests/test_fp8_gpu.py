"""FP8 forward on the HIP path vs the CPU oracle (needs an MI355X).

Quantisation is byte work: codes and scales must equal the oracle's bit for
bit (oracle.fp8.quantize_blocks, which takes its rounding decisions in float32
as the GPU does).  Attention on the codes is compared with exact fp64
attention on the dequantised operands: every output element within the bound
of oracle.fp8.fp8_out_bound (the error of rounding probabilities to E4M3), with
5% slack for float32 arithmetic, plus 2^-8 of the value for the bf16 output
rounding and 1e-5; lse within 1e-3; rows with no key exactly 0 and -inf.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import oracle.fp8 as OF
import workloads as W
from test_parity_gpu import to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def np_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


QUANT_CASES = [(130, 3, False, "rows", 128), (130, 3, True, "rows", 128), (200, 2, False, "vt", 128),
               (64, 1, True, "vt", 128), (1, 2, False, "rows", 128), (65, 2, True, "vt", 128),
               (300, 2, True, "rows", 128),
               (130, 3, True, "rows", 64), (200, 2, False, "vt", 64), (65, 2, True, "vt", 64),
               (130, 3, True, "rows", 256), (200, 2, False, "vt", 256), (65, 2, True, "vt", 256),
               (1, 1, True, "rows", 256)]


@pytest.mark.parametrize("N,H,turn,layout,d", QUANT_CASES, ids=lambda x: str(x))
def test_quantize_bit_exact(N, H, turn, layout, d):
    x = np_bf16((2, N, H, d), seed=N + H + d)
    if N >= 128:
        x[0, 64:128, 0] = 0.0            # a zero block
        x[1, 64:128, 1 % H] *= 1e-3      # a quiet block
        x[1, 70, 0, 5] = 300.0           # an outlier
    signs = W.hadamard_signs(d, seed=N) if turn else None
    codes, scales = ea.attn_fp8_quantize(x.to(DEV), signs=None if signs is None else signs.to(DEV), layout=layout)
    torch.cuda.synchronize()
    ref_c, ref_s = OF.quantize_blocks(to64(x), None if signs is None else signs.numpy().astype(np.float64))
    if layout == "vt":
        ref_c = OF.vt_layout(ref_c)
    got = codes.cpu().numpy()
    assert got.shape == ref_c.shape
    assert np.array_equal(got, ref_c), f"{int((got != ref_c).sum())} codes differ"
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref_s)


def check_fp8(case, causal, turn, seed, rows=None):
    """Run the FP8 path on a dense case and compare with the oracle (all rows, or sampled rows)."""
    d = case["q"].shape[-1]
    scale = d ** -0.5
    signs = W.hadamard_signs(d, seed) if turn else None
    q, k, v = (case[x] for x in "qkv")
    sd = None if signs is None else signs.to(DEV)
    qc, qs = ea.attn_fp8_quantize(q.to(DEV), signs=sd)
    kc, ks = ea.attn_fp8_quantize(k.to(DEV), signs=sd)
    vc, vs = ea.attn_fp8_quantize(v.to(DEV), layout="vt")
    out, lse = ea.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=causal, softmax_scale=scale, incoherent=turn)
    torch.cuda.synchronize()
    sg = None if signs is None else signs.numpy().astype(np.float64)
    rq, rqs = OF.quantize_blocks(to64(q), sg)
    rk, rks = OF.quantize_blocks(to64(k), sg)
    rv, rvs = OF.quantize_blocks(to64(v), None)
    # the operands the kernel read are the oracle's, bit for bit
    assert np.array_equal(qc.cpu().numpy(), rq) and np.array_equal(kc.cpu().numpy(), rk)
    assert np.array_equal(vc.cpu().numpy(), OF.vt_layout(rv))
    kw = dict(causal=causal, softmax_scale=scale, incoherent=turn)
    o, l = to64(out), to64(lse)
    if rows is None:
        ref_o, ref_l = OF.attention_fp8_ref(rq, rk, rv, rqs, rks, rvs, **kw)
        bound = OF.fp8_out_bound(rq, rk, rv, rqs, rks, rvs, **kw)
        got_o, got_l = o, l
    else:
        sc = scale / d if turn else scale
        ref_o, ref_l = oracle.attention_rows(OF.dequantize(rq, rqs), OF.dequantize(rk, rks), OF.dequantize(rv, rvs),
                                             rows, causal=causal, softmax_scale=sc)
        bound = OF.fp8_out_bound(rq, rk, rv, rqs, rks, rvs, rows=rows, **kw)
        got_o = np.array([o[b, i, h] for b, h, i in rows])
        got_l = np.array([l[b, h, i] for b, h, i in rows])
    err = np.abs(got_o - ref_o)
    tol = 1.05 * bound + 2.0 ** -8 * np.abs(ref_o) + 1e-5
    assert np.all(np.isfinite(got_o)), "non-finite output"
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3f}, max err {err.max():.3e}"
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.max(np.abs(got_l[~empty] - ref_l[~empty]), initial=0.0) <= 1e-3
    if empty.any():
        rows_empty = empty if rows is not None else empty.transpose(0, 2, 1)  # lse [B, H, N] -> out [B, N, H]
        assert np.all(got_o[rows_empty] == 0)
    return float(np.mean(err)), float(np.mean(bound))


SHAPES = [
    # (B, Nq, Nk, Hq, Hkv, causal, incoherent)
    (1, 128, 128, 2, 2, True, True),
    (2, 200, 333, 4, 2, True, False),
    (1, 300, 300, 4, 1, False, True),
    (1, 65, 700, 2, 2, True, True),
    (1, 700, 65, 2, 1, True, True),     # leading rows see no key
    (1, 1, 900, 8, 2, True, False),
    (1, 513, 1030, 2, 2, False, False),
    (1, 100, 30, 2, 2, False, True),    # fewer keys than one tile
    (1, 100, 30, 2, 2, True, True),     # ... causal: the first 70 rows see nothing
    (2, 64, 64, 16, 1, True, True),     # MQA, one tile
    (1, 250, 2000, 8, 2, True, True),   # Nk >> Nq: bottom-right rows see long prefixes
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_fp8_small(shape):
    B, Nq, Nk, Hq, Hkv, causal, turn = shape
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, 128, seed=Nq + 3 * Nk)
    check_fp8(case, causal, turn, seed=Nq)


SHAPES_D = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, incoherent)
    (1, 128, 128, 2, 2, 64, True, True),
    (2, 200, 333, 4, 2, 64, True, False),
    (1, 700, 65, 2, 1, 64, True, True),
    (1, 513, 1030, 2, 2, 64, False, True),
    (1, 128, 128, 2, 2, 256, True, True),
    (2, 200, 333, 4, 2, 256, True, False),
    (1, 700, 65, 2, 1, 256, True, True),
    (1, 100, 30, 2, 2, 256, True, True),
    (1, 513, 1030, 2, 2, 256, False, True),
    (1, 1, 900, 8, 2, 256, True, False),
]


@pytest.mark.parametrize("shape", SHAPES_D, ids=lambda s: "x".join(map(str, s)))
def test_fwd_fp8_head_dims(shape):
    B, Nq, Nk, Hq, Hkv, d, causal, turn = shape
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed=Nq + 3 * Nk + d)
    check_fp8(case, causal, turn, seed=Nq + d)


def test_fwd_fp8_key_outliers_and_quiet_tiles():
    """K with 1% of rows x3 (the GQA workload's recipe) and a V tile 1000x quieter than the rest."""
    case = W.dense_case(1, 256, 640, 4, 2, 128, seed=77, k_outlier_frac=0.01)
    case["v"][0, 128:192] = (case["v"][0, 128:192].float() * 1e-3).to(torch.bfloat16)
    check_fp8(case, True, True, seed=5)
    check_fp8(case, True, False, seed=5)


def test_fwd_fp8_prefill_workload_sampled():
    """The causal MHA prefill workload (B=4, H=16, N=4096, d=128) with incoherent processing:
    all codes bit for bit, sampled rows against the oracle."""
    case = W.config_case("mha_causal_b4_h16_n4096_d128", device="cpu")
    rows = [(0, 0, 0), (0, 5, 63), (1, 15, 64), (2, 7, 2047), (3, 3, 4095), (3, 15, 1000), (1, 0, 4000)]
    check_fp8(case, True, True, seed=9, rows=rows)


@pytest.mark.parametrize("d", [64, 256])
def test_fwd_fp8_head_dims_long_sampled(d):
    """d = 64 and 256 over 2048 causal keys (many tiles and query tiles, GQA), all codes bit for bit,
    sampled rows against the oracle."""
    case = W.dense_case(2, 2048, 2048, 8, 2, d, seed=31 + d, k_outlier_frac=0.01)
    rows = [(0, 0, 0), (0, 7, 255), (1, 3, 256), (1, 4, 1023), (0, 2, 2047), (1, 6, 1500), (0, 5, 777)]
    check_fp8(case, True, True, seed=17, rows=rows)


def _fp8_forward(case, causal, turn, seed):
    d = case["q"].shape[-1]
    signs = W.hadamard_signs(d, seed).to(DEV) if turn else None
    qc, qs = ea.attn_fp8_quantize(case["q"].to(DEV), signs=signs)
    kc, ks = ea.attn_fp8_quantize(case["k"].to(DEV), signs=signs)
    vc, vs = ea.attn_fp8_quantize(case["v"].to(DEV), layout="vt")
    out, lse = ea.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=causal, softmax_scale=d ** -0.5, incoherent=turn)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


FP8_VS_DEFINITION = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, incoherent, key-outlier fraction)
    (1, 512, 512, 4, 2, 128, True, True, 0.0),
    (1, 512, 512, 4, 2, 128, True, False, 0.0),
    (1, 300, 900, 4, 1, 128, False, True, 0.01),
    (1, 256, 640, 4, 2, 64, True, True, 0.01),
    (1, 256, 640, 4, 2, 256, True, False, 0.0),
]


@pytest.mark.parametrize("shape", FP8_VS_DEFINITION, ids=lambda s: "x".join(map(str, s)))
def test_fwd_fp8_against_bf16_definition(shape):
    """The FP8 path end to end against the fp64 definition on the unquantised bf16
    inputs, by the pages' rule: at most twice the error of the lower-precision
    reference (exact attention on the same E4M3 block-quantised operands, which
    uses no constant of the kernel) plus the bf16 rounding of the output."""
    B, Nq, Nk, Hq, Hkv, d, causal, turn, frac = shape
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed=Nq + Nk + d, k_outlier_frac=frac)
    out, lse = _fp8_forward(case, causal, turn, seed=7)
    q, k, v = (to64(case[x]) for x in "qkv")
    hi_o, hi_l = oracle.attention_ref(q, k, v, causal=causal, softmax_scale=d ** -0.5)
    sg = W.hadamard_signs(d, 7).numpy().astype(np.float64) if turn else None
    rq, rqs = OF.quantize_blocks(q, sg)
    rk, rks = OF.quantize_blocks(k, sg)
    rv, rvs = OF.quantize_blocks(v, None)
    lo_o, lo_l = OF.attention_fp8_ref(rq, rk, rv, rqs, rks, rvs, causal=causal, softmax_scale=d ** -0.5,
                                      incoherent=turn)
    fin = np.isfinite(hi_l)
    e_gpu, e_lo = np.abs(out - hi_o), np.abs(lo_o - hi_o)
    print(f"fp8 vs definition {shape}: max {e_gpu.max():.4f} (lo {e_lo.max():.4f}), "
          f"mean {e_gpu.mean():.5f} (lo {e_lo.mean():.5f})")
    assert np.all(np.isfinite(out))
    assert e_gpu.max() <= 2 * e_lo.max() + 2.0 ** -8 * np.abs(hi_o).max()
    assert e_gpu.mean() <= 2 * e_lo.mean() + 2.0 ** -9 * np.abs(hi_o).mean()
    assert np.abs(lse[fin] - hi_l[fin]).max() <= 2 * np.abs(lo_l[fin] - hi_l[fin]).max() + 1e-3


def test_fwd_fp8_incoherence_lowers_error_on_feature_outliers():
    """Four feature channels of Q and K twenty times larger than the rest: the
    turn must cut the FP8 path's mean error against the definition to at most
    2/3 of the error without it ("FlashAttention-3 and PagedAttention: IO-Aware
    Attention Kernels (2026)", "FlashAttention-3": 2.6x lower error)."""
    case = W.dense_case(1, 512, 512, 4, 2, 128, seed=123)
    g = torch.Generator().manual_seed(3)
    ch = torch.randperm(128, generator=g)[:4]
    for t in ("q", "k"):
        x = case[t].float()
        x[..., ch] *= 20.0
        case[t] = x.to(torch.bfloat16)
    q, k, v = (to64(case[x]) for x in "qkv")
    hi_o, _ = oracle.attention_ref(q, k, v, causal=True, softmax_scale=128 ** -0.5)
    errs = []
    for turn in (False, True):
        out, _ = _fp8_forward(case, True, turn, seed=11)
        errs.append(float(np.mean(np.abs(out - hi_o))))
    print(f"fp8 feature outliers: mean error without turn {errs[0]:.4f}, with turn {errs[1]:.4f}")
    assert errs[1] <= (2.0 / 3.0) * errs[0], errs
