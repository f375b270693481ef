"""Gradients on the HIP path vs the CPU fp64 oracle (needs an MI355X).

Tolerance, following "Deep Dive - FlashAttention", "Backward recomputes tiles
on purpose" (the tests there bound the error by twice the error of a
lower-precision PyTorch reference against a higher-precision path, with an
extra absolute allowance): for each of dq, dk and dv,

    max |gpu - oracle|  <= 2 * max |bf16 reference - oracle|  + 1e-3 * G
    mean |gpu - oracle| <= 2 * mean |bf16 reference - oracle| + 1e-4 * G

with G the largest |oracle| over dq, dk and dv together, where the bf16 reference is plain PyTorch autograd on the CPU over the same
bf16 inputs with every tensor kept in bf16 (scores, probabilities, output),
and the oracle is oracle.attention_bwd_ref in fp64.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def to64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def bf16_reference(q, k, v, dout, *, causal, scale, cu_q=None, cu_k=None, heads=None):
    """PyTorch autograd in bf16 on the CPU, per sequence; float64 numpy grads.

    Layouts as the library's.  heads restricts the query heads (and their K/V
    heads); other entries stay zero.
    """
    varlen = cu_q is not None
    q4, k4, v4, g4 = (t[None] if varlen else t for t in (q, k, v, dout))
    hq, hkv = q4.shape[2], k4.shape[2]
    grp = hq // hkv
    hs = list(range(hq)) if heads is None else list(heads)
    dq, dk, dv = (np.zeros(t.shape) for t in (q4, k4, v4))
    seqs = ([(0, int(cu_q[i]), int(cu_q[i + 1] - cu_q[i]), int(cu_k[i]), int(cu_k[i + 1] - cu_k[i]))
             for i in range(len(cu_q) - 1)] if varlen else
            [(b, 0, q4.shape[1], 0, k4.shape[1]) for b in range(q4.shape[0])])
    for bb, qo, nq, ko, nk in seqs:
        if nq == 0 or nk == 0:
            continue
        kvs = sorted({h // grp for h in hs})
        Q = q4[bb, qo:qo + nq, hs].permute(1, 0, 2).clone().requires_grad_(True)
        K = k4[bb, ko:ko + nk, kvs].permute(1, 0, 2).clone().requires_grad_(True)
        V = v4[bb, ko:ko + nk, kvs].permute(1, 0, 2).clone().requires_grad_(True)
        idx = torch.tensor([kvs.index(h // grp) for h in hs])
        Ke, Ve = K[idx], V[idx]
        S = (Q @ Ke.transpose(-1, -2)) * scale
        keep = torch.from_numpy(oracle.causal_keep(nq, nk)) if causal else torch.ones(nq, nk, dtype=torch.bool)
        has = keep.any(dim=-1, keepdim=True)
        S = torch.where(keep, S, torch.full_like(S, -float("inf")))
        S = torch.where(has, S, torch.zeros_like(S))
        P = torch.softmax(S, dim=-1).masked_fill(~keep, 0.0)
        O = P @ Ve
        O.backward(g4[bb, qo:qo + nq, hs].permute(1, 0, 2))
        for n, h in enumerate(hs):
            dq[bb, qo:qo + nq, h] = Q.grad[n].double().numpy()
        for n, h in enumerate(kvs):
            dk[bb, ko:ko + nk, h] += K.grad[n].double().numpy()
            dv[bb, ko:ko + nk, h] += V.grad[n].double().numpy()
    if varlen:
        return dq[0], dk[0], dv[0]
    return dq, dk, dv


def assert_grads(gpu, ref, low, tag, mask=None):
    # The absolute allowance is taken relative to the largest reference
    # gradient of the problem (dq, dk and dv together): a gradient that is
    # exactly zero (a row with a single visible key has dS = P (dP - D) = 0)
    # still leaves room for the fp32 rounding of dP - D.
    sel = []
    for name, g, r, lo in zip(("dq", "dk", "dv"), gpu, ref, low):
        if mask is not None:
            g, r, lo = g[mask[name]], r[mask[name]], lo[mask[name]]
        sel.append((name, g, r, lo))
    scale = max([np.max(np.abs(r)) for _, _, r, _ in sel if r.size] + [1e-30])
    for name, g, r, lo in sel:
        if r.size == 0:
            continue
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite"
        e_gpu, e_low = np.abs(g - r), np.abs(lo - r)
        assert e_gpu.max() <= 2 * e_low.max() + 1e-3 * scale, (
            f"{tag} {name}: max err {e_gpu.max():.3e} vs bf16 reference {e_low.max():.3e} (scale {scale:.3e})")
        assert e_gpu.mean() <= 2 * e_low.mean() + 1e-4 * scale, (
            f"{tag} {name}: mean err {e_gpu.mean():.3e} vs bf16 reference {e_low.mean():.3e}")


def run_dense(B, Nq, Nk, Hq, Hkv, d, causal, seed, heads=None, k_outlier_frac=0.0):
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed, k_outlier_frac=k_outlier_frac)
    g = torch.Generator().manual_seed(seed + 1000)
    dout = torch.randn(case["q"].shape, generator=g).to(torch.bfloat16)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    out, lse = ea.attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, out, lse, dout.to(DEV), causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    kvh = None if heads is None else sorted({h // (Hq // Hkv) for h in heads})
    ref = oracle.attention_bwd_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), to64(dout),
                                   causal=causal, softmax_scale=scale, kv_heads=kvh)
    low = bf16_reference(case["q"], case["k"], case["v"], dout, causal=causal, scale=scale, heads=heads)
    mask = None
    if heads is not None:
        mask = {"dq": (slice(None), slice(None), heads), "dk": (slice(None), slice(None), kvh),
                "dv": (slice(None), slice(None), kvh)}
    assert_grads((to64(dq), to64(dk), to64(dv)), ref, low, f"dense B{B} Nq{Nq} Nk{Nk} Hq{Hq} Hkv{Hkv} d{d} c{causal}", mask)
    return dq, dk, dv


SMALL = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (1, 128, 128, 2, 2, 128, True),
    (1, 128, 128, 2, 2, 64, True),
    (2, 65, 200, 4, 2, 128, True),     # bottom-right corner, ragged tiles
    (1, 300, 7, 2, 1, 64, True),       # leading rows with no key
    (1, 257, 513, 3, 1, 128, False),   # MQA, ragged, non-causal
    (1, 1, 1000, 8, 1, 128, True),     # one query row
    (1, 200, 200, 8, 2, 64, False),
    (2, 96, 33, 4, 4, 128, False),
    (1, 128, 128, 2, 2, 256, True),
    (2, 65, 200, 4, 2, 256, True),     # d = 256: ragged, GQA, bottom-right corner
    (1, 257, 300, 3, 1, 256, False),   # d = 256: MQA, non-causal
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bwd_dense_small(shape):
    run_dense(*shape, seed=sum(shape))


@pytest.mark.parametrize("shape", [(3, 300, 300, 32, 32, 128, True), (2, 200, 260, 64, 16, 64, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_four_head_groups(shape):
    """(sequence, head) counts that are multiples of 32, so each XCD runs its
    heads four at a time in the dK/dV kernel (B x Hkv = 96 and 32) and the dQ
    kernel (B x Hq = 96 and 128)."""
    run_dense(*shape, seed=900 + sum(shape))


def test_bwd_gqa_medium_with_key_outliers():
    run_dense(1, 1024, 1024, 8, 2, 128, True, seed=31, k_outlier_frac=0.01)


def test_bwd_long_causal_sampled_heads():
    """A 4096-token causal head pair at the prefill workload's shape, two heads checked."""
    run_dense(1, 4096, 4096, 4, 4, 128, True, seed=41, heads=[0, 3])


def test_bwd_prefill_workload_sampled():
    """The shape and launch configuration bench.py times for the backward (B=4, H=16,
    N=4096, d=128, causal): every batch of two heads checked against the oracle."""
    run_dense(4, 4096, 4096, 16, 16, 128, True, seed=2, heads=[0, 9])


@pytest.mark.parametrize("d", [128, 64, 256])
def test_bwd_varlen(d):
    lens = [(3, 100), (0, 5), (64, 64), (129, 300), (1, 1), (70, 0)]
    nq = [a for a, _ in lens]
    nk = [b for _, b in lens]
    case = W.varlen_case(nq, nk, 4, 2, d, seed=900 + d)
    g = torch.Generator().manual_seed(77 + d)
    dout = torch.randn(case["q"].shape, generator=g).to(torch.bfloat16)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    cq, ck = case["cu_seqlens_q"].to(DEV), case["cu_seqlens_k"].to(DEV)
    kw = dict(cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=case["max_seqlen_q"],
              max_seqlen_k=case["max_seqlen_k"], causal=True, softmax_scale=scale)
    out, lse = ea.attn_fwd(q, k, v, **kw)
    dq, dk, dv = ea.attn_bwd(q, k, v, out, lse, dout.to(DEV), **kw)
    torch.cuda.synchronize()
    cqh, ckh = case["cu_seqlens_q"].numpy(), case["cu_seqlens_k"].numpy()
    ref = oracle.attention_bwd_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), to64(dout),
                                   causal=True, softmax_scale=scale, cu_seqlens_q=cqh, cu_seqlens_k=ckh)
    low = bf16_reference(case["q"], case["k"], case["v"], dout, causal=True, scale=scale,
                         cu_q=cqh, cu_k=ckh)
    assert_grads((to64(dq), to64(dk), to64(dv)), ref, low, f"varlen d{d}")
    # rows with no key and keys no row sees get exactly zero
    assert torch.all(dq[cqh[5]:cqh[6]] == 0).item()
    assert torch.all(dk[ckh[1]:ckh[2]] == 0).item() and torch.all(dv[ckh[1]:ckh[2]] == 0).item()


def test_bwd_deterministic():
    a = run_dense(1, 256, 384, 4, 2, 128, True, seed=5)
    b = run_dense(1, 256, 384, 4, 2, 128, True, seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_single_visible_key():
    """Nq > Nk with one key: only the last rows see it, each row has a single
    visible key, so dS = P (dP - D) vanishes and dq is exactly zero in exact
    arithmetic (the allowance then comes from dk and dv's scale)."""
    run_dense(2, 52, 1, 8, 2, 128, True, seed=130)
    run_dense(1, 40, 3, 4, 4, 64, True, seed=131)
