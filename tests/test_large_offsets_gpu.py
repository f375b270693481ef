"""Element offsets past 2^31 on the HIP path (needs an MI355X).

Every kernel forms its addresses from 64-bit element offsets.  These tests
put small seeded cases behind large filler regions, so that their query, key,
value, output and gradient elements, or their cache pages, sit past element
2^31 of their tensors, and compare them with the oracle on the small cases
alone.  The fillers have closed-form results: zero queries, keys and values
give uniform weights, a zero output and lse = ln(number of keys); rows that
see no key give out = 0 and lse = -inf; with a zero output gradient every
filler gradient is exactly zero.

About 35 GB of device memory for the packed forward and backward, 9 GB for
each paged case; a few seconds in all.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W
from test_bwd_gpu import assert_grads, bf16_reference
from test_kvcache_gpu import assert_same_bits, call, tables
from test_parity_gpu import assert_close, decode_parity, to64
from test_window_paged_gpu import paged_prefill_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LIMIT = 2 ** 31


def test_packed_forward_and_backward_offsets_past_2_31():
    """Three packed sequences, 32 query and 32 K/V heads, d = 128: one query
    row over 540,000 zero keys, 530,000 zero query rows over one zero key, then
    a seeded 150 x 333 causal case whose first query element sits at
    530,001 * 32 * 128 and first key element at 540,001 * 32 * 128, both past
    2^31."""
    hq = hkv = 32
    d = 128
    n_fill_k, n_fill_q = 540_000, 530_000
    real_q, real_k = 150, 333
    nq = [1, n_fill_q, real_q]
    nk = [n_fill_k, 1, real_k]
    tq, tk = sum(nq), sum(nk)
    q_off, k_off = tq - real_q, tk - real_k
    assert q_off * hq * d >= LIMIT and k_off * hkv * d >= LIMIT
    case = W.varlen_case([real_q], [real_k], hq, hkv, d, seed=4242)
    g = torch.Generator().manual_seed(4243)
    dout_real = torch.randn(case["q"].shape, generator=g).to(torch.bfloat16)
    scale = d ** -0.5
    print(f"packed offsets: tq={tq} tk={tk} q_off={q_off} k_off={k_off}", flush=True)

    bf16 = torch.bfloat16
    q = torch.zeros((tq, hq, d), dtype=bf16, device=DEV)
    k = torch.zeros((tk, hkv, d), dtype=bf16, device=DEV)
    v = torch.zeros((tk, hkv, d), dtype=bf16, device=DEV)
    q[q_off:] = case["q"].to(DEV)
    k[k_off:] = case["k"].to(DEV)
    v[k_off:] = case["v"].to(DEV)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=DEV)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(nk)]), dtype=torch.int32, device=DEV)
    kw = dict(cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=max(nq), max_seqlen_k=max(nk), causal=True,
              softmax_scale=scale)
    out, lse = ea.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()

    cqh, ckh = case["cu_seqlens_q"].numpy(), case["cu_seqlens_k"].numpy()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), causal=True,
                                        softmax_scale=scale, cu_seqlens_q=cqh, cu_seqlens_k=ckh)
    assert_close(to64(out[q_off:]), to64(lse[:, q_off:]), ref_o, ref_l, "packed past 2^31")
    # fillers: zero output everywhere; the single row of sequence 0 weighs all
    # its keys equally; in sequence 1 only the last row sees the key
    assert torch.all(out[:q_off] == 0).item()
    lse0 = to64(lse[:, 0])
    assert np.all(np.abs(lse0 - math.log(n_fill_k)) <= 1e-4), lse0[:4]
    lse1 = lse[:, 1:1 + n_fill_q]
    assert torch.all(torch.isneginf(lse1[:, :-1])).item()
    assert torch.all(lse1[:, -1] == 0).item()

    dout = torch.zeros_like(q)
    dout[q_off:] = dout_real.to(DEV)
    print("packed offsets: backward", flush=True)
    dq, dk, dv = ea.attn_bwd(q, k, v, out, lse, dout, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), to64(dout_real),
                                   causal=True, softmax_scale=scale, cu_seqlens_q=cqh, cu_seqlens_k=ckh)
    low = bf16_reference(case["q"], case["k"], case["v"], dout_real, causal=True, scale=scale, cu_q=cqh,
                         cu_k=ckh)
    assert_grads((to64(dq[q_off:]), to64(dk[k_off:]), to64(dv[k_off:])), ref, low, "packed past 2^31")
    assert torch.all(dq[:q_off] == 0).item()
    assert torch.all(dk[:k_off] == 0).item() and torch.all(dv[:k_off] == 0).item()


def _shift_pages(cache, first_page):
    """The case's pages moved to physical ids first_page.. of a larger cache
    (zero below them); the block table is shifted to match."""
    kc, vc = cache["k_cache"], cache["v_cache"]
    n = kc.shape[0]
    big_k = torch.zeros((first_page + n,) + tuple(kc.shape[1:]), dtype=kc.dtype, device=DEV)
    big_v = torch.zeros_like(big_k)
    big_k[first_page:] = kc.to(DEV)
    big_v[first_page:] = vc.to(DEV)
    out = dict(cache)
    out["k_cache"], out["v_cache"] = big_k, big_v
    out["block_table"] = (cache["block_table"] + first_page).to(torch.int32)
    return out


def test_decode_pages_past_2_31():
    """Split-KV decode and combine reading pages whose first element is past
    2^31 (Hkv = 8, d = 128: page 8192 starts at element 2^31), including the
    NaN poison page behind every request's last page."""
    hkv, d = 8, 128
    page_elems = 256 * hkv * d
    first = LIMIT // page_elems
    case = W.decode_case([300, 4096, 1, 2049, 700], 32, hkv, d, seed=4244, poison=True, extra_table_cols=1)
    big = _shift_pages(case, first)
    print(f"decode pages from {first}: cache {tuple(big['k_cache'].shape)}", flush=True)
    for chunk in (256, 1024):
        decode_parity(big, chunk)


def test_paged_prefill_pages_past_2_31():
    """Packed query rows against a paged cache whose pages start past element
    2^31, compared with the oracle on the original cache."""
    hq, hkv, d = 8, 8, 128
    first = LIMIT // (256 * hkv * d)
    nk = [300, 1, 2049, 600]
    nq = [300, 1, 17, 200]
    q, cq, c = paged_prefill_case(nq, nk, hq, hkv, d, seed=4245)
    big = _shift_pages(c, first)
    scale = d ** -0.5
    print(f"paged prefill pages from {first}: cache {tuple(big['k_cache'].shape)}", flush=True)
    out, lse = ea.attn_fwd_paged(q.to(DEV), big["k_cache"], big["v_cache"], big["block_table"].to(DEV),
                                 cq.to(DEV), c["seqlens_k"].to(DEV), max_seqlen_q=max(nq), causal=True,
                                 softmax_scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.paged_prefill_ref(to64(q), to64(c["k_cache"]), to64(c["v_cache"]),
                                            c["block_table"].numpy(), cq.numpy(), c["seqlens_k"].numpy(),
                                            causal=True, softmax_scale=scale)
    assert_close(to64(out), to64(lse), ref_o, ref_l, "paged prefill past 2^31")


def test_append_rotary_decode_pages_past_2_31():
    """In-place append with rotary turns writing pages from id 8192 on: the
    cache bytes bit for bit against the oracle's appended cache, every page
    below untouched, and the decode output at the forward bar."""
    hkv, d = 8, 128
    first = LIMIT // (256 * hkv * d)
    lens = [0, 1, 255, 256, 1000, 3000]
    case = W.append_case(lens, 32, hkv, d, seed=4246, poison=True, extra_table_cols=1)
    cos, sin, cos_h, sin_h = tables(128, 3100)
    rkw = dict(rotary_cos=cos_h, rotary_sin=sin_h, rotary_dim=128, interleaved=False)
    kc_ref, vc_ref = oracle.append_ref(to64(case["k_new"]), to64(case["v_new"]), to64(case["k_cache"]),
                                       to64(case["v_cache"]), case["block_table"].numpy(), lens, **rkw)
    ref_o, ref_l, ref_q = oracle.decode_append_ref(
        to64(case["q"]), to64(case["k_new"]), to64(case["v_new"]), to64(case["k_cache"]),
        to64(case["v_cache"]), case["block_table"].numpy(), lens, softmax_scale=d ** -0.5, **rkw)
    big = _shift_pages(case, first)
    dev = {x: (big[x] if x in ("k_cache", "v_cache") else big[x].to(DEV))
           for x in ("q", "k_new", "v_new", "k_cache", "v_cache", "block_table", "seqlens_k")}
    print(f"append pages from {first}: cache {tuple(big['k_cache'].shape)}", flush=True)
    out, lse, q_rot = call(case, dev, cos, sin, False, 512)
    torch.cuda.synchronize()
    assert_same_bits(dev["k_cache"][first:], kc_ref, "append past 2^31 k_cache")
    assert_same_bits(dev["v_cache"][first:], vc_ref, "append past 2^31 v_cache")
    assert torch.all(dev["k_cache"][:first] == 0).item() and torch.all(dev["v_cache"][:first] == 0).item()
    assert_same_bits(q_rot, ref_q, "append past 2^31 q_rot")
    assert_close(to64(out), to64(lse), ref_o, ref_l, "append past 2^31")
