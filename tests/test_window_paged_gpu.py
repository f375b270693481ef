"""Local-window and paged prefill on the HIP path vs the CPU fp64 oracle (needs an MI355X).

Same tolerances as the forward parity tests: max |out - ref| <= 1.5e-2, mean
<= 1e-3, |lse - ref| <= 1e-3, rows with no allowed key exactly out = 0 and
lse = -inf.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W
from test_parity_gpu import assert_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

WINDOWED = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, window)
    (1, 300, 300, 4, 2, 128, True, (64, -1)),     # sliding window, causal
    (1, 257, 513, 2, 1, 64, False, (100, 50)),    # two-sided, Nq < Nk
    (2, 65, 200, 4, 2, 128, True, (0, 0)),        # a single key per row
    (1, 200, 90, 2, 2, 128, False, (0, 0)),       # Nq > Nk: leading rows see nothing
    (1, 128, 1000, 2, 2, 256, True, (17, -1)),
    (1, 1000, 1000, 8, 1, 128, True, (255, -1)),  # window of exactly four 64-key tiles
    (1, 333, 333, 2, 2, 64, False, (-1, 40)),     # right side only
]


@pytest.mark.parametrize("shape", WINDOWED, ids=lambda s: "x".join(map(str, s[:7])) + f"w{s[7][0]}_{s[7][1]}")
def test_window_dense(shape):
    B, Nq, Nk, Hq, Hkv, d, causal, window = shape
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed=Nq + Nk + d)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    out, lse = ea.attn_fwd(q, k, v, causal=causal, softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]),
                                        causal=causal, softmax_scale=scale, window=window)
    o = to64(out)
    empty = np.isneginf(ref_l)
    if empty.any():
        bb, hh, ii = np.nonzero(empty)
        assert np.all(o[bb, ii, hh] == 0)
    assert_close(o, to64(lse), ref_o, ref_l, f"window {shape}")


@pytest.mark.parametrize("d", [128, 64])
def test_window_varlen(d):
    nq = [3, 0, 64, 129, 1, 70, 400]
    nk = [100, 5, 64, 300, 1, 0, 1600]
    case = W.varlen_case(nq, nk, 4, 2, d, seed=500 + d)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    cq, ck = case["cu_seqlens_q"].to(DEV), case["cu_seqlens_k"].to(DEV)
    out, lse = ea.attn_fwd(q, k, v, cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=case["max_seqlen_q"],
                           max_seqlen_k=case["max_seqlen_k"], causal=True, softmax_scale=scale,
                           window=(96, -1))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), causal=True,
                                        softmax_scale=scale, cu_seqlens_q=case["cu_seqlens_q"].numpy(),
                                        cu_seqlens_k=case["cu_seqlens_k"].numpy(), window=(96, -1))
    assert_close(to64(out), to64(lse), ref_o, ref_l, f"window varlen d{d}")


def paged_prefill_case(nq, nk, hq, hkv, d, seed, poison=True):
    """A paged cache from the decode generator plus packed new query rows."""
    cache = W.decode_case(nk, hq, hkv, d, seed, page=256, poison=poison, extra_table_cols=1)
    g = torch.Generator().manual_seed(seed + 7)
    tq = int(sum(nq))
    q = torch.randn((tq, hq, d), generator=g).to(torch.bfloat16)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32)
    return q, cq, cache


@pytest.mark.parametrize("d,causal,window", [(128, True, (-1, -1)), (64, True, (200, -1)),
                                             (256, False, (-1, -1)), (128, False, (300, 10)),
                                             (256, True, (-1, -1))])
def test_paged_prefill(d, causal, window):
    nk = [300, 1, 2049, 512, 4100]
    nq = [300, 1, 17, 0, 1025]  # the new rows are the last keys of each sequence
    q, cq, c = paged_prefill_case(nq, nk, 8, 2, d, seed=60 + d)
    scale = d ** -0.5
    dev = {x: c[x].to(DEV) for x in ("k_cache", "v_cache", "block_table", "seqlens_k")}
    out, lse = ea.attn_fwd_paged(q.to(DEV), dev["k_cache"], dev["v_cache"], dev["block_table"],
                                 cq.to(DEV), dev["seqlens_k"], max_seqlen_q=max(nq), causal=causal,
                                 softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.paged_prefill_ref(to64(q), to64(c["k_cache"]), to64(c["v_cache"]),
                                            c["block_table"].numpy(), cq.numpy(), c["seqlens_k"].numpy(),
                                            causal=causal, softmax_scale=scale, window=window)
    assert_close(to64(out), to64(lse), ref_o, ref_l, f"paged d{d} c{causal} w{window}")


def test_paged_prefill_bad_page_is_nan():
    """An out-of-range page id poisons the rows that read it; other sequences are unaffected."""
    nk = [600, 300]
    nq = [100, 300]
    q, cq, c = paged_prefill_case(nq, nk, 4, 4, 128, seed=99, poison=False)
    table = c["block_table"].clone()
    table[0, 1] = c["num_pages"] + 5  # keys 256..511 of sequence 0
    out, lse = ea.attn_fwd_paged(q.to(DEV), c["k_cache"].to(DEV), c["v_cache"].to(DEV), table.to(DEV),
                                 cq.to(DEV), c["seqlens_k"].to(DEV), max_seqlen_q=max(nq), causal=True,
                                 softmax_scale=128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isnan(out[:100].float()).all().item()
    ref_o, ref_l = oracle.paged_prefill_ref(to64(q), to64(c["k_cache"]), to64(c["v_cache"]),
                                            c["block_table"].numpy(), cq.numpy(), c["seqlens_k"].numpy(),
                                            causal=True, softmax_scale=128 ** -0.5, sequences=[1])
    assert_close(to64(out)[100:], to64(lse)[:, 100:], ref_o[100:], ref_l[:, 100:], "paged, good sequence")


def test_window_none_is_bitwise_attn_fwd():
    """window = (-1, -1) through attn_fwd_ex gives attn_fwd's results bit for bit."""
    case = W.dense_case(1, 300, 300, 4, 2, 128, seed=3)
    q, k, v = (case[x].to(DEV) for x in "qkv")
    a = ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.1)
    lib = ea.lib()
    out, lse = torch.empty_like(q), torch.empty_like(a[1])
    st = lib.attn_fwd_ex(ea._ptr(q), ea._ptr(k), ea._ptr(v), None, None, None, None, 1, 300, 300, 4, 2,
                         128, 256, 0, 0, 1, -1, -1, 0.1, ea._ptr(out), ea._ptr(lse),
                         ea._stream(None, q.device))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(out, a[0]) and torch.equal(lse, a[1])


@pytest.mark.parametrize("n_seqs", [64, 70])
def test_paged_prefill_many_sequences(n_seqs):
    """Paged prefill over batches at and past the length-ranking limit (64 sequences)."""
    rng = np.random.default_rng(900 + n_seqs)
    nk = [int(x) for x in rng.integers(1, 700, size=n_seqs)]
    nq = [min(int(x), n) for x, n in zip(rng.integers(0, 200, size=n_seqs), nk)]
    q, cq, c = paged_prefill_case(nq, nk, 4, 2, 128, seed=950 + n_seqs)
    scale = 128 ** -0.5
    dev = {x: c[x].to(DEV) for x in ("k_cache", "v_cache", "block_table", "seqlens_k")}
    out, lse = ea.attn_fwd_paged(q.to(DEV), dev["k_cache"], dev["v_cache"], dev["block_table"],
                                 cq.to(DEV), dev["seqlens_k"], max_seqlen_q=max(nq), causal=True,
                                 softmax_scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.paged_prefill_ref(to64(q), to64(c["k_cache"]), to64(c["v_cache"]),
                                            c["block_table"].numpy(), cq.numpy(), c["seqlens_k"].numpy(),
                                            causal=True, softmax_scale=scale)
    assert_close(to64(out), to64(lse), ref_o, ref_l, f"paged, {n_seqs} sequences")
