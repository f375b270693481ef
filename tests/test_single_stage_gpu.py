"""LDS-race check: the forward kernel rebuilt with a single LDS stage
(libattn_single_stage.so, built beside libattn.so by the same build) loads each
tile only after every wave has finished the previous one.  It performs the same
arithmetic in the same order, so its outputs must equal the double-buffered
kernel's bit for bit; a difference would mean a wave read a stage while the
next tile's loads were landing in it.  Both libraries are called through the C
ABI (needs an MI355X)."""
import contextlib
import ctypes

import pytest
import torch

import exact_io_aware_07_amd as ea
from exact_io_aware_07_amd import build as B
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@contextlib.contextmanager
def single_stage_library():
    handle = ctypes.CDLL(B.LIB_SINGLE_STAGE)
    for name, (args, res) in ea._SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = res
    saved = ea.lib()
    ea._lib = handle
    try:
        yield
    finally:
        ea._lib = saved


def both(fn):
    a = fn()
    torch.cuda.synchronize()
    with single_stage_library():
        b = fn()
        torch.cuda.synchronize()
    return a, b


DENSE = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, window)
    # Grids of at most 128 workgroups with enough keys run in split-key mode
    # (each wave its own stages): the first three.
    (2, 1024, 1024, 4, 4, 128, True, (-1, -1)),
    (1, 700, 1500, 8, 2, 128, True, (-1, -1)),
    (1, 513, 777, 4, 1, 64, False, (-1, -1)),
    # Shared stages: d = 256, a narrow window, and grids over 128 workgroups.
    (1, 600, 600, 4, 2, 256, True, (-1, -1)),
    (1, 1024, 1024, 4, 2, 128, True, (255, -1)),
    (2, 2048, 2048, 16, 4, 128, True, (-1, -1)),
    (2, 1024, 1030, 16, 16, 64, False, (-1, -1)),
]


@pytest.mark.parametrize("shape", DENSE, ids=lambda s: "x".join(map(str, s)))
def test_single_stage_bitwise_dense(shape):
    Bn, Nq, Nk, Hq, Hkv, d, causal, window = shape
    c = W.dense_case(Bn, Nq, Nk, Hq, Hkv, d, seed=700 + Nq + d, device=DEV)
    (o1, l1), (o2, l2) = both(lambda: ea.attn_fwd(c["q"], c["k"], c["v"], causal=causal, softmax_scale=d ** -0.5,
                                                  window=window))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_single_stage_bitwise_varlen(d):
    nq = [300, 0, 1, 900, 77]
    nk = [1200, 5, 64, 900, 300]
    c = W.varlen_case(nq, nk, 8, 2, d, seed=720 + d, device=DEV)
    kw = dict(cu_seqlens_q=c["cu_seqlens_q"].to(DEV), cu_seqlens_k=c["cu_seqlens_k"].to(DEV),
              max_seqlen_q=max(nq), max_seqlen_k=max(nk), causal=True, softmax_scale=d ** -0.5)
    (o1, l1), (o2, l2) = both(lambda: ea.attn_fwd(c["q"], c["k"], c["v"], **kw))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_single_stage_bitwise_paged():
    lens = [700, 1300, 256]
    nq = [100, 300, 256]
    c = W.decode_case(lens, 8, 2, 128, seed=731, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(732)
    q = torch.randn((sum(nq), 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    cu = torch.tensor([0, nq[0], nq[0] + nq[1], sum(nq)], dtype=torch.int32, device=DEV)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in c.items()}
    (o1, l1), (o2, l2) = both(lambda: ea.attn_fwd_paged(q, dev["k_cache"], dev["v_cache"], dev["block_table"], cu,
                                                        dev["seqlens_k"], max_seqlen_q=max(nq), causal=True,
                                                        softmax_scale=128 ** -0.5))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
