"""Randomised shapes, streams and graph capture on the HIP path vs the CPU oracle (needs an MI355X).

Each seed draws one configuration (mode, head dim, head counts, lengths,
causal, window; decode lengths and chunk) small enough for the oracle to
finish in seconds, and compares with the parity bar of test_parity_gpu.
The stream and graph tests check that every call runs on the caller's stream
and that a captured graph replays to the same bits as eager calls.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W
from test_parity_gpu import assert_close, decode_parity, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def draw_fwd(seed):
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([64, 128, 256]))
    hkv = int(r.integers(1, 4))
    hq = hkv * int(r.choice([1, 2, 4, 8]))
    causal = bool(r.integers(0, 2))
    window = (-1, -1)
    if r.random() < 0.35:
        window = (int(r.integers(0, 300)), int(r.choice([-1, int(r.integers(0, 50))])))
    if r.random() < 0.5:
        shape = dict(mode="dense", B=int(r.integers(1, 4)), Nq=int(r.integers(1, 700)), Nk=int(r.integers(1, 700)))
    else:
        n = int(r.integers(1, 6))
        shape = dict(mode="varlen", nq=[int(x) for x in r.integers(0, 400, size=n)],
                     nk=[int(x) for x in r.integers(0, 600, size=n)])
    return dict(d=d, hq=hq, hkv=hkv, causal=causal, window=window, **shape)


@pytest.mark.parametrize("seed", range(24))
def test_fwd_random(seed):
    c = draw_fwd(seed)
    d, scale = c["d"], c["d"] ** -0.5
    kw = dict(causal=c["causal"], softmax_scale=scale, window=c["window"])
    if c["mode"] == "dense":
        case = W.dense_case(c["B"], c["Nq"], c["Nk"], c["hq"], c["hkv"], d, seed=seed)
        q, k, v = (case[x].to(DEV) for x in "qkv")
        out, lse = ea.attn_fwd(q, k, v, **kw)
        ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), **kw)
    else:
        case = W.varlen_case(c["nq"], c["nk"], c["hq"], c["hkv"], d, seed=seed)
        q, k, v = (case[x].to(DEV) for x in "qkv")
        out, lse = ea.attn_fwd(q, k, v, cu_seqlens_q=case["cu_seqlens_q"].to(DEV),
                               cu_seqlens_k=case["cu_seqlens_k"].to(DEV), max_seqlen_q=case["max_seqlen_q"],
                               max_seqlen_k=case["max_seqlen_k"], **kw)
        ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]),
                                            cu_seqlens_q=case["cu_seqlens_q"].numpy(),
                                            cu_seqlens_k=case["cu_seqlens_k"].numpy(), **kw)
    torch.cuda.synchronize()
    assert_close(to64(out), to64(lse), ref_o, ref_l, f"seed {seed}: {c}")


@pytest.mark.parametrize("seed", range(8))
def test_decode_random(seed):
    r = np.random.default_rng(2000 + seed)
    d = int(r.choice([64, 128, 256]))
    hkv = int(r.integers(1, 5))
    hq = hkv * int(r.choice([1, 2, 4, 8, 16]))
    lens = [int(x) for x in r.integers(0, 3000, size=int(r.integers(1, 7)))]
    chunk = 256 * int(r.integers(1, 9))
    decode_parity(W.decode_case(lens, hq, hkv, d, seed=seed, poison=True, extra_table_cols=1), chunk)


@pytest.mark.parametrize("seed", range(6))
def test_bwd_random(seed):
    from test_bwd_gpu import run_dense
    r = np.random.default_rng(3000 + seed)
    d = int(r.choice([64, 128, 256]))
    hkv = int(r.integers(1, 3))
    hq = hkv * int(r.choice([1, 2, 4]))
    run_dense(int(r.integers(1, 3)), int(r.integers(1, 300)), int(r.integers(1, 300)), hq, hkv, d,
              bool(r.integers(0, 2)), seed=seed)


def test_calls_run_on_the_callers_stream():
    """A call made under another stream gives the same bits as on the default stream."""
    case = W.dense_case(2, 300, 500, 8, 2, 128, seed=11)
    q, k, v = (case[x].to(DEV) for x in "qkv")
    ref = ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.1)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.1)
    s.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_graph_capture_replays_match_eager():
    """Prefill and split + combine decode captured in one graph; three replays with new inputs
    copied in between, each equal bit for bit to the eager calls on those inputs."""
    pc = W.dense_case(1, 512, 512, 4, 2, 128, seed=21)
    dc = W.decode_case([700, 1, 2049, 300], 8, 2, 128, seed=22)
    q, k, v = (pc[x].to(DEV) for x in "qkv")
    dq, kc, vc = dc["q"].to(DEV), dc["k_cache"].to(DEV), dc["v_cache"].to(DEV)
    bt, sl = dc["block_table"].to(DEV), dc["seqlens_k"].to(DEV)
    chunk, n = 512, ea.attn_decode_num_splits(2049, 512)
    out, lse = torch.empty_like(q), torch.empty((1, 4, 512), dtype=torch.float32, device=DEV)
    po = torch.empty((n, 4, 8, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((n, 4, 8), dtype=torch.float32, device=DEV)
    dout, dlse = torch.empty_like(dq), torch.empty((4, 8), dtype=torch.float32, device=DEV)

    def work():
        ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.09, out=out, lse=lse)
        ea.attn_decode_splitkv(dq, kc, vc, bt, sl, chunk_tokens=chunk, num_splits=n, softmax_scale=0.09,
                               out_partial=po, lse_partial=pl)
        ea.attn_decode_combine(po, pl, sl, chunk_tokens=chunk, out=dout, lse=dlse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    gen = torch.Generator(device=DEV).manual_seed(5)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        dq.copy_(torch.randn(dq.shape, generator=gen, device=DEV).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, dout, dlse)]
        work()  # eager on the same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, (out, lse, dout, dlse)):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
    # and the replayed prefill is right
    ref_o, ref_l = oracle.attention_ref(to64(q), to64(k), to64(v), causal=True, softmax_scale=0.09)
    assert_close(to64(got[0]), to64(got[1]), ref_o, ref_l, "graph replay")
