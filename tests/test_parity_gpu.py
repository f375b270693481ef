"""HIP path vs the CPU fp64 oracle, element by element (needs an MI355X).

Tolerances (bf16 out, fp32 lse): max |out - ref| <= 1.5e-2, mean |out - ref|
<= 1e-3, |lse - ref| <= 1e-3; rows with no allowed key must give out == 0 and
lse == -inf on both sides.  Small and ragged shapes are compared in full;
the full-size workloads are launched exactly as the benchmark launches them
and compared on every element as well (the oracle computes them in full).
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

OUT_MAX_ABS = 1.5e-2
OUT_MEAN_ABS = 1e-3
LSE_ABS = 1e-3

DEV = "cuda:0"


def to64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def assert_close(out, lse, ref_out, ref_lse, tag=""):
    o = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(o)), f"{tag}: non-finite output"
    d = np.abs(o - ref_out)
    assert d.max(initial=0.0) <= OUT_MAX_ABS, f"{tag}: max |diff| {d.max():.3e}"
    assert (d.mean() if d.size else 0.0) <= OUT_MEAN_ABS, f"{tag}: mean |diff| {d.mean():.3e}"
    l = np.asarray(lse, dtype=np.float64)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty), f"{tag}: empty-row pattern differs"
    fin = ~empty
    ld = np.abs(l[fin] - ref_lse[fin])
    assert ld.max(initial=0.0) <= LSE_ABS, f"{tag}: max |lse diff| {ld.max(initial=0):.3e}"


def dense_parity(B, Nq, Nk, Hq, Hkv, d, causal, seed, k_outlier_frac=0.0):
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed, k_outlier_frac=k_outlier_frac)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    out, lse = ea.attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]),
                                        causal=causal, softmax_scale=scale)
    lse_np = to64(lse)
    o_np = to64(out)
    # Empty rows: out exactly zero.
    empty = np.isneginf(ref_l)  # [B, Hq, Nq]
    if empty.any():
        bb, hh, ii = np.nonzero(empty)
        assert np.all(o_np[bb, ii, hh] == 0)
    assert_close(o_np, lse_np, ref_o, ref_l, f"dense B{B} Nq{Nq} Nk{Nk} Hq{Hq} Hkv{Hkv} d{d} c{causal}")


SMALL_DENSE = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (2, 7, 300, 4, 2, 128, True),      # short query over a longer cache (bottom-right)
    (2, 300, 7, 4, 2, 128, True),      # Nq > Nk: leading rows have no key
    (1, 257, 513, 2, 1, 64, True),     # ragged tails on both axes
    (1, 257, 513, 2, 1, 256, False),
    (1, 129, 129, 3, 3, 256, True),
    (1, 1, 1000, 8, 1, 128, True),     # one query row, many keys (MQA)
    (2, 384, 384, 32, 1, 64, True),    # MQA, 32 query heads on one K/V head
    (1, 600, 1100, 8, 2, 128, False),
    (1, 1000, 1000, 4, 4, 128, True),
    (1, 64, 65, 4, 1, 256, True),
    (2, 600, 700, 4, 2, 256, True),    # d = 256: three 256-row query tiles, ragged tails
]


@pytest.mark.parametrize("shape", SMALL_DENSE, ids=lambda s: "x".join(map(str, s)))
def test_dense_small(shape):
    B, Nq, Nk, Hq, Hkv, d, causal = shape
    dense_parity(B, Nq, Nk, Hq, Hkv, d, causal, seed=100 + sum(shape[:6]))


# Dense launches whose (sequence, head) count is a multiple of 32 run each
# XCD's heads four at a time: one, three and four groups of four heads per
# XCD, ragged query tiles, GQA groups aligned with the four-head groups and not.
FOUR_HEAD_GROUPS = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (1, 300, 700, 32, 32, 64, True),
    (3, 600, 600, 32, 8, 128, True),
    (2, 260, 260, 48, 16, 256, False),
    (4, 333, 333, 32, 4, 128, True),
]


@pytest.mark.parametrize("shape", FOUR_HEAD_GROUPS, ids=lambda s: "x".join(map(str, s)))
def test_dense_four_head_groups(shape):
    B, Nq, Nk, Hq, Hkv, d, causal = shape
    dense_parity(B, Nq, Nk, Hq, Hkv, d, causal, seed=700 + sum(shape[:6]))


def test_config_noncausal_mha_full():
    c = W.CONFIGS["mha_noncausal_b1_h4_n512_d64"]
    dense_parity(c["B"], c["Nq"], c["Nk"], c["Hq"], c["Hkv"], c["d"], c["causal"], c["seed"])


@pytest.mark.parametrize("name", ["mha_causal_b4_h16_n4096_d128", "gqa_causal_b2_hq32_hkv8_n8192_d128_koutliers"])
def test_config_dense_full(name):
    """The full-size dense workload, launched as the benchmark launches it, against
    the oracle on every element (max and mean |diff| over the whole output)."""
    case = W.config_case(name, device=DEV)
    out, lse = ea.attn_fwd(case["q"], case["k"], case["v"], causal=case["causal"],
                           softmax_scale=case["scale"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]),
                                        causal=case["causal"], softmax_scale=case["scale"])
    assert_close(to64(out), to64(lse), ref_o, ref_l, name)
    # Every row of a square causal problem sees at least its own key.
    assert np.isfinite(ref_l).all()


def varlen_parity(nq, nk, Hq, Hkv, d, causal, seed, sample=None):
    case = W.varlen_case(nq, nk, Hq, Hkv, d, seed)
    scale = d ** -0.5
    q, k, v = (case[x].to(DEV) for x in "qkv")
    cq, ck = case["cu_seqlens_q"].to(DEV), case["cu_seqlens_k"].to(DEV)
    out, lse = ea.attn_fwd(q, k, v, cu_seqlens_q=cq, cu_seqlens_k=ck,
                           max_seqlen_q=max(max(nq), 1), max_seqlen_k=max(nk), causal=causal,
                           softmax_scale=scale)
    torch.cuda.synchronize()
    tag = f"varlen d{d} c{causal} n{len(nq)}"
    if sample is None:
        ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]),
                                            causal=causal, softmax_scale=scale,
                                            cu_seqlens_q=case["cu_seqlens_q"].numpy(),
                                            cu_seqlens_k=case["cu_seqlens_k"].numpy())
        o_np, l_np = to64(out), to64(lse)
        empty = np.isneginf(ref_l)  # [Hq, TQ]
        if empty.any():
            hh, rr = np.nonzero(empty)
            assert np.all(o_np[rr, hh] == 0)
        assert_close(o_np, l_np, ref_o, ref_l, tag)
        return
    rng = np.random.default_rng(seed)
    rows = set()
    for s in range(len(nq)):
        if nq[s]:
            rows.add((s, int(rng.integers(Hq)), 0))
            rows.add((s, int(rng.integers(Hq)), nq[s] - 1))
    while len(rows) < sample:
        s = int(rng.integers(len(nq)))
        if nq[s]:
            rows.add((s, int(rng.integers(Hq)), int(rng.integers(nq[s]))))
    rows = sorted(rows)
    ref_o, ref_l = oracle.attention_rows(to64(case["q"]), to64(case["k"]), to64(case["v"]), rows,
                                         causal=causal, softmax_scale=scale,
                                         cu_seqlens_q=case["cu_seqlens_q"].numpy(),
                                         cu_seqlens_k=case["cu_seqlens_k"].numpy())
    cu = case["cu_seqlens_q"].tolist()
    o_cpu, l_cpu = out.to("cpu"), lse.to("cpu")
    got = np.stack([to64(o_cpu[cu[s] + i, h]) for s, h, i in rows])
    got_l = np.array([float(l_cpu[h, cu[s] + i]) for s, h, i in rows])
    assert_close(got, got_l, ref_o, ref_l, tag)
    assert torch.isfinite(out).all().item()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_small_edge_lengths(d):
    # Includes empty sequences, one-token sequences and Nq > Nk (empty rows).
    nq = [1, 0, 5, 70, 300, 2, 130, 1]
    nk = [1, 4, 0, 33, 600, 1, 129, 700]
    varlen_parity(nq, nk, 8, 2, d, True, seed=31 + d)
    varlen_parity(nq, nk, 8, 8, d, False, seed=32 + d)


@pytest.mark.parametrize("d", [128, 64, 256])
def test_config_varlen_chunked_prefill_full(d):
    """All 16 packed sequences and all 32 query heads at each head dim, every element."""
    c = W.CONFIGS["varlen_chunked_prefill_16seq_hq32_hkv8"]
    nq, nk = W.varlen_lengths(c["n_seqs"], c["nk_lo"], c["nk_hi"], c["q_div"], c["seed"])
    varlen_parity(nq, nk, c["Hq"], c["Hkv"], d, True, seed=c["seed"] * 1000 + d)


def oracle_decode(case, req):
    """The oracle on the listed requests only, from a copy of just their pages."""
    page = case["page"]
    table = case["block_table"].to("cpu")
    lens = case["seqlens_k"].to("cpu").tolist()
    used = {b: table[b, :-(-lens[b] // page)].tolist() for b in req}
    pages = sorted({p for b in req for p in used[b]})
    if not pages:
        pages = [0]
    remap = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long, device=case["k_cache"].device)
    kc = to64(case["k_cache"].index_select(0, idx))
    vc = to64(case["v_cache"].index_select(0, idx))
    width = max([len(u) for u in used.values()] + [1])
    sub_table = np.zeros((len(req), width), dtype=np.int64)
    for n, b in enumerate(req):
        sub_table[n, :len(used[b])] = [remap[p] for p in used[b]]
    q = to64(case["q"])[req]
    return oracle.decode_ref(q, kc, vc, sub_table, [lens[b] for b in req],
                             softmax_scale=case["d"] ** -0.5)


def decode_parity(case, chunk, requests=None):
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in case.items()}
    max_len = int(case["seqlens_k"].max())
    n = max(1, ea.attn_decode_num_splits(max_len, chunk))
    po, pl = ea.attn_decode_splitkv(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                                    dev["seqlens_k"], chunk_tokens=chunk, num_splits=n,
                                    softmax_scale=case["d"] ** -0.5)
    out, lse = ea.attn_decode_combine(po, pl, dev["seqlens_k"], chunk_tokens=chunk)
    torch.cuda.synchronize()
    req = list(range(case["B"])) if requests is None else list(requests)
    ref_o, ref_l = oracle_decode(case, req)
    o_cpu, l_cpu = to64(out), to64(lse)
    assert_close(o_cpu[req], l_cpu[req], ref_o, ref_l, f"decode chunk{chunk}")
    empty = np.isneginf(ref_l)
    if empty.any():
        assert np.all(o_cpu[req][empty] == 0)
    return out, lse


@pytest.mark.parametrize("poison", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_small(d, poison):
    lens = [1, 255, 256, 257, 1000, 3000, 0, 513]
    case = W.decode_case(lens, 8, 2, d, seed=50 + d, poison=poison, extra_table_cols=2)
    for chunk in (256, 512, 1024, 4096):
        decode_parity(case, chunk)


def test_decode_mqa_and_wide_groups():
    lens = [700, 1, 2049]
    decode_parity(W.decode_case(lens, 32, 1, 128, seed=61), 512)   # g = 32
    decode_parity(W.decode_case(lens, 64, 1, 128, seed=62), 512)   # g = 64
    decode_parity(W.decode_case(lens, 4, 4, 128, seed=63), 256)    # MHA, g = 1
    decode_parity(W.decode_case(lens, 16, 1, 128, seed=64), 1024)  # g = 16: one full column block


@pytest.mark.parametrize("hq,hkv,d", [(12, 3, 64), (9, 3, 128), (24, 1, 256), (64, 1, 64), (40, 5, 256)],
                         ids=lambda x: str(x))
def test_decode_odd_head_counts_and_groups(hq, hkv, d):
    """Odd K/V head counts (one head per workgroup) and wide groups at every d."""
    lens = [300, 1, 2049, 4096]
    decode_parity(W.decode_case(lens, hq, hkv, d, seed=80 + hq + d, poison=True), 1024)


def test_config_decode_full():
    """All 64 requests of the paged decode workload with the heuristic chunk (the
    benchmark's launch), against the unsplit oracle; the oracle runs on groups
    of eight requests to bound host memory."""
    case = W.config_case("paged_decode_b64_hq32_hkv8_d128", device=DEV)
    lens = case["seqlens_k"].tolist()
    chunk = ea.attn_decode_default_chunk(case["B"], case["Hkv"], max(lens),
                                         torch.cuda.get_device_properties(0).multi_processor_count)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in case.items()}
    n = max(1, ea.attn_decode_num_splits(max(lens), chunk))
    po, pl = ea.attn_decode_splitkv(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                                    dev["seqlens_k"], chunk_tokens=chunk, num_splits=n,
                                    softmax_scale=case["d"] ** -0.5)
    out, lse = ea.attn_decode_combine(po, pl, dev["seqlens_k"], chunk_tokens=chunk)
    torch.cuda.synchronize()
    o_cpu, l_cpu = to64(out), to64(lse)
    ref_o = np.zeros_like(o_cpu)
    ref_l = np.zeros_like(l_cpu)
    for g0 in range(0, case["B"], 8):
        req = list(range(g0, min(case["B"], g0 + 8)))
        ref_o[req], ref_l[req] = oracle_decode(case, req)
    assert_close(o_cpu, l_cpu, ref_o, ref_l, f"decode workload chunk {chunk}")


def test_decode_chunk_invariance():
    """Different split counts agree with each other (and with the oracle above).

    Chunkings differ in where each chunk's softmax shift sits, so the bf16
    rounding of the probabilities falls differently; each chunk divides by
    the sum of its rounded probabilities and the combine is fp32.  They must
    agree within the oracle bar itself (not twice it), with mean |diff|
    <= 1e-4 and lse within 1e-4."""
    case = W.decode_case([5000, 17, 2300, 4096], 8, 2, 128, seed=71)
    runs = [decode_parity(case, c) for c in (256, 768, 4096, 8192)]
    o0, l0 = runs[0][0].float(), runs[0][1]
    for o, l in runs[1:]:
        d = (o.float() - o0).abs()
        print(f"chunk invariance: max {d.max().item():.3e} mean {d.mean().item():.3e} "
              f"lse {(l - l0).abs().max().item():.3e}")
        assert d.max().item() <= OUT_MAX_ABS
        assert d.mean().item() <= 1e-4
        assert (l - l0).abs().max().item() <= 1e-4


def test_mixed_shape_order_is_stable():
    """Shape A, then B, then A again: A's results are bitwise identical."""
    a = W.dense_case(1, 200, 300, 128, 2, 128, seed=81)
    b = W.dense_case(1, 200, 300, 64, 1, 128, seed=82)
    run = lambda c: ea.attn_fwd(*(c[x].to(DEV) for x in "qkv"), causal=True, softmax_scale=128 ** -0.5)
    o1, l1 = run(a)
    ob, lb = run(b)
    o2, l2 = run(a)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_o, ref_l = oracle.attention_ref(to64(b["q"]), to64(b["k"]), to64(b["v"]), causal=True,
                                        softmax_scale=128 ** -0.5)
    assert_close(to64(ob), to64(lb), ref_o, ref_l, "mixed B")


def test_lse_optional_and_deterministic():
    c = W.dense_case(2, 333, 444, 4, 2, 128, seed=91)
    q, k, v = (c[x].to(DEV) for x in "qkv")
    o1, _ = ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.1, return_lse=False)
    o2, l2 = ea.attn_fwd(q, k, v, causal=True, softmax_scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ref_o, ref_l = oracle.attention_ref(to64(c["q"]), to64(c["k"]), to64(c["v"]), causal=True,
                                        softmax_scale=0.1)
    assert_close(to64(o2), to64(l2), ref_o, ref_l, "scale 0.1")


def test_extreme_scale_and_constant_rows():
    """Large score magnitudes exercise the rescale path; equal keys give mean(V)."""
    c = W.dense_case(1, 256, 700, 2, 1, 64, seed=93)
    q, k, v = (c[x].to(DEV) for x in "qkv")
    out, lse = ea.attn_fwd(q, k, v, causal=True, softmax_scale=4.0)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(c["q"]), to64(c["k"]), to64(c["v"]), causal=True,
                                        softmax_scale=4.0)
    assert_close(to64(out), to64(lse), ref_o, ref_l, "scale 4")
    k1 = c["k"].clone()
    k1[:] = k1[:, :1]
    out, lse = ea.attn_fwd(q, k1.to(DEV), v, causal=False, softmax_scale=0.125)
    torch.cuda.synchronize()
    mean_v = c["v"].double().mean(dim=1)  # [B, Hkv, d]
    got = out.to("cpu").double()
    assert (got - mean_v[:, None, :, :]).abs().max().item() <= OUT_MAX_ABS
    ql = (c["q"].double() * k1[:, :1].double()).sum(-1) * 0.125  # [B, Nq, Hq]
    assert (lse.to("cpu").double() - (ql.permute(0, 2, 1) + math.log(700))).abs().max().item() <= LSE_ABS


@pytest.mark.parametrize("n_seqs", [64, 65, 150])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_many_sequences(n_seqs, d):
    """Packed batches at and past the size for which the kernel ranks its work items
    by sequence length (64 sequences); lengths include empty and one-token
    sequences, Nq > Nk and multi-tile queries. Every element is compared."""
    rng = np.random.default_rng(7000 + n_seqs + d)
    nk = [int(x) for x in rng.integers(0, 300, size=n_seqs)]
    nq = [min(int(x), 300) for x in rng.integers(0, 320, size=n_seqs)]
    nk[0], nq[0] = 0, 5        # rows with no keys
    nk[1], nq[1] = 1, 1
    nk[-1], nq[-1] = 299, 299  # several 128- or 256-row query tiles
    varlen_parity(nq, nk, 8, 2, d, True, seed=7100 + n_seqs + d)


# Launches whose usual grid has at most 128 workgroups (256 query rows per
# workgroup at d = 128, 128 at d = 64) and at least 8 key tiles (256 keys at
# d = 128, 512 at d = 64) run in split-key mode: four waves share 32 query
# rows and each walks a quarter of the keys, then their states are merged.
SPLIT_DENSE = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, window)
    (1, 2048, 2048, 4, 4, 64, True, (-1, -1)),
    (2, 128, 8192, 16, 4, 128, True, (-1, -1)),
    (1, 64, 16384, 32, 8, 128, True, (-1, -1)),
    (1, 300, 1000, 8, 1, 128, False, (-1, -1)),   # ragged tiles, MQA
    (1, 1000, 600, 4, 2, 64, True, (-1, -1)),     # Nq > Nk: rows with no keys
    (1, 512, 4096, 4, 4, 128, True, (300, -1)),   # a window wider than 8 tiles
    (3, 33, 777, 2, 2, 128, False, (-1, -1)),     # one short query tile per sequence
    (2, 300, 4096, 32, 8, 128, True, (-1, -1)),   # B x Hq = 64: two groups of four heads per XCD
    (1, 200, 2048, 64, 16, 64, True, (-1, -1)),   # the same at d = 64
]


@pytest.mark.parametrize("shape", SPLIT_DENSE, ids=lambda s: "x".join(map(str, s[:7])))
def test_split_key_mode_dense(shape):
    B, Nq, Nk, Hq, Hkv, d, causal, window = shape
    case = W.dense_case(B, Nq, Nk, Hq, Hkv, d, seed=8000 + Nq + d, device=DEV)
    out, lse = ea.attn_fwd(case["q"], case["k"], case["v"], causal=causal, softmax_scale=d ** -0.5,
                           window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_ref(to64(case["q"]), to64(case["k"]), to64(case["v"]), causal=causal,
                                        softmax_scale=d ** -0.5, window=window)
    o = to64(out)
    empty = np.isneginf(ref_l)
    if empty.any():
        bb, hh, ii = np.nonzero(empty)
        assert np.all(o[bb, ii, hh] == 0)
    assert_close(o, to64(lse), ref_o, ref_l, f"split-key {shape}")


@pytest.mark.parametrize("d", [64, 128])
def test_split_key_mode_varlen(d):
    """Packed batches with a small grid: one long-context chunk, an empty sequence, a short one."""
    nq = [200, 0, 17, 3]
    nk = [5000, 700, 17, 900]
    varlen_parity(nq, nk, 8, 2, d, True, seed=8100 + d)
    varlen_parity([150], [4000], 4, 4, d, False, seed=8200 + d)
