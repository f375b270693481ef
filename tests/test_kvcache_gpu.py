"""In-place cache append + rotary decode (attn_decode_kvcache) vs the CPU oracle (needs an MI355X).

Stored values are compared bit for bit: the appended key rows (turned in
float32 and rounded to bf16 on both sides), the appended value rows, the
turned queries, and every cache row the call must not touch.  The decode
output uses the forward parity bar: max |out - ref| <= 1.5e-2, mean <= 1e-3,
|lse - ref| <= 1e-3.
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


def bits(t):
    """bf16 tensor -> int16 bit patterns on the CPU."""
    return t.detach().to("cpu").contiguous().view(torch.int16)


def ref_bits(x):
    """float64 values that are bf16-exact -> int16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).view(torch.int16)


def assert_same_bits(gpu, ref64, tag):
    g = bits(gpu)
    nan_g = torch.isnan(gpu.detach().to("cpu").float())
    nan_r = torch.from_numpy(np.isnan(ref64))
    assert torch.equal(nan_g, nan_r), f"{tag}: NaN positions differ"
    r = ref_bits(np.nan_to_num(ref64))
    diff = (g != r) & ~nan_g
    assert not diff.any().item(), f"{tag}: {int(diff.sum())} values differ in their bits"


def tables(rot, max_pos):
    if not rot:
        return None, None, None, None
    cos, sin = W.rotary_tables(max_pos, rot)
    return cos.to(DEV), sin.to(DEV), cos.double().numpy(), sin.double().numpy()


def call(case, dev, cos, sin, inter, chunk=None):
    return ea.attn_decode_kvcache(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                                  dev["block_table"], dev["seqlens_k"],
                                  max_seqlen_k=int(case["seqlens_k"].max()),
                                  softmax_scale=case["d"] ** -0.5, rotary_cos=cos, rotary_sin=sin,
                                  rotary_interleaved=inter, chunk_tokens=chunk)


def to_dev(case):
    return {k: v.to(DEV) for k, v in case.items() if torch.is_tensor(v)}


@pytest.mark.parametrize("d,rot,inter", [(128, 128, False), (128, 128, True), (128, 64, False),
                                         (64, 64, True), (256, 128, False), (256, 256, True), (128, 0, False)],
                         ids=lambda x: str(x))
def test_kvcache_small(d, rot, inter):
    lens = [0, 1, 255, 256, 1000, 3000, 511, 17]
    case = W.append_case(lens, 8, 2, d, seed=700 + d + rot, poison=True, extra_table_cols=1)
    cos, sin, cos_h, sin_h = tables(rot, 3100)
    rkw = dict(rotary_cos=cos_h, rotary_sin=sin_h, rotary_dim=rot, interleaved=inter)
    kc_ref, vc_ref = oracle.append_ref(to64(case["k_new"]), to64(case["v_new"]), to64(case["k_cache"]),
                                       to64(case["v_cache"]), case["block_table"].numpy(), lens, **rkw)
    ref_o, ref_l, ref_q = oracle.decode_append_ref(
        to64(case["q"]), to64(case["k_new"]), to64(case["v_new"]), to64(case["k_cache"]),
        to64(case["v_cache"]), case["block_table"].numpy(), lens, softmax_scale=d ** -0.5, **rkw)
    for chunk in (256, 1024):
        dev = to_dev(case)
        first = None
        for _ in range(2):  # a repeated call rewrites the same rows and gives the same result
            out, lse, q_rot = call(case, dev, cos, sin, inter, chunk)
            torch.cuda.synchronize()
            if first is None:
                first = (out.clone(), lse.clone())
            else:
                assert torch.equal(out, first[0]) and torch.equal(lse, first[1])
        tag = f"d{d} rot{rot} inter{inter} chunk{chunk}"
        assert_same_bits(dev["k_cache"], kc_ref, f"{tag} k_cache")
        assert_same_bits(dev["v_cache"], vc_ref, f"{tag} v_cache")
        if rot:
            assert_same_bits(q_rot, ref_q, f"{tag} q_rot")
        else:
            assert q_rot is None
        assert_close(to64(out), to64(lse), ref_o, ref_l, tag)


def test_kvcache_gqa_shapes():
    """Wide groups and MHA, both layouts."""
    for hq, hkv, inter in [(32, 1, False), (4, 4, True), (12, 3, False)]:
        lens = [700, 1, 2049]
        case = W.append_case(lens, hq, hkv, 128, seed=800 + hq, poison=True)
        cos, sin, cos_h, sin_h = tables(128, 2100)
        dev = to_dev(case)
        out, lse, q_rot = call(case, dev, cos, sin, inter, 512)
        torch.cuda.synchronize()
        ref_o, ref_l, ref_q = oracle.decode_append_ref(
            to64(case["q"]), to64(case["k_new"]), to64(case["v_new"]), to64(case["k_cache"]),
            to64(case["v_cache"]), case["block_table"].numpy(), lens, softmax_scale=128 ** -0.5,
            rotary_cos=cos_h, rotary_sin=sin_h, rotary_dim=128, interleaved=inter)
        assert_same_bits(q_rot, ref_q, f"hq{hq} hkv{hkv} q_rot")
        assert_close(to64(out), to64(lse), ref_o, ref_l, f"hq{hq} hkv{hkv}")


def test_kvcache_three_steps():
    """A decode loop: three steps, the caller advancing seqlens_k by one each time."""
    lens0 = [5, 254, 1023, 0, 511]
    case = W.append_case([n + 2 for n in lens0], 8, 2, 128, seed=901, poison=True)
    case["seqlens_k"] = torch.tensor(lens0, dtype=torch.int32)
    cos, sin, cos_h, sin_h = tables(128, 1100)
    rkw = dict(rotary_cos=cos_h, rotary_sin=sin_h, rotary_dim=128, interleaved=False)
    dev = to_dev(case)
    kc_ref, vc_ref = to64(case["k_cache"]), to64(case["v_cache"])
    table = case["block_table"].numpy()
    g = torch.Generator().manual_seed(902)
    for step in range(3):
        lens = [n + step for n in lens0]
        q = torch.randn(case["q"].shape, generator=g).to(torch.bfloat16)
        kn = torch.randn(case["k_new"].shape, generator=g).to(torch.bfloat16)
        vn = torch.randn(case["v_new"].shape, generator=g).to(torch.bfloat16)
        dev.update(q=q.to(DEV), k_new=kn.to(DEV), v_new=vn.to(DEV),
                   seqlens_k=torch.tensor(lens, dtype=torch.int32, device=DEV))
        out, lse, _ = ea.attn_decode_kvcache(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                                             dev["v_cache"], dev["block_table"], dev["seqlens_k"],
                                             max_seqlen_k=max(lens), softmax_scale=128 ** -0.5,
                                             rotary_cos=cos, rotary_sin=sin)
        torch.cuda.synchronize()
        ref_o, ref_l, _ = oracle.decode_append_ref(to64(q), to64(kn), to64(vn), kc_ref, vc_ref, table, lens,
                                                   softmax_scale=128 ** -0.5, **rkw)
        assert_close(to64(out), to64(lse), ref_o, ref_l, f"step {step}")
        kc_ref, vc_ref = oracle.append_ref(to64(kn), to64(vn), kc_ref, vc_ref, table, lens, **rkw)
    assert_same_bits(dev["k_cache"], kc_ref, "k_cache after three steps")
    assert_same_bits(dev["v_cache"], vc_ref, "v_cache after three steps")


def test_kvcache_bad_requests_are_nan():
    """Requests that cannot append get NaN and write nothing; the others are exact."""
    lens = [300, 40, 700, 10, 20]
    case = W.append_case(lens, 4, 2, 128, seed=903)
    max_pos = 305
    table = case["block_table"].clone()
    table[1, 0] = case["num_pages"] + 3          # new position's page id out of range
    seq = case["seqlens_k"].clone()
    seq[2] = table.shape[1] * 256                # no room left in the table
    seq[3] = 500                                 # beyond the rotary table (max_pos 305)
    seq[4] = -1                                  # negative length
    cos, sin, cos_h, sin_h = tables(128, max_pos)
    dev = to_dev(case)
    dev["block_table"], dev["seqlens_k"] = table.to(DEV), seq.to(DEV)
    out, lse, q_rot = ea.attn_decode_kvcache(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                                             dev["v_cache"], dev["block_table"], dev["seqlens_k"],
                                             max_seqlen_k=int(seq.max()), softmax_scale=128 ** -0.5,
                                             rotary_cos=cos, rotary_sin=sin)
    torch.cuda.synchronize()
    assert torch.isnan(out[1:].float()).all().item() and torch.isnan(lse[1:]).all().item()
    assert torch.isnan(q_rot[1:].float()).all().item()
    rkw = dict(rotary_cos=cos_h, rotary_sin=sin_h, rotary_dim=128, interleaved=False)
    kc_ref, vc_ref = oracle.append_ref(to64(case["k_new"][:1]), to64(case["v_new"][:1]), to64(case["k_cache"]),
                                       to64(case["v_cache"]), table[:1].numpy(), lens[:1], **rkw)
    assert_same_bits(dev["k_cache"], kc_ref, "k_cache, only request 0 appends")
    assert_same_bits(dev["v_cache"], vc_ref, "v_cache, only request 0 appends")
    ref_o, ref_l, ref_q = oracle.decode_append_ref(
        to64(case["q"][:1]), to64(case["k_new"][:1]), to64(case["v_new"][:1]), to64(case["k_cache"]),
        to64(case["v_cache"]), table[:1].numpy(), lens[:1], softmax_scale=128 ** -0.5, **rkw)
    assert_close(to64(out[:1]), to64(lse[:1]), ref_o, ref_l, "good request")


def test_kvcache_config_sampled():
    """The paged decode workload (64 requests, 4096..32768 cached keys, Hq 32, Hkv 8, d 128) with
    one appended token each and a full-width rotary turn: every appended row and turned query
    bit for bit, no other cache row changed, and sampled requests against the oracle."""
    c = W.CONFIGS["paged_decode_b64_hq32_hkv8_d128"]
    lens = W.decode_lengths(c["B"], c["nk_lo"], c["nk_hi"], c["seed"])
    case = W.append_case(lens, c["Hq"], c["Hkv"], c["d"], seed=c["seed"], device=DEV)
    case["seqlens_k"] = case["seqlens_k"].to(DEV)
    page = case["page"]
    table = case["block_table"]
    order = np.argsort(lens)
    req = sorted({int(order[0]), int(order[-1]), 5, 17, 40})
    # the oracle's view of the sampled requests, taken before the call changes the caches
    used = {b: table[b, :-(-(lens[b] + 1) // page)].tolist() for b in req}
    pages = sorted({p for b in req for p in used[b]})
    remap = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long, device=DEV)
    kc_sub, vc_sub = to64(case["k_cache"].index_select(0, idx)), to64(case["v_cache"].index_select(0, idx))
    sub_table = np.zeros((len(req), max(len(u) for u in used.values())), dtype=np.int64)
    for n, b in enumerate(req):
        sub_table[n, :len(used[b])] = [remap[p] for p in used[b]]
    k_before, v_before = case["k_cache"].clone(), case["v_cache"].clone()
    cos, sin, cos_h, sin_h = tables(128, max(lens) + 1)
    dev = {k: case[k] for k in ("q", "k_new", "v_new", "k_cache", "v_cache", "seqlens_k")}
    dev["block_table"] = table.to(DEV)
    out, lse, q_rot = call(case, dev, cos, sin, False)
    torch.cuda.synchronize()
    rkw = dict(rotary_dim=128, interleaved=False)
    q64, kn64 = to64(case["q"]), to64(case["k_new"])
    assert_same_bits(q_rot, oracle.round_bf16(oracle.rotary_f32(q64, cos_h, sin_h, lens, **rkw)), "q_rot")
    phys = torch.tensor([int(table[b, lens[b] // page]) for b in range(len(lens))], device=DEV)
    off = torch.tensor([lens[b] % page for b in range(len(lens))], device=DEV)
    assert_same_bits(case["k_cache"][phys, off], oracle.round_bf16(oracle.rotary_f32(kn64, cos_h, sin_h, lens, **rkw)),
                     "appended keys")
    assert torch.equal(bits(case["v_cache"][phys, off]), bits(case["v_new"]))
    for after, before in ((case["k_cache"], k_before), (case["v_cache"], v_before)):
        changed = (after.view(torch.int16) != before.view(torch.int16)).any(dim=-1).nonzero()
        got = {(int(p), int(o), int(h)) for p, o, h in changed.tolist()}
        allowed = {(int(p), int(o), h) for p, o in zip(phys.tolist(), off.tolist()) for h in range(c["Hkv"])}
        assert got <= allowed, f"{len(got - allowed)} rows changed that the append must not touch"
    del k_before, v_before
    sub = {b: n for n, b in enumerate(req)}
    ref_o, ref_l, _ = oracle.decode_append_ref(
        q64[req], kn64[req], to64(case["v_new"])[req], kc_sub, vc_sub, sub_table, [lens[b] for b in req],
        softmax_scale=128 ** -0.5, rotary_cos=cos_h, rotary_sin=sin_h, **rkw)
    o, l = to64(out), to64(lse)
    assert_close(o[req], l[req], ref_o, ref_l, "config sampled")
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(lse).all().item()
    assert sub  # sampled requests exist
