"""The C ABI on the host: symbols, status codes and argument validation (no GPU).

Every call here fails host-side validation (or is a pure host helper), so no
kernel is ever launched and the fake device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

import exact_io_aware_07_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000)
FAKE3 = ctypes.c_void_p(0x30000)
OUT = ctypes.c_void_p(0x40000000)
LSE = ctypes.c_void_p(0x50000000)
NULL = None


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = ea.lib()
    names = header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = ea.lib()
    assert lib.attn_abi_version() == 1
    for code, name in ea.STATUS.items():
        assert lib.attn_status_str(code).decode() == name
    assert lib.attn_status_str(99).decode() == "ATTN_ERR_UNKNOWN"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, cq=NULL, ck=NULL, batch=1, mq=8, mk=8, hq=4, hkv=2, d=128,
             causal=1, scale=0.125, out=OUT, lse=LSE)
    a.update(kw)
    lib = ea.lib()
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["batch"], a["mq"], a["mk"],
                        a["hq"], a["hkv"], a["d"], a["causal"], a["scale"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(out=NULL), 1), (dict(cq=FAKE), 1),
    (dict(batch=0), 2), (dict(mq=0), 2), (dict(mk=0), 2), (dict(hq=0), 2), (dict(hkv=0), 2),
    (dict(hq=6, hkv=4), 2), (dict(causal=2), 2),
    (dict(d=96), 3), (dict(d=512), 3), (dict(d=0), 3),
    (dict(scale=0.0), 4), (dict(scale=-1.0), 4), (dict(scale=float("inf")), 4),
    (dict(scale=float("nan")), 4),
    (dict(out=FAKE), 5), (dict(lse=OUT), 5), (dict(out=ctypes.c_void_p(0x10000 + 64)), 5),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code
    msg = ea.lib().attn_last_error().decode()
    assert msg


def dec(**kw):
    a = dict(q=FAKE, kc=FAKE2, vc=FAKE3, bt=ctypes.c_void_p(0x60000), sl=ctypes.c_void_p(0x70000),
             batch=2, hq=8, hkv=2, d=128, page=256, maxp=4, npages=8, chunk=512, nsplit=2,
             scale=0.1, po=OUT, pl=LSE)
    a.update(kw)
    return ea.lib().attn_decode_splitkv(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["batch"],
                                        a["hq"], a["hkv"], a["d"], a["page"], a["maxp"], a["npages"],
                                        a["chunk"], a["nsplit"], a["scale"], a["po"], a["pl"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(bt=NULL), 1), (dict(sl=NULL), 1), (dict(pl=NULL), 1),
    (dict(batch=0), 2), (dict(nsplit=0), 2), (dict(npages=0), 2), (dict(hq=6, hkv=4), 2),
    (dict(hq=130, hkv=2), 3), (dict(page=16), 3), (dict(chunk=300), 3), (dict(chunk=0), 3),
    (dict(d=80), 3), (dict(scale=0.0), 4), (dict(pl=ctypes.c_void_p(0x40000000 + 1024)), 5),
])
def test_decode_split_rejects(kw, code):
    assert dec(**kw) == code


def comb(**kw):
    a = dict(po=FAKE, pl=FAKE2, sl=FAKE3, batch=2, hq=8, d=128, chunk=512, nsplit=2, out=OUT, lse=LSE)
    a.update(kw)
    return ea.lib().attn_decode_combine(a["po"], a["pl"], a["sl"], a["batch"], a["hq"], a["d"],
                                        a["chunk"], a["nsplit"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(po=NULL), 1), (dict(out=NULL), 1), (dict(batch=0), 2), (dict(nsplit=0), 2),
    (dict(d=32), 3), (dict(chunk=100), 3), (dict(out=FAKE), 5), (dict(lse=OUT), 5),
])
def test_decode_combine_rejects(kw, code):
    assert comb(**kw) == code


def fwd_ex(**kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, cq=NULL, ck=NULL, bt=NULL, sk=NULL, batch=1, mq=8, mk=8, hq=4,
             hkv=2, d=128, page=256, maxp=4, npages=8, causal=1, wl=-1, wr=-1, scale=0.125, out=OUT,
             lse=LSE)
    a.update(kw)
    return ea.lib().attn_fwd_ex(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["bt"], a["sk"], a["batch"],
                                a["mq"], a["mk"], a["hq"], a["hkv"], a["d"], a["page"], a["maxp"],
                                a["npages"], a["causal"], a["wl"], a["wr"], a["scale"], a["out"], a["lse"],
                                None)


PAGED = dict(bt=FAKE, cq=FAKE2, sk=FAKE3, k=ctypes.c_void_p(0x11000), v=ctypes.c_void_p(0x12000))


@pytest.mark.parametrize("kw,code", [
    (dict(wl=-2), 2), (dict(wr=-5), 2), (dict(sk=FAKE), 1), (dict(q=NULL), 1), (dict(d=96), 3),
    (dict(PAGED, cq=NULL), 1), (dict(PAGED, sk=NULL), 1), (dict(PAGED, ck=FAKE), 1),
    (dict(PAGED, page=128), 3), (dict(PAGED, maxp=0), 2), (dict(PAGED, npages=0), 2),
    (dict(PAGED, wl=-3), 2), (dict(PAGED, out=FAKE), 5),
])
def test_fwd_ex_rejects(kw, code):
    assert fwd_ex(**kw) == code


def _at(i):
    return ctypes.c_void_p(0x1000000 * (i + 1))   # 16 MiB apart: no two regions overlap


def kvc(**kw):
    """attn_decode_kvcache with B=2, Hq=8, Hkv=2, d=128, 4 pages, 2 splits; every case fails validation."""
    a = dict(q=_at(0), kn=_at(1), vn=_at(2), kc=_at(3), vc=_at(4), bt=_at(5), sl=_at(6), cos=NULL, sin=NULL,
             rot=0, inter=0, maxpos=0, batch=2, hq=8, hkv=2, d=128, page=256, maxp=2, npages=4, chunk=256,
             nsplit=2, scale=0.125, qrot=NULL, po=_at(7), pl=_at(8), out=_at(9), lse=_at(10))
    a.update(kw)
    return ea.lib().attn_decode_kvcache(
        a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["sl"], a["cos"], a["sin"], a["rot"], a["inter"],
        a["maxpos"], a["batch"], a["hq"], a["hkv"], a["d"], a["page"], a["maxp"], a["npages"], a["chunk"],
        a["nsplit"], a["scale"], a["qrot"], a["po"], a["pl"], a["out"], a["lse"], None)


ROPE = dict(rot=64, cos=_at(11), sin=_at(12), qrot=_at(13), maxpos=100)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(kn=NULL), 1), (dict(vn=NULL), 1), (dict(kc=NULL), 1), (dict(vc=NULL), 1),
    (dict(bt=NULL), 1), (dict(sl=NULL), 1), (dict(po=NULL), 1), (dict(pl=NULL), 1), (dict(out=NULL), 1),
    (dict(ROPE, cos=NULL), 1), (dict(ROPE, sin=NULL), 1), (dict(ROPE, qrot=NULL), 1),
    (dict(batch=0), 2), (dict(hq=6, hkv=4), 2), (dict(nsplit=0), 2), (dict(ROPE, rot=3), 2),
    (dict(ROPE, rot=256), 2), (dict(ROPE, rot=-2), 2), (dict(ROPE, maxpos=0), 2), (dict(inter=2), 2),
    (dict(d=96), 3), (dict(page=128), 3), (dict(chunk=100), 3), (dict(hq=130, hkv=2), 3),
    (dict(scale=0.0), 4), (dict(ROPE, scale=float("nan")), 4),
    (dict(kc=_at(0)), 5), (dict(vc=ctypes.c_void_p(0x4000000 + 64)), 5), (dict(out=_at(0)), 5),
    (dict(lse=_at(9)), 5), (dict(ROPE, qrot=_at(11)), 5), (dict(ROPE, out=_at(13)), 5),
    (dict(po=_at(1)), 5), (dict(pl=_at(5)), 5), (dict(ROPE, kc=_at(12)), 5),
])
def test_decode_kvcache_rejects(kw, code):
    assert kvc(**kw) == code


def fp8q(**kw):
    a = dict(x=_at(0), signs=NULL, batch=2, n=100, h=3, d=128, layout=0, codes=_at(1), scales=_at(2))
    a.update(kw)
    return ea.lib().attn_fp8_quantize(a["x"], a["signs"], a["batch"], a["n"], a["h"], a["d"], a["layout"],
                                      a["codes"], a["scales"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=NULL), 1), (dict(codes=NULL), 1), (dict(scales=NULL), 1),
    (dict(batch=0), 2), (dict(n=0), 2), (dict(h=-1), 2), (dict(layout=2), 2),
    (dict(d=32), 3), (dict(d=96, layout=1), 3), (dict(d=512), 3),
    (dict(codes=_at(0)), 5), (dict(scales=ctypes.c_void_p(0x1000000 + 100)), 5), (dict(signs=_at(1)), 5),
    (dict(scales=ctypes.c_void_p(0x2000000 + 64)), 5),
])
def test_fp8_quantize_rejects(kw, code):
    assert fp8q(**kw) == code


def fp8f(**kw):
    a = dict(q=_at(0), k=_at(1), v=_at(2), qs=_at(3), ks=_at(4), vs=_at(5), batch=1, nq=100, nk=120, hq=4,
             hkv=2, d=128, causal=1, inc=1, scale=0.1, out=_at(6), lse=_at(7))
    a.update(kw)
    return ea.lib().attn_fwd_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["batch"], a["nq"], a["nk"],
                                 a["hq"], a["hkv"], a["d"], a["causal"], a["inc"], a["scale"], a["out"], a["lse"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(v=NULL), 1), (dict(vs=NULL), 1), (dict(out=NULL), 1),
    (dict(batch=0), 2), (dict(nk=0), 2), (dict(hq=6, hkv=4), 2), (dict(causal=2), 2), (dict(inc=-1), 2),
    (dict(d=32), 3), (dict(d=192), 3), (dict(scale=0.0), 4), (dict(scale=float("inf")), 4),
    (dict(out=_at(0)), 5), (dict(lse=_at(5)), 5), (dict(lse=ctypes.c_void_p(0x7000000 + 8)), 5),
])
def test_fwd_fp8_rejects(kw, code):
    assert fp8f(**kw) == code


def test_fp8_sizes():
    lib = ea.lib()
    assert lib.attn_fp8_num_blocks(1) == 1 and lib.attn_fp8_num_blocks(64) == 1 and lib.attn_fp8_num_blocks(65) == 2
    assert lib.attn_fp8_num_blocks(0) == 0
    assert lib.attn_fp8_codes_bytes(2, 100, 3, 128, 0) == 2 * 100 * 3 * 128
    assert lib.attn_fp8_codes_bytes(2, 100, 3, 128, 1) == 2 * 3 * 128 * 128
    assert lib.attn_fp8_codes_bytes(2, 100, 3, 128, 2) == 0


DQ = ctypes.c_void_p(0x60000000)
DK = ctypes.c_void_p(0x70000000)
DV = ctypes.c_void_p(0x78000000)
WS = ctypes.c_void_p(0x7c000000)


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, out=OUT, lse=LSE, dout=ctypes.c_void_p(0x58000000), cq=NULL,
             ck=NULL, batch=1, mq=8, mk=8, tq=8, hq=4, hkv=2, d=128, causal=1, scale=0.125, dq=DQ,
             dk=DK, dv=DV, ws=WS, wsb=8 * 8 * 4)
    a.update(kw)
    return ea.lib().attn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["cq"], a["ck"],
                             a["batch"], a["mq"], a["mk"], a["tq"], a["hq"], a["hkv"], a["d"],
                             a["causal"], a["scale"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(lse=NULL), 1), (dict(dout=NULL), 1), (dict(dv=NULL), 1), (dict(ws=NULL), 1),
    (dict(ck=FAKE), 1),
    (dict(batch=0), 2), (dict(tq=0), 2), (dict(tq=9), 2), (dict(hq=6, hkv=4), 2), (dict(causal=3), 2),
    (dict(wsb=8 * 8 * 4 - 1), 2),
    (dict(d=32), 3), (dict(d=96), 3),
    (dict(scale=0.0), 4),
    (dict(dq=FAKE), 5), (dict(dk=FAKE3), 5), (dict(dv=DK), 5), (dict(ws=DQ), 5), (dict(dq=OUT), 5),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_bytes():
    lib = ea.lib()
    assert lib.attn_bwd_workspace_bytes(1000, 32) == 2 * 1000 * 32 * 4
    assert lib.attn_bwd_workspace_bytes(0, 32) == 0 and lib.attn_bwd_workspace_bytes(5, -1) == 0


def test_host_helpers():
    assert ea.attn_decode_num_splits(32768, 2048) == 16
    assert ea.attn_decode_num_splits(32769, 2048) == 17
    assert ea.attn_decode_num_splits(0, 256) == 0
    for args in [(64, 8, 32768, 256), (1, 1, 100, 256), (2, 32, 1 << 20, 304)]:
        c = ea.attn_decode_default_chunk(*args)
        assert c >= 256 and c % 256 == 0
    # 32 split waves per compute unit, chunks lengthened toward 2048 tokens
    # while 8 waves per compute unit remain; small batches keep short chunks.
    assert ea.attn_decode_default_chunk(64, 8, 32768, 256) == 2048
    assert ea.attn_decode_default_chunk(64, 8, 8192, 256) == 2048
    assert ea.attn_decode_default_chunk(64, 8, 2048, 256) == 512
    assert ea.attn_decode_default_chunk(1, 8, 32768, 256) == 256
    assert ea.attn_decode_default_chunk(1, 1, 1 << 20, 256) == 512
    assert ea.attn_decode_workspace_bytes(64, 32, 128, 16) == 16 * 64 * 32 * 129 * 4


def test_cu_seqlens_validator():
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int32)
    ea.attn_check_cu_seqlens(good, total=10, max_seqlen=7)
    for bad, total, mx in [([1, 3, 3, 10], 10, 7), ([0, 3, 2, 10], 10, 8), ([0, 3, 3, 10], 11, 7),
                           ([0, 3, 3, 10], 10, 6)]:
        with pytest.raises(ea.AttnError) as e:
            ea.attn_check_cu_seqlens(torch.tensor(bad, dtype=torch.int32), total=total, max_seqlen=mx)
        assert e.value.status == 7


def test_block_table_validator():
    table = torch.tensor([[3, 1, 0], [2, 9, 9]], dtype=torch.int32)
    ea.attn_check_block_table(table, torch.tensor([700, 256], dtype=torch.int32), num_pages=4)
    for lens in ([700, 257], [769, 10], [-1, 5]):
        with pytest.raises(ea.AttnError) as e:
            ea.attn_check_block_table(table, torch.tensor(lens, dtype=torch.int32), num_pages=4)
        assert e.value.status == 7


def test_python_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attn_fwd(q, q, q, causal=False, softmax_scale=0.125)


ODD = ctypes.c_void_p(0x10000 + 2)   # 2-byte aligned: fine for no tensor


@pytest.mark.parametrize("call,kw", [
    (fwd, dict(q=ODD)), (fwd, dict(out=ctypes.c_void_p(0x40000000 + 8))), (fwd, dict(lse=ctypes.c_void_p(0x50000000 + 2))),
    (fwd_ex, dict(PAGED, bt=ODD)), (dec, dict(kc=ODD)), (dec, dict(sl=ctypes.c_void_p(0x70000 + 1))),
    (comb, dict(po=ctypes.c_void_p(0x10000 + 4))), (bwd, dict(ws=ctypes.c_void_p(0x7c000000 + 8))),
    (kvc, dict(q=ODD)), (kvc, dict(ROPE, cos=ctypes.c_void_p(0xB000000 + 2))), (fp8q, dict(x=ODD)),
    (fp8q, dict(signs=ctypes.c_void_p(0x3000000 + 4))), (fp8f, dict(v=ctypes.c_void_p(0x3000000 + 8))),
])
def test_misaligned_pointers_rejected(call, kw):
    """Misaligned tensors are refused before any launch (ATTN_ERR_UNSUPPORTED)."""
    assert call(**kw) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(src=NULL), 1), (dict(sink=NULL), 1), (dict(nbytes=0), 2), (dict(nbytes=100), 2),
    (dict(src=ctypes.c_void_p(0x10000 + 8)), 3),
])
def test_ceiling_read_rejects(kw, code):
    a = dict(src=FAKE, nbytes=1 << 20, sink=OUT)
    a.update(kw)
    assert ea.lib().attn_ceiling_read(a["src"], a["nbytes"], a["sink"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(ops=NULL), 1), (dict(sink=NULL), 1), (dict(waves=6), 2), (dict(waves=0), 2), (dict(iters=0), 2),
    (dict(ops=ctypes.c_void_p(0x10000 + 4)), 3),
])
@pytest.mark.parametrize("fn", ["attn_ceiling_mfma_bf16", "attn_ceiling_mfma_fp8"])
def test_ceiling_mfma_rejects(fn, kw, code):
    a = dict(ops=FAKE, waves=8, iters=10, sink=OUT)
    a.update(kw)
    assert getattr(ea.lib(), fn)(a["ops"], a["waves"], a["iters"], a["sink"], None) == code


def dec_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE2, vc=FAKE3, bt=ctypes.c_void_p(0x60000), sl=ctypes.c_void_p(0x70000),
             batch=2, hq=8, hkv=2, d=128, page=256, maxp=4, npages=8, chunk=512, nsplit=2,
             scale=0.1, out=OUT, lse=LSE)
    a.update(kw)
    return ea.lib().attn_decode_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["batch"], a["hq"],
                                        a["hkv"], a["d"], a["page"], a["maxp"], a["npages"], a["chunk"],
                                        a["nsplit"], a["scale"], a["out"], a["lse"], None)


# Only checks that fail before the scratch address is looked up (no HIP call).
@pytest.mark.parametrize("kw,code", [
    (dict(out=NULL), 1), (dict(batch=0), 2), (dict(hq=0), 2), (dict(nsplit=0), 2), (dict(d=96), 3),
    (dict(out=ctypes.c_void_p(0x40000000 + 8)), 3), (dict(lse=ctypes.c_void_p(0x50000000 + 2)), 3),
])
def test_decode_noalloc_rejects(kw, code):
    assert dec_noalloc(**kw) == code
    assert ea.lib().attn_last_error().decode()


def test_decode_noalloc_rejects_partials_beyond_scratch():
    """Partials larger than the library's array are refused with a clear message."""
    lib = ea.lib()
    limit = ea.DECODE_NOALLOC_SCRATCH_BYTES
    # 64 requests x 32 heads x d=128: one split needs 64*32*129*4 = 1,056,768 bytes.
    per_split = lib.attn_decode_workspace_bytes(64, 32, 128, 1)
    fits = limit // per_split
    too_many = fits + 1
    assert lib.attn_decode_workspace_bytes(64, 32, 128, too_many) > limit
    assert dec_noalloc(batch=64, hq=32, hkv=8, nsplit=too_many) == 2
    msg = lib.attn_last_error().decode()
    assert "scratch" in msg and str(limit) in msg


def test_noalloc_scratch_constant_matches_header():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    m = re.search(r"#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ea.DECODE_NOALLOC_SCRATCH_BYTES
