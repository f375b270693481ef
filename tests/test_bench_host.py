"""Host logic of bench.py (no GPU): FLOP and byte formulas, the committed-traffic
loader and writer, and the one-GPU guard.

The exact FLOP counts are checked against the oracle's own keep masks (the
bottom-right causal rule), counted pair by pair.
"""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle.attention as oa  # noqa: E402


@pytest.mark.parametrize("nq,nk", [(1, 1), (5, 5), (3, 7), (7, 3), (64, 200), (0, 4)])
def test_prefill_flops_exact_counts_allowed_pairs(nq, nk):
    case = dict(B=2, Hq=3, Hkv=3, Nq=nq, Nk=nk, d=16, causal=True)
    pairs = int(oa.causal_keep(nq, nk).sum()) if nq and nk else 0
    assert bench.prefill_flops_exact(case) == 4.0 * 16 * pairs * 2 * 3
    case["causal"] = False
    assert bench.prefill_flops_exact(case) == 4.0 * 16 * nq * nk * 2 * 3


def test_prefill_flops_metric():
    case = dict(B=4, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=128, causal=True)
    assert bench.prefill_flops(case) == 274877906944.0  # 4 N^2 d / 2 per head, 64 heads
    # The exact count adds the diagonal: N (N + 1) / 2 pairs per head.
    assert bench.prefill_flops_exact(case) == 4.0 * 128 * (4096 * 4097 // 2) * 64


def test_varlen_flops_exact_counts_allowed_pairs():
    rng = np.random.default_rng(3)
    nq = [int(x) for x in rng.integers(1, 40, size=6)]
    nk = [q + int(x) for q, x in zip(nq, rng.integers(0, 50, size=6))]
    case = dict(nq=nq, nk=nk, Hq=4, Hkv=2, d=32)
    pairs = sum(int(oa.causal_keep(a, b).sum()) for a, b in zip(nq, nk))
    assert bench.varlen_flops_exact(case) == 4.0 * 32 * pairs * 4
    assert bench.varlen_flops(case) == sum(4.0 * a * b * 32 / 2 for a, b in zip(nq, nk)) * 4
    tq, tk = sum(nq), sum(nk)
    assert bench.varlen_bytes(case) == 2 * (2 * tq * 4 * 32 + 2 * tk * 2 * 32) + 4 * 4 * tq


def test_prefill_and_decode_bytes():
    case = dict(B=2, Hq=4, Hkv=2, Nq=10, Nk=12, d=8, causal=True)
    q = 2 * 10 * 4 * 8
    kv = 2 * 12 * 2 * 8
    assert bench.prefill_bytes(case) == 2 * (2 * q + 2 * kv) + 4 * 2 * 4 * 10

    class Lens:
        def tolist(self):
            return [300, 5, 256]
    dc = dict(seqlens_k=Lens(), B=3, Hq=8, Hkv=2, d=16, page=256)
    kv_b = (300 + 5 + 256) * 2 * 16 * 2 * 2
    qo = 2 * 3 * 8 * 16 * 2
    lse = 4 * 3 * 8
    table = 4 * (2 + 1 + 1) + 4 * 3
    assert bench.decode_bytes(dc) == kv_b + qo + lse + table


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, val in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_write_and_load_traffic(tmp_path, monkeypatch):
    out = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(out))
    mib = 8
    # The copy kernel reads and writes 8 MiB; the counters report half of the
    # reads (FETCH_SIZE) and all of the writes (WRITE_SIZE), in KiB.
    fetch = [("__amd_rocclr_copyBuffer", mib * 1024 / 2), ("__amd_rocclr_copyBuffer", 1.0),
             ("void attn::attn_fwd_kernel<128, 1>(p)", 100.0), ("void attn::attn_fwd_kernel<128, 1>(p)", 300.0),
             ("void attn::attn_fwd_fp8_kernel<128>(p)", 999.0)]
    write = [("__amd_rocclr_copyBuffer", mib * 1024.0), ("void attn::attn_fwd_kernel<128, 1>(p)", 50.0),
             ("void attn::attn_fwd_kernel<128, 1>(p)", 50.0)]
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", fetch)
    _counter_csv(wcsv, "WRITE_SIZE", write)
    cmd = "rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --legs c1 --copy-calibration-mib 8"
    assert bench.write_traffic([("c1", str(fcsv), str(wcsv))], mib, [cmd, "other --legs c3 x"]) == 0
    rec = json.loads(out.read_text())
    leg = rec["legs"]["c1"]
    assert leg["copy_calibration"]["fetch_scale"] == 2.0 and leg["copy_calibration"]["write_scale"] == 1.0
    k = leg["kernels"]["attn_fwd_kernel"]
    # mean fetch 200 KiB x 2, mean write 50 KiB x 1
    assert k["hbm_bytes_per_launch"] == (200 * 2 + 50) * 1024
    assert "attn_fwd_fp8_kernel" not in leg["kernels"]  # no WRITE_SIZE rows for it
    assert leg["commands"] == [cmd]
    digest = bench.source_digest()
    assert rec["source_digest"] == digest
    assert bench.load_traffic("c1", "attn_fwd_kernel", digest) == (200 * 2 + 50) * 1024
    assert bench.load_traffic("c1", "attn_fwd_kernel", "another-digest") is None
    assert bench.load_traffic("c3", "attn_fwd_kernel", digest) is None
    assert bench.traffic_sum("c1", ["attn_fwd_kernel", "attn_bwd_dq_kernel"], digest) is None


def test_write_traffic_needs_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "t.json"))
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", [("void attn::attn_fwd_kernel<1>(p)", 1.0)])
    _counter_csv(wcsv, "WRITE_SIZE", [("void attn::attn_fwd_kernel<1>(p)", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic([("c1", str(fcsv), str(wcsv))], 8, [])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
