"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  1. attn_fwd on the causal MHA prefill workload (B=4, H=16, N=4096, d=128,
     bf16 N(0,1)), and
  2. attn_decode_splitkv + attn_decode_combine on the paged decode workload
     (B=64, Hq=32, Hkv=8, d=128, 256-token pages, per-request length uniform
     in [4096, 32768]).
Each kernel is bracketed by HIP events recorded on the stream it is launched
on (torch's current stream).  The headline value is the prefill throughput in
TFLOP/s (4*Nq*Nk*d per head, halved for causal); the decode leg reports HBM
GB/s over its algorithmic bytes (K/V rows used, q, out, lse, block table and
lengths).

Every other workload is timed as a leg of its own after the step (per-launch
mean, p50 and p95, roofline against the published peak, counter traffic):
the non-causal d=64 case, the causal GQA N=8192 case with key outliers, the
packed chunked prefill at d = 128, 64 and 256, and the widened rows (backward,
decode with append + rotary, FP8 forward).  The CPU oracle is timed on a
bounded sample of every workload as a reported baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 50] [--legs step,c1,...]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
WARM_MS = 200.0             # wall time of untimed calls before each leg apart from the step
PREFILL = "mha_causal_b4_h16_n4096_d128"
DECODE = "paged_decode_b64_hq32_hkv8_d128"
NONCAUSAL = "mha_noncausal_b1_h4_n512_d64"
GQA = "gqa_causal_b2_hq32_hkv8_n8192_d128_koutliers"
VARLEN = "varlen_chunked_prefill_16seq_hq32_hkv8"
# Legs: the step (prefill + decode, the headline) and the separately timed ones.
LEGS = ["step", "c1", "c3", "c4_d128", "c4_d64", "c4_d256", "backward", "kvcache", "fp8", "ceilings"]
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["attn_tile.h", "attn_launch.h", "attn_udiv.h", "attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip", "attn_fp8.hip"]


def source_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_io_aware_07_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_flops(case):
    """Metric FLOPs: 4*Nq*Nk*d per (sequence, head), halved when causal."""
    per_head = 4.0 * case["Nq"] * case["Nk"] * case["d"]
    if case["causal"]:
        per_head /= 2
    return per_head * case["B"] * case["Hq"]


def prefill_flops_exact(case):
    """4*d per allowed (query, key) pair (bottom-right causal)."""
    nq, nk = case["Nq"], case["Nk"]
    if not case["causal"]:
        pairs = nq * nk
    else:
        pairs = sum(max(0, min(nk, i + nk - nq + 1)) for i in range(nq))
    return 4.0 * case["d"] * pairs * case["B"] * case["Hq"]


def prefill_bytes(case):
    """Compulsory traffic: read Q, K, V once; write out once and lse once."""
    B, Nq, Nk, Hq, Hkv, d = (case[x] for x in ("B", "Nq", "Nk", "Hq", "Hkv", "d"))
    return 2 * (2 * B * Nq * Hq * d + 2 * B * Nk * Hkv * d) + 4 * B * Hq * Nq


def decode_bytes(case):
    """K/V rows actually used, q, out, lse, used block-table entries and lengths."""
    lens = case["seqlens_k"].tolist()
    Hq, Hkv, d, page = case["Hq"], case["Hkv"], case["d"], case["page"]
    kv = sum(lens) * Hkv * d * 2 * 2
    qo = 2 * case["B"] * Hq * d * 2
    lse = 4 * case["B"] * Hq
    table = 4 * sum(-(-n // page) for n in lens) + 4 * case["B"]
    return kv + qo + lse + table


def load_traffic(leg, kernel_key, digest):
    """HBM bytes per launch of one kernel of one leg, from the committed
    rocprofv3 counter runs of that leg, if they match the current sources."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest:
        return None
    k = rec.get("legs", {}).get(leg, {}).get("kernels", {}).get(kernel_key)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


# Counter key -> substring of the rocprofv3 kernel name ("<" keeps attn_fwd_kernel
# apart from attn_fwd_fp8_kernel).  Each leg is profiled in a run of its own
# (bench.py --legs LEG), so per-launch figures average only that leg's
# dispatches.
TRAFFIC_KERNELS = {
    "attn_fwd_kernel": "attn_fwd_kernel<",
    "attn_decode_split_kernel": "attn_decode_split_kernel<",
    "attn_decode_combine_kernel": "attn_decode_combine_kernel<",
    "attn_decode_append_kernel": "attn_decode_append_kernel<",
    "attn_bwd_dkdv": "attn_bwd_dkdv_",  # attn_bwd_dkdv_kernel (d = 64) or attn_bwd_dkdv_pair_kernel (d = 128)
    "attn_bwd_dq_kernel": "attn_bwd_dq_kernel<",
    "attn_fwd_fp8_kernel": "attn_fwd_fp8_kernel<",
    "attn_fp8_quant_kernel": "attn_fp8_quant_kernel<",
}


def traffic_sum(leg, keys, digest):
    """Sum of the per-launch HBM bytes of several kernels of a leg, or None if any is missing."""
    vals = [load_traffic(leg, k, digest) for k in keys]
    return None if any(v is None for v in vals) else sum(vals)


def _counter_rows(path, counter):
    """(kernel name, value in KiB) per dispatch from a rocprofv3 counter_collection.csv."""
    import csv

    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(runs, copy_mib, commands):
    """Merge rocprofv3 --pmc runs into profiles/hbm_traffic.json.

    runs: (leg, fetch_csv, write_csv) per leg, each pair from two runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of `bench.py --legs LEG
    --copy-calibration-mib N`.  The calibration copy (a same-dtype tensor
    copy, which the HIP runtime runs as its copyBuffer blit kernel) reads and
    writes N MiB exactly once; the ratio of that size to what each counter
    reports for it scales the counter for the attention kernels of the same
    run.  It is the copyBuffer dispatch with the largest counter value.
    """
    digest = source_digest()
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
        if rec.get("source_digest") != digest or "legs" not in rec:
            rec = None
    except (OSError, ValueError):
        rec = None
    if rec is None:
        rec = {"source_digest": digest, "legs": {}}
    expect_kib = copy_mib * 1024.0

    def calib(rows):
        copies = [v for n, v in rows if "copyBuffer" in n]
        if not copies:
            raise SystemExit("no copy kernel in the counter file: run bench.py with --copy-calibration-mib")
        measured = max(copies)
        return expect_kib / measured, measured

    for leg, fetch_csv, write_csv in runs:
        fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
        write = _counter_rows(write_csv, "WRITE_SIZE")
        fr, fm = calib(fetch)
        wr, wm = calib(write)
        kernels = {}
        for key, pat in TRAFFIC_KERNELS.items():
            fv = [v for n, v in fetch if pat in n]
            wv = [v for n, v in write if pat in n]
            if not fv or not wv:
                continue
            f_kib = sum(fv) / len(fv)
            w_kib = sum(wv) / len(wv)
            kernels[key] = {
                "dispatches": [len(fv), len(wv)],
                "fetch_kib_per_launch": round(f_kib, 1),
                "write_kib_per_launch": round(w_kib, 1),
                "hbm_bytes_per_launch": int(round((f_kib * fr + w_kib * wr) * 1024)),
            }
        rec["legs"][leg] = {
            "commands": [c for c in commands if f"--legs {leg} " in c + " "],
            "copy_calibration": {"mib": copy_mib, "fetch_kib_measured": fm, "write_kib_measured": wm,
                                 "fetch_scale": round(fr, 4), "write_scale": round(wr, 4)},
            "kernels": kernels,
        }
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


def time_backward(ea, pc, out, lse, stream, torch, digest, reps=20):
    """attn_bwd on the prefill workload, timed apart from the step.

    Gradients are a widening of the path (not part of the step above).  FLOPs
    follow the usual convention of 2.5x the forward's (five products of the
    forward's size: two recomputed, three gradient products).
    """
    g = torch.Generator(device=pc["q"].device).manual_seed(99)
    dout = torch.randn(pc["q"].shape, generator=g, device=pc["q"].device).to(torch.bfloat16)
    total_q = pc["B"] * pc["Nq"]
    ws = torch.empty(ea.attn_bwd_workspace_bytes(total_q, pc["Hq"]), dtype=torch.uint8, device=pc["q"].device)
    dq, dk, dv = (torch.empty_like(pc[x]) for x in "qkv")
    kw = dict(causal=pc["causal"], softmax_scale=pc["scale"], dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
    warm_up(lambda: ea.attn_bwd(pc["q"], pc["k"], pc["v"], out, lse, dout, **kw), torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        ea.attn_bwd(pc["q"], pc["k"], pc["v"], out, lse, dout, **kw)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    flops = 2.5 * prefill_flops(pc)
    tf = flops / (ms * 1e-3) / 1e12
    n_qo = pc["B"] * pc["Nq"] * pc["Hq"] * pc["d"]
    n_kv = pc["B"] * pc["Nk"] * pc["Hkv"] * pc["d"]
    # read q, out, dout, k, v and lse; write dq, dk, dv (bf16)
    alg = 2 * (3 * n_qo + 2 * n_kv) + 4 * pc["B"] * pc["Hq"] * pc["Nq"] + 2 * (n_qo + 2 * n_kv)
    return {"kernel_ms_mean": round(ms, 4), "value": round(tf, 2),
            "unit": "TFLOP/s", "flops": flops, "flops_convention": "2.5x the forward metric FLOPs",
            "algorithmic_bytes": alg,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_sum("backward", ["attn_bwd_dkdv", "attn_bwd_dq_kernel"], digest)},
            "workload": PREFILL}


def kvcache_bytes(case, rotary_dim):
    """Algorithmic bytes of a decode step that appends one token per request:
    the cached K/V rows read, the new key and value read once and written once
    into the cache, q read, out and lse written, the used table entries,
    lengths and cos/sin rows.  The turned-query round trip is overhead."""
    lens = case["seqlens_k"].tolist()
    B, Hq, Hkv, d, page = case["B"], case["Hq"], case["Hkv"], case["d"], case["page"]
    kv = sum(lens) * Hkv * d * 2 * 2
    new = 2 * (2 * B * Hkv * d * 2)
    qo = 2 * B * Hq * d * 2 + 4 * B * Hq
    table = 4 * sum(-(-(n + 1) // page) for n in lens) + 4 * B
    rot = B * (rotary_dim // 2) * 4 * 2
    return kv + new + qo + table + rot


def time_decode_kvcache(ea, W, dev, props, stream, torch, digest, reps=20):
    """attn_decode_kvcache (append + rotary, split, combine in one call) on the
    paged decode workload's lengths with one appended token per request and a
    rotary turn over all 128 features; timed apart from the step."""
    c = W.CONFIGS[DECODE]
    lens = W.decode_lengths(c["B"], c["nk_lo"], c["nk_hi"], c["seed"])
    kc = W.append_case(lens, c["Hq"], c["Hkv"], c["d"], seed=c["seed"], device=dev)
    table, seq = kc["block_table"].to(dev), kc["seqlens_k"].to(dev)
    cos, sin = (t.to(dev) for t in W.rotary_tables(max(lens) + 1, c["d"]))
    total = max(lens) + 1
    chunk = ea.attn_decode_default_chunk(c["B"], c["Hkv"], total, props.multi_processor_count)
    n = ea.attn_decode_num_splits(total, chunk)
    bufs = dict(q_rot=torch.empty_like(kc["q"]),
                out_partial=torch.empty((n, c["B"], c["Hq"], c["d"]), dtype=torch.float32, device=dev),
                lse_partial=torch.empty((n, c["B"], c["Hq"]), dtype=torch.float32, device=dev),
                out=torch.empty_like(kc["q"]), lse=torch.empty((c["B"], c["Hq"]), dtype=torch.float32, device=dev))

    def run():
        ea.attn_decode_kvcache(kc["q"], kc["k_new"], kc["v_new"], kc["k_cache"], kc["v_cache"], table, seq,
                               max_seqlen_k=max(lens), softmax_scale=c["d"] ** -0.5, rotary_cos=cos,
                               rotary_sin=sin, chunk_tokens=chunk, stream=stream, **bufs)

    warm_up(run, torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    nbytes = kvcache_bytes(kc, c["d"])
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"call_ms_mean": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
            "algorithmic_bytes": nbytes, "chunk_tokens": chunk, "splits": n,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_sum("kvcache", ["attn_decode_append_kernel", "attn_decode_split_kernel"], digest)},
            "workload": DECODE + " with one appended token per request, rotary over all 128 features"}


PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)


def time_fp8(ea, W, pc, stream, torch, digest, reps=20):
    """FP8 forward on the prefill workload, timed apart from the step: the three
    quantisation passes (Q and K turned by seeded random signs, V into the V^T
    layout) and attn_fwd_fp8, each bracketed by events.  FLOPs as the bf16
    metric (the same attention)."""
    signs = W.hadamard_signs(pc["d"], 9, device=pc["q"].device)
    q, k, v = pc["q"], pc["k"], pc["v"]
    qc, qs = ea.attn_fp8_quantize(q, signs=signs, stream=stream)
    kc, ks = ea.attn_fp8_quantize(k, signs=signs, stream=stream)
    vc, vs = ea.attn_fp8_quantize(v, layout="vt", stream=stream)
    out = torch.empty_like(q)
    lse = torch.empty((pc["B"], pc["Hq"], pc["Nq"]), dtype=torch.float32, device=q.device)

    def quant():
        ea.attn_fp8_quantize(q, signs=signs, codes=qc, scales=qs, stream=stream)
        ea.attn_fp8_quantize(k, signs=signs, codes=kc, scales=ks, stream=stream)
        ea.attn_fp8_quantize(v, layout="vt", codes=vc, scales=vs, stream=stream)

    def attn():
        ea.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=pc["causal"], softmax_scale=pc["scale"], incoherent=True,
                        out=out, lse=lse, stream=stream)

    warm_up(lambda: (quant(), attn()), torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        quant()
        e[1].record(stream)
        attn()
        e[2].record(stream)
    torch.cuda.synchronize()
    q_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    a_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    flops = prefill_flops(pc)
    tf = flops / (a_ms * 1e-3) / 1e12
    qbytes = 3 * 3 * q.numel()  # read bf16 (2 B), write codes (1 B), three tensors
    nb = -(-pc["Nq"] // 64)
    # read the three code tensors and their block scales, write out (bf16) and lse
    alg = 3 * q.numel() + 3 * 4 * pc["B"] * pc["Hq"] * nb + 2 * q.numel() + 4 * pc["B"] * pc["Hq"] * pc["Nq"]
    return {"kernel_ms_mean": round(a_ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
            "algorithmic_bytes": alg,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": load_traffic("fp8", "attn_fwd_fp8_kernel", digest)},
            "quantize_ms_mean": round(q_ms, 4), "quantize_gbs": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
            "end_to_end_tflops": round(flops / ((q_ms + a_ms) * 1e-3) / 1e12, 2),
            "workload": PREFILL + ", E4M3, 64-row block scales, Q and K turned by a random-sign Hadamard transform"}


def measure_ceilings(ea, torch, dev, stream, read_gib=4, waves=2048, iters=4096, reps=4):
    """Measured ceilings on this GPU (include/attn_ceiling.h): a streaming read
    of read_gib GiB, and bf16 matrix cores on random operands, two waves per
    SIMD of four independent accumulator chains."""
    def timed(fn):
        fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return sum(e[0].elapsed_time(e[1]) for e in ev) / reps

    src = torch.zeros(read_gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(ea.lib().attn_ceiling_read_sink_words(read_gib << 30), dtype=torch.int32, device=dev)
    r_ms = timed(lambda: ea.ceiling_read(src, sink, stream=stream))
    nbytes = src.numel()
    del src
    g = torch.Generator(device=dev).manual_seed(7)
    ops = torch.randn((waves, 64, 64), generator=g, device=dev).to(torch.bfloat16).view(torch.int32)
    sinkf = torch.empty(waves * 64, dtype=torch.float32, device=dev)
    m_ms = timed(lambda: ea.ceiling_mfma_bf16(ops, iters, sink=sinkf, stream=stream))
    flops = waves * iters * 32 * 32768.0
    ops8 = torch.randn((waves, 64, 256), generator=g, device=dev).to(torch.float8_e4m3fn).view(torch.int32)
    f_ms = timed(lambda: ea.ceiling_mfma_fp8(ops8, iters, sink=sinkf, stream=stream))
    flops8 = waves * iters * 32 * 131072.0
    return {"hbm_read_gbs": round(nbytes / (r_ms * 1e-3) / 1e9, 1), "read_bytes": nbytes,
            "mfma_bf16_random_tflops": round(flops / (m_ms * 1e-3) / 1e12, 1),
            "mfma_fp8_random_tflops": round(flops8 / (f_ms * 1e-3) / 1e12, 1), "mfma_waves": waves,
            "mfma_iters": iters,
            "method": "each wave streams a contiguous 512 KiB of a 4 GiB buffer, 8 16-byte loads in flight per "
                      "lane; 4 independent v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x64_f8f6f4) chains per wave on "
                      "N(0,1) bf16 (E4M3) operands, 2 waves per SIMD (64 KiB of LDS per 4-wave workgroup keeps the "
                      "grid spread over all CUs)"}


def add_measured(roof, ceiling):
    """Beside the published peak: the same rate against the measured ceiling."""
    if roof is not None and ceiling:
        roof["peak_measured"] = ceiling
        roof["frac_measured"] = round(roof["achieved"] / ceiling, 4)


def _cpu_info():
    """(BLAS/OpenMP threads the oracle runs with, CPU model)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return threads, cpu


def _cpu_record(value, unit, sample):
    threads, cpu = _cpu_info()
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "sample": sample,
            "cpu": cpu, "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_dense(case, name, budget_s):
    """The fp64 oracle on whole (batch, head) pairs of a dense workload, until
    the time budget is spent; metric FLOPs of the pairs done / time."""
    import numpy as np
    import torch

    import oracle

    q, k, v = (case[x].to("cpu", dtype=torch.float32).numpy() for x in "qkv")
    B, Hq = case["B"], case["Hq"]
    pairs = [(b, h) for h in range(Hq) for b in range(B)]
    done = 0
    t0 = time.perf_counter()
    for b, h in pairs:
        hk = h // (Hq // case["Hkv"])
        oracle.attention_ref(q[b:b + 1, :, h:h + 1].astype(np.float64),
                             k[b:b + 1, :, hk:hk + 1].astype(np.float64),
                             v[b:b + 1, :, hk:hk + 1].astype(np.float64),
                             causal=case["causal"], softmax_scale=case["scale"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    elapsed = time.perf_counter() - t0
    per_head = prefill_flops(case) / (B * Hq)
    masked = " (materialising S, masked half included)" if case["causal"] else " (materialising S)"
    return _cpu_record(per_head * done / elapsed / 1e12, "TFLOP/s",
                       f"{done} of {B * Hq} (batch, head) pairs of {name}, each the full "
                       f"{case['Nq']}x{case['Nk']} problem in fp64 NumPy{masked}, {elapsed:.1f} s; "
                       f"metric FLOPs as on the GPU")


def cpu_baseline_varlen(case, name, budget_s):
    """The fp64 oracle on whole (sequence, head) pairs of the packed workload,
    longest sequences first, until the time budget is spent."""
    import numpy as np
    import torch

    import oracle

    q, k, v = (case[x].to("cpu", dtype=torch.float32).numpy() for x in "qkv")
    cq, ck = case["cu_seqlens_q"].tolist(), case["cu_seqlens_k"].tolist()
    Hq, g = case["Hq"], case["Hq"] // case["Hkv"]
    order = sorted(range(len(case["nq"])), key=lambda s: -case["nk"][s])
    flops = 0.0
    done = 0
    t0 = time.perf_counter()
    for s in order:
        for h in range(Hq):
            nq, nk = case["nq"][s], case["nk"][s]
            oracle.attention_ref(q[None, cq[s]:cq[s + 1], h:h + 1].astype(np.float64),
                                 k[None, ck[s]:ck[s + 1], h // g:h // g + 1].astype(np.float64),
                                 v[None, ck[s]:ck[s + 1], h // g:h // g + 1].astype(np.float64),
                                 causal=True, softmax_scale=case["scale"])
            flops += 4.0 * nq * nk * case["d"] / 2
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    elapsed = time.perf_counter() - t0
    return _cpu_record(flops / elapsed / 1e12, "TFLOP/s",
                       f"{done} of {len(order) * Hq} (sequence, head) pairs of {name} at d={case['d']}, "
                       f"longest sequences first, in fp64 NumPy (materialising S), {elapsed:.1f} s; "
                       f"metric FLOPs (halved for causal) as on the GPU")


def cpu_baseline_decode(case, budget_s):
    """The fp64 decode oracle (gather, then the definition, unsplit) on whole
    requests until the time budget is spent; algorithmic bytes / time.  Each
    request's pages are copied out of the cache before its timed call."""
    import numpy as np
    import torch

    import oracle

    lens = case["seqlens_k"].tolist()
    page = case["page"]
    table = case["block_table"].to("cpu")
    nbytes = 0
    done = 0
    elapsed = 0.0
    for b in range(case["B"]):
        n_pages = -(-lens[b] // page)
        idx = table[b, :n_pages].to(case["k_cache"].device, torch.long)
        kc = case["k_cache"].index_select(0, idx).to("cpu", torch.float32).numpy()
        vc = case["v_cache"].index_select(0, idx).to("cpu", torch.float32).numpy()
        q = case["q"][b:b + 1].to("cpu", torch.float32).numpy()
        t0 = time.perf_counter()
        oracle.decode_ref(q.astype(np.float64), kc, vc, np.arange(n_pages)[None], [lens[b]],
                          softmax_scale=case["scale"])
        elapsed += time.perf_counter() - t0
        nbytes += (lens[b] * case["Hkv"] * case["d"] * 4 + 2 * case["Hq"] * case["d"] * 2 + 4 * case["Hq"]
                   + 4 * n_pages + 4)
        done += 1
        if elapsed >= budget_s:
            break
    return _cpu_record(nbytes / elapsed / 1e9, "GB/s",
                       f"{done} of {case['B']} requests of {DECODE} (each over all its cached keys, "
                       f"{sum(lens[:done])} keys in all) in fp64 NumPy, {elapsed:.1f} s of oracle time; "
                       f"the request's algorithmic bytes as on the GPU")


def varlen_flops(case):
    """Metric FLOPs of a packed causal batch: 4*Nq*Nk*d per (sequence, head), halved."""
    return sum(4.0 * nq * nk * case["d"] / 2 for nq, nk in zip(case["nq"], case["nk"])) * case["Hq"]


def varlen_flops_exact(case):
    """4*d per allowed (query, key) pair, bottom-right causal per sequence."""
    pairs = 0
    for nq, nk in zip(case["nq"], case["nk"]):
        pairs += sum(max(0, min(nk, i + nk - nq + 1)) for i in range(nq))
    return 4.0 * case["d"] * pairs * case["Hq"]


def varlen_bytes(case):
    """Compulsory traffic of a packed batch: Q, K, V read once, out and lse written once."""
    tq, tk = sum(case["nq"]), sum(case["nk"])
    return 2 * (2 * tq * case["Hq"] * case["d"] + 2 * tk * case["Hkv"] * case["d"]) + 4 * case["Hq"] * tq


def warm_up(fn, torch, min_ms=WARM_MS):
    """Call fn until at least min_ms of wall time has passed (synchronising
    every few calls): the GPU's clocks settle over tens of milliseconds of
    work, so a leg that ran only a few warm-up calls would be timed on a
    clock still ramping up."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms or n >= 4000:
            return n


def time_launches(fn, stream, torch, reps):
    """Per-launch times (ms) of fn, each bracketed by events on `stream`,
    after warm_up."""
    warm_up(fn, torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev]


def _stats(ms):
    mean = sum(ms) / len(ms)
    srt = sorted(ms)
    pct = lambda p: srt[min(len(srt) - 1, int(round(p * (len(srt) - 1))))]
    return mean, pct(0.5), pct(0.95)


def graph_launch_ms(fn, torch, per_graph=20, reps=20):
    """Device time per launch of fn (which launches on torch's current stream):
    a HIP graph of per_graph back-to-back launches is replayed reps times, each
    replay bracketed by events; the host's per-call overhead is not in it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    warm_up(g.replay, torch)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / per_graph)
    return ms


def fwd_leg(ea, case, workload, leg, stream, torch, digest, flops, flops_exact, nbytes, reps=20, graph=False):
    """One attn_fwd workload timed on its own: per-launch mean, p50, p95.  With
    graph=True (a launch shorter than the binding's host overhead) the kernel
    time comes from graph replays and the eager per-call time is reported as
    call_ms_mean."""
    kw = dict(causal=case["causal"], softmax_scale=case["scale"])
    if "cu_seqlens_q" in case:
        kw.update(cu_seqlens_q=case["cu_seqlens_q"], cu_seqlens_k=case["cu_seqlens_k"],
                  max_seqlen_q=case["max_seqlen_q"], max_seqlen_k=case["max_seqlen_k"])
    out, lse = ea.attn_fwd(case["q"], case["k"], case["v"], stream=stream, **kw)
    ms = time_launches(lambda: ea.attn_fwd(case["q"], case["k"], case["v"], out=out, lse=lse, stream=stream, **kw),
                       stream, torch, reps)
    extra = {}
    if graph:
        extra["call_ms_mean"] = round(sum(ms) / len(ms), 4)
        extra["timing"] = ("kernel_ms_*: HIP-graph replays of 20 back-to-back launches (device time per launch); "
                           "call_ms_mean: eager calls through the Python binding, each bracketed by events")
        ms = graph_launch_ms(lambda: ea.attn_fwd(case["q"], case["k"], case["v"], out=out, lse=lse, **kw), torch)
    mean, p50, p95 = _stats(ms)
    tf = flops / (mean * 1e-3) / 1e12
    return {"workload": workload, "kernel_ms_mean": round(mean, 4), "kernel_ms_p50": round(p50, 4),
            "kernel_ms_p95": round(p95, 4), **extra, "value": round(tf, 2), "unit": "TFLOP/s",
            "flops_metric": flops, "flops_exact": flops_exact,
            "tflops_exact": round(flops_exact / (mean * 1e-3) / 1e12, 2), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic(leg, "attn_fwd_kernel", digest)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help=f"comma-separated legs to run (default: all of {','.join(LEGS)}); "
                         "the headline value needs 'step'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (for counter scaling)")
    ap.add_argument("--write-traffic", nargs=3, action="append", metavar=("LEG", "FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: merge two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a `--legs LEG --copy-calibration-mib N` run into "
                         "profiles/hbm_traffic.json (repeatable), then exit")
    ap.add_argument("--traffic-commands", nargs="*", default=[],
                    help="with --write-traffic: the profiler commands, stored with the figures")
    args = ap.parse_args()
    if args.write_traffic:
        if not args.copy_calibration_mib:
            print("--write-traffic needs the --copy-calibration-mib value of the profiled runs",
                  file=sys.stderr)
            return 2
        return write_traffic(args.write_traffic, args.copy_calibration_mib, args.traffic_commands)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2
    legs = [x for x in args.legs.split(",") if x]
    unknown = [x for x in legs if x not in LEGS]
    if unknown:
        print(f"unknown legs {unknown}; choose from {LEGS}", file=sys.stderr)
        return 2
    cpu = not args.no_cpu_baseline

    import torch

    import exact_io_aware_07_amd as ea
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream(dev)
    digest = source_digest()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: {n * 4} bytes read and written", file=sys.stderr, flush=True)
        del src, dst

    rec = {
        "metric": "attn fwd TFLOP/s (bf16 d=128 causal, % MFMA peak); decode HBM GB/s",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL},
    }
    pc = None
    if "step" in legs or "backward" in legs or "fp8" in legs:
        pc = W.config_case(PREFILL, device=dev)
        out = torch.empty_like(pc["q"])
        lse = torch.empty((pc["B"], pc["Hq"], pc["Nq"]), dtype=torch.float32, device=dev)
        ea.attn_fwd(pc["q"], pc["k"], pc["v"], causal=pc["causal"], softmax_scale=pc["scale"],
                    out=out, lse=lse, stream=stream)

    if "step" in legs:
        dc = W.config_case(DECODE, device=dev)
        dc_dev = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in dc.items()}
        max_len = int(dc["seqlens_k"].max())
        chunk = ea.attn_decode_default_chunk(dc["B"], dc["Hkv"], max_len, props.multi_processor_count)
        n_splits = ea.attn_decode_num_splits(max_len, chunk)
        part_o = torch.empty((n_splits, dc["B"], dc["Hq"], dc["d"]), dtype=torch.float32, device=dev)
        part_l = torch.empty((n_splits, dc["B"], dc["Hq"]), dtype=torch.float32, device=dev)
        dout = torch.empty((dc["B"], dc["Hq"], dc["d"]), dtype=torch.bfloat16, device=dev)
        dlse = torch.empty((dc["B"], dc["Hq"]), dtype=torch.float32, device=dev)

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            ea.attn_fwd(pc["q"], pc["k"], pc["v"], causal=pc["causal"], softmax_scale=pc["scale"],
                        out=out, lse=lse, stream=stream)
            if ev:
                ev[1].record(stream)
            ea.attn_decode_splitkv(dc_dev["q"], dc_dev["k_cache"], dc_dev["v_cache"],
                                   dc_dev["block_table"], dc_dev["seqlens_k"], chunk_tokens=chunk,
                                   num_splits=n_splits, softmax_scale=dc["scale"], out_partial=part_o,
                                   lse_partial=part_l, stream=stream)
            if ev:
                ev[2].record(stream)
            ea.attn_decode_combine(part_o, part_l, dc_dev["seqlens_k"], chunk_tokens=chunk, out=dout,
                                   lse=dlse, stream=stream)
            if ev:
                ev[3].record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_peak = torch.cuda.max_memory_allocated(dev)
        pre = [e[0].elapsed_time(e[1]) for e in events]
        spl = [e[1].elapsed_time(e[2]) for e in events]
        cmb = [e[2].elapsed_time(e[3]) for e in events]
        pre_ms, pre_p50, pre_p95 = _stats(pre)
        spl_ms, _, spl_p95 = _stats(spl)
        cmb_ms = sum(cmb) / len(cmb)
        flops = prefill_flops(pc)
        tflops = flops / (pre_ms * 1e-3) / 1e12
        dbytes = decode_bytes(dc)
        split_gbs = dbytes / (spl_ms * 1e-3) / 1e9
        decode_gbs = dbytes / ((spl_ms + cmb_ms) * 1e-3) / 1e9
        rec.update({
            "value": round(tflops, 2),
            "ms_per_step": round(wall * 1e3 / args.steps, 4),
            "peak_device_memory_bytes_step": step_peak,
            "config": {"workload": PREFILL, "B": pc["B"], "Hq": pc["Hq"], "Hkv": pc["Hkv"],
                       "Nq": pc["Nq"], "Nk": pc["Nk"], "d": pc["d"], "causal": pc["causal"],
                       "decode_workload": DECODE, "decode_chunk_tokens": chunk,
                       "decode_splits": n_splits},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic("step", "attn_fwd_kernel", digest)},
            "prefill": {"kernel_ms_mean": round(pre_ms, 4), "kernel_ms_p50": round(pre_p50, 4),
                        "kernel_ms_p95": round(pre_p95, 4), "flops_metric": flops,
                        "flops_exact": prefill_flops_exact(pc),
                        "tflops_exact": round(prefill_flops_exact(pc) / (pre_ms * 1e-3) / 1e12, 2),
                        "algorithmic_bytes": prefill_bytes(pc)},
            "decode": {"workload": DECODE, "value": round(decode_gbs, 1), "unit": "GB/s",
                       "split_ms_mean": round(spl_ms, 4), "combine_ms_mean": round(cmb_ms, 4),
                       "split_ms_p95": round(spl_p95, 4),
                       "algorithmic_bytes": dbytes,
                       "roofline": {"bound": "hbm", "achieved": round(split_gbs, 1),
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                                    "traffic": load_traffic("step", "attn_decode_split_kernel", digest)}},
        })
        print(f"step: prefill {pre_ms:.4f} ms ({tflops:.1f} TFLOP/s), decode split {spl_ms:.4f} ms "
              f"({split_gbs:.0f} GB/s)", file=sys.stderr, flush=True)
        # Cold-cache samples (reported beside the warm figures, never as the
        # value): a 512 MiB fill before each launch evicts the L2s and the
        # 256 MB Infinity Cache, so every input comes from HBM.
        flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        cold_pre, cold_dec = [], []
        for i in range(5):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            flush.fill_(float(i))
            ev[0].record(stream)
            ea.attn_fwd(pc["q"], pc["k"], pc["v"], causal=pc["causal"], softmax_scale=pc["scale"],
                        out=out, lse=lse, stream=stream)
            ev[1].record(stream)
            flush.fill_(float(i) + 0.5)
            ev[2].record(stream)
            ea.attn_decode_splitkv(dc_dev["q"], dc_dev["k_cache"], dc_dev["v_cache"],
                                   dc_dev["block_table"], dc_dev["seqlens_k"], chunk_tokens=chunk,
                                   num_splits=n_splits, softmax_scale=dc["scale"], out_partial=part_o,
                                   lse_partial=part_l, stream=stream)
            ea.attn_decode_combine(part_o, part_l, dc_dev["seqlens_k"], chunk_tokens=chunk, out=dout,
                                   lse=dlse, stream=stream)
            ev[3].record(stream)
            torch.cuda.synchronize()
            cold_pre.append(ev[0].elapsed_time(ev[1]))
            cold_dec.append(ev[2].elapsed_time(ev[3]))
        del flush
        cold_pre_ms = sum(cold_pre) / len(cold_pre)
        cold_dec_ms = sum(cold_dec) / len(cold_dec)
        rec["prefill"]["cold_kernel_ms_mean"] = round(cold_pre_ms, 4)
        rec["prefill"]["cold_tflops"] = round(flops / (cold_pre_ms * 1e-3) / 1e12, 2)
        rec["decode"]["cold_ms_mean"] = round(cold_dec_ms, 4)
        rec["decode"]["cold_value"] = round(dbytes / (cold_dec_ms * 1e-3) / 1e9, 1)
        rec["decode"]["cold_note"] = ("cold_*: 5 samples, a 512 MiB fill before each launch (outside the "
                                      "events) evicts the L2s and the Infinity Cache")
        del part_o, part_l
        if cpu:
            rec["decode"]["cpu_baseline"] = cpu_baseline_decode(dc, budget_s=6.0)
        del dc, dc_dev

    extra = {}
    if "c1" in legs:
        c = W.config_case(NONCAUSAL, device=dev)
        extra["noncausal_d64"] = fwd_leg(ea, c, NONCAUSAL, "c1", stream, torch, digest, prefill_flops(c),
                                         prefill_flops_exact(c), prefill_bytes(c), reps=50, graph=True)
        extra["noncausal_d64"]["note"] = ("2048 query rows: 64 workgroups of 4 waves in split-key mode on 256 "
                                          "compute units; latency bound")
        if cpu:
            extra["noncausal_d64"]["cpu_baseline"] = cpu_baseline_dense(c, NONCAUSAL, budget_s=2.0)
        del c
    if "c3" in legs:
        c = W.config_case(GQA, device=dev)
        extra["gqa_n8192"] = fwd_leg(ea, c, GQA, "c3", stream, torch, digest, prefill_flops(c),
                                     prefill_flops_exact(c), prefill_bytes(c))
        if cpu:
            extra["gqa_n8192"]["cpu_baseline"] = cpu_baseline_dense(c, GQA, budget_s=8.0)
        del c
    for d in (128, 64, 256):
        leg = f"c4_d{d}"
        if leg not in legs:
            continue
        c = W.config_case(VARLEN, device=dev, d=d)
        for x in ("cu_seqlens_q", "cu_seqlens_k"):
            c[x] = c[x].to(dev)
        extra[f"varlen_d{d}"] = fwd_leg(ea, c, f"{VARLEN} d={d}", leg, stream, torch, digest, varlen_flops(c),
                                        varlen_flops_exact(c), varlen_bytes(c))
        extra[f"varlen_d{d}"]["note"] = ("value uses the metric formula (halved for causal); tflops_exact "
                                         "counts the allowed pairs (bottom-right causal with Nq = Nk/4)")
        if cpu:
            extra[f"varlen_d{d}"]["cpu_baseline"] = cpu_baseline_varlen(c, VARLEN, budget_s=5.0)
        del c
    for key, leg in extra.items():
        print(f"{key}: {leg['kernel_ms_mean']:.4f} ms, {leg['value']:.1f} TFLOP/s "
              f"(exact {leg['tflops_exact']:.1f})", file=sys.stderr, flush=True)
    rec["configs"] = extra

    bwd = time_backward(ea, pc, out, lse, stream, torch, digest) if "backward" in legs else None
    kvc = time_decode_kvcache(ea, W, dev, props, stream, torch, digest) if "kvcache" in legs else None
    fp8 = time_fp8(ea, W, pc, stream, torch, digest) if "fp8" in legs else None
    ceil = measure_ceilings(ea, torch, dev, stream) if "ceilings" in legs else None
    rec["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "cus": props.multi_processor_count, "torch": torch.__version__,
                     "hip": getattr(torch.version, "hip", None)}
    rec["kernel_source_digest"] = digest
    if ceil is not None:
        rec["ceilings"] = ceil
        for r in [rec.get("roofline")] + [x["roofline"] for x in extra.values()]:
            add_measured(r, ceil["mfma_bf16_random_tflops"])
        if "decode" in rec:
            add_measured(rec["decode"]["roofline"], ceil["hbm_read_gbs"])
        if bwd is not None:
            add_measured(bwd["roofline"], ceil["mfma_bf16_random_tflops"])
        if kvc is not None:
            add_measured(kvc["roofline"], ceil["hbm_read_gbs"])
        if fp8 is not None:
            add_measured(fp8["roofline"], ceil["mfma_fp8_random_tflops"])
    if bwd is not None:
        rec["backward"] = bwd
    if kvc is not None:
        rec["decode_kvcache"] = kvc
    if fp8 is not None:
        rec["fp8_forward"] = fp8
    if cpu and "step" in legs:
        rec["cpu_baseline"] = cpu_baseline_dense(pc, PREFILL, budget_s=12.0)
    rec["peak_device_memory_bytes"] = torch.cuda.max_memory_allocated(dev)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
