"""Seeded synthetic attention inputs.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it without sharing any of the method.

Recipe: every tensor entry is drawn as float32 N(0, 1) from a torch.Generator
seeded per case and rounded once to bfloat16 (round to nearest even).  The
oracle reads back the very same bfloat16 values, upcast exactly to float64.
Tensors that are generated on a GPU use that device's generator, so their
values differ from a CPU draw with the same seed; the distribution does not.
"""
import torch

PAGE_SIZE = 256

# The five workloads (shapes, masks, head layouts and length mixes).
CONFIGS = {
    "mha_noncausal_b1_h4_n512_d64": dict(kind="dense", B=1, Hq=4, Hkv=4, Nq=512, Nk=512, d=64,
                                 causal=False, seed=1),
    "mha_causal_b4_h16_n4096_d128": dict(kind="dense", B=4, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=128,
                               causal=True, seed=2),
    "gqa_causal_b2_hq32_hkv8_n8192_d128_koutliers": dict(kind="dense", B=2, Hq=32, Hkv=8, Nq=8192, Nk=8192,
                                        d=128, causal=True, seed=3, k_outlier_frac=0.01,
                                        k_outlier_scale=3.0),
    "varlen_chunked_prefill_16seq_hq32_hkv8": dict(kind="varlen", n_seqs=16, nk_lo=256, nk_hi=8192,
                                      q_div=4, Hq=32, Hkv=8, d=128, causal=True, seed=4),
    "paged_decode_b64_hq32_hkv8_d128": dict(kind="decode", B=64, Hq=32, Hkv=8, d=128, nk_lo=4096,
                                    nk_hi=32768, page=PAGE_SIZE, seed=5),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, g, device):
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


def dense_case(B, Nq, Nk, Hq, Hkv, d, seed, *, device="cpu", k_outlier_frac=0.0,
               k_outlier_scale=3.0):
    """q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d] bf16.

    With k_outlier_frac > 0, floor(frac * B * Nk * Hkv) key rows (one row is
    the d-vector at one (b, n, kv head)) are picked without replacement and
    their float32 draws multiplied by k_outlier_scale before rounding.
    """
    g = _gen(seed, device)
    q = _randn_bf16((B, Nq, Hq, d), g, device)
    k32 = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32, device=device)
    v = _randn_bf16((B, Nk, Hkv, d), g, device)
    n_out = int(k_outlier_frac * B * Nk * Hkv)
    if n_out:
        rows = torch.randperm(B * Nk * Hkv, generator=g, device=device)[:n_out]
        flat = k32.view(B * Nk * Hkv, d)
        flat[rows] *= k_outlier_scale
    k = k32.to(torch.bfloat16)
    return dict(q=q, k=k, v=v, B=B, Nq=Nq, Nk=Nk, Hq=Hq, Hkv=Hkv, d=d)


def varlen_lengths(n_seqs, lo, hi, q_div, seed):
    """Per-sequence key lengths uniform on the integers [lo, hi]; Nq = Nk // q_div."""
    g = _gen(seed, "cpu")
    nk = torch.randint(lo, hi + 1, (n_seqs,), generator=g).tolist()
    nq = [n // q_div for n in nk]
    return nq, nk


def _cumsum(lengths):
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def varlen_case(nq_list, nk_list, Hq, Hkv, d, seed, *, device="cpu"):
    """Packed q [sum Nq, Hq, d], k and v [sum Nk, Hkv, d] with int32 cu_seqlens."""
    g = _gen(seed, device)
    cu_q, cu_k = _cumsum(nq_list), _cumsum(nk_list)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _randn_bf16((tq, Hq, d), g, device)
    k = _randn_bf16((tk, Hkv, d), g, device)
    v = _randn_bf16((tk, Hkv, d), g, device)
    return dict(q=q, k=k, v=v, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                max_seqlen_q=max(nq_list) if nq_list else 0,
                max_seqlen_k=max(nk_list) if nk_list else 0,
                nq=list(nq_list), nk=list(nk_list), Hq=Hq, Hkv=Hkv, d=d)


def decode_lengths(B, lo, hi, seed):
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def decode_case(seqlens, Hq, Hkv, d, seed, *, page=PAGE_SIZE, device="cpu", poison=False,
                extra_table_cols=0):
    """Paged cache for one-token decode.

    Request b uses ceil(seqlens[b] / page) logical pages; the pool holds
    exactly their total P, and logical pages take physical ids in the order of
    a seeded random permutation of range(P).  block_table is int32
    [B, max pages (+ extra_table_cols)]; entries past a request's pages are 0,
    or, with poison=True, point at one extra page P filled with NaN, and every
    cache row past a request's length in its last page is NaN as well.
    """
    B = len(seqlens)
    g = _gen(seed, device)
    q = _randn_bf16((B, Hq, d), g, device)
    pages = [-(-int(n) // page) for n in seqlens]
    P = sum(pages)
    n_pool = P + (1 if poison else 0)
    k_cache = _randn_bf16((n_pool, page, Hkv, d), g, device)
    v_cache = _randn_bf16((n_pool, page, Hkv, d), g, device)
    perm = torch.randperm(P, generator=g, device=device).to("cpu")
    width = max(pages) + extra_table_cols if pages else 1
    fill = P if poison else 0
    table = torch.full((B, width), fill, dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    if poison:
        nan = float("nan")
        k_cache[P] = nan
        v_cache[P] = nan
        for b, n in enumerate(seqlens):
            used = int(n) % page
            if used:
                last = int(table[b, pages[b] - 1])
                k_cache[last, used:] = nan
                v_cache[last, used:] = nan
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
                seqlens_k=torch.tensor([int(n) for n in seqlens], dtype=torch.int32),
                B=B, Hq=Hq, Hkv=Hkv, d=d, page=page, num_pages=n_pool)


def rotary_tables(max_pos, rotary_dim, base=10000.0, device="cpu"):
    """float32 cos/sin tables [max_pos, rotary_dim / 2] of RoFormer's angles.

    Pair i at position p turns by p * base ** (-2 i / rotary_dim); the angles
    and their cosines and sines are formed in float64 and rounded once.  These
    are inputs (a model's choice of frequencies), not part of the method.
    """
    i = torch.arange(rotary_dim // 2, dtype=torch.float64)
    theta = base ** (-2.0 * i / rotary_dim)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * theta[None, :]
    return (torch.cos(ang).to(torch.float32).to(device), torch.sin(ang).to(torch.float32).to(device))


def append_case(seqlens, Hq, Hkv, d, seed, *, device="cpu", poison=False, extra_table_cols=0):
    """Inputs of one decode step that appends a token to each request.

    The paged cache is decode_case's for lengths seqlens[b] + 1, so each
    request's table already names the page of its new position; seqlens_k is
    set to seqlens (the keys cached before the step), and the row at position
    seqlens[b] holds random data that the append overwrites.  k_new, v_new
    [B, Hkv, d] are bf16 N(0, 1) from their own seeded generator.
    """
    case = decode_case([int(n) + 1 for n in seqlens], Hq, Hkv, d, seed, device=device, poison=poison,
                       extra_table_cols=extra_table_cols)
    case["seqlens_k"] = torch.tensor([int(n) for n in seqlens], dtype=torch.int32)
    g = _gen(seed + 500, device)
    case["k_new"] = _randn_bf16((len(seqlens), Hkv, d), g, device)
    case["v_new"] = _randn_bf16((len(seqlens), Hkv, d), g, device)
    return case


def hadamard_signs(d, seed, device="cpu"):
    """int8 [d] of +-1 drawn from a seeded generator: the random sign vector of
    incoherent processing (an input the caller chooses)."""
    g = _gen(seed, "cpu")
    return (torch.randint(0, 2, (d,), generator=g, dtype=torch.int64) * 2 - 1).to(torch.int8).to(device)


def config_case(name, *, device="cpu", d=None, poison=False):
    """Materialise one of CONFIGS (d overrides the head dim of the varlen case)."""
    c = CONFIGS[name]
    if c["kind"] == "dense":
        case = dense_case(c["B"], c["Nq"], c["Nk"], c["Hq"], c["Hkv"], c["d"], c["seed"],
                          device=device, k_outlier_frac=c.get("k_outlier_frac", 0.0),
                          k_outlier_scale=c.get("k_outlier_scale", 3.0))
        case.update(causal=c["causal"], scale=c["d"] ** -0.5)
        return case
    if c["kind"] == "varlen":
        dd = c["d"] if d is None else d
        nq, nk = varlen_lengths(c["n_seqs"], c["nk_lo"], c["nk_hi"], c["q_div"], c["seed"])
        case = varlen_case(nq, nk, c["Hq"], c["Hkv"], dd, c["seed"] * 1000 + dd, device=device)
        case.update(causal=c["causal"], scale=dd ** -0.5)
        return case
    lens = decode_lengths(c["B"], c["nk_lo"], c["nk_hi"], c["seed"])
    case = decode_case(lens, c["Hq"], c["Hkv"], c["d"], c["seed"], page=c["page"],
                       device=device, poison=poison)
    case.update(scale=c["d"] ** -0.5)
    return case
