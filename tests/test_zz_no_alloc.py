"""attn_decode_noalloc (partials in the library's own device array) against
attn_decode_splitkv + attn_decode_combine with a caller workspace, and against
the fp64 oracle (needs an MI355X).

Two calls in a row, the second with a smaller input, so that the second call
runs over the array the first one left behind: both must equal the workspace
path bit for bit (the same kernels on the same inputs) and meet the oracle
tolerances (max |out - ref| <= 1.5e-2, mean <= 1e-3, |lse - ref| <= 1e-3).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def to64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def run_both(case, chunk):
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in case.items()}
    max_len = int(case["seqlens_k"].max())
    scale = case["d"] ** -0.5
    out_n, lse_n = ea.attn_decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                                          dev["seqlens_k"], max_seqlen_k=max_len, softmax_scale=scale,
                                          chunk_tokens=chunk)
    out_w, lse_w = ea.attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                                  dev["seqlens_k"], max_seqlen_k=max_len, softmax_scale=scale,
                                  chunk_tokens=chunk)
    torch.cuda.synchronize()
    return out_n, lse_n, out_w, lse_w


def check_oracle(case, out, lse):
    ref_o, ref_l = oracle.decode_ref(to64(case["q"]), to64(case["k_cache"]), to64(case["v_cache"]),
                                     case["block_table"].numpy(), case["seqlens_k"].numpy(),
                                     softmax_scale=case["d"] ** -0.5)
    o, l = to64(out), to64(lse)
    assert np.isfinite(o).all()
    d = np.abs(o - ref_o)
    assert d.max() <= 1.5e-2 and d.mean() <= 1e-3, (d.max(), d.mean())
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(o[empty] == 0)
    assert np.abs(l[~empty] - ref_l[~empty]).max(initial=0.0) <= 1e-3


def test_noalloc_matches_workspace_path_twice_second_smaller():
    big = W.decode_case([4000, 1, 2500, 0, 7000, 300], 16, 4, 128, seed=301, poison=True)
    small = W.decode_case([900, 17], 8, 2, 128, seed=302, poison=True)
    for case, chunk in ((big, 512), (small, 256)):
        out_n, lse_n, out_w, lse_w = run_both(case, chunk)
        assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
        check_oracle(case, out_n, lse_n)


@pytest.mark.parametrize("d", [64, 256])
def test_noalloc_other_head_dims(d):
    case = W.decode_case([1500, 64, 3000], 8, 1, d, seed=310 + d)
    out_n, lse_n, out_w, lse_w = run_both(case, 1024)
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
    check_oracle(case, out_n, lse_n)


def test_noalloc_rejects_oversized_partials_on_gpu():
    case = W.decode_case([600, 300], 8, 2, 128, seed=320)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in case.items()}
    with pytest.raises(ea.AttnError, match="scratch"):
        # 256-token chunks over a length that needs more splits than the array holds.
        ea.attn_decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                               dev["seqlens_k"], max_seqlen_k=(ea.DECODE_NOALLOC_SCRATCH_BYTES // (2 * 8 * 129 * 4) + 1) * 256,
                               softmax_scale=0.1, chunk_tokens=256)
