"""The measurement kernels of include/attn_ceiling.h compute what they claim (needs an MI355X).

The read kernel's sink words are the XOR of each 512 KiB chunk, checked with
numpy on a buffer with a ragged last chunk.  The matrix-core kernels, given
fragments that each hold one small integer, must return the exact sum that
their four chains of fragment pairs imply (every product entry is K * a * b,
K = 16 for bf16 and 64 for E4M3).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_07_amd as ea

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHUNK = 512 * 1024


def test_read_sink_is_xor_of_each_chunk():
    nbytes = 3 * CHUNK + 48
    host = np.random.default_rng(3).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = ea.ceiling_read(src)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = [np.bitwise_xor.reduce(host[i:i + CHUNK // 4]) for i in range(0, host.size, CHUNK // 4)]
    assert got.tolist() == [int(x) for x in want]


def expected_sink(vals, iters, k):
    per_lane = sum(16 * iters * sum(k * vals[(j + c) % 8] * vals[(j + 2 * c + 1) % 8] for j in range(8))
                   for c in range(4))
    return 2 * per_lane  # each lane adds the sum of the lane 64 threads on


# (element type, K of one product, values per lane per fragment, binding)
@pytest.mark.parametrize("dtype,k,per_frag,fn", [(torch.bfloat16, 16, 8, "ceiling_mfma_bf16"),
                                                 (torch.float8_e4m3fn, 64, 32, "ceiling_mfma_fp8")])
def test_mfma_sink_matches_the_fragment_schedule(dtype, k, per_frag, fn):
    waves, iters = 8, 3
    vals = np.arange(1, 9, dtype=np.float64)  # fragment i holds the value i + 1 in every slot
    frag = torch.tensor(vals, dtype=torch.float32).to(dtype).view(1, 1, 8, 1).expand(waves, 64, 8, per_frag)
    ops = frag.contiguous().view(waves, 64, 8 * per_frag).view(torch.int32).to(DEV)
    sink = getattr(ea, fn)(ops, iters)
    torch.cuda.synchronize()
    want = expected_sink(vals, iters, k)
    assert want < 2**24  # every partial sum is an exact fp32 integer
    assert torch.equal(sink.cpu(), torch.full((waves * 64,), want, dtype=torch.float32))
