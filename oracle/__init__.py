"""CPU fp64 oracle for exact attention -- test infrastructure, not product code.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It shares no code with the HIP path: it computes the
plain, materialising definition of scaled dot-product attention in float64
with NumPy, one (sequence, query head) at a time.

Sources (page title, section):
  * "Deep Dive - FlashAttention": "Exact attention without an n x n workspace",
    "Two tiles by hand", "The public interface is several kernels",
    "Backward recomputes tiles on purpose" (the gradients), "Causal 2.1 is the
    decode gotcha" (the local window),
    "Paged KV is a lookup, not a cache manager" (also the in-place cache append).
  * "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)":
    "Runnable Example: Measuring the IO Gap", "Decode-Time Kernels".
  * "Flash Attention: A Complete Architectural Autopsy": "Part 1", "FP8 Path and
    Quantization" (module fp8).
  * "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
    "FlashAttention-3": block quantisation and incoherent processing (module fp8).
  * "FlashAttention: Part 1": sections 2.2, 3.5, 4.1, 4.2 (rotary embedding as a
    transform of Q and K before attention; module kvcache).

Parity status: every function here is pinned by the tests in
tests/test_oracle_pins.py except two conventions the pages leave open (the
lse of a row with no allowed key, and the packed [Hq, total_q] lse layout of
variable-length batches); those two are "parity unpinned".  The rotary
formula and the bf16 rounding of rotated rows are readings (the pages give
neither); they are pinned to hand-worked turns, RoFormer's relative-position
property, a hand-worked float32 rounding case with the float64 error bound,
and PyTorch's float32 -> bfloat16 conversion.  Module fp8 (E4M3 codec, the
float32 Walsh-Hadamard turn, block quantisation, the V^T layout, attention on
dequantised operands and the bound on the error of rounding probabilities to
E4M3) is pinned to PyTorch's float8_e4m3fn, scipy's Hadamard matrix, hand-worked
codes and positions, and a slow tile model of the probability rounding.
"""
from .attention import (  # noqa: F401
    kv_head_for_queries,
    causal_keep,
    attention_ref,
    attention_rows,
    paged_gather,
    decode_ref,
    attention_bwd_ref,
    window_keep,
    paged_prefill_ref,
)
from .kvcache import (  # noqa: F401
    round_bf16,
    rotary_ref,
    rotary_f32,
    append_ref,
    decode_append_ref,
)
