"""Exact attention for AMD MI355X (gfx950): Python binding of libattn.so.

The functions below only marshal arguments (shape checks, device pointers,
the current HIP stream) and call the C ABI declared in include/attn.h; every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: when libattn.so is missing or fails to load, every call
raises.

    out, lse = attn_fwd(q, k, v, causal=True, softmax_scale=d ** -0.5)
    out, lse = attn_fwd(q, k, v, cu_seqlens_q=cq, cu_seqlens_k=ck,
                        max_seqlen_q=mq, max_seqlen_k=mk, causal=True, softmax_scale=s)
    part_o, part_l = attn_decode_splitkv(q, k_cache, v_cache, block_table, seqlens_k,
                                         chunk_tokens=c, num_splits=n, softmax_scale=s)
    out, lse = attn_decode_combine(part_o, part_l, seqlens_k, chunk_tokens=c)
    dq, dk, dv = attn_bwd(q, k, v, out, lse, dout, causal=True, softmax_scale=s)
"""
import contextlib
import ctypes
import os

import torch

__all__ = [
    "AttnError", "lib", "lib_path", "attn_fwd", "attn_fwd_paged", "attn_bwd", "attn_bwd_workspace_bytes",
    "attn_decode_splitkv", "attn_decode_combine",
    "attn_decode", "attn_decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES", "attn_decode_num_splits", "attn_decode_default_chunk",
    "attn_decode_workspace_bytes", "attn_check_cu_seqlens", "attn_check_block_table",
    "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# EXACT_ATTN_LIBRARY selects another build of the same sources (the tests run
# the ABI checks against a host-sanitizer build this way).
lib_path = os.environ.get("EXACT_ATTN_LIBRARY") or os.path.join(_HERE, "libattn.so")

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_SCALE", 5: "ATTN_ERR_ALIAS", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_DATA",
}

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

_SIGNATURES = {
    "attn_abi_version": ([], _I),
    "attn_status_str": ([_I], ctypes.c_char_p),
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "attn_fwd_ex": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                     _P, _P, _P], _I),
    "attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                  _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "attn_bwd_workspace_bytes": ([_I, _I], ctypes.c_size_t),
    "attn_decode_splitkv": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "attn_decode_combine": ([_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "attn_decode_noalloc": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "attn_decode_kvcache": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                             _I, _I, _I, _F, _P, _P, _P, _P, _P, _P], _I),
    "attn_fp8_quantize": ([_P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "attn_fp8_codes_bytes": ([_I, _I, _I, _I, _I], ctypes.c_size_t),
    "attn_fp8_num_blocks": ([_I], _I),
    "attn_fwd_fp8": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "attn_ceiling_read_sink_words": ([ctypes.c_size_t], ctypes.c_size_t),
    "attn_ceiling_read": ([_P, ctypes.c_size_t, _P, _P], _I),
    "attn_ceiling_mfma_bf16": ([_P, _I, _I, _P, _P], _I),
    "attn_ceiling_mfma_fp8": ([_P, _I, _I, _P, _P], _I),
    "attn_ceiling_last_error": ([], ctypes.c_char_p),
    "attn_decode_num_splits": ([_I, _I], _I),
    "attn_decode_default_chunk": ([_I, _I, _I, _I], _I),
    "attn_decode_workspace_bytes": ([_I, _I, _I, _I], ctypes.c_size_t),
    "attn_check_cu_seqlens": ([_P, _I, _I, _I], _I),
    "attn_check_block_table": ([_P, _P, _I, _I, _I, _I], _I),
}

_lib = None

# ATTN_DECODE_NOALLOC_SCRATCH_BYTES of include/attn.h.
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnError(RuntimeError):
    """A non-OK status from libattn.so."""

    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded libattn.so (ctypes), raising if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is missing: build it with `python -m exact_io_aware_07_amd.build`")
        handle = ctypes.CDLL(lib_path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(status):
    if status != 0:
        raise AttnError(status, lib().attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on(dev):
    """Make dev the current device for a call (a no-op context when it already is)."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def attn_fwd(q, k, v, *, causal, softmax_scale, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None, out=None, lse=None, return_lse=True,
             window=(-1, -1), stream=None):
    """Forward pass; returns (out, lse) (lse is None when return_lse is False).

    Dense: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] -> out like q, lse [B, Hq, Nq].
    Packed: q [TQ, Hq, d], k/v [TK, Hkv, d] with int32 cu_seqlens_q/k [B + 1]
    and max_seqlen_q/k -> out like q, lse [Hq, TQ].
    window: (left, right) local window, -1 for an unbounded side.
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    varlen = cu_seqlens_q is not None
    if varlen != (cu_seqlens_k is not None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    if varlen:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
        _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
        if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
            raise ValueError("packed mode expects q [TQ,Hq,d] and k, v [TK,Hkv,d]")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("packed mode needs max_seqlen_q and max_seqlen_k")
        batch = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() != batch + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
        _, hq, d = q.shape
        hkv = k.shape[1]
        mq, mk = int(max_seqlen_q), int(max_seqlen_k)
        lse_shape = (hq, q.shape[0])
    else:
        if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
            raise ValueError("dense mode expects q [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d]")
        batch, mq, hq, d = q.shape
        mk, hkv = k.shape[1], k.shape[2]
        if k.shape[0] != batch:
            raise ValueError("q and k batch sizes differ")
        lse_shape = (batch, hq, mq)
    if k.shape[-1] != d:
        raise ValueError("q and k head dims differ")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if return_lse:
        if lse is None:
            lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
        else:
            _need(lse, "lse", torch.float32, dev)
            if tuple(lse.shape) != lse_shape:
                raise ValueError(f"lse must have shape {lse_shape}")
    else:
        lse = None
    if q.numel() == 0:
        return out, lse
    wl, wr = (int(x) for x in window)
    with _on(dev):
        if wl == -1 and wr == -1:
            st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                batch, mq, mk, hq, hkv, d, 1 if causal else 0, float(softmax_scale),
                                _ptr(out), _ptr(lse), _stream(stream, dev))
        else:
            st = lib().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                   None, None, batch, mq, mk, hq, hkv, d, 256, 0, 0,
                                   1 if causal else 0, wl, wr, float(softmax_scale), _ptr(out),
                                   _ptr(lse), _stream(stream, dev))
    _check(st)
    return out, lse


def attn_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, *, max_seqlen_q,
                   causal, softmax_scale, window=(-1, -1), out=None, lse=None, stream=None):
    """Paged prefill: packed new rows q [TQ, Hq, d] (cu_seqlens_q [B + 1]) against
    caches [P, 256, Hkv, d] through block_table int32 [B, maxp], with seqlens_k
    int32 [B] cached keys per sequence (including the new rows).
    Returns (out [TQ, Hq, d], lse [Hq, TQ])."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expects q [TQ,Hq,d] and caches [P,page,Hkv,d]")
    batch = cu_seqlens_q.numel() - 1
    if seqlens_k.numel() != batch or block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("seqlens_k and block_table must have one entry / row per sequence")
    tq, hq, d = q.shape
    num_pages, page, hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("q and cache head dims differ")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, tq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    if tq == 0:
        return out, lse
    wl, wr = (int(x) for x in window)
    with _on(dev):
        st = lib().attn_fwd_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), None,
                               _ptr(block_table), _ptr(seqlens_k), batch, int(max_seqlen_q), 0, hq, hkv,
                               d, page, block_table.shape[1], num_pages, 1 if causal else 0, wl, wr,
                               float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st)
    return out, lse


def attn_bwd_workspace_bytes(total_q, num_heads_q):
    return lib().attn_bwd_workspace_bytes(int(total_q), int(num_heads_q))


def attn_bwd(q, k, v, out, lse, dout, *, causal, softmax_scale, cu_seqlens_q=None,
             cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd from its saved out and lse and dout = dL/d(out).

    Layouts as attn_fwd (out and dout like q, lse as attn_fwd returned it).
    workspace: optional uint8 GPU tensor of at least attn_bwd_workspace_bytes(TQ, Hq)
    bytes; allocated here when not given.
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    if out.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("out and dout must have q's shape, v k's shape")
    varlen = cu_seqlens_q is not None
    if varlen != (cu_seqlens_k is not None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    if varlen:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
        _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed mode expects q [TQ,Hq,d] and k, v [TK,Hkv,d]")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("packed mode needs max_seqlen_q and max_seqlen_k")
        batch = cu_seqlens_q.numel() - 1
        total_q, hq, d = q.shape
        hkv = k.shape[1]
        mq, mk = int(max_seqlen_q), int(max_seqlen_k)
        lse_shape = (hq, total_q)
    else:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense mode expects q [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d]")
        batch, mq, hq, d = q.shape
        mk, hkv = k.shape[1], k.shape[2]
        total_q = batch * mq
        lse_shape = (batch, hq, mq)
    if tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must have shape {lse_shape}")
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _need(t, name, torch.bfloat16, dev)
            if t.shape != like.shape:
                raise ValueError(f"{name} has the wrong shape")
        outs.append(t)
    dq, dk, dv = outs
    need = attn_bwd_workspace_bytes(total_q, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
    if q.numel() == 0:
        return dq, dk, dv
    with _on(dev):
        st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                            _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, mq, mk, total_q, hq, hkv,
                            d, 1 if causal else 0, float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st)
    return dq, dk, dv


def attn_decode_num_splits(max_seqlen_k, chunk_tokens):
    return lib().attn_decode_num_splits(int(max_seqlen_k), int(chunk_tokens))


def attn_decode_default_chunk(batch, num_heads_kv, max_seqlen_k, num_cus=0):
    return lib().attn_decode_default_chunk(int(batch), int(num_heads_kv), int(max_seqlen_k),
                                           int(num_cus))


def attn_decode_workspace_bytes(batch, num_heads_q, head_dim, num_splits):
    return lib().attn_decode_workspace_bytes(int(batch), int(num_heads_q), int(head_dim),
                                             int(num_splits))


def attn_decode_splitkv(q, k_cache, v_cache, block_table, seqlens_k, *, chunk_tokens, num_splits,
                        softmax_scale, out_partial=None, lse_partial=None, stream=None):
    """Split pass: q [B, Hq, d]; caches [P, 256, Hkv, d]; block_table int32 [B, maxp];
    seqlens_k int32 [B].  Returns (out_partial [n, B, Hq, d], lse_partial [n, B, Hq])."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expects q [B,Hq,d] and caches [P,page,Hkv,d]")
    batch, hq, d = q.shape
    num_pages, page, hkv, dk = k_cache.shape
    if dk != d or block_table.dim() != 2 or block_table.shape[0] != batch or seqlens_k.shape != (batch,):
        raise ValueError("inconsistent decode shapes")
    n = int(num_splits)
    if out_partial is None:
        out_partial = torch.empty((n, batch, hq, d), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((n, batch, hq), dtype=torch.float32, device=dev)
    _need(out_partial, "out_partial", torch.float32, dev)
    _need(lse_partial, "lse_partial", torch.float32, dev)
    if out_partial.numel() < n * batch * hq * d or lse_partial.numel() < n * batch * hq:
        raise ValueError("partial buffers are too small for num_splits")
    with _on(dev):
        st = lib().attn_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(seqlens_k), batch, hq, hkv, d, page,
                                       block_table.shape[1], num_pages, int(chunk_tokens), n,
                                       float(softmax_scale), _ptr(out_partial), _ptr(lse_partial),
                                       _stream(stream, dev))
    _check(st)
    return out_partial, lse_partial


def attn_decode_combine(out_partial, lse_partial, seqlens_k, *, chunk_tokens, out=None, lse=None,
                        return_lse=True, stream=None):
    """Combine pass: returns (out [B, Hq, d] bf16, lse [B, Hq] fp32)."""
    dev = out_partial.device
    _need(out_partial, "out_partial", torch.float32, dev)
    _need(lse_partial, "lse_partial", torch.float32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    n, batch, hq, d = out_partial.shape
    if tuple(lse_partial.shape) != (n, batch, hq):
        raise ValueError("lse_partial must be [num_splits, B, Hq]")
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    with _on(dev):
        st = lib().attn_decode_combine(_ptr(out_partial), _ptr(lse_partial), _ptr(seqlens_k), batch,
                                       hq, d, int(chunk_tokens), n, _ptr(out), _ptr(lse),
                                       _stream(stream, dev))
    _check(st)
    return out, lse


def attn_decode(q, k_cache, v_cache, block_table, seqlens_k, *, max_seqlen_k, softmax_scale,
                chunk_tokens=None, stream=None):
    """Split + combine in one call (two kernel launches on the same stream)."""
    if chunk_tokens is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        chunk_tokens = attn_decode_default_chunk(q.shape[0], k_cache.shape[2], max_seqlen_k, cus)
    n = max(1, attn_decode_num_splits(max_seqlen_k, chunk_tokens))
    po, pl = attn_decode_splitkv(q, k_cache, v_cache, block_table, seqlens_k,
                                 chunk_tokens=chunk_tokens, num_splits=n,
                                 softmax_scale=softmax_scale, stream=stream)
    return attn_decode_combine(po, pl, seqlens_k, chunk_tokens=chunk_tokens, stream=stream)


def attn_decode_noalloc(q, k_cache, v_cache, block_table, seqlens_k, *, max_seqlen_k, softmax_scale,
                        chunk_tokens=None, out=None, lse=None, return_lse=True, stream=None):
    """Split + combine with the partials in the library's own device array: the C call
    allocates nothing (pass `out` and `lse` to allocate nothing here either)."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expects q [B,Hq,d] and caches [P,page,Hkv,d]")
    batch, hq, d = q.shape
    num_pages, page, hkv, dk = k_cache.shape
    if dk != d or block_table.dim() != 2 or block_table.shape[0] != batch or seqlens_k.shape != (batch,):
        raise ValueError("inconsistent decode shapes")
    if chunk_tokens is None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        chunk_tokens = attn_decode_default_chunk(batch, hkv, max_seqlen_k, cus)
    n = max(1, attn_decode_num_splits(max_seqlen_k, chunk_tokens))
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    with _on(dev):
        st = lib().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(seqlens_k), batch, hq, hkv, d, page, block_table.shape[1],
                                       num_pages, int(chunk_tokens), n, float(softmax_scale), _ptr(out),
                                       _ptr(lse), _stream(stream, dev))
    _check(st)
    return out, lse


def attn_decode_kvcache(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, *, max_seqlen_k,
                        softmax_scale, rotary_cos=None, rotary_sin=None, rotary_interleaved=False,
                        chunk_tokens=None, q_rot=None, out_partial=None, lse_partial=None, out=None,
                        lse=None, return_lse=True, stream=None):
    """Append one token per request to the paged cache (in place), then decode.

    q [B, Hq, d]; k_new, v_new [B, Hkv, d] bf16; caches [P, 256, Hkv, d] bf16
    (updated); block_table int32 [B, maxp]; seqlens_k int32 [B], keys cached
    before the call (the new token goes to position seqlens_k[b]; seqlens_k is
    not changed).  max_seqlen_k bounds seqlens_k (before the append) and sizes
    the splits.  rotary_cos/rotary_sin float32 [max_pos, rotary_dim / 2] turn q
    and the new key at their position (None: no rotary).  Returns (out, lse,
    q_rot); q_rot is None without rotary.
    """
    dev = q.device
    for t, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expects q [B,Hq,d] and caches [P,page,Hkv,d]")
    batch, hq, d = q.shape
    num_pages, page, hkv, dk = k_cache.shape
    if (dk != d or tuple(k_new.shape) != (batch, hkv, d) or v_new.shape != k_new.shape
            or block_table.dim() != 2 or block_table.shape[0] != batch or seqlens_k.shape != (batch,)):
        raise ValueError("inconsistent decode shapes")
    rot = 0
    max_pos = 0
    if (rotary_cos is None) != (rotary_sin is None):
        raise ValueError("give both rotary_cos and rotary_sin, or neither")
    if rotary_cos is not None:
        _need(rotary_cos, "rotary_cos", torch.float32, dev)
        _need(rotary_sin, "rotary_sin", torch.float32, dev)
        if rotary_cos.dim() != 2 or rotary_sin.shape != rotary_cos.shape:
            raise ValueError("rotary tables must both be [max_pos, rotary_dim / 2]")
        max_pos, rot = rotary_cos.shape[0], 2 * rotary_cos.shape[1]
        if q_rot is None:
            q_rot = torch.empty_like(q)
        _need(q_rot, "q_rot", torch.bfloat16, dev)
        if q_rot.shape != q.shape:
            raise ValueError("q_rot must have q's shape")
    else:
        q_rot = None
    total = int(max_seqlen_k) + 1
    if chunk_tokens is None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        chunk_tokens = attn_decode_default_chunk(batch, hkv, total, cus)
    n = max(1, attn_decode_num_splits(total, chunk_tokens))
    if out_partial is None:
        out_partial = torch.empty((n, batch, hq, d), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((n, batch, hq), dtype=torch.float32, device=dev)
    _need(out_partial, "out_partial", torch.float32, dev)
    _need(lse_partial, "lse_partial", torch.float32, dev)
    if out_partial.numel() < n * batch * hq * d or lse_partial.numel() < n * batch * hq:
        raise ValueError("partial buffers are too small")
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    with _on(dev):
        st = lib().attn_decode_kvcache(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seqlens_k), _ptr(rotary_cos), _ptr(rotary_sin), rot, int(bool(rotary_interleaved)),
            max_pos, batch, hq, hkv, d, page, block_table.shape[1], num_pages, int(chunk_tokens), n,
            float(softmax_scale), _ptr(q_rot), _ptr(out_partial), _ptr(lse_partial), _ptr(out),
            _ptr(lse), _stream(stream, dev))
    _check(st)
    return out, lse, q_rot


def attn_fp8_num_blocks(seqlen):
    return lib().attn_fp8_num_blocks(int(seqlen))


def attn_fp8_quantize(x, *, signs=None, layout="rows", codes=None, scales=None, stream=None):
    """Block-quantise x [B, N, H, d] bf16 (d in {64, 128, 256}) to E4M3 codes
    (uint8) and float32 block scales [B, H, ceil(N / 64)].  signs: int8 [d] of
    +-1 to turn the rows first (Q and K), or None.  layout "rows": codes
    [B, N, H, d]; "vt": codes [B, H, d, Np] in the V^T layout attn_fwd_fp8
    reads."""
    dev = x.device
    _need(x, "x", torch.bfloat16, dev)
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, d]")
    B, N, H, d = x.shape
    lay = {"rows": 0, "vt": 1}[layout]
    nb = attn_fp8_num_blocks(N)
    shape = (B, N, H, d) if lay == 0 else (B, H, d, 64 * nb)
    if codes is None:
        codes = torch.empty(shape, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.float32, dev)
    if tuple(codes.shape) != shape or tuple(scales.shape) != (B, H, nb):
        raise ValueError("codes/scales have the wrong shape")
    if signs is not None:
        _need(signs, "signs", torch.int8, dev)
        if tuple(signs.shape) != (d,):
            raise ValueError("signs must be [head_dim]")
    with _on(dev):
        st = lib().attn_fp8_quantize(_ptr(x), _ptr(signs), B, N, H, d, lay, _ptr(codes), _ptr(scales),
                                     _stream(stream, dev))
    _check(st)
    return codes, scales


def attn_fwd_fp8(q_codes, k_codes, v_codes_t, q_scales, k_scales, v_scales, *, causal, softmax_scale,
                 incoherent, out=None, lse=None, return_lse=True, stream=None):
    """Attention forward on attn_fp8_quantize's codes: q [B, Nq, Hq, d] and
    k [B, Nk, Hkv, d] in the row layout, v in the V^T layout [B, Hkv, d, Np]
    (d in {64, 128, 256}).  Returns (out [B, Nq, Hq, d] bf16, lse [B, Hq, Nq])."""
    dev = q_codes.device
    for t, n in ((q_codes, "q_codes"), (k_codes, "k_codes"), (v_codes_t, "v_codes_t")):
        _need(t, n, torch.uint8, dev)
    for t, n in ((q_scales, "q_scales"), (k_scales, "k_scales"), (v_scales, "v_scales")):
        _need(t, n, torch.float32, dev)
    if q_codes.dim() != 4 or k_codes.dim() != 4 or v_codes_t.dim() != 4:
        raise ValueError("codes must be 4-d")
    B, Nq, Hq, d = q_codes.shape
    Bk, Nk, Hkv, dk = k_codes.shape
    nbq, nbk = attn_fp8_num_blocks(Nq), attn_fp8_num_blocks(Nk)
    if (Bk != B or dk != d or tuple(v_codes_t.shape) != (B, Hkv, d, 64 * nbk)
            or tuple(q_scales.shape) != (B, Hq, nbq) or tuple(k_scales.shape) != (B, Hkv, nbk)
            or tuple(v_scales.shape) != (B, Hkv, nbk)):
        raise ValueError("inconsistent FP8 operand shapes")
    if out is None:
        out = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    with _on(dev):
        st = lib().attn_fwd_fp8(_ptr(q_codes), _ptr(k_codes), _ptr(v_codes_t), _ptr(q_scales), _ptr(k_scales),
                                _ptr(v_scales), B, Nq, Nk, Hq, Hkv, d, int(bool(causal)), int(bool(incoherent)),
                                float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st)
    return out, lse


def attn_fp8_forward(q, k, v, *, causal, softmax_scale, signs=None, stream=None):
    """Quantise bf16 q, k, v ([B, N, H, d]) and run attn_fwd_fp8: Q and K turned
    by `signs` (incoherent processing) when given.  Returns (out, lse)."""
    qc, qs = attn_fp8_quantize(q, signs=signs, layout="rows", stream=stream)
    kc, ks = attn_fp8_quantize(k, signs=signs, layout="rows", stream=stream)
    vc, vs = attn_fp8_quantize(v, layout="vt", stream=stream)
    return attn_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=causal, softmax_scale=softmax_scale,
                        incoherent=signs is not None, stream=stream)


def ceiling_read(src, sink=None, stream=None):
    """Measurement helper: stream-read every byte of the GPU tensor `src`
    (contiguous, size a multiple of 16 bytes).  Returns the sink tensor."""
    dev = src.device
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(lib().attn_ceiling_read_sink_words(src.numel() * src.element_size()), dtype=torch.int32,
                           device=dev)
    with _on(dev):
        st = lib().attn_ceiling_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, lib().attn_ceiling_last_error().decode())
    return sink


def _ceiling_mfma(fn, words, operands, iters, sink, stream):
    dev = operands.device
    _need(operands, "operands", torch.int32, dev)
    waves = operands.shape[0]
    if tuple(operands.shape) != (waves, 64, words):
        raise ValueError(f"operands must be [waves, 64, {words}]")
    if sink is None:
        sink = torch.empty(waves * 64, dtype=torch.float32, device=dev)
    with _on(dev):
        st = fn(_ptr(operands), waves, int(iters), _ptr(sink), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, lib().attn_ceiling_last_error().decode())
    return sink


def ceiling_mfma_bf16(operands, iters, sink=None, stream=None):
    """Measurement helper: bf16 matrix-core loop on `operands` (int32 GPU tensor
    [waves, 64, 32] of random bf16 pairs).  Returns the sink tensor [waves * 64]."""
    return _ceiling_mfma(lib().attn_ceiling_mfma_bf16, 32, operands, iters, sink, stream)


def ceiling_mfma_fp8(operands, iters, sink=None, stream=None):
    """Measurement helper: E4M3 matrix-core loop on `operands` (int32 GPU tensor
    [waves, 64, 64] of finite E4M3 codes, four per word).  Returns the sink
    tensor [waves * 64]."""
    return _ceiling_mfma(lib().attn_ceiling_mfma_fp8, 64, operands, iters, sink, stream)


def attn_check_cu_seqlens(cu_seqlens, total, max_seqlen):
    """Host-side validator over a CPU int32 tensor; raises AttnError on bad offsets."""
    cu = cu_seqlens.to("cpu", torch.int32).contiguous()
    _check(lib().attn_check_cu_seqlens(_ptr(cu), cu.numel() - 1, int(total), int(max_seqlen)))


def attn_check_block_table(block_table, seqlens_k, num_pages, page_size=256):
    """Host-side validator over CPU copies; raises AttnError on bad page ids or lengths."""
    t = block_table.to("cpu", torch.int32).contiguous()
    s = seqlens_k.to("cpu", torch.int32).contiguous()
    _check(lib().attn_check_block_table(_ptr(t), _ptr(s), t.shape[0], t.shape[1], int(num_pages),
                                        int(page_size)))
