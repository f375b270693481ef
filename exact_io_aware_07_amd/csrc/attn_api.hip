// Host side of the C ABI declared in include/attn.h: argument validation,
// status reporting and kernel dispatch.  Nothing here allocates device
// memory or synchronises; errors are returned before any launch.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/attn.h"
#include "attn_launch.h"

#include <algorithm>
#include <mutex>

// Partials of attn_decode_noalloc: a file-scope device array, so that the
// call needs no allocation.  Each GPU the library runs on holds its own copy
// (ATTN_DECODE_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code never
// passes this name to a kernel: its device address comes from
// hipGetSymbolAddress, once per device (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

attn_status_t ok() {
    g_last_error[0] = '\0';
    return ATTN_OK;
}

bool head_dim_supported(int d) { return d == 64 || d == 128 || d == 256; }

// [a, a + na) and [b, b + nb) overlap (byte ranges; empty ranges never do).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

// True if any non-null pointer is not a multiple of `a` bytes.
template <typename... P>
bool misaligned(uintptr_t a, P... ps) {
    return ((ps != nullptr && (reinterpret_cast<uintptr_t>(ps) & (a - 1)) != 0) || ...);
}

attn_status_t fail_align() {
    return fail(ATTN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned (int32 arrays, lse, scales "
                "and rotary tables 4-byte, FP8 signs 8-byte)");
}

attn_status_t check_scale(float s) {
    if (!isfinite(s) || !(s > 0.0f)) return fail(ATTN_ERR_SCALE, "softmax_scale must be finite and > 0 (got %g)", s);
    return ATTN_OK;
}

attn_status_t hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for later calls.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

attn_status_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || addr == nullptr)
            return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = addr;
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
        case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE";
        case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
        case ATTN_ERR_DATA: return "ATTN_ERR_DATA";
        default: return "ATTN_ERR_UNKNOWN";
    }
}

const char* attn_last_error(void) { return g_last_error; }

attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, const int32_t* block_table, const int32_t* seqlens_k,
                          int batch, int max_seqlen_q, int max_seqlen_k, int num_heads_q, int num_heads_kv,
                          int head_dim, int page_size, int max_pages_per_seq, int num_pages, int causal,
                          int window_left, int window_right, float softmax_scale, void* out, float* lse,
                          void* stream) {
    if (!q || !k || !v || !out) return fail(ATTN_ERR_NULL, "q, k, v and out must be non-NULL");
    if (misaligned(16, q, k, v, out) || misaligned(4, lse, cu_seqlens_q, cu_seqlens_k, block_table, seqlens_k))
        return fail_align();
    const bool paged = block_table != nullptr;
    const bool varlen = cu_seqlens_q != nullptr;
    if (paged) {
        if (!cu_seqlens_q || cu_seqlens_k || !seqlens_k)
            return fail(ATTN_ERR_NULL, "paged mode needs cu_seqlens_q and seqlens_k, and no cu_seqlens_k");
        if (page_size != 256) return fail(ATTN_ERR_UNSUPPORTED, "page_size=%d, only 256 is supported", page_size);
        if (max_pages_per_seq < 1 || num_pages < 1)
            return fail(ATTN_ERR_SHAPE, "max_pages_per_seq=%d num_pages=%d", max_pages_per_seq, num_pages);
    } else {
        if (seqlens_k) return fail(ATTN_ERR_NULL, "seqlens_k is only for paged mode (block_table set)");
        if (varlen != (cu_seqlens_k != nullptr))
            return fail(ATTN_ERR_NULL, "cu_seqlens_q and cu_seqlens_k must both be NULL or both be set");
    }
    if (batch < 1 || max_seqlen_q < 1 || max_seqlen_k < (varlen ? 0 : 1) || num_heads_q < 1 ||
        num_heads_kv < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d max_seqlen_q=%d max_seqlen_k=%d "
                    "num_heads_q=%d num_heads_kv=%d", batch, max_seqlen_q, max_seqlen_k,
                    num_heads_q, num_heads_kv);
    if (num_heads_q % num_heads_kv)
        return fail(ATTN_ERR_SHAPE, "num_heads_kv=%d does not divide num_heads_q=%d", num_heads_kv,
                    num_heads_q);
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim=%d not in {64,128,256}", head_dim);
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_SHAPE, "causal must be 0 or 1 (got %d)", causal);
    if (window_left < -1 || window_right < -1)
        return fail(ATTN_ERR_SHAPE, "window sides must be >= -1 (got %d, %d)", window_left, window_right);
    attn_status_t st = check_scale(softmax_scale);
    if (st != ATTN_OK) return st;
    // Aliasing: byte ranges are known in dense mode; packed and paged modes
    // know only the start pointers on the host.
    if (!varlen) {
        const size_t nq = (size_t)batch * max_seqlen_q, nk = (size_t)batch * max_seqlen_k;
        const size_t qbytes = nq * num_heads_q * head_dim * 2;
        const size_t kbytes = nk * num_heads_kv * head_dim * 2;
        const size_t lbytes = (size_t)batch * num_heads_q * max_seqlen_q * 4;
        if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k, kbytes) ||
            overlap(out, qbytes, v, kbytes) || overlap(lse, lbytes, out, qbytes) ||
            overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
            overlap(lse, lbytes, v, kbytes))
            return fail(ATTN_ERR_ALIAS, "out/lse overlap an input or each other");
    } else if (out == q || out == k || out == v || (void*)lse == out || (const void*)lse == q ||
               (const void*)lse == k || (const void*)lse == v) {
        return fail(ATTN_ERR_ALIAS, "out/lse alias an input or each other");
    }
    attn::FwdParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.batch = batch;
    p.max_q = max_seqlen_q;
    p.max_k = max_seqlen_k;
    p.hq = num_heads_q;
    p.hkv = num_heads_kv;
    p.scale = softmax_scale;
    p.wl = window_left;
    p.wr = window_right;
    p.block_table = block_table;
    p.seqlens_k = seqlens_k;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    return hip_status(attn::launch_fwd(p, head_dim, causal != 0, varlen, paged, static_cast<hipStream_t>(stream)),
                      "attn_fwd launch");
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                       const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k,
                       int num_heads_q, int num_heads_kv, int head_dim, int causal,
                       float softmax_scale, void* out, float* lse, void* stream) {
    return attn_fwd_ex(q, k, v, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, batch, max_seqlen_q,
                       max_seqlen_k, num_heads_q, num_heads_kv, head_dim, 256, 0, 0, causal, -1, -1,
                       softmax_scale, out, lse, stream);
}

size_t attn_bwd_workspace_bytes(int total_q, int num_heads_q) {
    if (total_q < 1 || num_heads_q < 1) return 0;
    return (size_t)2 * total_q * num_heads_q * 4;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int num_heads_q,
                       int num_heads_kv, int head_dim, int causal, float softmax_scale, void* dq,
                       void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
        return fail(ATTN_ERR_NULL, "every tensor argument of attn_bwd must be non-NULL");
    if (misaligned(16, q, k, v, out, dout, dq, dk, dv, workspace) || misaligned(4, lse, cu_seqlens_q, cu_seqlens_k))
        return fail_align();
    const bool varlen = cu_seqlens_q != nullptr;
    if (varlen != (cu_seqlens_k != nullptr))
        return fail(ATTN_ERR_NULL, "cu_seqlens_q and cu_seqlens_k must both be NULL or both be set");
    if (batch < 1 || max_seqlen_q < 1 || max_seqlen_k < (varlen ? 0 : 1) || num_heads_q < 1 ||
        num_heads_kv < 1 || total_q < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d max_seqlen_q=%d max_seqlen_k=%d "
                    "total_q=%d num_heads_q=%d num_heads_kv=%d", batch, max_seqlen_q, max_seqlen_k,
                    total_q, num_heads_q, num_heads_kv);
    if (!varlen && (long)total_q != (long)batch * max_seqlen_q)
        return fail(ATTN_ERR_SHAPE, "dense mode needs total_q = batch * max_seqlen_q (%ld), got %d",
                    (long)batch * max_seqlen_q, total_q);
    if (num_heads_q % num_heads_kv)
        return fail(ATTN_ERR_SHAPE, "num_heads_kv=%d does not divide num_heads_q=%d", num_heads_kv,
                    num_heads_q);
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: head_dim=%d not in {64,128,256}", head_dim);
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_SHAPE, "causal must be 0 or 1 (got %d)", causal);
    attn_status_t st = check_scale(softmax_scale);
    if (st != ATTN_OK) return st;
    const size_t need = attn_bwd_workspace_bytes(total_q, num_heads_q);
    if (workspace_bytes < need)
        return fail(ATTN_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    // Outputs against inputs, the workspace and each other.  Byte ranges are
    // known from total_q; packed K/V totals are not, so K-like ranges use
    // start pointers only there.
    const size_t qbytes = (size_t)total_q * num_heads_q * head_dim * 2;
    const size_t lbytes = (size_t)total_q * num_heads_q * 4;
    const size_t kbytes = varlen ? 1 : (size_t)batch * max_seqlen_k * num_heads_kv * head_dim * 2;
    const void* ins_q[] = {q, out, dout};
    for (const void* x : ins_q)
        if (overlap(dq, qbytes, x, qbytes) || overlap(dk, kbytes, x, qbytes) || overlap(dv, kbytes, x, qbytes))
            return fail(ATTN_ERR_ALIAS, "dq/dk/dv overlap an input");
    const void* ins_k[] = {k, v};
    for (const void* x : ins_k)
        if (overlap(dq, qbytes, x, kbytes) || overlap(dk, kbytes, x, kbytes) || overlap(dv, kbytes, x, kbytes))
            return fail(ATTN_ERR_ALIAS, "dq/dk/dv overlap an input");
    if (overlap(dq, qbytes, lse, lbytes) || overlap(dk, kbytes, lse, lbytes) || overlap(dv, kbytes, lse, lbytes) ||
        overlap(dq, qbytes, workspace, need) || overlap(dk, kbytes, workspace, need) ||
        overlap(dv, kbytes, workspace, need) || overlap(dq, qbytes, dk, kbytes) ||
        overlap(dq, qbytes, dv, kbytes) || overlap(dk, kbytes, dv, kbytes) ||
        overlap(workspace, need, q, qbytes) || overlap(workspace, need, out, qbytes) ||
        overlap(workspace, need, dout, qbytes) || overlap(workspace, need, lse, lbytes))
        return fail(ATTN_ERR_ALIAS, "dq/dk/dv/workspace overlap an input or each other");
    attn::BwdParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.out = static_cast<const uint16_t*>(out);
    p.lse = lse;
    p.dout = static_cast<const uint16_t*>(dout);
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    p.lse2 = static_cast<float*>(workspace);
    p.dsum = static_cast<float*>(workspace) + (size_t)total_q * num_heads_q;
    p.batch = batch;
    p.max_q = max_seqlen_q;
    p.max_k = max_seqlen_k;
    p.total_q = total_q;
    p.hq = num_heads_q;
    p.hkv = num_heads_kv;
    p.scale = softmax_scale;
    return hip_status(attn::launch_bwd(p, head_dim, causal != 0, varlen, static_cast<hipStream_t>(stream)),
                      "attn_bwd launch");
}

attn_status_t attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seqlens_k, int batch,
                                  int num_heads_q, int num_heads_kv, int head_dim, int page_size,
                                  int max_pages_per_seq, int num_pages, int chunk_tokens,
                                  int num_splits, float softmax_scale, float* out_partial,
                                  float* lse_partial, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seqlens_k || !out_partial || !lse_partial)
        return fail(ATTN_ERR_NULL, "every pointer argument of attn_decode_splitkv must be non-NULL");
    if (misaligned(16, q, k_cache, v_cache, out_partial) || misaligned(4, block_table, seqlens_k, lse_partial))
        return fail_align();
    if (batch < 1 || num_heads_q < 1 || num_heads_kv < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
        num_splits < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d num_heads_q=%d num_heads_kv=%d "
                    "max_pages_per_seq=%d num_pages=%d num_splits=%d", batch, num_heads_q,
                    num_heads_kv, max_pages_per_seq, num_pages, num_splits);
    if (num_heads_q % num_heads_kv)
        return fail(ATTN_ERR_SHAPE, "num_heads_kv=%d does not divide num_heads_q=%d", num_heads_kv,
                    num_heads_q);
    if (num_heads_q / num_heads_kv > 64)
        return fail(ATTN_ERR_UNSUPPORTED, "more than 64 query heads per K/V head");
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim=%d not in {64,128,256}", head_dim);
    if (page_size != 256) return fail(ATTN_ERR_UNSUPPORTED, "page_size must be 256 (got %d)", page_size);
    if (chunk_tokens < page_size || chunk_tokens % page_size)
        return fail(ATTN_ERR_UNSUPPORTED, "chunk_tokens=%d is not a positive multiple of page_size",
                    chunk_tokens);
    attn_status_t st = check_scale(softmax_scale);
    if (st != ATTN_OK) return st;
    const size_t obytes = (size_t)num_splits * batch * num_heads_q * head_dim * 4;
    const size_t lbytes = (size_t)num_splits * batch * num_heads_q * 4;
    if (overlap(out_partial, obytes, lse_partial, lbytes))
        return fail(ATTN_ERR_ALIAS, "out_partial and lse_partial overlap");
    attn::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k_cache = static_cast<const uint16_t*>(k_cache);
    p.v_cache = static_cast<const uint16_t*>(v_cache);
    p.block_table = block_table;
    p.seqlens = seqlens_k;
    p.out_part = out_partial;
    p.lse_part = lse_partial;
    p.batch = batch;
    p.hq = num_heads_q;
    p.hkv = num_heads_kv;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    p.chunk = chunk_tokens;
    p.n_splits = num_splits;
    p.scale = softmax_scale;
    return hip_status(attn::launch_decode_split(p, head_dim, static_cast<hipStream_t>(stream)),
                      "attn_decode_splitkv launch");
}

attn_status_t attn_decode_combine(const float* out_partial, const float* lse_partial,
                                  const int32_t* seqlens_k, int batch, int num_heads_q,
                                  int head_dim, int chunk_tokens, int num_splits, void* out,
                                  float* lse, void* stream) {
    if (!out_partial || !lse_partial || !seqlens_k || !out)
        return fail(ATTN_ERR_NULL, "out_partial, lse_partial, seqlens_k and out must be non-NULL");
    if (misaligned(16, out_partial, out) || misaligned(4, lse_partial, seqlens_k, lse)) return fail_align();
    if (batch < 1 || num_heads_q < 1 || num_splits < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d num_heads_q=%d num_splits=%d",
                    batch, num_heads_q, num_splits);
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim=%d not in {64,128,256}", head_dim);
    if (chunk_tokens < 256 || chunk_tokens % 256)
        return fail(ATTN_ERR_UNSUPPORTED, "chunk_tokens=%d is not a positive multiple of 256",
                    chunk_tokens);
    const size_t obytes = (size_t)batch * num_heads_q * head_dim * 2;
    const size_t lbytes = (size_t)batch * num_heads_q * 4;
    const size_t pobytes = (size_t)num_splits * batch * num_heads_q * head_dim * 4;
    const size_t plbytes = (size_t)num_splits * batch * num_heads_q * 4;
    if (overlap(out, obytes, out_partial, pobytes) || overlap(out, obytes, lse_partial, plbytes) ||
        overlap(lse, lbytes, out, obytes) || overlap(lse, lbytes, out_partial, pobytes) ||
        overlap(lse, lbytes, lse_partial, plbytes))
        return fail(ATTN_ERR_ALIAS, "out/lse overlap the partials or each other");
    attn::CombineParams p{};
    p.out_part = out_partial;
    p.lse_part = lse_partial;
    p.seqlens = seqlens_k;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.batch = batch;
    p.hq = num_heads_q;
    p.chunk = chunk_tokens;
    p.n_splits = num_splits;
    return hip_status(attn::launch_decode_combine(p, head_dim, static_cast<hipStream_t>(stream)),
                      "attn_decode_combine launch");
}

attn_status_t attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seqlens_k, int batch,
                                  int num_heads_q, int num_heads_kv, int head_dim, int page_size,
                                  int max_pages_per_seq, int num_pages, int chunk_tokens,
                                  int num_splits, float softmax_scale, void* out, float* lse,
                                  void* stream) {
    // Host-only checks first (no HIP call before the sizes are known to fit).
    if (!out) return fail(ATTN_ERR_NULL, "out must be non-NULL");
    if (misaligned(16, out) || misaligned(4, lse)) return fail_align();
    if (batch < 1 || num_heads_q < 1 || num_splits < 1 || !head_dim_supported(head_dim))
        return fail(batch < 1 || num_heads_q < 1 || num_splits < 1 ? ATTN_ERR_SHAPE : ATTN_ERR_UNSUPPORTED,
                    "batch=%d num_heads_q=%d num_splits=%d head_dim=%d", batch, num_heads_q, num_splits,
                    head_dim);
    const size_t obytes = (size_t)num_splits * batch * num_heads_q * head_dim * 4;
    const size_t need = attn_decode_workspace_bytes(batch, num_heads_q, head_dim, num_splits);
    if (need > (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_SHAPE, "partials need %zu bytes, more than the %zu-byte scratch of "
                    "attn_decode_noalloc (use attn_decode_splitkv with a workspace)", need,
                    (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES);
    void* base = nullptr;
    attn_status_t st = scratch_on_current_device(&base);
    if (st != ATTN_OK) return st;
    float* out_partial = static_cast<float*>(base);
    float* lse_partial = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + obytes);
    // The split validates every remaining argument before it launches; the
    // combine's checks are covered by those above, so only its launch can fail.
    st = attn_decode_splitkv(q, k_cache, v_cache, block_table, seqlens_k, batch, num_heads_q,
                             num_heads_kv, head_dim, page_size, max_pages_per_seq, num_pages,
                             chunk_tokens, num_splits, softmax_scale, out_partial, lse_partial, stream);
    if (st != ATTN_OK) return st;
    return attn_decode_combine(out_partial, lse_partial, seqlens_k, batch, num_heads_q, head_dim,
                               chunk_tokens, num_splits, out, lse, stream);
}

attn_status_t attn_decode_kvcache(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const int32_t* block_table, const int32_t* seqlens_k,
                                  const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                                  int rotary_interleaved, int rotary_max_pos, int batch,
                                  int num_heads_q, int num_heads_kv, int head_dim, int page_size,
                                  int max_pages_per_seq, int num_pages, int chunk_tokens,
                                  int num_splits, float softmax_scale, void* q_rot,
                                  float* out_partial, float* lse_partial, void* out, float* lse,
                                  void* stream) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !seqlens_k || !out_partial ||
        !lse_partial || !out)
        return fail(ATTN_ERR_NULL, "q, k_new, v_new, the caches, block_table, seqlens_k, the partials "
                    "and out must be non-NULL");
    if (rotary_dim != 0 && (!rotary_cos || !rotary_sin || !q_rot))
        return fail(ATTN_ERR_NULL, "rotary_dim > 0 needs rotary_cos, rotary_sin and q_rot");
    if (misaligned(16, q, k_new, v_new, k_cache, v_cache, q_rot, out_partial, out) ||
        misaligned(4, block_table, seqlens_k, rotary_cos, rotary_sin, lse_partial, lse))
        return fail_align();
    if (batch < 1 || num_heads_q < 1 || num_heads_kv < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
        num_splits < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d num_heads_q=%d num_heads_kv=%d "
                    "max_pages_per_seq=%d num_pages=%d num_splits=%d", batch, num_heads_q,
                    num_heads_kv, max_pages_per_seq, num_pages, num_splits);
    if (num_heads_q % num_heads_kv)
        return fail(ATTN_ERR_SHAPE, "num_heads_kv=%d does not divide num_heads_q=%d", num_heads_kv,
                    num_heads_q);
    if (num_heads_q / num_heads_kv > 64)
        return fail(ATTN_ERR_UNSUPPORTED, "more than 64 query heads per K/V head");
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim=%d not in {64,128,256}", head_dim);
    if (page_size != 256) return fail(ATTN_ERR_UNSUPPORTED, "page_size must be 256 (got %d)", page_size);
    if (chunk_tokens < page_size || chunk_tokens % page_size)
        return fail(ATTN_ERR_UNSUPPORTED, "chunk_tokens=%d is not a positive multiple of page_size",
                    chunk_tokens);
    if (rotary_dim < 0 || rotary_dim % 2 || rotary_dim > head_dim)
        return fail(ATTN_ERR_SHAPE, "rotary_dim=%d must be even and in [0, head_dim=%d]", rotary_dim,
                    head_dim);
    if (rotary_dim > 0 && rotary_max_pos < 1)
        return fail(ATTN_ERR_SHAPE, "rotary_max_pos=%d must be >= 1", rotary_max_pos);
    if (rotary_interleaved != 0 && rotary_interleaved != 1)
        return fail(ATTN_ERR_SHAPE, "rotary_interleaved must be 0 or 1");
    attn_status_t st = check_scale(softmax_scale);
    if (st != ATTN_OK) return st;

    // Every written region must be disjoint from every other region.
    const size_t qb = (size_t)batch * num_heads_q * head_dim * 2;
    const size_t kb = (size_t)batch * num_heads_kv * head_dim * 2;
    const size_t cb = (size_t)num_pages * page_size * num_heads_kv * head_dim * 2;
    const size_t tb = (size_t)rotary_max_pos * (size_t)(rotary_dim / 2) * 4;
    struct Region { const void* p; size_t n; bool written; };
    const Region reg[] = {
        {q, qb, false}, {k_new, kb, false}, {v_new, kb, false},
        {block_table, (size_t)batch * max_pages_per_seq * 4, false}, {seqlens_k, (size_t)batch * 4, false},
        {rotary_dim ? rotary_cos : nullptr, tb, false}, {rotary_dim ? rotary_sin : nullptr, tb, false},
        {k_cache, cb, true}, {v_cache, cb, true}, {rotary_dim ? q_rot : nullptr, qb, true},
        {out_partial, (size_t)num_splits * batch * num_heads_q * head_dim * 4, true},
        {lse_partial, (size_t)num_splits * batch * num_heads_q * 4, true},
        {out, qb, true}, {lse, (size_t)batch * num_heads_q * 4, true},
    };
    const int nreg = (int)(sizeof(reg) / sizeof(reg[0]));
    for (int i = 0; i < nreg; ++i)
        for (int j = i + 1; j < nreg; ++j)
            if ((reg[i].written || reg[j].written) && overlap(reg[i].p, reg[i].n, reg[j].p, reg[j].n))
                return fail(ATTN_ERR_ALIAS, "argument regions %d and %d overlap (a written region must "
                            "not overlap any other argument)", i, j);

    const hipStream_t s = static_cast<hipStream_t>(stream);
    attn::AppendParams a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.block_table = block_table;
    a.seqlens = seqlens_k;
    a.rot_cos = rotary_cos;
    a.rot_sin = rotary_sin;
    a.q_rot = static_cast<uint16_t*>(q_rot);
    a.batch = batch;
    a.hq = num_heads_q;
    a.hkv = num_heads_kv;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    a.rot_dim = rotary_dim;
    a.interleaved = rotary_interleaved;
    a.max_pos = rotary_max_pos;
    st = hip_status(attn::launch_decode_append(a, head_dim, s), "attn_decode_kvcache append launch");
    if (st != ATTN_OK) return st;

    attn::DecodeParams p{};
    p.q = rotary_dim ? static_cast<const uint16_t*>(q_rot) : static_cast<const uint16_t*>(q);
    p.k_cache = static_cast<const uint16_t*>(k_cache);
    p.v_cache = static_cast<const uint16_t*>(v_cache);
    p.block_table = block_table;
    p.seqlens = seqlens_k;
    p.out_part = out_partial;
    p.lse_part = lse_partial;
    p.batch = batch;
    p.hq = num_heads_q;
    p.hkv = num_heads_kv;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    p.chunk = chunk_tokens;
    p.n_splits = num_splits;
    p.scale = softmax_scale;
    p.len_add = 1;
    p.len_limit = rotary_dim ? rotary_max_pos : 0;
    st = hip_status(attn::launch_decode_split(p, head_dim, s), "attn_decode_kvcache split launch");
    if (st != ATTN_OK) return st;

    attn::CombineParams c{};
    c.out_part = out_partial;
    c.lse_part = lse_partial;
    c.seqlens = seqlens_k;
    c.out = static_cast<uint16_t*>(out);
    c.lse = lse;
    c.batch = batch;
    c.hq = num_heads_q;
    c.chunk = chunk_tokens;
    c.n_splits = num_splits;
    c.len_add = 1;
    return hip_status(attn::launch_decode_combine(c, head_dim, s), "attn_decode_kvcache combine launch");
}

int attn_fp8_num_blocks(int seqlen) {
    if (seqlen <= 0) return 0;
    return (int)(((long)seqlen + 63) / 64);
}

size_t attn_fp8_codes_bytes(int batch, int seqlen, int num_heads, int head_dim, int layout) {
    if (batch < 1 || seqlen < 1 || num_heads < 1 || head_dim < 1 || (layout != 0 && layout != 1)) return 0;
    const size_t n = layout == 0 ? (size_t)seqlen : (size_t)attn_fp8_num_blocks(seqlen) * 64;
    return (size_t)batch * n * num_heads * head_dim;
}

attn_status_t attn_fp8_quantize(const void* x, const int8_t* signs, int batch, int seqlen, int num_heads,
                                int head_dim, int layout, void* codes, float* scales, void* stream) {
    if (!x || !codes || !scales) return fail(ATTN_ERR_NULL, "x, codes and scales must be non-NULL");
    if (misaligned(16, x, codes) || misaligned(8, signs) || misaligned(4, scales)) return fail_align();
    if (batch < 1 || seqlen < 1 || num_heads < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d seqlen=%d num_heads=%d", batch, seqlen,
                    num_heads);
    if (layout != 0 && layout != 1) return fail(ATTN_ERR_SHAPE, "layout must be 0 (rows) or 1 (V^T)");
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "FP8 path: head_dim=%d not in {64,128,256}", head_dim);
    const size_t xb = (size_t)batch * seqlen * num_heads * head_dim * 2;
    const size_t cb = attn_fp8_codes_bytes(batch, seqlen, num_heads, head_dim, layout);
    const size_t sb = (size_t)batch * num_heads * attn_fp8_num_blocks(seqlen) * 4;
    if (overlap(codes, cb, x, xb) || overlap(codes, cb, signs, (size_t)head_dim) || overlap(scales, sb, x, xb) ||
        overlap(scales, sb, signs, (size_t)head_dim) || overlap(codes, cb, scales, sb))
        return fail(ATTN_ERR_ALIAS, "codes/scales overlap an input or each other");
    attn::Fp8QuantParams p{};
    p.x = static_cast<const uint16_t*>(x);
    p.signs = signs;
    p.codes = static_cast<uint8_t*>(codes);
    p.scales = scales;
    p.batch = batch;
    p.n = seqlen;
    p.heads = num_heads;
    return hip_status(attn::launch_fp8_quant(p, head_dim, layout == 1, static_cast<hipStream_t>(stream)),
                      "attn_fp8_quantize launch");
}

attn_status_t attn_fwd_fp8(const void* q_codes, const void* k_codes, const void* v_codes_t,
                           const float* q_scales, const float* k_scales, const float* v_scales, int batch,
                           int seqlen_q, int seqlen_k, int num_heads_q, int num_heads_kv, int head_dim,
                           int causal, int incoherent, float softmax_scale, void* out, float* lse,
                           void* stream) {
    if (!q_codes || !k_codes || !v_codes_t || !q_scales || !k_scales || !v_scales || !out)
        return fail(ATTN_ERR_NULL, "codes, scales and out must be non-NULL");
    if (misaligned(16, q_codes, k_codes, v_codes_t, out) || misaligned(4, q_scales, k_scales, v_scales, lse))
        return fail_align();
    if (batch < 1 || seqlen_q < 1 || seqlen_k < 1 || num_heads_q < 1 || num_heads_kv < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range: batch=%d seqlen_q=%d seqlen_k=%d num_heads_q=%d "
                    "num_heads_kv=%d", batch, seqlen_q, seqlen_k, num_heads_q, num_heads_kv);
    if (num_heads_q % num_heads_kv)
        return fail(ATTN_ERR_SHAPE, "num_heads_kv=%d does not divide num_heads_q=%d", num_heads_kv,
                    num_heads_q);
    if ((causal != 0 && causal != 1) || (incoherent != 0 && incoherent != 1))
        return fail(ATTN_ERR_SHAPE, "causal and incoherent must be 0 or 1");
    if (!head_dim_supported(head_dim))
        return fail(ATTN_ERR_UNSUPPORTED, "FP8 path: head_dim=%d not in {64,128,256}", head_dim);
    attn_status_t st = check_scale(softmax_scale);
    if (st != ATTN_OK) return st;
    const size_t ob = (size_t)batch * seqlen_q * num_heads_q * head_dim * 2;
    const size_t lb = (size_t)batch * num_heads_q * seqlen_q * 4;
    const size_t qb = attn_fp8_codes_bytes(batch, seqlen_q, num_heads_q, head_dim, 0);
    const size_t kb = attn_fp8_codes_bytes(batch, seqlen_k, num_heads_kv, head_dim, 0);
    const size_t vb = attn_fp8_codes_bytes(batch, seqlen_k, num_heads_kv, head_dim, 1);
    const size_t qsb = (size_t)batch * num_heads_q * attn_fp8_num_blocks(seqlen_q) * 4;
    const size_t ksb = (size_t)batch * num_heads_kv * attn_fp8_num_blocks(seqlen_k) * 4;
    const void* ins[6] = {q_codes, k_codes, v_codes_t, q_scales, k_scales, v_scales};
    const size_t inb[6] = {qb, kb, vb, qsb, ksb, ksb};
    for (int i = 0; i < 6; ++i)
        if (overlap(out, ob, ins[i], inb[i]) || overlap(lse, lb, ins[i], inb[i]))
            return fail(ATTN_ERR_ALIAS, "out/lse overlap an input");
    if (overlap(out, ob, lse, lb)) return fail(ATTN_ERR_ALIAS, "out and lse overlap");
    if ((long)head_dim * attn_fp8_num_blocks(seqlen_k) * 64 > 0xffffffffL)
        return fail(ATTN_ERR_UNSUPPORTED, "seqlen_k too large for 32-bit tile offsets");
    attn::Fp8FwdParams p{};
    p.q = static_cast<const uint8_t*>(q_codes);
    p.k = static_cast<const uint8_t*>(k_codes);
    p.vt = static_cast<const uint8_t*>(v_codes_t);
    p.q_scale = q_scales;
    p.k_scale = k_scales;
    p.v_scale = v_scales;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.batch = batch;
    p.nq = seqlen_q;
    p.nk = seqlen_k;
    p.hq = num_heads_q;
    p.hkv = num_heads_kv;
    p.np = attn_fp8_num_blocks(seqlen_k) * 64;
    p.nbq = attn_fp8_num_blocks(seqlen_q);
    p.nbk = attn_fp8_num_blocks(seqlen_k);
    p.scale = incoherent ? softmax_scale / (float)head_dim : softmax_scale;
    return hip_status(attn::launch_fwd_fp8(p, head_dim, causal != 0, static_cast<hipStream_t>(stream)),
                      "attn_fwd_fp8 launch");
}

int attn_decode_num_splits(int max_seqlen_k, int chunk_tokens) {
    if (max_seqlen_k <= 0 || chunk_tokens <= 0) return 0;
    return (int)(((long)max_seqlen_k + chunk_tokens - 1) / chunk_tokens);
}

int attn_decode_default_chunk(int batch, int num_heads_kv, int max_seqlen_k, int num_cus) {
    if (num_cus <= 0) num_cus = 256;
    if (batch < 1) batch = 1;
    if (num_heads_kv < 1) num_heads_kv = 1;
    if (max_seqlen_k < 1) return 256;
    // One split wave per (K/V head, chunk, request).  Aim for about 32 of them
    // per compute unit over the longest request, then lengthen chunks shorter
    // than eight pages as far as still leaves 8 waves per compute unit: with
    // the non-temporal K/V stream, longer chunks read faster and shrink the
    // combine (measured with 64 requests on 256 compute units: 2048-token
    // chunks beat 1024 by 2% on 4K-32K mixed caches and by 6% on uniform 8K
    // caches; 512 was slowest everywhere), while small batches keep short
    // chunks, which they need to fill the GPU.
    const long units = (long)batch * num_heads_kv;
    auto round_page = [](long c) { return ((c + 255) / 256) * 256; };
    const long splits = std::max(1L, (32L * num_cus + units - 1) / units);
    long chunk = round_page(((long)max_seqlen_k + splits - 1) / splits);
    const long splits_min = std::max(1L, (8L * num_cus + units - 1) / units);
    const long chunk_cap = round_page(((long)max_seqlen_k + splits_min - 1) / splits_min);
    chunk = std::max(chunk, std::min(2048L, chunk_cap));
    if (chunk < 256) chunk = 256;
    if (chunk > 16384) chunk = 16384;
    return (int)chunk;
}

size_t attn_decode_workspace_bytes(int batch, int num_heads_q, int head_dim, int num_splits) {
    if (batch < 1 || num_heads_q < 1 || head_dim < 1 || num_splits < 1) return 0;
    return (size_t)num_splits * batch * num_heads_q * ((size_t)head_dim + 1) * 4;
}

attn_status_t attn_check_cu_seqlens(const int32_t* cu, int batch, int total, int max_seqlen) {
    if (!cu) return fail(ATTN_ERR_NULL, "cu_seqlens is NULL");
    if (batch < 1 || total < 0) return fail(ATTN_ERR_SHAPE, "batch=%d total=%d", batch, total);
    if (cu[0] != 0) return fail(ATTN_ERR_DATA, "cu_seqlens[0]=%d, expected 0", cu[0]);
    for (int b = 0; b < batch; ++b) {
        const long len = (long)cu[b + 1] - cu[b];
        if (len < 0) return fail(ATTN_ERR_DATA, "cu_seqlens decreases at %d", b + 1);
        if (len > max_seqlen)
            return fail(ATTN_ERR_DATA, "sequence %d has length %ld > max_seqlen %d", b, len, max_seqlen);
    }
    if (cu[batch] != total)
        return fail(ATTN_ERR_DATA, "cu_seqlens[%d]=%d, expected the packed total %d", batch, cu[batch], total);
    return ok();
}

attn_status_t attn_check_block_table(const int32_t* table, const int32_t* seqlens, int batch,
                                     int max_pages_per_seq, int num_pages, int page_size) {
    if (!table || !seqlens) return fail(ATTN_ERR_NULL, "block_table and seqlens must be non-NULL");
    if (batch < 1 || max_pages_per_seq < 1 || num_pages < 1 || page_size < 1)
        return fail(ATTN_ERR_SHAPE, "counts out of range");
    for (int b = 0; b < batch; ++b) {
        const long n = seqlens[b];
        if (n < 0 || n > (long)max_pages_per_seq * page_size)
            return fail(ATTN_ERR_DATA, "seqlens[%d]=%ld outside [0, %ld]", b, n,
                        (long)max_pages_per_seq * page_size);
        const long used = (n + page_size - 1) / page_size;
        for (long i = 0; i < used; ++i) {
            const int id = table[(long)b * max_pages_per_seq + i];
            if (id < 0 || id >= num_pages)
                return fail(ATTN_ERR_DATA, "block_table[%d][%ld]=%d outside [0, %d)", b, i, id, num_pages);
        }
    }
    return ok();
}

}  // extern "C"
