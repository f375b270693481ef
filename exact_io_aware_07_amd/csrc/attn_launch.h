// Kernel parameter blocks and launchers (internal to libattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_udiv.h"

namespace attn {

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* cu_q;  // null in dense mode
    const int32_t* cu_k;
    uint16_t* out;
    float* lse;  // may be null
    int batch, max_q, max_k, hq, hkv;
    int n_qtiles;  // filled in by the launcher
    float scale;
    int wl = -1, wr = -1;  // local window (left, right); -1: unbounded side
    // Paged prefill: k and v are [num_pages, 256, hkv, d] caches.
    const int32_t* block_table = nullptr;
    const int32_t* seqlens_k = nullptr;
    int max_pages = 0, num_pages = 0;
    // Divisors of the work-item mapping, filled in by the launcher: query
    // heads per XCD (dense: (sequence, head) pairs per XCD), heads (dense:
    // sequences x heads), query heads, sequences, query heads per K/V head,
    // and the work items of a four-head group on one XCD (4 x query tiles).
    UDiv dv_hpx, dv_bh, dv_hq, dv_batch, dv_grp, dv_gt;
};

struct DecodeParams {
    const uint16_t* q;
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* seqlens;
    float* out_part;
    float* lse_part;
    int batch, hq, hkv, max_pages, num_pages, chunk, n_splits;
    float scale;
    int len_add = 0;    // keys appended just before this launch: request b attends over seqlens[b] + len_add
    int len_limit = 0;  // > 0: a request attending over more keys than this is invalid (NaN)
};

// In-place append of one new token per request, with optional rotary turns.
struct AppendParams {
    const uint16_t* q;      // [batch, hq, d]
    const uint16_t* k_new;  // [batch, hkv, d]
    const uint16_t* v_new;
    uint16_t* k_cache;      // [num_pages, 256, hkv, d]
    uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* seqlens;  // position of the new token = keys cached before the call
    const float* rot_cos;    // [max_pos, rot_dim / 2]; unused when rot_dim == 0
    const float* rot_sin;
    uint16_t* q_rot;         // [batch, hq, d]; written when rot_dim > 0
    int batch, hq, hkv, max_pages, num_pages;
    int rot_dim, interleaved, max_pos;
};

struct CombineParams {
    const float* out_part;
    const float* lse_part;
    const int32_t* seqlens;
    uint16_t* out;
    float* lse;  // may be null
    int batch, hq, chunk, n_splits;
    int len_add = 0;  // as in DecodeParams
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const float* lse;
    const uint16_t* dout;
    const int32_t* cu_q;  // null in dense mode
    const int32_t* cu_k;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* lse2;  // workspace [hq][total_q]: lse * log2(e), +inf for rows with no key
    float* dsum;  // workspace [hq][total_q]: rowsum(dout * out)
    int batch, max_q, max_k, total_q, hq, hkv;
    int n_tiles;  // filled in by the launchers (query tiles or key tiles)
    float scale;
    // Divisors of each kernel's work-item mapping, filled in by the launcher:
    // (sequences x heads) and heads of the grid (K/V heads for dK/dV, query
    // heads for dQ), query heads per K/V head (grp), and the work items of a
    // four-head group on one XCD (4 x n_tiles).
    UDiv dv_bh, dv_h, dv_grp, dv_gt;
    int grp = 1;
};

// FP8 block quantisation of a bf16 [batch, n, heads, 128] tensor.
struct Fp8QuantParams {
    const uint16_t* x;
    const int8_t* signs;  // +-1 per feature: turn by H(s * x) first; null: no turn
    uint8_t* codes;       // row layout [batch, n, heads, d] or V^T layout [batch, heads, d, np]
    float* scales;        // [batch, heads, ceil(n / 64)]
    int batch, n, heads;
};

// FP8 attention forward (dense, head_dim d in {64, 128, 256}).
struct Fp8FwdParams {
    const uint8_t* q;   // [batch, nq, hq, d]
    const uint8_t* k;   // [batch, nk, hkv, d]
    const uint8_t* vt;  // [batch, hkv, d, np]
    const float* q_scale;  // [batch, hq, nbq]
    const float* k_scale;  // [batch, hkv, nbk]
    const float* v_scale;  // [batch, hkv, nbk]
    uint16_t* out;      // [batch, nq, hq, d] bf16
    float* lse;         // [batch, hq, nq] or null
    int batch, nq, nk, hq, hkv;
    int n_qtiles;       // filled in by the launcher
    int np, nbq, nbk;
    float scale;        // softmax scale on the scores of the (turned) operands
    // Divisors of the work-item mapping, filled in by the launcher (see
    // FwdParams): (sequence, head) pairs per XCD, sequences x heads, query
    // heads, query heads per K/V head.
    UDiv dv_hpx, dv_bh, dv_hq, dv_grp;
};

hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, bool varlen, bool paged, hipStream_t s);
hipError_t launch_fp8_quant(const Fp8QuantParams& p, int head_dim, bool vt, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int head_dim, bool causal, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, bool varlen, hipStream_t s);
hipError_t launch_decode_split(const DecodeParams& p, int head_dim, hipStream_t s);
hipError_t launch_decode_combine(const CombineParams& p, int head_dim, hipStream_t s);
hipError_t launch_decode_append(const AppendParams& p, int head_dim, hipStream_t s);

}  // namespace attn
