/*
 * Exact attention forward pass and split-KV paged decode for AMD MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every tensor argument is a device pointer to memory
 * the caller allocated; the library never allocates, frees or synchronises.
 * Every call only validates its arguments on the host and then enqueues
 * kernels on `stream` (a hipStream_t; NULL means the null stream), so it
 * returns before the work is done.  Calls are stateless and may be made from
 * several host threads at once.  No call aborts or throws: failures are
 * reported through attn_status_t, and attn_last_error() gives the calling
 * thread's message for its last failing call.
 *
 * Element types: bf16 tensors are IEEE bfloat16 stored as 16-bit words;
 * lse and the decode partials are IEEE float32.  All tensors are dense and
 * row-major in the layouts documented below (no strides are accepted).
 * Alignment: bf16, float32 partial and FP8 code tensors (and workspaces) are
 * read and written with 16-byte vector accesses and must start on a 16-byte
 * boundary; int32 arrays, lse, scales and rotary tables on a 4-byte one, the
 * FP8 signs on an 8-byte one (allocations from the HIP allocator or PyTorch
 * are).  A misaligned pointer gives ATTN_ERR_UNSUPPORTED.
 *
 * What is computed (the definition the results are checked against):
 *   for each sequence and query head h, with K/V head kvh = h / (Hq / Hkv),
 *     S = softmax_scale * Q K^T, entries outside the allowed set set to -inf,
 *     out = softmax(S) V row by row, lse = log(sum_j exp(S_ij)) (natural log).
 *   The causal mask is bottom-right aligned: query row i of a sequence with
 *   Nq queries and Nk keys may see key j exactly when j <= i + Nk - Nq.
 *   A row with no allowed key gets out = 0 and lse = -inf.
 * Sources ("Deep Dive - FlashAttention": "Exact attention without an n x n
 * workspace", "The public interface is several kernels", "Causal 2.1 is the
 * decode gotcha", "Paged KV is a lookup, not a cache manager";
 * "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)":
 * "Decode-Time Kernels: Flash-Decoding, GQA and MLA").
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                               */
    ATTN_ERR_SHAPE = 2,       /* a count or length is out of range, or Hq % Hkv != 0      */
    ATTN_ERR_UNSUPPORTED = 3, /* head_dim, page size, chunk or pointer alignment not supported */
    ATTN_ERR_SCALE = 4,       /* softmax_scale is not finite or not > 0                    */
    ATTN_ERR_ALIAS = 5,       /* an output overlaps an input or the other output           */
    ATTN_ERR_HIP = 6,         /* the HIP runtime refused a launch (see attn_last_error)    */
    ATTN_ERR_DATA = 7         /* a host-side validator found invalid offsets or page ids   */
} attn_status_t;

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

/* Static name of a status code; never NULL. */
const char* attn_status_str(int status);

/* Message of the calling thread's last failing call ("" if none); valid
 * until that thread's next call into the library. */
const char* attn_last_error(void);

/*
 * attn_fwd -- prefill / chunked-prefill forward pass with online softmax.
 *
 * Each workgroup owns one tile of query rows of one (sequence, query head)
 * and streams the key/value tiles past it, keeping the running row maximum,
 * running sum and output accumulator on chip; no score matrix reaches memory
 * ("Deep Dive - FlashAttention", "Exact attention without an n x n
 * workspace"; "Flash Attention: A Complete Architectural Autopsy", "The
 * Online Softmax Recurrence").  Tiles wholly above the causal boundary are
 * skipped ("FlashAttention: Part 1", section 3.5).
 *
 * Dense mode (cu_seqlens_q == cu_seqlens_k == NULL):
 *   q   [batch, max_seqlen_q, num_heads_q,  head_dim] bf16
 *   k,v [batch, max_seqlen_k, num_heads_kv, head_dim] bf16
 *   out [batch, max_seqlen_q, num_heads_q,  head_dim] bf16
 *   lse [batch, num_heads_q, max_seqlen_q] float32, or NULL if not wanted
 *   Every sequence has exactly max_seqlen_q queries and max_seqlen_k keys.
 * Packed variable-length mode (both cu_seqlens non-NULL):
 *   cu_seqlens_q, cu_seqlens_k: int32 device arrays of batch + 1 entries,
 *     starting at 0, nondecreasing, ending at the packed totals TQ and TK;
 *     sequence s owns rows [cu[s], cu[s+1]) ("Deep Dive - FlashAttention",
 *     "Paged KV is a lookup, not a cache manager").  The same pointer may be
 *     given twice.  max_seqlen_q / max_seqlen_k must be >= every length.
 *   q   [TQ, num_heads_q,  head_dim] bf16,  k,v [TK, num_heads_kv, head_dim] bf16
 *   out [TQ, num_heads_q,  head_dim] bf16,  lse [num_heads_q, TQ] float32 or NULL
 *   The offsets are read on the device and are not validated there: offsets
 *   that break the rules above are undefined behaviour (attn_check_cu_seqlens
 *   checks a host copy).
 * causal: 0 = no mask, 1 = bottom-right aligned causal mask (per sequence).
 * Requirements: batch >= 1, max_seqlen_q >= 1, max_seqlen_k >= 0 (dense:
 *   >= 1), num_heads_kv >= 1 dividing num_heads_q, head_dim in {64,128,256},
 *   softmax_scale finite and > 0, out distinct from q/k/v and not overlapping
 *   lse.  Errors are returned before anything is enqueued.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int batch, int max_seqlen_q, int max_seqlen_k,
                       int num_heads_q, int num_heads_kv, int head_dim,
                       int causal, float softmax_scale,
                       void* out, float* lse, void* stream);

/*
 * attn_fwd_ex -- attn_fwd with a local window and an optional paged K/V cache.
 *
 * Local window ("Deep Dive - FlashAttention", "Causal 2.1 is the decode
 * gotcha"): query row i of a sequence with Nq queries and Nk keys sees key j
 * when i + Nk - Nq - window_left <= j <= i + Nk - Nq + window_right; a side
 * of -1 is unbounded, and causal = 1 further restricts the right side to
 * j <= i + Nk - Nq.  window_left = window_right = -1 is attn_fwd.  Rows that
 * see no key get out = 0 and lse = -inf.  Key tiles outside every row's
 * window are not read.
 *
 * Paged prefill (block_table non-NULL): new query rows against a paged cache
 * that already holds their keys ("Deep Dive - FlashAttention", "Paged KV is
 * a lookup, not a cache manager"; "FlashAttention-3 and PagedAttention:
 * IO-Aware Attention Kernels (2026)", "Block tables and what the kernel
 * does").  k, v are k_cache, v_cache [num_pages, page_size, num_heads_kv,
 * head_dim] bf16; block_table int32 [batch, max_pages_per_seq]; seqlens_k
 * int32 [batch] device array of cached keys per sequence (the last Nq of
 * which belong to the sequence's new rows, so masks align bottom-right);
 * queries are packed: cu_seqlens_q required, cu_seqlens_k must be NULL; out
 * [TQ, Hq, d], lse [Hq, TQ].  page_size must be 256.  A page id outside
 * [0, num_pages) in a tile a workgroup reads, or a length beyond
 * max_pages_per_seq * page_size, turns that workgroup's rows into NaN (never
 * a fault); cache rows past seqlens_k are never used.
 * Without block_table, seqlens_k must be NULL and the other arguments are as
 * in attn_fwd (page_size, max_pages_per_seq and num_pages are ignored).
 * window_left, window_right >= -1, else ATTN_ERR_SHAPE.
 */
attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* block_table, const int32_t* seqlens_k,
                          int batch, int max_seqlen_q, int max_seqlen_k,
                          int num_heads_q, int num_heads_kv, int head_dim,
                          int page_size, int max_pages_per_seq, int num_pages,
                          int causal, int window_left, int window_right, float softmax_scale,
                          void* out, float* lse, void* stream);

/*
 * attn_fp8_quantize -- block quantisation to FP8 (E4M3) with optional
 * incoherent processing ("FlashAttention-3 and PagedAttention: IO-Aware
 * Attention Kernels (2026)", "FlashAttention-3": FP8 with one scale per block
 * and a random orthogonal transform that spreads outliers first; "Flash
 * Attention: A Complete Architectural Autopsy", "FP8 Path and Quantization":
 * a tile's scale comes from its absolute maximum).
 *
 *   x       [batch, seqlen, num_heads, head_dim] bf16 (finite values)
 *   signs   NULL, or int8 [head_dim] of +1/-1: each row is first turned to
 *           H (s * x), H the unnormalised Sylvester-ordered Walsh-Hadamard
 *           matrix, computed in float32 by butterflies (stage h = 1, 2, 4, ...,
 *           head_dim/2; the pair (x[i], x[i+h]) with i & h == 0 becomes
 *           (x[i] + x[i+h], x[i] - x[i+h])).  Give Q and K the same signs and
 *           V none; attn_fwd_fp8's `incoherent` then divides the scale by d.
 *   layout  0: codes [batch, seqlen, num_heads, head_dim] (for Q and K);
 *           1: codes [batch, num_heads, head_dim, Np], Np = 64 *
 *           attn_fp8_num_blocks(seqlen) (for V): inside every 64-key block,
 *           byte p = 32 h + 16 kb + 4 g + e (0 <= h, kb < 2, g, e < 4) of a row
 *           holds key 32 kb + 8 g + 4 h + e; padding keys hold code 0.
 *   codes   uint8 E4M3 ("fn": bias 7, max 448, no infinities) codes, round to
 *           nearest even; attn_fp8_codes_bytes(...) bytes, written
 *   scales  float32 [batch, num_heads, attn_fp8_num_blocks(seqlen)], written:
 *           for each block of 64 consecutive rows of one (sequence, head),
 *           amax = max |x| (after the turn), scale = amax / 448 and code =
 *           E4M3(x * (448 / amax)) with the product rounded to float32; a
 *           block of zeros gets scale 0 and codes 0.  value ~ code * scale.
 * Requirements: head_dim in {64, 128, 256} (ATTN_ERR_UNSUPPORTED), positive
 * counts, layout 0 or 1 (ATTN_ERR_SHAPE); codes and scales must not overlap x, signs
 * or each other (ATTN_ERR_ALIAS).
 */
attn_status_t attn_fp8_quantize(const void* x, const int8_t* signs, int batch, int seqlen, int num_heads,
                                int head_dim, int layout, void* codes, float* scales, void* stream);

/* Bytes of attn_fp8_quantize's codes for a layout (0 for invalid sizes), and
 * the number of 64-row blocks of a sequence (ceil(seqlen / 64), 0 if <= 0). */
size_t attn_fp8_codes_bytes(int batch, int seqlen, int num_heads, int head_dim, int layout);
int attn_fp8_num_blocks(int seqlen);

/*
 * attn_fwd_fp8 -- attention forward on FP8 operands from attn_fp8_quantize
 * (dense batches; "Flash Attention: A Complete Architectural Autopsy", "FP8
 * Path and Quantization": scores are formed from the FP8 operands and
 * dequantised to fp32 for the softmax; the online softmax is that of
 * attn_fwd).
 *
 *   q_codes, k_codes  layout 0 codes of Q [batch, seqlen_q, num_heads_q, d]
 *                     and K [batch, seqlen_k, num_heads_kv, d], d = head_dim
 *   v_codes_t         layout 1 codes of V [batch, num_heads_kv, d, Np]
 *   q/k/v_scales      their block scales
 *   incoherent        1 if Q and K were turned (same signs): the scores of the
 *                     turned operands are d times the original ones, so
 *                     softmax_scale / d is applied
 *   out, lse          as attn_fwd in dense mode (bf16 out, float32 lse in
 *                     nats, lse may be NULL); causal masks align bottom-right
 * The probabilities are rounded to E4M3 for the P V product, after scaling by
 * 64 * s_v / max(s_v) of the V tile (which folds the V scales into P); the
 * softmax shift is raised only when a tile's maximum exceeds it by more than
 * 2 in log2 units, so they are at most 4 before that scaling, and the row
 * sums use the unrounded values.  Results equal exact attention on the
 * dequantised operands within the error of that rounding (2^-4 relative per
 * probability, 2^-10 absolute below 2^-6).
 * Requirements: head_dim in {64, 128, 256} (ATTN_ERR_UNSUPPORTED); others as
 * attn_fwd.
 */
attn_status_t attn_fwd_fp8(const void* q_codes, const void* k_codes, const void* v_codes_t,
                           const float* q_scales, const float* k_scales, const float* v_scales, int batch,
                           int seqlen_q, int seqlen_k, int num_heads_q, int num_heads_kv, int head_dim,
                           int causal, int incoherent, float softmax_scale, void* out, float* lse,
                           void* stream);

/*
 * attn_bwd -- gradients of attn_fwd by recomputation.
 *
 * From the forward's saved q, k, v, out and lse and the upstream gradient
 * dout = dL/d(out), rebuild each probability tile as exp(S - lse) under the
 * same mask and form dV = P^T dout, dP = dout V^T, dS = P * (dP - D) with
 * D = rowsum(dout * out), dQ = scale * dS K, dK = scale * dS^T Q ("Deep Dive
 * - FlashAttention", "Backward recomputes tiles on purpose").  A K/V head
 * shared by a group of query heads receives the sum over its group.  Rows
 * with no allowed key (lse = -inf) contribute nothing.
 *
 * Layouts and modes are those of attn_fwd: q, out, dout, dq like q; k, v, dk,
 * dv like k; lse as attn_fwd wrote it (required, not NULL).  total_q is the
 * number of query rows: batch * max_seqlen_q in dense mode, the packed total
 * TQ = cu_seqlens_q[batch] in packed mode (the caller knows it from the size
 * of q; a different value is undefined behaviour).
 * workspace: device memory of at least attn_bwd_workspace_bytes(total_q,
 *   num_heads_q) bytes, owned by the caller; its contents on entry do not
 *   matter and it is overwritten.
 * dq, dk, dv (bf16, written; round to nearest even) must not overlap any
 * input, the workspace or each other.  Calls that share a workspace on one
 * stream are ordered; on different streams they race.
 * Requirements: those of attn_fwd (head_dim in {64, 128, 256};
 * ATTN_ERR_UNSUPPORTED otherwise); workspace_bytes too small gives
 * ATTN_ERR_SHAPE.  Errors are returned before anything is enqueued.
 */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                       int num_heads_q, int num_heads_kv, int head_dim,
                       int causal, float softmax_scale,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_bwd needs: two float32 values (the row sum D and the
 * base-2 lse) per query row and query head; 0 for non-positive sizes. */
size_t attn_bwd_workspace_bytes(int total_q, int num_heads_q);

/*
 * attn_decode_splitkv -- one-token decode over a paged KV cache, split along
 * the cached keys ("FlashAttention-3 and PagedAttention: IO-Aware Attention
 * Kernels (2026)", "Why decode starves the GPU" and "How GQA and MLA reshape
 * the problem": chunks of the cache run in parallel, each emitting a partial
 * output and its log-sum-exp; all query heads that share a K/V head are
 * processed together so each cache row is read once).
 *
 *   q            [batch, num_heads_q, head_dim] bf16 (one new token per request)
 *   k_cache,
 *   v_cache      [num_pages, page_size, num_heads_kv, head_dim] bf16
 *   block_table  [batch, max_pages_per_seq] int32: logical page p of request
 *                b lives in physical page block_table[b * max_pages_per_seq + p]
 *                ("Deep Dive - FlashAttention", "Paged KV is a lookup, not a
 *                cache manager")
 *   seqlens_k    [batch] int32, cached keys per request (0 allowed)
 *   chunk_tokens keys per split; a positive multiple of page_size
 *   num_splits   leading dimension of the partials; must be >=
 *                ceil(max_b seqlens_k[b] / chunk_tokens) (see
 *                attn_decode_num_splits)
 *   out_partial  [num_splits, batch, num_heads_q, head_dim] float32 (written)
 *   lse_partial  [num_splits, batch, num_heads_q] float32 (written)
 * Split c of request b covers keys [c*chunk_tokens, min(seqlens_k[b],
 * (c+1)*chunk_tokens)); splits starting at or past seqlens_k[b] are not
 * written.  A written partial holds the softmax-normalised output over its
 * keys and the natural-log lse of those keys.  Cache rows at or past
 * seqlens_k[b], and table entries past ceil(seqlens_k[b]/page_size), are
 * never used as data, so they may hold anything, NaN included.  A page id
 * outside [0, num_pages), or a length beyond max_pages_per_seq * page_size
 * or num_splits * chunk_tokens, turns that request's results into NaN (it
 * never faults).  Requirements: page_size == 256, num_heads_q / num_heads_kv
 * <= 64, head_dim in {64,128,256}; others as attn_fwd.
 */
attn_status_t attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seqlens_k,
                                  int batch, int num_heads_q, int num_heads_kv, int head_dim,
                                  int page_size, int max_pages_per_seq, int num_pages,
                                  int chunk_tokens, int num_splits, float softmax_scale,
                                  float* out_partial, float* lse_partial, void* stream);

/*
 * attn_decode_combine -- merge the split partials of attn_decode_splitkv.
 * With L = log(sum_c exp(lse_c)) over the ceil(seqlens_k[b] / chunk_tokens)
 * written splits, out = sum_c exp(lse_c - L) * out_c and lse = L (the
 * rescaling identity of "FlashAttention-3 and PagedAttention: IO-Aware
 * Attention Kernels (2026)", "Why decode starves the GPU").  Only written
 * splits are read.  A request with no keys gets out = 0 and lse = -inf.
 *   out [batch, num_heads_q, head_dim] bf16, lse [batch, num_heads_q] float32
 *   (lse may be NULL).  The other arguments must equal those given to the
 *   attn_decode_splitkv call that produced the partials.
 */
attn_status_t attn_decode_combine(const float* out_partial, const float* lse_partial,
                                  const int32_t* seqlens_k, int batch, int num_heads_q,
                                  int head_dim, int chunk_tokens, int num_splits,
                                  void* out, float* lse, void* stream);

/*
 * attn_decode_noalloc -- attn_decode_splitkv followed by attn_decode_combine,
 * with the partials kept in a device array inside the library instead of a
 * caller workspace.  For callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the call allocates and frees nothing.
 *
 * Arguments are those of attn_decode_splitkv without out_partial and
 * lse_partial, plus out and lse as in attn_decode_combine.  The partials
 * (attn_decode_workspace_bytes(batch, num_heads_q, head_dim, num_splits)
 * bytes) must fit in ATTN_DECODE_NOALLOC_SCRATCH_BYTES, else ATTN_ERR_SHAPE
 * is returned before any HIP call.  The array is per GPU (the current
 * device; `stream` must belong to it), is held from the first call on that
 * GPU until the process ends, and is shared by every call on that GPU: calls
 * on one stream are ordered, calls that overlap on different streams of the
 * same GPU race and give undefined results.  Every partial the combine reads
 * is written by the split of the same call, so nothing needs clearing.
 * Errors in the arguments are returned before anything is enqueued; a failed
 * combine launch can leave the split enqueued.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
attn_status_t attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seqlens_k,
                                  int batch, int num_heads_q, int num_heads_kv, int head_dim,
                                  int page_size, int max_pages_per_seq, int num_pages,
                                  int chunk_tokens, int num_splits, float softmax_scale,
                                  void* out, float* lse, void* stream);

/*
 * attn_decode_kvcache -- one decode step that first appends the new token to
 * the paged cache in place, with optional rotary embedding, then decodes over
 * the cache including it ("Deep Dive - FlashAttention", "Paged KV is a
 * lookup, not a cache manager": the cached-decode call can update the cache
 * in place and apply rotary embeddings, into space the caller reserved;
 * "FlashAttention: Part 1", sections 4.1 and 4.2: rotary embedding turns Q
 * and K by position before attention).
 *
 *   q            [batch, num_heads_q, head_dim] bf16, the new token's queries
 *   k_new, v_new [batch, num_heads_kv, head_dim] bf16, its key and value
 *   k_cache,
 *   v_cache      [num_pages, page_size, num_heads_kv, head_dim] bf16, updated
 *                in place
 *   block_table, as in attn_decode_splitkv
 *   seqlens_k    [batch] int32: keys cached BEFORE this call.  The new token
 *                takes position p = seqlens_k[b]: its key and value are
 *                written to row p % page_size of page block_table[b][p /
 *                page_size], and request b then attends over p + 1 keys.
 *                seqlens_k is not modified; the caller advances it.
 *   rotary_dim   0 (no rotary: the key is stored and the query used as given)
 *                or an even number <= head_dim of leading features to turn.
 *                Feature pairs are (i, i + rotary_dim/2) when
 *                rotary_interleaved == 0, (2i, 2i+1) when 1; pair i at
 *                position p turns (a, b) into (a cos - b sin, a sin + b cos)
 *                with cos = rotary_cos[p * rotary_dim/2 + i] and likewise sin
 *                (float32 tables [rotary_max_pos, rotary_dim/2], the caller's
 *                frequencies).  Both q and the new key turn at position p, in
 *                float32, and are rounded to bf16 (nearest even).
 *   q_rot        [batch, num_heads_q, head_dim] bf16, written with the turned
 *                queries when rotary_dim > 0 (may be NULL when 0)
 *   chunk_tokens, num_splits, out_partial, lse_partial: as in
 *                attn_decode_splitkv, for lengths seqlens_k[b] + 1
 *                (num_splits >= ceil((max_b seqlens_k[b] + 1) / chunk_tokens))
 *   out, lse     as in attn_decode_combine (lse may be NULL)
 * A request whose position is negative, has no room (p >= max_pages_per_seq *
 * page_size, or p >= rotary_max_pos with rotary), or falls on a page id
 * outside [0, num_pages) writes nothing into the caches, gets NaN q_rot rows
 * and NaN out/lse; it never faults.  Requests must not share the cache row
 * they append to, and no request may read a row another request of the same
 * call appends (the writes would race).  Every written region (caches,
 * q_rot, partials, out, lse) must be disjoint from every other argument
 * (ATTN_ERR_ALIAS).  Requirements otherwise as attn_decode_splitkv.
 * Enqueues three kernels (append, split, combine) on the stream; argument
 * errors are returned before any of them, a launch failure after the first
 * can leave the earlier ones enqueued.
 */
attn_status_t attn_decode_kvcache(const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const int32_t* block_table,
                                  const int32_t* seqlens_k, const float* rotary_cos,
                                  const float* rotary_sin, int rotary_dim, int rotary_interleaved,
                                  int rotary_max_pos, int batch, int num_heads_q, int num_heads_kv,
                                  int head_dim, int page_size, int max_pages_per_seq, int num_pages,
                                  int chunk_tokens, int num_splits, float softmax_scale,
                                  void* q_rot, float* out_partial, float* lse_partial, void* out,
                                  float* lse, void* stream);

/* ceil(max_seqlen_k / chunk_tokens), the smallest valid num_splits (0 if
 * max_seqlen_k <= 0 or chunk_tokens <= 0). */
int attn_decode_num_splits(int max_seqlen_k, int chunk_tokens);

/* A chunk size (a multiple of 256) that gives a few workgroups per compute
 * unit for the given batch, K/V head count and longest cached length; the
 * split count is free ("FlashAttention-3 and PagedAttention: IO-Aware
 * Attention Kernels (2026)", "Why decode starves the GPU"), results do not
 * depend on it beyond rounding.  num_cus <= 0 means 256. */
int attn_decode_default_chunk(int batch, int num_heads_kv, int max_seqlen_k, int num_cus);

/* Bytes of out_partial plus lse_partial for these sizes. */
size_t attn_decode_workspace_bytes(int batch, int num_heads_q, int head_dim, int num_splits);

/* Host-side validators (they read host arrays only and never touch the GPU).
 * attn_check_cu_seqlens: cu[0] == 0, nondecreasing, cu[batch] == total, and
 * every length <= max_seqlen.  attn_check_block_table: every used entry
 * (ceil(seqlens[b] / page_size) per request) lies in [0, num_pages) and
 * every seqlens[b] is in [0, max_pages_per_seq * page_size].  Both return
 * ATTN_OK or ATTN_ERR_DATA (ATTN_ERR_NULL / ATTN_ERR_SHAPE for bad calls). */
attn_status_t attn_check_cu_seqlens(const int32_t* cu_seqlens_host, int batch, int total,
                                    int max_seqlen);
attn_status_t attn_check_block_table(const int32_t* block_table_host,
                                     const int32_t* seqlens_host, int batch,
                                     int max_pages_per_seq, int num_pages, int page_size);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
