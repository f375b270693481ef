/*
 * Measured ceilings for the attention kernels' rooflines (libattn.so).
 *
 * Not part of the attention method: kernels that measure, on the machine
 * at hand, the rates the attention kernels are bound by, so that each kernel
 * can be reported against the measured ceiling as well as the published peak
 * ("Deep Dive - FlashAttention", "Benchmark the path you will ship";
 * "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
 * "Runnable Example: Measuring the IO Gap": measure rather than assume).
 * Conventions (device pointers, stream, status codes) as in attn.h.
 */
#ifndef EXACT_ATTN_CEILING_H
#define EXACT_ATTN_CEILING_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `sink` that attn_ceiling_read writes for `bytes` bytes: one per
 * 512 KiB chunk (one wave each). */
size_t attn_ceiling_read_sink_words(size_t bytes);

/*
 * Streaming read of `bytes` bytes at `src` (16-byte aligned, a positive
 * multiple of 16; the content is irrelevant): each wave reads its own
 * contiguous 512 KiB chunk with eight 16-byte loads in flight per lane and
 * writes the XOR of what it read to sink[wave] (uint32,
 * attn_ceiling_read_sink_words(bytes) words, written).  Rate = bytes /
 * kernel time.
 */
attn_status_t attn_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * `waves` waves (a positive multiple of 4; 2048 fills an MI355X two waves per
 * SIMD, the occupancy of the attention kernels) each run `iters` iterations
 * of 32 v_mfma_f32_32x32x16_bf16 products (32768 FLOP each) in four
 * independent accumulator chains, operands cycled among 8 fragments of 8 bf16
 * per lane taken from `operands`: uint32 [waves, 64 lanes, 32] (finite random
 * bf16 values, which toggle the multipliers as real data does).
 * sink: float [waves * 64], written with each lane's accumulator sum plus
 * that of the lane 64 threads further on in its workgroup.  The kernel holds
 * 64 KiB of LDS per 4-wave workgroup so that no more than two workgroups
 * share a compute unit.
 * Rate = waves * iters * 32 * 32768 / kernel time.
 */
attn_status_t attn_ceiling_mfma_bf16(const uint32_t* operands, int waves, int iters, float* sink, void* stream);

/*
 * As attn_ceiling_mfma_bf16 for E4M3 operands: v_mfma_f32_32x32x64_f8f6f4
 * products (131072 FLOP each), 8 fragments of 32 E4M3 codes per lane from
 * `operands`: uint32 [waves, 64 lanes, 64] (finite codes; no NaN byte 0x7F or
 * 0xFF).  Rate = waves * iters * 32 * 131072 / kernel time.
 */
attn_status_t attn_ceiling_mfma_fp8(const uint32_t* operands, int waves, int iters, float* sink, void* stream);

/* The calling thread's message for its last failing ceiling call. */
const char* attn_ceiling_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_CEILING_H */
