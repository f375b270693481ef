// Measured ceilings of the resources the attention kernels are bound by
// (gfx950): streaming HBM reads, and bf16 and E4M3 matrix-core throughput on
// random operands.  Not part of the method: the benchmark reports each kernel's
// rate against these as well as against the published peaks ("Deep Dive -
// FlashAttention", "Benchmark the path you will ship", and "FlashAttention-3
// and PagedAttention: IO-Aware Attention Kernels (2026)", "Runnable Example:
// Measuring the IO Gap": measure on the machine rather than assume).

#include "../../include/attn_ceiling.h"
#include "attn_tile.h"

#include <stdarg.h>
#include <stdio.h>

namespace {

constexpr int kChunkBytes = 512 * 1024;  // contiguous bytes streamed by one wave
constexpr int kUnroll = 8;               // 16-byte loads in flight per lane

// One wave per 64-thread workgroup streams its own contiguous 512 KiB chunk,
// eight 16-byte non-temporal loads in flight per lane (the policy the decode
// kernel uses for its read-once K/V stream), and folds what it read into one
// word (so the loads cannot be dropped).
__global__ __launch_bounds__(64) void ceiling_read_kernel(const attn::u32x4* src, long n16, uint32_t* sink) {
    const int lane = threadIdx.x;
    const long base = (long)blockIdx.x * (kChunkBytes / 16);
    const long end = base + kChunkBytes / 16 < n16 ? base + kChunkBytes / 16 : n16;
    attn::u32x4 acc = {0u, 0u, 0u, 0u};
    long i = base + lane;
    for (; i + 64 * (kUnroll - 1) < end; i += 64 * kUnroll) {
        attn::u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(&src[i + 64 * u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < end; i += 64) acc ^= __builtin_nontemporal_load(&src[i]);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
    if (lane == 0) sink[blockIdx.x] = x;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One 32x32 matrix-core product: bf16 (v_mfma_f32_32x32x16_bf16, 16 bytes of
// operand per lane) or E4M3 (v_mfma_f32_32x32x64_f8f6f4 with format 0 for both
// operands, 32 bytes per lane).
template <bool FP8>
struct CeilOp;
template <>
struct CeilOp<false> {
    using Frag = attn::u32x4;
    static constexpr int WORDS = 4;
    static __device__ __forceinline__ Frag load(const uint32_t* w) { return Frag{w[0], w[1], w[2], w[3]}; }
    static __device__ __forceinline__ attn::f32x16 mma(const Frag& a, const Frag& b, const attn::f32x16& c) {
        return attn::mfma32(a, b, c);
    }
};
template <>
struct CeilOp<true> {
    using Frag = i32x8;
    static constexpr int WORDS = 8;
    static __device__ __forceinline__ Frag load(const uint32_t* w) {
        return Frag{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
    static __device__ __forceinline__ attn::f32x16 mma(const Frag& a, const Frag& b, const attn::f32x16& c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// Four accumulator chains of 32x32 products per wave, operands cycled among
// eight fragments of random values per lane (values that toggle the
// multipliers as real data does; constant operands run at a higher clock),
// 32 products per iteration.
template <bool FP8>
__global__ __launch_bounds__(256) void ceiling_mfma_kernel(const uint32_t* ops, int iters, float* sink) {
    using Op = CeilOp<FP8>;
    // 64 KiB of LDS per workgroup (of 160 KiB per CU) leaves room for two
    // workgroups per CU, so the grid spreads two waves onto every SIMD instead
    // of piling more onto some compute units and leaving others idle.
    __shared__ float spread[16384];
    const int lane = threadIdx.x & 63;
    const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint32_t* my = ops + (w * 64 + lane) * (8 * Op::WORDS);
    typename Op::Frag f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = Op::load(my + Op::WORDS * i);
    attn::f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = Op::mma(f[(j + c) & 7], f[(j + 2 * c + 1) & 7], acc[c]);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    spread[threadIdx.x * 64] = s;
    __syncthreads();
    sink[w * 64 + lane] = spread[((threadIdx.x + 64) & 255) * 64] + s;
}

thread_local char g_err[256] = "";

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

attn_status_t launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ATTN_OK;
}

template <bool FP8>
attn_status_t ceiling_mfma(const uint32_t* operands, int waves, int iters, float* sink, void* stream,
                           const char* what) {
    if (!operands || !sink) return fail(ATTN_ERR_NULL, "operands and sink must be non-NULL");
    if (((uintptr_t)operands & 15u) || ((uintptr_t)sink & 3u))
        return fail(ATTN_ERR_UNSUPPORTED, "misaligned pointer");
    if (waves < 4 || waves % 4 || iters < 1)
        return fail(ATTN_ERR_SHAPE, "waves must be a positive multiple of 4 and iters >= 1");
    hipLaunchKernelGGL(ceiling_mfma_kernel<FP8>, dim3(waves / 4), dim3(256), 0, static_cast<hipStream_t>(stream),
                       operands, iters, sink);
    return launched(what);
}

}  // namespace

extern "C" {

size_t attn_ceiling_read_sink_words(size_t bytes) { return (bytes + kChunkBytes - 1) / kChunkBytes; }

attn_status_t attn_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink) return fail(ATTN_ERR_NULL, "src and sink must be non-NULL");
    if (((uintptr_t)src & 15u) || ((uintptr_t)sink & 3u)) return fail(ATTN_ERR_UNSUPPORTED, "misaligned pointer");
    if (bytes == 0 || bytes % 16) return fail(ATTN_ERR_SHAPE, "bytes must be a positive multiple of 16");
    const size_t waves = attn_ceiling_read_sink_words(bytes);
    if (waves > 0x7fffffffu) return fail(ATTN_ERR_SHAPE, "too many bytes");
    hipLaunchKernelGGL(ceiling_read_kernel, dim3((unsigned)waves), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const attn::u32x4*>(src), (long)(bytes / 16), sink);
    return launched("attn_ceiling_read launch");
}

attn_status_t attn_ceiling_mfma_bf16(const uint32_t* operands, int waves, int iters, float* sink, void* stream) {
    return ceiling_mfma<false>(operands, waves, iters, sink, stream, "attn_ceiling_mfma_bf16 launch");
}

attn_status_t attn_ceiling_mfma_fp8(const uint32_t* operands, int waves, int iters, float* sink, void* stream) {
    return ceiling_mfma<true>(operands, waves, iters, sink, stream, "attn_ceiling_mfma_fp8 launch");
}

const char* attn_ceiling_last_error(void) { return g_err; }

}  // extern "C"
