// Device building blocks shared by the prefill and decode kernels (gfx950).
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   D[32x32] += A[32x16] * B[16x32]
//   A operand: lane l holds A[l % 32][8 * (l / 32) + 0..7]   (8 bf16, 16 bytes)
//   B operand: lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   D result:  lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//
// Scores are formed transposed, S^T = K Q^T (A = K rows, B = Q^T), so every
// lane owns one query row (column l % 32) and sixteen of its key scores: row
// max and row sum are in-lane work plus one swap between the two lane halves.
// The output is kept transposed too, O^T = V^T P^T, so the S^T registers feed
// the B operand of the second product directly (no trip through LDS) and the
// per-row rescale multiplies whole lanes.
//
// The key order inside a 32-key block is whatever makes the S^T registers a
// valid B operand: for the 16-key step c of block kb, lane half h holds keys
// 32*kb + 16*c + {4h..4h+3, 8+4h..8+4h+3}.  V stays row-major in LDS and is
// read transposed (ds_read_b64_tr_b16) in exactly that key order
// (read_vt_frag_tr).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A row's shift is only raised when a tile's maximum exceeds it by more than
// this many powers of two, so exp2(s - shift) <= 2^8 stays far inside fp32 and
// bf16 range; the result is the same operator whatever shift is used, because
// numerator and denominator carry the same factor.
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_permlane32_swap with both operands = x leaves each lane holding the pair
// {x[l], x[l ^ 32]} (one in each result), so a symmetric op of the two
// results combines the two halves of a query row.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + the sum of the eight bf16 values packed in w (four pairs), each pair
// added by one v_dot2c_f32_bf16 against (1, 1): the products are exact and the
// sum is taken in fp32.  The components are named one by one: indexing w with
// the counter of an unrolled loop under __builtin_bit_cast made this compiler
// read w.x four times.
__device__ __forceinline__ float add_bf16x8(const u32x4& w, float acc) {
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), one, acc, false);
    return acc;
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Buffer resource over [base, base + bytes); raw loads at or past `bytes`
// return zeros (gfx9 descriptor word 3: 32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// A 16-byte raw buffer load with the non-temporal cache policy (nt: bit 1 of
// the policy operand on gfx950), for data that is read exactly once: a
// streamed K/V cache no other workgroup reads should not displace cached
// lines (measured on the paged decode: 7% faster than the default policy).
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

__device__ __forceinline__ u32x4 lds_read16(const char* base, uint32_t off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}

// XOR swizzle of 16-byte chunks for an LDS row of NCHUNK chunks.  Rows that
// consecutive lanes read at the same logical chunk land in distinct bank
// groups both for 128-byte and 256-byte-per-clock LDS: rows r..r+7 map to 8
// distinct chunks, and rows r..r+15 to 16 distinct 16-byte slots of a 256-byte
// window.  Depends on the low four row bits only.
template <int NCHUNK>
__device__ __forceinline__ uint32_t swz(uint32_t row) {
    if constexpr (NCHUNK == 4) {
        return ((row >> 1) ^ (row >> 2)) & 3u;
    } else if constexpr (NCHUNK == 8) {
        return (row & 7u) ^ ((row >> 3) & 1u);
    } else {
        static_assert(NCHUNK >= 16, "row too short");
        return row & 15u;
    }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS tiles (no register staging).
//
// K and V tiles are both stored row-major [BC][D] (row = key), 16-byte chunks
// XOR-swizzled per row.  A 16-byte buffer load with the LDS flag writes the 64
// lanes' data to 1 KiB of LDS in lane order at a wave-uniform base, so each
// lane fetches whichever global chunk belongs at its LDS slot; 16 consecutive
// lanes still cover one 256-byte row, so the reads stay coalesced.  Rows past
// the resource size (keys past the end) arrive as zeros.
//
// V is read back transposed with ds_read_b64_tr_b16.  Within each group of 16
// lanes that instruction hands output lane j, element k, the element (j % 4)
// of the 8 bytes addressed by source lane 4k + j / 4.  So when source lane s
// addresses V[key0 + s / 4][d0 + 4 * (s % 4) .. +3], output lane j receives
// V[key0 .. key0 + 3][d0 + j]: four consecutive keys of one d column, i.e. half
// of a V^T A-operand fragment.

typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); exp and lgkm counters left unconstrained).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Buffer resource words for [base, base + bytes): 48-bit base, stride 0,
// num_records = bytes, gfx9 word 3 (32-bit data format, no swizzle).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// One 16-byte-per-lane buffer load straight into LDS: lane i's data lands at
// LDS byte lds_base + 16 * i (lds_base is wave-uniform and goes to M0).
// Written as inline assembly so that the compiler does not track these LDS
// writes: it would otherwise drain every outstanding load before LDS reads it
// cannot prove unrelated.  Every consumer waits explicitly (wait_vmem)
// before reading a stage and synchronises as needed.
// M0 is saved and restored around the load (M0 is a reserved register that a
// clobber list does not protect; the load takes its value at issue), and one
// wait state separates the M0 write from the load, as GFX9-family parts
// require between an SALU write of M0 and an LDS-DMA instruction.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds_base, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voff), "s"(rsrc)
        : "memory");
}

// Swizzle for V rows read by ds_read_b64_tr_b16: one instruction touches 8
// consecutive key rows and a 64-byte window of each; this spreads the eight
// windows evenly over the banks (two per 64-byte bank group).
template <int NCHUNK>
__device__ __forceinline__ uint32_t swz_tr(uint32_t row) {
    if constexpr (NCHUNK == 8) {
        return 4u * ((row >> 1) & 1u);
    } else {
        static_assert(NCHUNK >= 16, "row too short");
        return 4u * (row & 3u);
    }
}

template <int D, int BC, int NW>
struct KVDirect {
    static constexpr uint32_t ROWB = D * 2;        // bytes per row
    static constexpr int CH = D / 8;               // 16-byte chunks per row
    static constexpr uint32_t K_BYTES = BC * ROWB;
    static constexpr uint32_t BYTES = 2 * K_BYTES; // K then V
    static constexpr int INSTR = K_BYTES / 1024;   // 1 KiB load instructions per tensor
    static constexpr int PER_WAVE = INSTR / NW;
    static constexpr int RPI = 1024 / ROWB;        // rows per instruction
    static_assert(INSTR % NW == 0, "each wave issues the same number of loads");

    // Issue this wave's share of the loads of one tile into the stage at LDS
    // byte address `st` (K at st, V at st + K_BYTES).  kbase/vbase: first row
    // of the tile; consecutive rows `stride_b` bytes apart; the first
    // `nvalid` rows are real keys.
    __device__ __forceinline__ static void issue(const uint16_t* kbase, const uint16_t* vbase,
                                                 uint32_t stride_b, int nvalid, uint32_t st,
                                                 int wave, int lane) {
        const uint32_t nrec = nvalid > 0 ? (uint32_t)(nvalid < BC ? nvalid : BC) * stride_b : 0u;
        const u32x4 rk = rsrc_words(kbase, nrec);
        const u32x4 rv = rsrc_words(vbase, nrec);
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int i = wave * PER_WAVE + j;
            const uint32_t row = i * RPI + lane / CH;
            const uint32_t pc = lane % CH;
            dma16(rk, st + i * 1024, row * stride_b + ((pc ^ swz<CH>(row)) * 16));
            dma16(rv, st + K_BYTES + i * 1024, row * stride_b + ((pc ^ swz_tr<CH>(row)) * 16));
        }
    }
};

// A operand of O^T = V^T P^T from a row-major V tile (see KVDirect).
template <int D>
__device__ __forceinline__ u32x4 read_vt_frag_tr(const char* vs, int db, int kb, int c, int lane) {
    constexpr int CH = D / 8;
    const uint32_t G = lane >> 4, s = lane & 15;
    const uint32_t d = 32 * db + 16 * (G & 1) + 4 * (s & 3);
    const uint32_t key = 32 * kb + 16 * c + 4 * (G >> 1) + (s >> 2);
    const uint32_t k2 = key + 8;
    const uint32_t a1 = key * (2 * D) + (((d >> 3) ^ swz_tr<CH>(key)) * 16) + (d & 7) * 2;
    const uint32_t a2 = k2 * (2 * D) + (((d >> 3) ^ swz_tr<CH>(k2)) * 16) + (d & 7) * 2;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(vs + a1));
    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(vs + a2));
    const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
    return u32x4{w1[0], w1[1], w2[0], w2[1]};
}

// A operand of S^T = K Q^T for key block kb (32 rows) and d-step s (16 wide).
template <int D>
__device__ __forceinline__ u32x4 read_k_frag(const char* ks, int kb, int s, int lane) {
    const uint32_t row = 32 * kb + (lane & 31), h = lane >> 5;
    return lds_read16(ks, row * (2 * D) + (((2 * s + h) ^ swz<D / 8>(row)) * 16));
}

// Key index (within the tile) of S^T register r of block kb for this lane.
__device__ __forceinline__ int score_key(int kb, int r, int lane) {
    return 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// ---- 16x16x32 matrix-core tiles (one-query decode) -------------------------
// v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 * (l / 16) + 0..7] and
// B[8 * (l / 16) + 0..7][l % 16]; result register r of lane l is
// D[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes that hold
// one column of a 16x16 result).  v_permlane16_swap with both operands = x
// leaves each lane holding {x[l], x[l ^ 16]}.
__device__ __forceinline__ float quad_max(float x) {
    x = pair_max(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float quad_sum(float x) {
    x = pair_sum(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Chunk swizzle of a row-major V tile that is read back with 16-lane
// transposed reads of 16 consecutive rows: 16-byte chunk c of row `row` sits
// in slot c ^ swz_v16<CH>(row), which puts those 16 rows' segments of one
// chunk on 16 different bank groups.
template <int CH>
__device__ __forceinline__ uint32_t swz_v16(uint32_t row) {
    if constexpr (CH == 8) {
        return (row >> 1) & 7u;  // 128-byte rows: odd rows already sit on the other 32 banks
    } else {
        static_assert(CH >= 16, "row too short");
        return row & 15u;
    }
}

// A operand of O^T = V^T P^T (16x16x32 shape) for d block db (16 rows of V^T)
// from a 32-key row-major V tile stored with swz_v16.  Contraction index
// 8 * (l / 16) + j maps to key 4 * (l / 16) + j for j < 4 and to key
// 16 + 4 * (l / 16) + (j - 4) for j >= 4: the keys a lane holds in the two
// 16-key blocks of S^T (result registers 0..3 of each block).
template <int D>
__device__ __forceinline__ u32x4 read_vt16_tr(const char* vs, int db, int lane) {
    constexpr int CH = D / 8;
    const uint32_t G = lane >> 4, s = lane & 15;
    const uint32_t d = 16 * db + 4 * (s & 3);
    const uint32_t k1 = 4 * G + (s >> 2);
    const uint32_t k2 = k1 + 16;
    const uint32_t a1 = k1 * (2 * D) + (((d >> 3) ^ swz_v16<CH>(k1)) * 16) + (d & 7) * 2;
    const uint32_t a2 = k2 * (2 * D) + (((d >> 3) ^ swz_v16<CH>(k2)) * 16) + (d & 7) * 2;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(vs + a1));
    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(vs + a2));
    const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
    return u32x4{w1[0], w1[1], w2[0], w2[1]};
}

// ---- output rows through LDS ------------------------------------------------
// A wave's 32 rows of a 32x32 accumulator set (lane l holds row l % 32, d
// values 32 db + 8 g + 4 (l / 32) .. + 3 in acc[db][4 g .. 4 g + 3]) scaled by
// mul (per lane, so per row), rounded to bf16 and written to rows [0, nrows)
// of dst (row r at dst + r * stride elements).  The rows go through the wave's
// own LDS region `ob` (32 * 64 * DB bytes; 16-byte chunks XOR-swizzled by
// row) so that each global store writes 16 bytes per lane and a group of
// lanes writes whole rows, instead of 8-byte pieces scattered over 32 rows.
// The caller makes sure no other wave still reads `ob`.
template <int DB>
__device__ __forceinline__ void store_rows_bf16_staged(char* ob, const f32x16 (&acc)[DB], float mul, int lane,
                                                       uint16_t* dst, long stride, int nrows) {
    constexpr int D = 32 * DB;
    constexpr int CHR = D / 8;          // 16-byte chunks per row
    constexpr int RPP = 1024 / (D * 2); // rows per 64-lane pass
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 w = {pack_bf16x2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                             pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
            const int ch = 4 * db + g;
            *reinterpret_cast<u32x2*>(ob + l32 * (D * 2) + ((ch ^ (l32 & (CHR - 1))) * 16) + h * 8) = w;
        }
#pragma unroll
    for (int i = 0; i < 32 / RPP; ++i) {
        const int r = i * RPP + lane / CHR, c = lane % CHR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * (D * 2) + ((c ^ (r & (CHR - 1))) * 16));
        if (r < nrows) *reinterpret_cast<u32x4*>(dst + (long)r * stride + c * 8) = v;
    }
}

}  // namespace attn
