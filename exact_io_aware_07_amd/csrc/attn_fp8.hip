// FP8 forward pass: block quantisation with incoherent processing, and the
// attention kernel on E4M3 operands (gfx950, head_dim 64, 128 or 256).
//
// "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
// "FlashAttention-3": FP8 with one scale per block and incoherent processing
// (a random orthogonal transform spreads outliers before quantisation).
// "Flash Attention: A Complete Architectural Autopsy", "FP8 Path and
// Quantization": each tile's scale comes from its absolute maximum, scores
// are formed from the FP8 operands and dequantised to fp32 for the softmax,
// and V tiles are quantised the same way.
//
// Quantisation runs as its own HBM-bound pass (one read of the bf16 tensor,
// one write of the codes) rather than inside the attention kernel: there the
// vector ALUs already limit the softmax, and a tile scale needs the whole
// tile's maximum before any of it can be converted.
//
// Formats (shared by both kernels):
//   codes   E4M3 ("fn": bias 7, max 448, no infinities), round to nearest even
//   blocks  64 consecutive rows of one (sequence, head); scale = amax / 448,
//           code = E4M3(x * (448 / amax)) with the product rounded to float32;
//           a zero block has scale 0 and codes 0
//   turn    x -> H (s * x) along d for Q and K: unnormalised Walsh-Hadamard
//           butterflies in float32, stage h = 1, 2, 4, ..., d / 2, the pair
//           (x[i], x[i+h]), i & h == 0, becoming (x[i] + x[i+h], x[i] - x[i+h]);
//           scores of turned operands are d times the original ones
//   Q, K    codes [B, N, H, d] (row layout)
//   V       codes [B, H, d, Np] (V^T layout, Np = N rounded up to 64): inside
//           every 64-key block, byte p = 32 h + 16 kb + 4 g + e holds key
//           32 kb + 8 g + 4 h + e, the order in which a lane holds the keys of
//           a score tile; padding keys are zero codes
//   scales  float32 [B, H, ceil(N / 64)]

#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kFp8Block = 64;
constexpr float kE4M3Max = 448.0f;
// The attention kernel's shift is raised only when a tile's maximum exceeds it
// by more than kFp8Rescale (log2 units), so probabilities are <= 2^kFp8Rescale;
// they are multiplied by 2^kFp8PScale before rounding to E4M3, which keeps the
// rounded values <= 256 (E4M3 max 448) and puts a probability 2^-12 below the
// shift at the bottom of the normal range.
constexpr float kFp8Rescale = 2.0f;
constexpr float kFp8PScale = 6.0f;

// D[32x32] += A[32x64] * B[64x32] on E4M3 operands (v_mfma_f32_32x32x64_f8f6f4,
// format 0 for both): lane l holds 32 bytes of row l % 32 of A and of column
// l % 32 of B; byte j of lane half h = l / 32 is one k index, the same for A
// and B (probed on the GPU), so the products pair byte (h, j) of A with byte
// (h, j) of B.  The result layout is the one of the 32x32x16 bf16 product.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two E4M3 codes (round to nearest even) of lo, hi into bytes 0-1 (hi_word
// false) or 2-3 (true) of `old`.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t cvt_fp8x2(float lo, float hi, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, (int)old, HI_WORD);
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

// Position, inside its 64-key block of a V^T row, of key k (0..63).
__device__ __forceinline__ uint32_t vt_pos_of_key(uint32_t k) {
    const uint32_t kb = k >> 5, g = (k >> 3) & 3u, h = (k >> 2) & 1u, e = k & 3u;
    return 32u * h + 16u * kb + 4u * g + e;
}

// ---- quantisation ----------------------------------------------------------------
// Value of lane (this lane ^ M) within the 16-lane group of a row, by DPP:
// M = 1, 2 are quad permutes, M = 8 rotates the 16-lane row by 8, and M = 4
// mirrors each half-row (i -> 7 - i) and then reverses each quad (i -> i ^ 3),
// which together map i to i ^ 4.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
    const int v = __float_as_int(x);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
    else if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));
    else {
        const int m = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);           // row_half_mirror
        return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false));  // quad_perm [3,2,1,0]
    }
}

// One cross-lane butterfly stage of the turn: the lane holding x[i] (bit M of
// its chunk index clear) keeps x[i] + x[i+h], its partner x[i] - x[i+h].
// other +- mine as one fused multiply-add with a +-1 factor: the product is
// exact, so the single rounding gives the same bits as the add or subtract.
// (M = 16, the partner 16 lanes away, is xstage16.)
template <int M>
__device__ __forceinline__ void xstage(float (&v)[4][8], bool low) {
    const float sgn = low ? 1.0f : -1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float mine = v[i][e];
            const float other = lane_xor<M>(mine);
            v[i][e] = __builtin_fmaf(mine, sgn, other);
        }
}

// The cross-lane stage with the partner 16 lanes away (d = 256):
// v_permlane16_swap of x with itself returns {x[l], x[l ^ 16]} in lanes of
// even 16-lane rows (bit 4 of the chunk index clear) and {x[l ^ 16], x[l]} in
// odd ones, so r0 + sgn * r1 is own + partner there and partner - own here.
__device__ __forceinline__ void xstage16(float (&v)[4][8], bool low) {
    const float sgn = low ? 1.0f : -1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i][e]), __float_as_uint(v[i][e]),
                                                            false, false);
            v[i][e] = __builtin_fmaf(__uint_as_float(r[1]), sgn, __uint_as_float(r[0]));
        }
}

// One workgroup (2 d threads) per (64-row block, head, sequence).  With
// L = d / 8 lanes per row, thread t holds rows 4 (t / L) .. + 3 of the block,
// values 8 (t % L) .. + 7 of each: a row's d values lie on L consecutive
// lanes (the butterflies' partners), and four consecutive rows are four
// consecutive keys of a V^T word.
template <int D, bool VT>
__global__ __launch_bounds__(2 * D) void attn_fp8_quant_kernel(Fp8QuantParams p) {
#pragma clang fp contract(off)
    constexpr int L = D / 8;         // lanes per row
    constexpr int NWQ = 2 * D / 64;  // waves per workgroup
    __shared__ float wmax[NWQ];
    __shared__ __attribute__((aligned(16))) uint8_t tile[VT ? D * kFp8Block : 16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nblk = (p.n + kFp8Block - 1) / kFp8Block;
    // Heads fastest: the workgroups that run together read whole rows (all
    // heads of the same 64 positions) rather than one head's 2 d bytes of
    // many rows (2-5% faster).
    const int h = blockIdx.x % p.heads;
    const int kb = (blockIdx.x / p.heads) % nblk;
    const int b = blockIdx.x / (p.heads * nblk);
    const int bh = b * p.heads + h;
    const int j = tid & (L - 1);  // 8-value chunk of the rows
    const int r0 = 4 * (tid / L);  // first of this thread's four rows

    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = kb * kFp8Block + r0 + i;
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        if (n < p.n) raw[i] = load16(p.x + (((long)b * p.n + n) * p.heads + h) * D + 8 * j);
    }
    float sg[8];
    if (p.signs != nullptr) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p.signs + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) sg[e] = (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
    }
    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[i][2 * e] = __uint_as_float(raw[i][e] << 16);
            v[i][2 * e + 1] = __uint_as_float(raw[i][e] & 0xffff0000u);
        }
    if (p.signs != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] *= sg[e];  // exact: +-1
            // in-lane stages h = 1, 2, 4
#pragma unroll
            for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((e & hs) == 0) {
                        const float a = v[i][e], c = v[i][e + hs];
                        v[i][e] = a + c;
                        v[i][e + hs] = a - c;
                    }
        }
        // cross-lane stages h = 8, 16, ..., d / 2: partner chunk j ^ (h / 8)
        xstage<1>(v, (j & 1) == 0);
        xstage<2>(v, (j & 2) == 0);
        xstage<4>(v, (j & 4) == 0);
        if constexpr (L > 8) xstage<8>(v, (j & 8) == 0);
        if constexpr (L > 16) xstage16(v, (j & 16) == 0);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    amax = wave_max_f(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int w = 1; w < NWQ; ++w) amax = fmaxf(amax, wmax[w]);
    const bool zero = !(amax > 0.0f);
    const float inv = zero ? 0.0f : kE4M3Max / amax;
    if (tid == 0) p.scales[(long)bh * nblk + kb] = zero ? 0.0f : amax / kE4M3Max;

    // codes of row i: lo = values 0..3, hi = values 4..7 (byte e = value e)
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = hi[i] = 0u;
        if (!zero && kb * kFp8Block + r0 + i < p.n) {  // padding rows are code 0 (a turned zero row can hold -0)
            // the second conversion overwrites bytes 2-3 of the first's seed
            lo[i] = cvt_fp8x2<false>(v[i][0] * inv, v[i][1] * inv, __float_as_uint(v[i][0]));
            lo[i] = cvt_fp8x2<true>(v[i][2] * inv, v[i][3] * inv, lo[i]);
            hi[i] = cvt_fp8x2<false>(v[i][4] * inv, v[i][5] * inv, __float_as_uint(v[i][4]));
            hi[i] = cvt_fp8x2<true>(v[i][6] * inv, v[i][7] * inv, hi[i]);
        }
    }
    if constexpr (!VT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = kb * kFp8Block + r0 + i;
            if (n < p.n)
                *reinterpret_cast<u32x2*>(p.codes + (((long)b * p.n + n) * p.heads + h) * D + 8 * j) =
                    u32x2{lo[i], hi[i]};
        }
    } else {
        // Rows r0 .. r0+3 are keys at positions pos .. pos+3 of the V^T block:
        // transpose the 4x4 bytes of each half so that word e holds value e of
        // the four rows, and write one word per value.
        const uint32_t pos = vt_pos_of_key((uint32_t)r0);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t* a = half ? hi : lo;
            const uint32_t t0 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);  // a0[0] a1[0] a0[1] a1[1]
            const uint32_t t1 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);  // a0[2] a1[2] a0[3] a1[3]
            const uint32_t t2 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
            const uint32_t t3 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
            const uint32_t w[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                                   __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<uint32_t*>(tile + (8 * j + 4 * half + e) * kFp8Block + pos) = w[e];
        }
        __syncthreads();
        const int np = nblk * kFp8Block;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 2 * D * i;      // 16-byte chunk of the d x 64 tile
            const int dd = c >> 2, q = c & 3;
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + dd * kFp8Block + 16 * q);
            *reinterpret_cast<u32x4*>(p.codes + ((long)bh * D + dd) * np + (long)kb * kFp8Block + 16 * q) = w;
        }
    }
}

template <int D>
static void launch_fp8_quant_d(const Fp8QuantParams& p, bool vt, unsigned grid, hipStream_t s) {
    if (vt)
        hipLaunchKernelGGL((attn_fp8_quant_kernel<D, true>), dim3(grid), dim3(2 * D), 0, s, p);
    else
        hipLaunchKernelGGL((attn_fp8_quant_kernel<D, false>), dim3(grid), dim3(2 * D), 0, s, p);
}

hipError_t launch_fp8_quant(const Fp8QuantParams& p, int head_dim, bool vt, hipStream_t s) {
    const long nblk = (p.n + kFp8Block - 1) / kFp8Block;
    const long grid = nblk * p.batch * p.heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    switch (head_dim) {
        case 64: launch_fp8_quant_d<64>(p, vt, (unsigned)grid, s); break;
        case 128: launch_fp8_quant_d<128>(p, vt, (unsigned)grid, s); break;
        case 256: launch_fp8_quant_d<256>(p, vt, (unsigned)grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- attention -----------------------------------------------------------------------
// The structure of the bf16 forward (waves of 32 query rows, 64-key tiles, two
// LDS stages filled by LDS-DMA, scores formed transposed so a lane owns a
// query row), with 4-wave workgroups at three waves per SIMD.  Per tile and wave: S^T = K Q^T in 4 MFMAs (2 key blocks x
// 2 d steps of 64) and O^T += V^T P^T in 4 (one per 32-row d block, all 64 keys
// at once).  The lane's 32 probabilities are rounded to E4M3 in register order,
// which is the key order of the V^T layout, so they are the B operand as they
// stand.  Differences from the bf16 kernel's softmax: the shift is raised when
// a tile's maximum exceeds it by more than kFp8Rescale, so probabilities are
// <= 4; they are multiplied by 64 * s_v(t) / max_t s_v(t) (folded into the
// exponent), which puts the V tile scale into P and keeps the E4M3 values
// <= 256; the row sum is kept from the unrounded values.
template <int D, bool CAUSAL, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_fp8_kernel(Fp8FwdParams p) {
    constexpr int BR = NW * 32, BC = 64;
    constexpr int KSD = D / 64;   // 64-wide d steps of S^T
    constexpr int DBD = D / 32;   // 32-row d blocks of O^T
    constexpr int KCH = D / 16;   // 16-byte chunks per K row
    constexpr int NI = D / 16;    // one-KiB loads per tensor and tile
    static_assert(NI % NW == 0, "each wave issues the same number of tile loads");
    constexpr uint32_t K_BYTES = BC * D, STAGE = 2 * K_BYTES;
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE];

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int BH = p.batch * p.hq;
    const int bid = blockIdx.x;
    int qt, bh;
    if ((BH & 7) == 0) {
        const int hpx = BH >> 3, x = bid & 7, kk = bid >> 3;
        const int kq = (int)udiv_apply(kk, p.dv_hpx);
        qt = p.n_qtiles - 1 - kq;
        bh = x * hpx + (kk - kq * hpx);
    } else {
        const int kq = (int)udiv_apply(bid, p.dv_bh);
        qt = p.n_qtiles - 1 - kq;
        bh = bid - kq * BH;
    }
    const int b = (int)udiv_apply(bh, p.dv_hq), hq = bh - b * p.hq;
    const int kvh = (int)udiv_apply(hq, p.dv_grp);
    const int Nq = p.nq, Nk = p.nk;
    const int q0 = qt * BR;
    if (q0 >= Nq) return;

    const long shift = (long)Nk - Nq;
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        if (!CAUSAL) return Nk - 1;
        const long hh = i + shift;
        return (int)(hh < Nk - 1 ? hh : Nk - 1);
    };
    const int last_row = min(q0 + BR, Nq) - 1;
    const int t_end = hi_of(last_row) < 0 ? 0 : hi_of(last_row) / BC + 1;

    const int wr0 = q0 + wave * 32;
    const bool wave_rows = wr0 < Nq;
    const int w_last_row = min(wr0 + 32, Nq) - 1;
    const int w_hi_max = hi_of(w_last_row), w_hi_min = hi_of(wr0);

    const uint32_t stride_k = (uint32_t)(p.hkv * D);  // bytes between key rows
    const uint8_t* kbase = p.k + ((long)b * Nk * p.hkv + kvh) * D;
    const uint8_t* vtbase = p.vt + ((long)b * p.hkv + kvh) * D * (long)p.np;
    const float* ks_row = p.k_scale + ((long)b * p.hkv + kvh) * p.nbk;
    const float* vs_row = p.v_scale + ((long)b * p.hkv + kvh) * p.nbk;

    auto issue_tile = [&](int t, uint32_t st) __attribute__((always_inline)) {
        const int key0 = t * BC;
        const int nvalid = Nk - key0;
        const uint32_t nrec = nvalid > 0 ? (uint32_t)(nvalid < BC ? nvalid : BC) * stride_k : 0u;
        const u32x4 rk = rsrc_words(kbase + (long)key0 * stride_k, nrec);
        const u32x4 rv = rsrc_words(vtbase + key0, (uint32_t)(D - 1) * (uint32_t)p.np + (uint32_t)BC);
        // each tile is 64 d bytes of K and as many of V^T: d / 16 one-KiB loads of each
#pragma unroll
        for (int jj = 0; jj < NI / NW; ++jj) {
            const int i = wave * (NI / NW) + jj;
            const uint32_t krow = (1024 / D) * i + lane / KCH, kc = lane % KCH;
            dma16(rk, st + 1024 * i, krow * stride_k + ((kc ^ swz<KCH>(krow)) * 16));
            const uint32_t vrow = 16 * i + (lane >> 2), vc = lane & 3;
            dma16(rv, st + K_BYTES + 1024 * i, vrow * (uint32_t)p.np + ((vc ^ swz<4>(vrow)) * 16));
        }
    };

    // Q^T fragments (B operand): lane half h holds d = 64 s + 32 h .. + 31 of its row.
    const int row = wr0 + l32;
    i32x8 qf[KSD];
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
        u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
        if (row < Nq) {
            const uint8_t* qrow = p.q + (((long)b * Nq + row) * p.hq + hq) * D + 64 * s + 32 * h;
            a = *reinterpret_cast<const u32x4*>(qrow);
            c = *reinterpret_cast<const u32x4*>(qrow + 16);
        }
        qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
    const float s_q = row < Nq ? p.q_scale[((long)b * p.hq + hq) * p.nbq + row / kFp8Block] : 0.0f;
    float svmax = 0.0f;
    for (int i = lane; i < p.nbk; i += 64) svmax = fmaxf(svmax, vs_row[i]);
    svmax = wave_max_f(svmax);
    const float vref = svmax > 0.0f ? svmax : 1.0f;
    const float log2_svmax = svmax > 0.0f ? __log2f(svmax) : 0.0f;
    const float c2q = p.scale * kLog2e * s_q;

    f32x16 oacc[DBD];
#pragma unroll
    for (int db = 0; db < DBD; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m_run = -INFINITY, l_part = 0.0f;

    // The K and V scales of a tile are loaded one step ahead, with the tile's
    // own loads, so that the end-of-step wait covers them: a load waited for
    // inside a step would also wait for the next tile's loads issued before it.
    float ks_cur = 0.0f, vs_cur = 0.0f;
    if (t_end > 0) {
        issue_tile(0, lds_addr(stage0));
        ks_cur = ks_row[0];
        vs_cur = vs_row[0];
    }
    wait_vmem();
    __syncthreads();

    auto step = [&](const int t, char* cur, char* nxt) __attribute__((always_inline)) {
        const char* ks = cur;
        const char* vs = cur + K_BYTES;
        float ks_nxt = 0.0f, vs_nxt = 0.0f;
        if (t + 1 < t_end) {
            issue_tile(t + 1, lds_addr(nxt));
            ks_nxt = ks_row[t + 1];
            vs_nxt = vs_row[t + 1];
        }
        const int k0 = t * BC;
        const bool active = wave_rows && k0 <= w_hi_max;
        if (active) {
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < KSD; ++s)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint32_t kr = 32 * kb + l32;
                    const uint32_t c0 = 4 * s + 2 * h;
                    const u32x4 a0 = lds_read16(ks, kr * D + ((c0 ^ swz<KCH>(kr)) * 16));
                    const u32x4 a1 = lds_read16(ks, kr * D + (((c0 + 1) ^ swz<KCH>(kr)) * 16));
                    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    sacc[kb] = mfma_fp8(a, qf[s], sacc[kb]);
                }
            // scores of the turned, dequantised operands in log2 units: S * c2t
            const float c2t = fmaxf(c2q * ks_cur, 1.17549435e-38f);
            if (k0 + BC - 1 > w_hi_min || k0 + BC > Nk) {
                // key = k0 + 4 (lane / 32) + a constant of (kb, r): one
                // comparison of that constant per element
                const int th = hi_of(row) - (k0 + score_key(0, 0, lane));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (score_key(kb, r, 0) > th) sacc[kb][r] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = pair_max(mx) * c2t;
            const bool raise = mx > m_run + kFp8Rescale;
            if (__builtin_amdgcn_ballot_w64(raise && m_run != -INFINITY)) {
                const float alpha = (raise && m_run != -INFINITY) ? exp2f(m_run - mx) : 1.0f;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < DBD; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            if (raise) m_run = mx;
            // V tile scale folded into P: P' = p * 64 * s_v(t) / max s_v
            const float sv = vs_cur;
            const float lg = kFp8PScale + ((sv > 0.0f && svmax > 0.0f) ? __log2f(sv) - log2_svmax : 0.0f);
            // sv <= svmax, so lg <= kFp8PScale and 2^-lg >= 2^-kFp8PScale is a
            // normal number: the hardware exponential needs no range scaling.
            const float inv_g = __builtin_amdgcn_exp2f(-lg);
            const float sh = (m_run == -INFINITY) ? 0.0f : m_run - lg;
            float rs;  // starts from the first probability (same value as 0 + p)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c2t, -sh));
                    sacc[kb][r] = e;
                    rs = (kb == 0 && r == 0) ? e : rs + e;
                }
            l_part = __builtin_fmaf(rs, inv_g, l_part);
            i32x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int kb = i >> 2, r0 = 4 * (i & 3);
                // bytes 2-3 of the first result are overwritten by the second,
                // so any seed works; this one costs no register move
                uint32_t w = cvt_fp8x2<false>(sacc[kb][r0], sacc[kb][r0 + 1], __float_as_uint(sacc[kb][r0]));
                w = cvt_fp8x2<true>(sacc[kb][r0 + 2], sacc[kb][r0 + 3], w);
                pb[i] = (int)w;
            }
#pragma unroll
            for (int db = 0; db < DBD; ++db) {
                const uint32_t vr = 32 * db + l32;
                const u32x4 a0 = lds_read16(vs, vr * BC + (((2 * h) ^ swz<4>(vr)) * 16));
                const u32x4 a1 = lds_read16(vs, vr * BC + (((2 * h + 1) ^ swz<4>(vr)) * 16));
                const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                oacc[db] = mfma_fp8(a, pb, oacc[db]);
            }
        }
        wait_vmem();
        __syncthreads();
        ks_cur = ks_nxt;
        vs_cur = vs_nxt;
    };
    for (int t = 0; t < t_end; t += 2) {
        step(t, stage0, stage1);
        if (t + 1 < t_end) step(t + 1, stage1, stage0);
    }

    const float l_tot = pair_sum(l_part);
    constexpr uint32_t WB = 32u * D * 2;  // a wave's output rows in bf16
    if constexpr ((NW / 2) * WB <= STAGE) {
        // Output rows through LDS (the wave's own region of the stages, free
        // after the last barrier): 16-byte stores of whole rows.
        char* const ob = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WB;
        const float inv = l_tot > 0.0f ? vref / (exp2f(kFp8PScale) * l_tot) : 0.0f;
        store_rows_bf16_staged<DBD>(ob, oacc, inv, lane, p.out + (((long)b * Nq + wr0) * p.hq + hq) * D,
                                    (long)p.hq * D, Nq - wr0);
        if (row < Nq && p.lse != nullptr && h == 0)
            p.lse[((long)b * p.hq + hq) * Nq + row] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        return;
    }
    if (row < Nq) {
        const float inv = l_tot > 0.0f ? vref / (exp2f(kFp8PScale) * l_tot) : 0.0f;
        uint16_t* orow = p.out + (((long)b * Nq + row) * p.hq + hq) * D;
#pragma unroll
        for (int db = 0; db < DBD; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                           pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * h) = w;
            }
        if (p.lse != nullptr && h == 0)
            p.lse[((long)b * p.hq + hq) * Nq + row] =
                l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// Four-wave workgroups (128 query rows) at three waves per SIMD (d = 128):
// the softmax's vector work limits this kernel, and a third wave per SIMD
// hides more of it than 8-wave workgroups at two per SIMD (measured +12% on
// the causal 4096-token workload at d = 128, although each tile is loaded by
// twice as many workgroups).  At d = 256 eight-wave workgroups (256 query
// rows, two waves per SIMD) fit the 256-register budget without spills and
// run 1.7x faster than four waves at one per SIMD on that workload (a second
// wave per SIMD hides the softmax; a four-wave workgroup at two per SIMD
// spills).
// d = 64: 113 VGPRs fit four waves per SIMD (3-4% over three).
#ifndef ATTN_FP8_CFG64
#define ATTN_FP8_CFG64 4, 4
#endif
#ifndef ATTN_FP8_CFG128
#define ATTN_FP8_CFG128 4, 3
#endif
#ifndef ATTN_FP8_CFG256
#define ATTN_FP8_CFG256 8, 2
#endif
template <int D> struct Fp8Cfg;  // {waves per workgroup, waves per SIMD}
template <> struct Fp8Cfg<64> { static constexpr int v[2] = {ATTN_FP8_CFG64}; };
template <> struct Fp8Cfg<128> { static constexpr int v[2] = {ATTN_FP8_CFG128}; };
template <> struct Fp8Cfg<256> { static constexpr int v[2] = {ATTN_FP8_CFG256}; };

template <int D>
static hipError_t launch_fwd_fp8_d(Fp8FwdParams p, bool causal, hipStream_t s) {
    constexpr int NW = Fp8Cfg<D>::v[0], WPE = Fp8Cfg<D>::v[1];
    p.n_qtiles = (p.nq + 32 * NW - 1) / (32 * NW);
    const long grid = (long)p.n_qtiles * p.batch * p.hq;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const int bh_all = p.batch * p.hq;  // below 2^31 after the check above
    p.dv_hpx = udiv_make(bh_all >= 8 ? bh_all >> 3 : 1);
    p.dv_bh = udiv_make(bh_all);
    p.dv_hq = udiv_make(p.hq);
    p.dv_grp = udiv_make(p.hkv > 0 ? p.hq / p.hkv : 1);
    if (causal)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, true, NW, WPE>), dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
    else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, false, NW, WPE>), dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int head_dim, bool causal, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_fwd_fp8_d<64>(p, causal, s);
        case 128: return launch_fwd_fp8_d<128>(p, causal, s);
        case 256: return launch_fwd_fp8_d<256>(p, causal, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
