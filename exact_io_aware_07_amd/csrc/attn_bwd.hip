// Backward pass of exact attention by recomputation (gfx950).
//
// "Deep Dive - FlashAttention", "Backward recomputes tiles on purpose": the
// forward keeps Q, K, V, the output O and the row log-sum-exp; the backward
// rebuilds each probability tile as P = exp(S - LSE) under the same mask and
// forms, with G = dL/dO,
//   dV = P^T G,   dP = G V^T,   dS = P * (dP - D),   D = rowsum(G * O),
//   dQ = scale * dS K,   dK = scale * dS^T Q.
// Masked probabilities, and their gradients, are zero.
//
// Three kernels:
//   attn_bwd_prep_kernel  D per (row, query head), and lse in log2 units
//                         (+inf for rows with no key, so their P is 0);
//   attn_bwd_dkdv_kernel  one workgroup per (key tile, K/V head, sequence):
//                         the tile's K and V stay in registers while the
//                         query tiles of every query head of the group stream
//                         through LDS; dK and dV accumulate in registers, so
//                         no atomics and a fixed summation order (d = 64);
//   attn_bwd_dkdv_pair_kernel  the same with each 32-key group split over two
//                         waves, one for P and dV, one for dS and dK (d = 128);
//   attn_bwd_dq_kernel    one workgroup per (query tile, query head,
//                         sequence), shaped like the forward: K/V tiles stream
//                         through LDS and dQ accumulates in registers.
// All products are bf16 MFMA with fp32 accumulation; P and dS are rounded to
// bf16 as the forward rounds P.

#include <type_traits>

#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

// Chunk swizzle for the backward's LDS tiles.  Each tile is read two ways:
// as 32-row fragments (16 consecutive rows per 16-lane group, one 16-byte
// chunk each) and with transposing 16-row reads (4 consecutive rows, four
// chunks each).  Data chunk c of row r sits in slot c ^ swz_b(r); swz_b
// takes all 16 values on 16 consecutive rows and moves each of 4 consecutive
// rows to a different group of 4 slots, so both patterns are conflict-free.
template <int CH>
__device__ __forceinline__ uint32_t swz_b(uint32_t row) {
    if constexpr (CH == 8) {
        return (((row >> 1) & 1u) << 2) | ((row >> 2) & 3u);  // 128-byte rows: odd rows use the other banks
    } else {
        // 256- and 512-byte rows start on the same bank, so the low four
        // slot bits alone decide the bank group.
        static_assert(CH == 16 || CH == 32, "backward tiles support d = 64, 128 and 256");
        return ((row & 3u) << 2) | ((row >> 2) & 3u);
    }
}

// Two row-major [ROWS, D] bf16 tiles (A then B) loaded HBM -> LDS with the
// buffer range check zero-filling rows at or past nvalid.
template <int D, int ROWS, int NW>
struct BwdTile {
    static constexpr uint32_t ROWB = 2 * D;
    static constexpr int CH = D / 8;
    static constexpr uint32_t A_BYTES = ROWS * ROWB;
    static constexpr uint32_t BYTES = 2 * A_BYTES;
    static constexpr int INSTR = A_BYTES / 1024;
    static constexpr int PER_WAVE = INSTR / NW;
    static constexpr int RPI = 1024 / ROWB;
    static_assert(INSTR % NW == 0, "each wave issues the same number of loads");

    __device__ __forceinline__ static void issue(const uint16_t* abase, const uint16_t* bbase,
                                                 uint32_t stride_b, int nvalid, uint32_t st, int wave,
                                                 int lane) {
        const uint32_t nrec = nvalid > 0 ? (uint32_t)(nvalid < ROWS ? nvalid : ROWS) * stride_b : 0u;
        const u32x4 ra = rsrc_words(abase, nrec);
        const u32x4 rb = rsrc_words(bbase, nrec);
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int i = wave * PER_WAVE + j;
            const uint32_t row = i * RPI + lane / CH;
            const uint32_t off = row * stride_b + (((lane % CH) ^ swz_b<CH>(row)) * 16);
            dma16(ra, st + i * 1024, off);
            dma16(rb, st + A_BYTES + i * 1024, off);
        }
    }
};

// 32-row fragment (operand rows 32 rb + l % 32, d values 16 s + 8 (l / 32) ..
// + 7) of a backward tile.
template <int D>
__device__ __forceinline__ u32x4 rd_row(const char* t, int rb, int s, int lane) {
    const uint32_t row = 32 * rb + (lane & 31), c = 2 * s + (lane >> 5);
    return lds_read16(t, row * (2 * D) + ((c ^ swz_b<D / 8>(row)) * 16));
}

// Transposed fragment: A operand whose rows are d (block db of 32) and whose
// 16 contraction indices are tile rows of step c of the 32-row block rb, in
// the order in which a 32x32 accumulator holds its rows (the order the
// forward uses for V^T).
template <int D>
__device__ __forceinline__ u32x4 rd_tr(const char* t, int db, int rb, int c, int lane) {
    constexpr int CH = D / 8;
    const uint32_t G = lane >> 4, s = lane & 15;
    const uint32_t d = 32 * db + 16 * (G & 1) + 4 * (s & 3);
    const uint32_t r1 = 32 * rb + 16 * c + 4 * (G >> 1) + (s >> 2);
    const uint32_t r2 = r1 + 8;
    const uint32_t a1 = r1 * (2 * D) + (((d >> 3) ^ swz_b<CH>(r1)) * 16) + (d & 7) * 2;
    const uint32_t a2 = r2 * (2 * D) + (((d >> 3) ^ swz_b<CH>(r2)) * 16) + (d & 7) * 2;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(t + a1));
    const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(t + a2));
    const u32x2 w1 = __builtin_bit_cast(u32x2, x1), w2 = __builtin_bit_cast(u32x2, x2);
    return u32x4{w1[0], w1[1], w2[0], w2[1]};
}

// Rows held by register r of a 32x32 accumulator in this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// bf16 B operands (two 16-row steps) from a 32x32 accumulator.
__device__ __forceinline__ void pack_acc(const f32x16& x, u32x4 (&w)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[c][j] = pack_bf16x2(x[8 * c + 2 * j], x[8 * c + 2 * j + 1]);
}

// Write a [32 rows of d, 32 columns] accumulator block (scaled) as bf16 into
// row `dst` of a [.., d] tensor: this lane's column, d values 32 db + 8 g +
// 4 (l / 32) .. + 3.
template <int DB>
__device__ __forceinline__ void store_rows_bf16(uint16_t* dst, const f32x16 (&acc)[DB], float mul, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w = {pack_bf16x2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                       pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
            *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * g + 4 * h) = w;
        }
}

// ---- D = rowsum(G * O) and lse in log2 units ---------------------------------
// One wave per 16 consecutive rows of one query head: LPI lanes form one
// row's dot product per pass, and the 16 results are gathered into lanes
// 0..15 so that each of the two workspace arrays gets one contiguous 64-byte
// write per wave (with one row per lane group and the heads interleaved, every
// 4-byte result landed in a sector of its own).  The head index runs fastest
// over the waves, so neighbouring waves read neighbouring head slices of the
// same rows and the grid sweeps O and G front to back; each byte is read once,
// with non-temporal loads.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdParams p) {
    constexpr int LPI = D / 8;        // lanes per row
    constexpr int RPP = 64 / LPI;     // rows per pass
    constexpr int PASSES = 16 / RPP;  // 16 rows per wave
    const int lane = threadIdx.x & 63;
    const long job = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int h = (int)(job % p.hq);
    const long r0 = (job / p.hq) * 16;
    if (r0 >= p.total_q) return;
    float xs[PASSES];
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const long row = r0 + pass * RPP + lane / LPI;
        float x = 0.0f;
        if (row < p.total_q) {
            const long off = (row * p.hq + h) * D + (lane % LPI) * 8;
            const u32x4 o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.out + off));
            const u32x4 g = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.dout + off));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x += __uint_as_float(o[j] << 16) * __uint_as_float(g[j] << 16);
                x += __uint_as_float(o[j] & 0xffff0000u) * __uint_as_float(g[j] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int m = LPI / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        xs[pass] = x;
    }
    // lane i < 16 takes row r0 + i: pass i / RPP, lane group i % RPP
    float mine = 0.0f;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const float t = __shfl(xs[pass], LPI * (lane % RPP), 64);
        if (lane / RPP == pass) mine = t;
    }
    const long row = r0 + lane;
    if (lane < 16 && row < p.total_q) {
        const long w = (long)h * p.total_q + row;
        p.dsum[w] = mine;
        long li;
        if (p.cu_q != nullptr) {
            li = w;  // packed lse layout [hq, total_q]
        } else {
            const long b = row / p.max_q, i = row % p.max_q;
            li = (b * p.hq + h) * p.max_q + i;
        }
        const float l = p.lse[li];
        p.lse2[w] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
}

// ---- dK, dV ----------------------------------------------------------------
// Wave w owns keys j0 + 32 w .. + 31 (lane l: key l % 32).  Per 64-row query
// block: S = Q K^T and dP = G V^T (query rows x this wave's keys), P, dS, then
// dV^T += G^T P and dK^T += Q^T dS with G and Q read transposed from LDS.
// Work item of a dK/dV or dQ workgroup: tile index (key tiles for dK/dV,
// query tiles counted from the last for dQ, so both run the heaviest causal
// tiles first) and (sequence, head) index bh < BH.  Workgroups are dealt to
// the 8 XCDs round-robin.  When each XCD's share of heads (BH / 8) is a
// multiple of 4, an XCD runs its heads four at a time, all tiles of the four
// together (tile-major within the group), so the workgroups that stream the
// same Q and dO (dK/dV) or K and V (dQ) rows run together while those rows
// are in the L2: on causal MHA B=4 H=16 N=4096, d=128 the dK/dV kernel's HBM
// fetch per launch fell from 732 to 433 MiB and the dQ kernel's from 563 to
// 405 MiB, with the same time.  Otherwise the tile index runs slowest and
// the heads fastest over the grid.
__device__ __forceinline__ void bwd_work_item(const BwdParams& p, int BH, int& tile, int& bh) {
    const int bid = blockIdx.x;
    if ((BH & 31) == 0) {
        const int x = bid & 7, kk = bid >> 3;
        const int g = (int)udiv_apply(kk, p.dv_gt);  // 4 * n_tiles items per group
        const int j = kk - g * 4 * p.n_tiles;
        tile = j >> 2;
        bh = x * (BH >> 3) + 4 * g + (j & 3);
    } else {
        tile = (int)udiv_apply(bid, p.dv_bh);
        bh = bid - tile * BH;
    }
}

template <int D, int NW, int WPE, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_bwd_dkdv_kernel(BwdParams p) {
    constexpr int QBLK = 64;       // query rows per LDS stage
    constexpr int KT = 32 * NW;    // keys per workgroup
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    using Tile = BwdTile<D, QBLK, NW>;
    constexpr uint32_t STAGE = Tile::BYTES + 2 * QBLK * 4;  // Q, G, then lse2 and D of the block
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;

    // Key tiles in ascending order: under a causal mask the first key tiles
    // are seen by the most query rows, so the heaviest work starts first.
    const int BH = p.batch * p.hkv;
    int kt, bh;
    bwd_work_item(p, BH, kt, bh);
    const int b = (int)udiv_apply(bh, p.dv_h);
    const int kvh = bh - b * p.hkv;
    int q_off, k_off, Nq, Nk;
    if constexpr (VARLEN) {
        q_off = p.cu_q[b];
        Nq = p.cu_q[b + 1] - q_off;
        k_off = p.cu_k[b];
        Nk = p.cu_k[b + 1] - k_off;
        Nq = Nq < 0 ? 0 : Nq;
        Nk = Nk < 0 ? 0 : Nk;
    } else {
        q_off = b * p.max_q;
        Nq = p.max_q;
        k_off = b * p.max_k;
        Nk = p.max_k;
    }
    const int j0 = kt * KT;
    if (j0 >= Nk) return;
    const int kw0 = j0 + 32 * wave;
    const int key = kw0 + l32;
    const int shift = Nk - Nq;  // causal: row i sees keys j <= i + shift

    // K and V fragments (B operands), resident for the whole loop.
    u32x4 kf[KS], vf[KS];
    {
        const long off = ((long)(k_off + key) * p.hkv + kvh) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
            if (key < Nk) {
                zk = load16(p.k + off + (2 * s + (lane >> 5)) * 8);
                zv = load16(p.v + off + (2 * s + (lane >> 5)) * 8);
            }
            kf[s] = zk;
            vf[s] = zv;
        }
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[db][r] = 0.0f;
            dv[db][r] = 0.0f;
        }

    // Query blocks that see at least one key of this workgroup.
    const int g = p.grp;
    int qb_lo = 0;
    if constexpr (CAUSAL) {
        const int i_min = j0 - shift;  // first row that sees key j0
        qb_lo = i_min > 0 ? i_min / QBLK : 0;
    }
    const int qb_hi = (Nq + QBLK - 1) / QBLK;
    const int n_qb = qb_hi > qb_lo ? qb_hi - qb_lo : 0;
    const int n_it = g * n_qb;
    const uint32_t stride_q = (uint32_t)p.hq * D * 2;
    const float c2 = p.scale * kLog2e;

    auto issue = [&](int it, char* st) __attribute__((always_inline)) {
        const int h = kvh * g + it / n_qb;
        const int qs = (qb_lo + it % n_qb) * QBLK;
        const long off = ((long)(q_off + qs) * p.hq + h) * D;
        Tile::issue(p.q + off, p.dout + off, stride_q, Nq - qs, lds_addr(st), wave, lane);
        if (wave == 0) {
            // lse2 rows to bytes [0, 256) after the tiles (lanes 0-15), D rows
            // to [256, 512) (lanes 16-31): an LDS-DMA lane writes at the M0
            // base + 16 * lane, and each instruction takes one range.
            const int nv = Nq - qs < QBLK ? Nq - qs : QBLK;
            const long w = (long)h * p.total_q + q_off + qs;
            const uint32_t voff = (uint32_t)(lane & 15) * 16;
            if (lane < 16) dma16(rsrc_words(p.lse2 + w, (uint32_t)nv * 4), lds_addr(st) + Tile::BYTES, voff);
            if (lane >= 16 && lane < 32)
                dma16(rsrc_words(p.dsum + w, (uint32_t)nv * 4), lds_addr(st) + Tile::BYTES, voff);
        }
    };

    if (n_it > 0) issue(0, stage0);
    wait_vmem();
    __syncthreads();

    auto step = [&](int it, char* cur, char* nxt) __attribute__((always_inline)) {
        if (it + 1 < n_it) issue(it + 1, nxt);
        const int qs = (qb_lo + it % n_qb) * QBLK;
        // This wave's first key is seen from row kw0 - shift on.
        const bool active = kw0 < Nk && (!CAUSAL || qs + QBLK - 1 >= kw0 - shift);
        if (active) {
            const char* qt = cur;
            const char* gt = cur + Tile::A_BYTES;
            const float* lv = reinterpret_cast<const float*>(cur + Tile::BYTES);
            const bool need_mask = (qs + QBLK > Nq) || (kw0 + 31 >= Nk) ||
                                   (CAUSAL && kw0 + 31 > qs + shift);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x16 sacc, pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[r] = 0.0f;
                    pacc[r] = 0.0f;
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sacc = mfma32(rd_row<D>(qt, rb, s, lane), kf[s], sacc);
                    pacc = mfma32(rd_row<D>(gt, rb, s, lane), vf[s], pacc);
                }
                // Q and G row reads kept six products ahead.
                __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
                for (int i = 0; i < 2 * KS - 6; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
                // lse2 and D of the 16 rows this lane holds: rows 32 rb + 8 q4 + 4 (l / 32) .. + 3.
                f32x4 l2[4], dd[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int r0 = 32 * rb + 8 * q4 + 4 * (lane >> 5);
                    l2[q4] = *reinterpret_cast<const f32x4*>(lv + r0);
                    dd[q4] = *reinterpret_cast<const f32x4*>(lv + QBLK + r0);
                }
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = qs + 32 * rb + acc_row(r, lane);
                        const bool keep = i < Nq && key < Nk && (!CAUSAL || key <= i + shift);
                        if (!keep) sacc[r] = -INFINITY;
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c2, -l2[r >> 2][r & 3]));
                    sacc[r] = pr;
                    pacc[r] = pr * (pacc[r] - dd[r >> 2][r & 3]);
                }
                u32x4 pp[2], pds[2];
                pack_acc(sacc, pp);
                pack_acc(pacc, pds);
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        dv[db] = mfma32(rd_tr<D>(gt, db, rb, c, lane), pp[c], dv[db]);
                        dk[db] = mfma32(rd_tr<D>(qt, db, rb, c, lane), pds[c], dk[db]);
                    }
                // Transposed reads kept two products ahead.
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 4 * DB - 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        }
        wait_vmem();
        __syncthreads();
    };
    for (int it = 0; it < n_it; it += 2) {
        step(it, stage0, stage1);
        if (it + 1 < n_it) step(it + 1, stage1, stage0);
    }

    {
        // dK then dV rows through the wave's own LDS region (the stages are
        // free after the last barrier): 16-byte stores of whole rows.
        constexpr uint32_t WB = 32u * D * 2;
        static_assert((NW / 2) * WB <= STAGE, "output staging fits the stages");
        char* const ob = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WB;
        const long off = ((long)(k_off + kw0) * p.hkv + kvh) * D;
        store_rows_bf16_staged<DB>(ob, dk, p.scale, lane, p.dk + off, (long)p.hkv * D, Nk - kw0);
        store_rows_bf16_staged<DB>(ob, dv, 1.0f, lane, p.dv + off, (long)p.hkv * D, Nk - kw0);
    }
}

// dK, dV with the work of each 32-key group split over a pair of waves, so
// that two waves per SIMD fit the registers (one wave holding both dK and dV
// and K and V needs about 360): wave w (w < NP) forms S = Q K^T, the mask
// and P = exp(S - lse), hands P to wave w + NP through LDS and accumulates
// dV^T += G^T P; wave w + NP forms dP = G V^T, dS = P o (dP - D) and
// accumulates dK^T += Q^T dS.  At d = 128 the two waves of a pair share a
// SIMD (waves w and w + 4 of an 8-wave workgroup, two waves per SIMD), so
// each one's vector work runs beside the other's matrix products; at d = 256
// one accumulator and the K or V fragments alone take a wave's registers at
// two waves per SIMD, so two pairs run at one wave per SIMD.  Same arithmetic
// and the same order of accumulation per register as attn_bwd_dkdv_kernel.
template <int D, int NP, int WPE, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(2 * NP * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_bwd_dkdv_pair_kernel(BwdParams p) {
    constexpr int NW = 2 * NP;
    constexpr int QBLK = 64;       // query rows per LDS stage
    constexpr int KT = 32 * NP;    // keys per workgroup
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    using Tile = BwdTile<D, QBLK, NW>;
    constexpr uint32_t STAGE = Tile::BYTES + 2 * QBLK * 4;  // Q, G, then lse2 and D of the block
    constexpr uint32_t XBYTES = 2 * 16 * 64 * 4;            // P of one pair: 2 blocks x 16 floats x 64 lanes
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage2[D == 128 ? STAGE : 16];  // d = 128 only
    __shared__ __attribute__((aligned(1024))) char xchg[NP * XBYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool side_p = wave < NP;  // P side (S, mask, exp, dV) or dS side (dP, dS, dK)
    const int pair = side_p ? wave : wave - NP;
    const int l32 = lane & 31;

    const int BH = p.batch * p.hkv;
    int kt, bh;
    bwd_work_item(p, BH, kt, bh);
    const int b = (int)udiv_apply(bh, p.dv_h);
    const int kvh = bh - b * p.hkv;
    int q_off, k_off, Nq, Nk;
    if constexpr (VARLEN) {
        q_off = p.cu_q[b];
        Nq = p.cu_q[b + 1] - q_off;
        k_off = p.cu_k[b];
        Nk = p.cu_k[b + 1] - k_off;
        Nq = Nq < 0 ? 0 : Nq;
        Nk = Nk < 0 ? 0 : Nk;
    } else {
        q_off = b * p.max_q;
        Nq = p.max_q;
        k_off = b * p.max_k;
        Nk = p.max_k;
    }
    const int j0 = kt * KT;
    if (j0 >= Nk) return;
    const int kw0 = j0 + 32 * pair;
    const int key = kw0 + l32;
    const int shift = Nk - Nq;  // causal: row i sees keys j <= i + shift

    // K (P side) or V (dS side) fragments of the pair's 32 keys, resident.
    u32x4 kv[KS];
    {
        const long off = ((long)(k_off + key) * p.hkv + kvh) * D;
        const uint16_t* src = side_p ? p.k : p.v;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (key < Nk) z = load16(src + off + (2 * s + (lane >> 5)) * 8);
            kv[s] = z;
        }
    }
    f32x16 acc[DB];  // dV^T (P side) or dK^T (dS side)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    const int g = p.grp;
    int qb_lo = 0;
    if constexpr (CAUSAL) {
        const int i_min = j0 - shift;
        qb_lo = i_min > 0 ? i_min / QBLK : 0;
    }
    const int qb_hi = (Nq + QBLK - 1) / QBLK;
    const int n_qb = qb_hi > qb_lo ? qb_hi - qb_lo : 0;
    const int n_it = g * n_qb;
    const uint32_t stride_q = (uint32_t)p.hq * D * 2;
    const float c2 = p.scale * kLog2e;
    // This pair's P: float index ((rb * 4 + q) * 64 + lane) * 4 + j holds register 4 q + j of block rb.
    f32x4* const xp = reinterpret_cast<f32x4*>(xchg + pair * XBYTES);

    auto issue = [&](int it, char* st) __attribute__((always_inline)) {
        const int h = kvh * g + it / n_qb;
        const int qs = (qb_lo + it % n_qb) * QBLK;
        const long off = ((long)(q_off + qs) * p.hq + h) * D;
        Tile::issue(p.q + off, p.dout + off, stride_q, Nq - qs, lds_addr(st), wave, lane);
        if (wave == 0) {
            const int nv = Nq - qs < QBLK ? Nq - qs : QBLK;
            const long w = (long)h * p.total_q + q_off + qs;
            const uint32_t voff = (uint32_t)(lane & 15) * 16;
            if (lane < 16) dma16(rsrc_words(p.lse2 + w, (uint32_t)nv * 4), lds_addr(st) + Tile::BYTES, voff);
            if (lane >= 16 && lane < 32)
                dma16(rsrc_words(p.dsum + w, (uint32_t)nv * 4), lds_addr(st) + Tile::BYTES, voff);
        }
    };

    if (n_it > 0) issue(0, stage0);
    wait_vmem();
    __syncthreads();

    // Phase 1 products of block it: S^T = K Q^T (P side) or dP^T = V G^T (dS
    // side), two accumulation chains interleaved, the LDS reads of the Q (G)
    // rows kept six products ahead.
    auto phase1_products = [&](const char* rows, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sacc[rb] = mfma32(rd_row<D>(rows, rb, s, lane), kv[s], sacc[rb]);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 2 * KS - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    };
    // P side, after phase 1: mask, P = exp2(S scale log2e - lse2), P to LDS
    // for the dS side, and P as bf16 B operands.
    auto make_p = [&](int qs, const float* lv, f32x16 (&sacc)[2], u32x4 (&pw)[2][2]) __attribute__((always_inline)) {
        const bool need_mask = (qs + QBLK > Nq) || (kw0 + 31 >= Nk) || (CAUSAL && kw0 + 31 > qs + shift);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = qs + 32 * rb + acc_row(r, lane);
                    const bool keep = i < Nq && key < Nk && (!CAUSAL || key <= i + shift);
                    if (!keep) sacc[rb][r] = -INFINITY;
                }
            }
            // lse2 of the 16 rows this lane holds: rows 32 rb + 8 q4 + 4 (l / 32) .. + 3.
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 l2 = *reinterpret_cast<const f32x4*>(lv + 32 * rb + 8 * q4 + 4 * (lane >> 5));
                f32x4 pr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pr[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rb][4 * q4 + j], c2, -l2[j]));
                    sacc[rb][4 * q4 + j] = pr[j];
                }
                xp[(rb * 4 + q4) * 64 + lane] = pr;
            }
            pack_acc(sacc[rb], pw[rb]);
        }
    };
    // dS side, after the barrier: dS = P o (dP - D) as bf16 B operands.
    auto make_ds = [&](const float* lv, f32x16 (&sacc)[2], u32x4 (&pw)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 pr = xp[(rb * 4 + q4) * 64 + lane];
                const f32x4 dd = *reinterpret_cast<const f32x4*>(lv + QBLK + 32 * rb + 8 * q4 + 4 * (lane >> 5));
#pragma unroll
                for (int j = 0; j < 4; ++j) sacc[rb][4 * q4 + j] = pr[j] * (sacc[rb][4 * q4 + j] - dd[j]);
            }
            pack_acc(sacc[rb], pw[rb]);
        }
    };
    // acc += rows^T B over the block's 64 rows: dV^T += G^T P or dK^T += Q^T dS,
    // the transposed LDS reads kept two products ahead.
    auto phase2_products = [&](const char* rows, const u32x4 (&pw)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] = mfma32(rd_tr<D>(rows, db, rb, c, lane), pw[rb][c], acc[db]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4 * DB - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    if constexpr (D == 128) {
        // Three stages.  The dS side adds dK^T for block it-1 in phase 1 of
        // step it, beside its own dP products and the P side's exponentials,
        // from that block's dS (kept in registers) and stage (the loads of
        // block it+1 go to the third stage).  Each side runs its own copy of
        // the loop, with the same barriers, so that registers one side needs
        // are not held on the other.  The order of accumulation into dK is
        // unchanged: bitwise-identical gradients.
        auto run = [&](auto side) __attribute__((always_inline)) {
            constexpr bool SP = decltype(side)::value;
            u32x4 ds_prev[2][2];
            bool act_prev = false;
            const char* qt_prev = stage0;
            auto step = [&](int it, char* cur, char* nxt) __attribute__((always_inline)) {
                if (it + 1 < n_it) issue(it + 1, nxt);
                const int qs = (qb_lo + it % n_qb) * QBLK;
                const bool active = kw0 < Nk && (!CAUSAL || qs + QBLK - 1 >= kw0 - shift);
                const char* qt = cur;
                const char* gt = cur + Tile::A_BYTES;
                const float* lv = reinterpret_cast<const float*>(cur + Tile::BYTES);
                f32x16 sacc[2];
                u32x4 pw[2][2];
                if (active) {
                    phase1_products(SP ? qt : gt, sacc);
                    if constexpr (SP) make_p(qs, lv, sacc, pw);
                }
                if constexpr (!SP) {
                    if (act_prev) phase2_products(qt_prev, ds_prev);
                }
                // P is in LDS for the dS side.
                __syncthreads();
                if (active) {
                    if constexpr (SP)
                        phase2_products(gt, pw);
                    else
                        make_ds(lv, sacc, ds_prev);
                }
                act_prev = active;
                qt_prev = qt;
                // The next block has landed, and the dS side has read P
                // before the P side overwrites it.
                wait_vmem();
                __syncthreads();
            };
            for (int it = 0; it < n_it; it += 3) {
                step(it, stage0, stage1);
                if (it + 1 < n_it) step(it + 1, stage1, stage2);
                if (it + 2 < n_it) step(it + 2, stage2, stage0);
            }
            if constexpr (!SP) {
                if (act_prev) phase2_products(qt_prev, ds_prev);
            }
        };
        if (side_p)
            run(std::true_type{});
        else
            run(std::false_type{});
    } else {
        // d = 256: two stages (three do not fit the LDS); both products of a
        // side within its step.
        auto step = [&](int it, char* cur, char* nxt) __attribute__((always_inline)) {
            if (it + 1 < n_it) issue(it + 1, nxt);
            const int qs = (qb_lo + it % n_qb) * QBLK;
            const bool active = kw0 < Nk && (!CAUSAL || qs + QBLK - 1 >= kw0 - shift);
            const char* qt = cur;
            const char* gt = cur + Tile::A_BYTES;
            const float* lv = reinterpret_cast<const float*>(cur + Tile::BYTES);
            f32x16 sacc[2];
            u32x4 pw[2][2];  // packed P (P side) or dS (dS side) B operands
            if (active) {
                phase1_products(side_p ? qt : gt, sacc);
                if (side_p) make_p(qs, lv, sacc, pw);
            }
            // P is in LDS for the dS side.
            __syncthreads();
            if (active) {
                if (!side_p) make_ds(lv, sacc, pw);
                phase2_products(side_p ? gt : qt, pw);
            }
            wait_vmem();
            __syncthreads();
        };
        for (int it = 0; it < n_it; it += 2) {
            step(it, stage0, stage1);
            if (it + 1 < n_it) step(it + 1, stage1, stage0);
        }
    }

    // dV (P side) or dK (dS side) rows through LDS: the dS side's last dK
    // products may still read a stage, so every wave first passes a barrier.
    __syncthreads();
    {
        constexpr uint32_t WB = 32u * D * 2;
        static_assert((NW / 2) * WB <= STAGE, "output staging fits the stages");
        char* const ob = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WB;
        const long off = ((long)(k_off + kw0) * p.hkv + kvh) * D;
        store_rows_bf16_staged<DB>(ob, acc, side_p ? 1.0f : p.scale, lane, (side_p ? p.dv : p.dk) + off,
                                   (long)p.hkv * D, Nk - kw0);
    }
}

// ---- dQ ------------------------------------------------------------------------
// Shaped like the forward: wave w owns query rows q0 + 32 w .. + 31 (lane l:
// row l % 32).  Per 64-key tile: S^T = K Q^T and dP^T = V G^T, P^T, dS^T,
// then dQ^T += K^T dS^T with K read transposed from LDS.
template <int D, int NW, int WPE, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_bwd_dq_kernel(BwdParams p) {
    constexpr int BC = 64;
    constexpr int KB = BC / 32;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int BR = 32 * NW;
    using Tile = BwdTile<D, BC, NW>;
    __shared__ __attribute__((aligned(1024))) char stage0[Tile::BYTES];
    __shared__ __attribute__((aligned(1024))) char stage1[Tile::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;

    // Heaviest query tiles first.
    const int BH = p.batch * p.hq;
    int qq, bh;
    bwd_work_item(p, BH, qq, bh);
    const int qt = p.n_tiles - 1 - qq;
    const int b = (int)udiv_apply(bh, p.dv_h);
    const int hq = bh - b * p.hq;
    const int kvh = (int)udiv_apply(hq, p.dv_grp);
    int q_off, k_off, Nq, Nk;
    if constexpr (VARLEN) {
        q_off = p.cu_q[b];
        Nq = p.cu_q[b + 1] - q_off;
        k_off = p.cu_k[b];
        Nk = p.cu_k[b + 1] - k_off;
        Nq = Nq < 0 ? 0 : Nq;
        Nk = Nk < 0 ? 0 : Nk;
    } else {
        q_off = b * p.max_q;
        Nq = p.max_q;
        k_off = b * p.max_k;
        Nk = p.max_k;
    }
    const int q0 = qt * BR;
    if (q0 >= Nq) return;
    int n_tiles = (Nk + BC - 1) / BC;
    if constexpr (CAUSAL) {
        const int kmax = min(q0 + BR, Nq) - 1 + Nk - Nq;
        n_tiles = kmax < 0 ? 0 : min(n_tiles, kmax / BC + 1);
    }
    const uint32_t stride_k = (uint32_t)p.hkv * D * 2;
    const uint16_t* kbase = p.k + ((long)k_off * p.hkv + kvh) * D;
    const uint16_t* vbase = p.v + ((long)k_off * p.hkv + kvh) * D;

    const int wr0 = q0 + 32 * wave;
    const bool wave_rows = wr0 < Nq;
    const int w_last_key = min(wr0 + 32, Nq) - 1 + Nk - Nq;
    const int w_first_key_lim = wr0 + Nk - Nq;
    const int row = wr0 + l32;

    // Q^T and G^T fragments (B operands), and this row's lse2 and D.
    u32x4 qf[KS], gf[KS];
    float l2 = INFINITY, dd = 0.0f;
    {
        const long off = ((long)(q_off + row) * p.hq + hq) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 zq = {0u, 0u, 0u, 0u}, zg = {0u, 0u, 0u, 0u};
            if (row < Nq) {
                zq = load16(p.q + off + (2 * s + (lane >> 5)) * 8);
                zg = load16(p.dout + off + (2 * s + (lane >> 5)) * 8);
            }
            qf[s] = zq;
            gf[s] = zg;
        }
        if (row < Nq) {
            const long w = (long)hq * p.total_q + q_off + row;
            l2 = p.lse2[w];
            dd = p.dsum[w];
        }
    }
    f32x16 dacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dacc[db][r] = 0.0f;
    const float c2 = p.scale * kLog2e;

    if (n_tiles > 0) Tile::issue(kbase, vbase, stride_k, Nk, lds_addr(stage0), wave, lane);
    wait_vmem();
    __syncthreads();

    auto step = [&](const int t, char* cur, char* nxt) __attribute__((always_inline)) {
        const char* ks = cur;
        const char* vs = cur + Tile::A_BYTES;
        if (t + 1 < n_tiles) {
            const long off = (long)(t + 1) * BC * p.hkv * D;
            Tile::issue(kbase + off, vbase + off, stride_k, Nk - (t + 1) * BC, lds_addr(nxt), wave, lane);
        }
        const int k0 = t * BC;
        const bool active = wave_rows && (!CAUSAL || k0 <= w_last_key);
        if (active) {
            const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > w_first_key_lim);
            const int lim = CAUSAL ? min(Nk - 1, row + Nk - Nq) : Nk - 1;
            // One 32-key block at a time keeps two accumulators live, not four.
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 sacc, pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[r] = 0.0f;
                    pacc[r] = 0.0f;
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sacc = mfma32(rd_row<D>(ks, kb, s, lane), qf[s], sacc);
                    pacc = mfma32(rd_row<D>(vs, kb, s, lane), gf[s], pacc);
                }
                if constexpr (D != 256) {  // (at d = 256 the reads ahead would spill)
                    // K and V row reads kept six products ahead.
                    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
                    for (int i = 0; i < 2 * KS - 6; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
                }
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (k0 + 32 * kb + acc_row(r, lane) > lim) sacc[r] = -INFINITY;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c2, -l2));
                    pacc[r] = pr * (pacc[r] - dd);
                }
                u32x4 pds[2];
                pack_acc(pacc, pds);
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        dacc[db] = mfma32(rd_tr<D>(ks, db, kb, c, lane), pds[c], dacc[db]);
                if constexpr (D != 256) {
                    // Transposed K reads kept three products ahead.
                    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
                    for (int i = 0; i < 2 * DB - 3; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                }
            }
        }
        wait_vmem();
        __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, stage0, stage1);
        if (t + 1 < n_tiles) step(t + 1, stage1, stage0);
    }

    {
        // dQ rows through LDS (the wave's own region of the stages, free after
        // the last barrier): 16-byte stores of whole rows.
        constexpr uint32_t WB = 32u * D * 2;
        static_assert((NW / 2) * WB <= Tile::BYTES, "output staging fits the stages");
        char* const ob = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WB;
        store_rows_bf16_staged<DB>(ob, dacc, p.scale, lane, p.dq + ((long)(q_off + wr0) * p.hq + hq) * D,
                                   (long)p.hq * D, Nq - wr0);
    }
}

// ---- launchers -------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_bwd_cfg(const BwdParams& p0, hipStream_t s) {
    constexpr int DKDV_NW = 4, DKDV_WPE = 2;  // d = 64: two 4-wave workgroups per CU
    // d = 128: 4 pairs at two waves per SIMD; d = 256: 2 pairs at one.
    constexpr int PAIR_NP = D == 256 ? 2 : 4, PAIR_WPE = D == 256 ? 1 : 2;
    // dQ: 8 waves at two per SIMD; at d = 256 the Q, G and dQ registers of a
    // 32-row wave take a SIMD's budget, so 4 waves at one per SIMD.
    constexpr int DQ_NW = D == 256 ? 4 : 8, DQ_WPE = D == 256 ? 1 : 2;
    BwdParams p = p0;
    p.grp = p.hkv > 0 ? p.hq / p.hkv : 1;
    p.dv_grp = udiv_make(p.grp);
    {
        const long waves = ((long)p.total_q + 15) / 16 * p.hq;  // 16 rows of one head per wave
        const long grid = (waves + 3) / 4;
        if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
        if (grid > 0) hipLaunchKernelGGL(attn_bwd_prep_kernel<D>, dim3((unsigned)grid), dim3(256), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        constexpr int KT = 32 * (D >= 128 ? PAIR_NP : DKDV_NW);
        p.n_tiles = (p.max_k + KT - 1) / KT;
        const long grid = (long)p.n_tiles * p.batch * p.hkv;
        if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
        p.dv_bh = udiv_make((uint32_t)((long)p.batch * p.hkv));  // below 2^31 after the check
        p.dv_h = udiv_make(p.hkv);
        p.dv_gt = udiv_make((uint32_t)(4L * p.n_tiles));  // used when B * Hkv is a multiple of 32
        if (grid > 0) {
            // d >= 128: one wave would hold both accumulators, so the work of
            // each 32-key group is split over a pair of waves.
            if constexpr (D >= 128)
                hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<D, PAIR_NP, PAIR_WPE, CAUSAL, VARLEN>),
                                   dim3((unsigned)grid), dim3(2 * PAIR_NP * 64), 0, s, p);
            else
                hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, DKDV_NW, DKDV_WPE, CAUSAL, VARLEN>),
                                   dim3((unsigned)grid), dim3(DKDV_NW * 64), 0, s, p);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        constexpr int BR = 32 * DQ_NW;
        p.n_tiles = (p.max_q + BR - 1) / BR;
        const long grid = (long)p.n_tiles * p.batch * p.hq;
        if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
        p.dv_bh = udiv_make((uint32_t)((long)p.batch * p.hq));  // below 2^31 after the check
        p.dv_h = udiv_make(p.hq);
        p.dv_gt = udiv_make((uint32_t)(4L * p.n_tiles));  // used when B * Hq is a multiple of 32
        if (grid > 0)
            hipLaunchKernelGGL((attn_bwd_dq_kernel<D, DQ_NW, DQ_WPE, CAUSAL, VARLEN>), dim3((unsigned)grid),
                               dim3(DQ_NW * 64), 0, s, p);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool varlen, hipStream_t s) {
    if (causal) return varlen ? launch_bwd_cfg<D, true, true>(p, s) : launch_bwd_cfg<D, true, false>(p, s);
    return varlen ? launch_bwd_cfg<D, false, true>(p, s) : launch_bwd_cfg<D, false, false>(p, s);
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, bool varlen, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_bwd_d<64>(p, causal, varlen, s);
        case 128: return launch_bwd_d<128>(p, causal, varlen, s);
        case 256: return launch_bwd_d<256>(p, causal, varlen, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
