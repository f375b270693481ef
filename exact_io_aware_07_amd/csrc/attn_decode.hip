// Split-KV one-token decode over a paged KV cache, and the combine step (gfx950).
//
// "FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels (2026)",
// "Why decode starves the GPU": with one query per request, batch x heads
// leaves most compute units idle, so the cached keys are cut into chunks that
// run in parallel, each emitting a partial output and its log-sum-exp; a
// second small kernel merges them with weights exp(lse_c - lse_total).
// "How GQA and MLA reshape the problem": the g = Hq / Hkv query heads that
// share a K/V head are processed as the rows of one tile, so every cache row
// is read from memory once for all of them.
// "Deep Dive - FlashAttention", "Paged KV is a lookup, not a cache manager":
// logical key t of request b is row t % page of physical page
// block_table[b][t / page].
//
#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

constexpr int kPage = 256;

// Build-time knobs of the split kernel (defaults are the measured best):
// keep the 8 K/V heads of a (request, chunk) on one XCD, and the waves per
// SIMD the register budget targets.
#ifndef ATTN_DEC_XCD_GROUP
#define ATTN_DEC_XCD_GROUP 0
#endif
#ifndef ATTN_DEC_WPE
#define ATTN_DEC_WPE 1
#endif

// Split kernel: one wave (one workgroup) per (chunk, K/V head, request).  The
// chunk is walked in tiles of 32 keys that never straddle a page; K and V of a
// tile go straight from HBM into LDS (16-byte buffer loads with the lds flag,
// zeros past the valid rows), V is read back transposed, and NS LDS stages
// keep NS - 1 tiles in flight while one is computed, so each wave sustains
// several tens of KiB of outstanding reads without any barrier.
template <int D, int QB, int NS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ATTN_DEC_WPE)))
void attn_decode_split_kernel(DecodeParams p) {
    constexpr int BC = 32;
    constexpr int DB = D / 32;
    constexpr int KS = D / 16;
    static_assert(kPage % BC == 0, "tiles must not straddle pages");
    static_assert(NS >= 2 && NS <= 4, "stage count");
    using Tile = KVDirect<D, BC, 1>;
    constexpr int LOADS = 2 * Tile::PER_WAVE;  // load instructions per tile
    static_assert((NS - 1) * LOADS < 64, "outstanding loads must fit vmcnt");
    // Distinct LDS objects, named statically after unrolling, so that the
    // compiler never waits for in-flight DMA before reading a resident stage.
    __shared__ __attribute__((aligned(1024))) char stage0[Tile::BYTES];
    __shared__ __attribute__((aligned(1024))) char stage1[Tile::BYTES];
    __shared__ __attribute__((aligned(1024))) char stage2[NS > 2 ? Tile::BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char stage3[NS > 3 ? Tile::BYTES : 16];

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    // The K/V heads of one (request, chunk) read interleaved rows of the same
    // cache pages, so they run close together in time.  Workgroups are dealt
    // to the 8 XCDs round-robin; with ATTN_DEC_XCD_GROUP the heads of a
    // (request, chunk) are also kept on one XCD (one L2).
    int kvh, unit;
#if ATTN_DEC_XCD_GROUP
    if (p.hkv == 8) {
        const int bid = blockIdx.x;
        kvh = (bid >> 3) & 7;
        unit = (bid & 7) | ((bid >> 6) << 3);
    } else {
        kvh = blockIdx.x % p.hkv;
        unit = blockIdx.x / p.hkv;
    }
#else
    kvh = blockIdx.x % p.hkv;
    unit = blockIdx.x / p.hkv;
#endif
    const int split = unit % p.n_splits;
    const int b = unit / p.n_splits;
    if (b >= p.batch) return;  // padding of the grouped grid
    const int g = p.hq / p.hkv;
    const int hq0 = kvh * g;

    int Nk = p.seqlens[b];
    bool bad = false;
    if (Nk < 0) {
        Nk = 0;
        bad = true;
    }
    const long cap = (long)p.max_pages * kPage;
    if (Nk > cap) {
        Nk = (int)cap;
        bad = true;
    }
    const int key_begin = split * p.chunk;
    if (key_begin >= Nk && !(bad && split == 0)) return;
    const int key_end = min(Nk, key_begin + p.chunk);
    const int n_tiles = key_end > key_begin ? (key_end - key_begin + BC - 1) / BC : 0;

    const long row_stride = (long)p.hkv * D;
    const uint32_t stride_b = (uint32_t)(row_stride * 2);
    const int32_t* table = p.block_table + (long)b * p.max_pages;

    // Q^T fragments: rows are the g query heads of this K/V head.
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = 32 * qb + l32;
        const uint16_t* qrow = p.q + ((long)b * p.hq + hq0 + j) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (j < g) z = load16(qrow + (2 * s + (lane >> 5)) * 8);
            qf[qb][s] = z;
        }
    }

    // Q must be in registers before any tile DMA is issued: otherwise the
    // compiler cannot tell the Q loads from the DMA loads and drains every
    // outstanding load before each tile's first MFMA.
    wait_vmem();

    f32x16 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.0f;
    float m_run[QB], l_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_part[qb] = 0.0f;
    }
    const float c2 = p.scale * kLog2e;

    // Issue the loads of tile t into stage st (page lookup included).
    auto issue = [&](int t, char* st) __attribute__((always_inline)) {
        const int key0 = key_begin + t * BC;
        const int phys = table[key0 / kPage];
        int nvalid = min(BC, key_end - key0);
        const uint16_t* kb = p.k_cache;
        const uint16_t* vb = p.v_cache;
        if (phys < 0 || phys >= p.num_pages) {
            bad = true;
            nvalid = 0;
        } else {
            const long row0 = (long)phys * kPage + key0 % kPage;
            kb = p.k_cache + row0 * row_stride + (long)kvh * D;
            vb = p.v_cache + row0 * row_stride + (long)kvh * D;
        }
        Tile::issue(kb, vb, stride_b, nvalid, lds_addr(st), 0, lane);
    };
    // Wait until tile t has landed: the loads of the later tiles already
    // issued (at most NS - 1 of them) may stay in flight.
    auto wait_tile = [&](int t) __attribute__((always_inline)) {
        const int later = min(NS - 1, n_tiles - 1 - t);
        if (later >= NS - 1) {
            wait_vmem_le<(NS - 1) * LOADS>();
            return;
        }
        if constexpr (NS > 3) {
            if (later == 2) {
                wait_vmem_le<2 * LOADS>();
                return;
            }
        }
        if constexpr (NS > 2) {
            if (later == 1) {
                wait_vmem_le<LOADS>();
                return;
            }
        }
        wait_vmem();
    };
    auto compute = [&](int t, const char* st) __attribute__((always_inline)) {
        const char* ks = st;
        const char* vs = st + Tile::K_BYTES;
        const int nvalid = min(BC, key_end - (key_begin + t * BC));
        // S^T = K Q^T, two interleaved accumulation chains over d.
        f32x16 sacc[QB], sacc2[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[qb][r] = 0.0f;
                sacc2[qb][r] = 0.0f;
            }
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            const u32x4 a0 = read_k_frag<D>(ks, 0, s, lane);
            const u32x4 a1 = read_k_frag<D>(ks, 0, s + 1, lane);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                sacc[qb] = mfma32(a0, qf[qb][s], sacc[qb]);
                sacc2[qb] = mfma32(a1, qf[qb][s + 1], sacc2[qb]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb] += sacc2[qb];
        if (nvalid < BC) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (score_key(0, r, lane) >= nvalid) sacc[qb][r] = -INFINITY;
        }
        u32x4 pb[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][r]);
            mx = pair_max(mx);
            const float m_new = mx * c2;
            const bool raise = m_new > m_run[qb] + kRescaleThreshold;
            const bool scale_old = raise && (m_run[qb] != -INFINITY);
            if (__builtin_amdgcn_ballot_w64(scale_old)) {
                const float alpha = scale_old ? exp2f(m_run[qb] - m_new) : 1.0f;
                l_part[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
            }
            if (raise) m_run[qb] = m_new;
            const float shift = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
            float rs = 0.0f;
            float e[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c2, -shift));
                rs += e[r];
            }
            l_part[qb] += rs;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(e[8 * c + 2 * j], e[8 * c + 2 * j + 1]);
                pb[qb][c] = w;
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 a = read_vt_frag_tr<D>(vs, db, 0, c, lane);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(a, pb[qb][c], oacc[db][qb]);
            }
    };

    // Tile t lives in stage t % NS.  Step t first refills the stage that held
    // tile t - 1 (finished in the previous step) with tile t + NS - 1.
    auto step = [&](int t, const char* cur, char* refill) __attribute__((always_inline)) {
        if (t + NS - 1 < n_tiles) issue(t + NS - 1, refill);
        wait_tile(t);
        compute(t, cur);
    };
    if (n_tiles > 0) issue(0, stage0);
    if (NS > 2 && 1 < n_tiles) issue(1, stage1);
    if (NS > 3 && 2 < n_tiles) issue(2, stage2);
    for (int t = 0; t < n_tiles; t += NS) {
        if constexpr (NS == 4) {
            step(t, stage0, stage3);
            if (t + 1 < n_tiles) step(t + 1, stage1, stage0);
            if (t + 2 < n_tiles) step(t + 2, stage2, stage1);
            if (t + 3 < n_tiles) step(t + 3, stage3, stage2);
        } else if constexpr (NS == 3) {
            step(t, stage0, stage2);
            if (t + 1 < n_tiles) step(t + 1, stage1, stage0);
            if (t + 2 < n_tiles) step(t + 2, stage2, stage1);
        } else {
            step(t, stage0, stage1);
            if (t + 1 < n_tiles) step(t + 1, stage1, stage0);
        }
    }

    // ---- write the normalised partial and its lse ----------------------------
    const long part_row = ((long)split * p.batch + b) * p.hq + hq0;
    const int h = lane >> 5;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = 32 * qb + l32;
        const float L = pair_sum(l_part[qb]);
        if (j < g) {
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            float* orow = p.out_part + (part_row + j) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = bad ? NAN : oacc[db][qb][4 * q4 + i] * inv;
                    *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * q4 + 4 * h) = w;
                }
            if (h == 0) {
                float lse = L > 0.0f ? (m_run[qb] + __log2f(L)) * kLn2 : -INFINITY;
                if (bad) lse = NAN;
                p.lse_part[part_row + j] = lse;
            }
        }
    }
}

// One workgroup (one wave) per (request, query head).
template <int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(CombineParams p) {
    constexpr int PER = D / 64;
    const int bh = blockIdx.x;
    const int b = bh / p.hq;
    const int lane = threadIdx.x;
    int Nk = p.seqlens[b];
    const int n = Nk > 0 ? (Nk + p.chunk - 1) / p.chunk : 0;
    const bool bad = Nk < 0 || n > p.n_splits;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
    float M = -INFINITY;
    bool nan_seen = false;
    for (int c = 0; c < n && !bad; ++c) {
        const float x = p.lse_part[((long)c * p.batch) * p.hq + bh];
        nan_seen |= (x != x);
        M = fmaxf(M, x);
    }
    float L = 0.0f;
    if (!bad && M != -INFINITY) {
        for (int c = 0; c < n; ++c) {
            const long row = ((long)c * p.batch) * p.hq + bh;
            const float x = p.lse_part[row];
            const float w = __expf(x - M);
            L += w;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += w * p.out_part[row * D + lane + 64 * i];
        }
    }
    const bool poison = bad || nan_seen;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t* orow = p.out + (long)bh * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float o = poison ? NAN : acc[i] * inv;
        const uint32_t packed = pack_bf16x2(o, 0.0f);
        orow[lane + 64 * i] = (uint16_t)(packed & 0xffffu);
    }
    if (p.lse != nullptr && lane == 0)
        p.lse[bh] = poison ? NAN : (L > 0.0f ? M + __logf(L) : -INFINITY);
}

template <int D, int QB, int NS>
static hipError_t launch_split_cfg(const DecodeParams& p, hipStream_t s) {
    if (p.n_splits <= 0 || p.batch <= 0) return hipSuccess;
    long grid = (long)p.n_splits * p.hkv * p.batch;
    if (ATTN_DEC_XCD_GROUP && p.hkv == 8) grid = (grid + 63) / 64 * 64;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_decode_split_kernel<D, QB, NS>), dim3((unsigned)grid), dim3(64), 0, s, p);
    return hipGetLastError();
}

// LDS stages per wave (tiles in flight + 1).
#ifndef ATTN_DEC_STAGES
#define ATTN_DEC_STAGES 3
#endif

template <int D>
static hipError_t launch_split_d(const DecodeParams& p, hipStream_t s) {
    constexpr int NS = D >= 256 ? 2 : ATTN_DEC_STAGES;
    const int g = p.hq / p.hkv;
    return g <= 32 ? launch_split_cfg<D, 1, NS>(p, s) : launch_split_cfg<D, 2, NS>(p, s);
}

hipError_t launch_decode_split(const DecodeParams& p, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_split_d<64>(p, s);
        case 128: return launch_split_d<128>(p, s);
        case 256: return launch_split_d<256>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_combine(const CombineParams& p, int head_dim, hipStream_t s) {
    const long grid = (long)p.batch * p.hq;
    if (grid <= 0) return hipSuccess;
    switch (head_dim) {
        case 64:
            hipLaunchKernelGGL(attn_decode_combine_kernel<64>, dim3(grid), dim3(64), 0, s, p);
            break;
        case 128:
            hipLaunchKernelGGL(attn_decode_combine_kernel<128>, dim3(grid), dim3(64), 0, s, p);
            break;
        case 256:
            hipLaunchKernelGGL(attn_decode_combine_kernel<256>, dim3(grid), dim3(64), 0, s, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
