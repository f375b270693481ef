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
// Split kernel: one workgroup per (chunk, K/V head, request).  The chunk is
// walked in tiles of BC = 32 * NW keys inside one page; each wave owns 32 keys
// of every tile and keeps its own online-softmax state over them (the query
// rows are few, so the keys are what gets divided).  At the end the waves'
// states are merged in LDS, in a fixed order, and the chunk's normalised
// output and lse are written.

#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

constexpr int kPage = 256;

template <int D, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_split_kernel(DecodeParams p) {
    constexpr int NT = NW * 64;
    constexpr int BC = 32 * NW;
    constexpr int DB = D / 32;
    constexpr int KS = D / 16;
    static_assert(kPage % BC == 0, "tiles must not straddle pages");
    using Tile = KVTile<D, BC, NT>;
    __shared__ __attribute__((aligned(16))) char smem[2 * Tile::BYTES];
    static_assert(32 * QB * D * 4 + 2 * 32 * QB * 4 <= 2 * Tile::BYTES, "merge buffer");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    // The K/V heads of one (request, chunk) are consecutive workgroups: their
    // rows interleave in the same cache pages, so they read those pages at
    // about the same time.
    const int kvh = blockIdx.x % p.hkv;
    const int split = (blockIdx.x / p.hkv) % p.n_splits;
    const int b = blockIdx.x / (p.hkv * p.n_splits);
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

    // Locate tile t: base row pointers and the number of valid keys.
    auto locate = [&](int t, const uint16_t*& kb, const uint16_t*& vb, int& nvalid) {
        const int key0 = key_begin + t * BC;
        const int phys = table[key0 / kPage];
        nvalid = min(BC, key_end - key0);
        if (phys < 0 || phys >= p.num_pages) {
            bad = true;
            nvalid = 0;
            kb = p.k_cache;
            vb = p.v_cache;
            return;
        }
        const long row0 = (long)phys * kPage + key0 % kPage;
        kb = p.k_cache + row0 * row_stride + (long)kvh * D;
        vb = p.v_cache + row0 * row_stride + (long)kvh * D;
    };

    Tile tile;
    int nvalid_cur = 0, nvalid_next = 0;
    if (n_tiles > 0) {
        const uint16_t *kb, *vb;
        locate(0, kb, vb, nvalid_cur);
        tile.load(kb, vb, row_stride, nvalid_cur, tid);
        tile.store(smem, smem + Tile::K_BYTES, tid);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        char* ks = smem + (t & 1) * Tile::BYTES;
        char* vs = ks + Tile::K_BYTES;
        if (t + 1 < n_tiles) {
            const uint16_t *kb, *vb;
            locate(t + 1, kb, vb, nvalid_next);
            tile.load(kb, vb, row_stride, nvalid_next, tid);
        }
        if (32 * wave < nvalid_cur) {
            f32x16 sacc[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[qb][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 a = read_k_frag<D>(ks, wave, s, lane);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb] = mfma32(a, qf[qb][s], sacc[qb]);
            }
            if (32 * wave + 32 > nvalid_cur) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (score_key(wave, r, lane) >= nvalid_cur) sacc[qb][r] = -INFINITY;
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
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c2, -shift));
                    sacc[qb][r] = e;
                    rs += e;
                }
                l_part[qb] += rs;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        w[j] = pack_bf16x2(sacc[qb][8 * c + 2 * j], sacc[qb][8 * c + 2 * j + 1]);
                    pb[qb][c] = w;
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 a = read_vt_frag<BC>(vs, db, wave, c, lane);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(a, pb[qb][c], oacc[db][qb]);
                }
        }
        if (t + 1 < n_tiles) {
            char* nks = smem + ((t + 1) & 1) * Tile::BYTES;
            tile.store(nks, nks + Tile::K_BYTES, tid);
        }
        nvalid_cur = nvalid_next;
        __syncthreads();
    }

    // ---- merge the waves' states (fixed order, deterministic) ----------------
    // LDS: mbuf[NW][32*QB] running shifts, then obuf[32*QB][D] and lbuf[32*QB].
    float* mbuf = reinterpret_cast<float*>(smem);
    float* obuf = mbuf + NW * 32 * QB;
    float* lbuf = obuf + 32 * QB * D;
    const int h = lane >> 5;
    if (h == 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mbuf[wave * 32 * QB + 32 * qb + l32] = m_run[qb];
    }
    __syncthreads();
    float wscale[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = 32 * qb + l32;
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mbuf[w * 32 * QB + j]);
        wscale[qb] = (m_run[qb] == -INFINITY) ? 0.0f : exp2f(m_run[qb] - M);
    }
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int j = 32 * qb + l32;
                if (j < g) {
                    const float lt = pair_sum(l_part[qb]) * wscale[qb];
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int d = 32 * db + 8 * (r >> 2) + 4 * h + (r & 3);
                            const float v = oacc[db][qb][r] * wscale[qb];
                            obuf[j * D + d] = (w == 0) ? v : obuf[j * D + d] + v;
                        }
                    if (h == 0) lbuf[j] = (w == 0) ? lt : lbuf[j] + lt;
                }
            }
        }
        __syncthreads();
    }
    // ---- write the normalised partial and its lse ----------------------------
    const long part_row = ((long)split * p.batch + b) * p.hq + hq0;
    for (int i = tid; i < g * D; i += NT) {
        const int j = i / D, d = i % D;
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mbuf[w * 32 * QB + j]);
        const float L = lbuf[j];
        float o = L > 0.0f ? obuf[j * D + d] / L : 0.0f;
        if (bad) o = NAN;
        p.out_part[(part_row + j) * D + d] = o;
        if (d == 0) {
            float lse = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
            if (bad) lse = NAN;
            p.lse_part[part_row + j] = lse;
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

template <int D, int QB, int NW>
static hipError_t launch_split_cfg(const DecodeParams& p, hipStream_t s) {
    if (p.n_splits <= 0 || p.batch <= 0) return hipSuccess;
    const long grid = (long)p.n_splits * p.hkv * p.batch;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_decode_split_kernel<D, QB, NW>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       s, p);
    return hipGetLastError();
}

#ifndef ATTN_DEC_NW
#define ATTN_DEC_NW 2
#endif

template <int D>
static hipError_t launch_split_d(const DecodeParams& p, hipStream_t s) {
    constexpr int NW = D >= 256 ? 2 : ATTN_DEC_NW;
    const int g = p.hq / p.hkv;
    return g <= 32 ? launch_split_cfg<D, 1, NW>(p, s) : launch_split_cfg<D, 2, NW>(p, s);
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
