// Prefill / chunked-prefill forward pass with online softmax (gfx950).
//
// One workgroup owns BR = NW * 32 * QB query rows of one (sequence, query
// head) and walks the key/value tiles of its K/V head
// ("Deep Dive - FlashAttention", "Exact attention without an n x n workspace":
// the query tile stays resident while (K_j, V_j) stream past; "FlashAttention-3
// and PagedAttention: IO-Aware Attention Kernels (2026)", "FlashAttention-2:
// better parallelism and work partitioning": query tiles in the outer loop,
// spread over workgroups).  Each wave owns 32 * QB whole query rows, so no
// softmax state crosses waves ("Flash Attention: A Complete Architectural
// Autopsy", "Fix 3: Warp-Level Work Partitioning").
//
// Per K/V tile (the recurrence of "Flash Attention: A Complete Architectural
// Autopsy", "The Online Softmax Recurrence"):
//   S^T = K Q^T on bf16 matrix cores, fp32 accumulate;
//   mask (only tiles that touch the causal diagonal or the end of the keys);
//   running max in log2 units; rescale O and l only when the max rises by more
//   than kRescaleThreshold (the conditional rescaling named in "Deep Dive -
//   FlashAttention", "FA1 through FA4 retune the same IO idea");
//   P = exp2(S * scale * log2(e) - m), l += rowsum P, O^T += V^T P^T.
// Tiles wholly above the causal boundary are never visited ("FlashAttention:
// Part 1", section 3.5).  K/V tiles are double-buffered in LDS: the global
// loads of tile t+1 are issued before tile t is computed.

#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

// K fragment reads issued ahead of the first score MFMA of a tile.
#ifndef ATTN_FWD_K_LEAD
#define ATTN_FWD_K_LEAD 8
#endif

template <int D, int QB, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_kernel(FwdParams p) {
    constexpr int NT = NW * 64;
    constexpr int ROWS_W = 32 * QB;
    constexpr int BR = NW * ROWS_W;
    constexpr int KB = BC / 32;  // 32-key blocks per tile
    constexpr int DB = D / 32;   // 32-wide d blocks of O^T
    constexpr int KS = D / 16;   // 16-wide d steps of S^T
    using Tile = KVDirect<D, BC, NW>;
    // Two LDS stages as distinct objects, and a loop unrolled by two so that
    // every access names its stage statically: the compiler can then see that
    // the next tile's LDS-DMA writes never alias the reads of the current
    // tile, and does not wait for them before those reads.
    __shared__ __attribute__((aligned(1024))) char stage0[Tile::BYTES];
    __shared__ __attribute__((aligned(1024))) char stage1[Tile::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int l32 = lane & 31;

    // Work item: heaviest query tiles first (workgroups are dealt to the 8
    // XCDs round-robin, and each XCD runs its share in launch order).
    const int BH = p.batch * p.hq;
    const int bid = blockIdx.x;
    int qt, b, hq;
    if constexpr (VARLEN) {
        // Sequences differ in length, so a block of whole sequences per XCD
        // would load the XCDs unevenly.  Work items (query tile, sequence)
        // run in query-tile-descending order and the query heads of each
        // item are spread over the XCDs: XCD x takes heads
        // [x*hq/8, (x+1)*hq/8), which also keeps a GQA group on one L2.
        int item;
        if ((p.hq & 7) == 0) {
            const int hpx = p.hq >> 3, x = bid & 7, kk = bid >> 3;
            item = kk / hpx;
            hq = x * hpx + kk % hpx;
        } else {
            item = bid / p.hq;
            hq = bid % p.hq;
        }
        qt = p.n_qtiles - 1 - item / p.batch;
        b = item % p.batch;
    } else {
        // Equal-length sequences: when the (sequence, head) count is a
        // multiple of 8, all query tiles of a head run on the same XCD, so
        // that head's K/V stays in one L2.
        int bh;
        if ((BH & 7) == 0) {
            const int hpx = BH >> 3, x = bid & 7, kk = bid >> 3;
            qt = p.n_qtiles - 1 - kk / hpx;
            bh = x * hpx + kk % hpx;
        } else {
            qt = p.n_qtiles - 1 - bid / BH;
            bh = bid % BH;
        }
        b = bh / p.hq;
        hq = bh % p.hq;
    }
    const int kvh = hq / (p.hq / p.hkv);

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

    // K/V tile range: tile t covers keys [t*BC, t*BC + BC).
    int n_tiles = (Nk + BC - 1) / BC;
    if constexpr (CAUSAL) {
        const int last_row = min(q0 + BR, Nq) - 1;
        const int kmax = last_row + Nk - Nq;  // last key any row of the tile may see
        n_tiles = kmax < 0 ? 0 : min(n_tiles, kmax / BC + 1);
    }

    const long kv_stride = (long)p.hkv * D;
    const uint32_t stride_b = (uint32_t)(kv_stride * 2);
    const uint16_t* kbase = p.k + ((long)k_off * p.hkv + kvh) * D;
    const uint16_t* vbase = p.v + ((long)k_off * p.hkv + kvh) * D;

    // This wave's rows and their key horizon.
    const int wr0 = q0 + wave * ROWS_W;
    const bool wave_rows = wr0 < Nq;
    const int w_last_key = min(wr0 + ROWS_W, Nq) - 1 + Nk - Nq;  // causal: last key the wave sees
    const int w_first_key_lim = wr0 + Nk - Nq;                    // causal: first row's last key

    // Q^T fragments (B operand), resident for the whole loop.
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
        const uint16_t* qrow = p.q + ((long)(q_off + row) * p.hq + hq) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < Nq) z = load16(qrow + (2 * s + (lane >> 5)) * 8);
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

    if (n_tiles > 0) Tile::issue(kbase, vbase, stride_b, Nk, lds_addr(stage0), wave, lane);
    wait_vmem();
    __syncthreads();

    auto step = [&](const int t, char* cur, char* nxt) __attribute__((always_inline)) {
        const char* ks = cur;
        const char* vs = cur + Tile::K_BYTES;
        if (t + 1 < n_tiles) {
            const long off = (long)(t + 1) * BC * kv_stride;
            Tile::issue(kbase + off, vbase + off, stride_b, Nk - (t + 1) * BC, lds_addr(nxt), wave, lane);
        }
        const int k0 = t * BC;
        const bool active = wave_rows && (!CAUSAL || k0 <= w_last_key);
        if (active) {
            // ---- S^T = K Q^T --------------------------------------------
            f32x16 sacc[KB][QB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const u32x4 a = read_k_frag<D>(ks, kb, s, lane);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma32(a, qf[qb][s], sacc[kb][qb]);
                }
            }
            // Keep the K fragment reads ATTN_FWD_K_LEAD MFMAs ahead of their
            // use so that LDS latency is not exposed before each MFMA.
            __builtin_amdgcn_sched_group_barrier(0x100, ATTN_FWD_K_LEAD, 0);  // DS read
#pragma unroll
            for (int i = 0; i < KS * KB - ATTN_FWD_K_LEAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, QB * ATTN_FWD_K_LEAD, 0);
            // ---- mask: only tiles crossing the diagonal or the key end ----
            const bool need_mask =
                (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > w_first_key_lim);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int row = wr0 + 32 * qb + l32;
                    const int lim = CAUSAL ? min(Nk - 1, row + Nk - Nq) : Nk - 1;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (k0 + score_key(kb, r, lane) > lim) sacc[kb][qb][r] = -INFINITY;
                }
            }
            // ---- online softmax --------------------------------------------
            u32x4 pb[KB][QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
                mx = pair_max(mx);
                const float m_new = mx * c2;  // -inf when the row has no key here
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
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][r], c2, -shift));
                        sacc[kb][qb][r] = e;
                        rs += e;
                    }
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        u32x4 w;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            w[j] = pack_bf16x2(sacc[kb][qb][8 * c + 2 * j], sacc[kb][qb][8 * c + 2 * j + 1]);
                        pb[kb][qb][c] = w;
                    }
                }
                l_part[qb] += rs;
            }
            // ---- O^T += V^T P^T ----------------------------------------------
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const u32x4 a = read_vt_frag_tr<D>(vs, db, kb, c, lane);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(a, pb[kb][qb][c], oacc[db][qb]);
                    }
        }
        // The next tile's loads (this wave's share) must have landed in LDS
        // before the barrier releases other waves to read them.
        wait_vmem();
        __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, stage0, stage1);
        if (t + 1 < n_tiles) step(t + 1, stage1, stage0);
    }

    // ---- epilogue: out = O / l (bf16, round to nearest even), lse in nats ----
    const int h = lane >> 5;
    const int total_q = VARLEN ? p.cu_q[p.batch] : 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
        const float l_tot = pair_sum(l_part[qb]);
        if (row < Nq) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            uint16_t* orow = p.out + ((long)(q_off + row) * p.hq + hq) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w = {pack_bf16x2(oacc[db][qb][4 * g] * inv, oacc[db][qb][4 * g + 1] * inv),
                               pack_bf16x2(oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * h) = w;
                }
            if (p.lse != nullptr && h == 0) {
                const float lse = l_tot > 0.0f ? (m_run[qb] + __log2f(l_tot)) * kLn2 : -INFINITY;
                if constexpr (VARLEN)
                    p.lse[(long)hq * total_q + q_off + row] = lse;
                else
                    p.lse[((long)b * p.hq + hq) * Nq + row] = lse;
            }
        }
    }
}

template <int D, int QB, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN>
static hipError_t launch_fwd_cfg(const FwdParams& p0, hipStream_t stream) {
    FwdParams p = p0;
    constexpr int BR = NW * 32 * QB;
    p.n_qtiles = (p.max_q + BR - 1) / BR;
    const long grid = (long)p.n_qtiles * p.batch * p.hq;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_kernel<D, QB, BC, NW, WPE, CAUSAL, VARLEN>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

template <int D, int QB, int BC, int NW, int WPE>
static hipError_t launch_fwd_d(const FwdParams& p, bool causal, bool varlen, hipStream_t s) {
    if (causal) {
        return varlen ? launch_fwd_cfg<D, QB, BC, NW, WPE, true, true>(p, s)
                      : launch_fwd_cfg<D, QB, BC, NW, WPE, true, false>(p, s);
    }
    return varlen ? launch_fwd_cfg<D, QB, BC, NW, WPE, false, true>(p, s)
                  : launch_fwd_cfg<D, QB, BC, NW, WPE, false, false>(p, s);
}

// Tile shapes per head dim: <QB (32-row blocks per wave), BC (keys per tile),
// NW (waves per workgroup), WPE (waves per SIMD the register budget targets)>.
#ifndef ATTN_FWD128_CFG
#define ATTN_FWD128_CFG 1, 64, 8, 2
#endif
#ifndef ATTN_FWD64_CFG
#define ATTN_FWD64_CFG 2, 64, 4, 2
#endif
#ifndef ATTN_FWD256_CFG
#define ATTN_FWD256_CFG 1, 32, 4, 1
#endif

hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, bool varlen, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_fwd_d<64, ATTN_FWD64_CFG>(p, causal, varlen, s);
        case 128: return launch_fwd_d<128, ATTN_FWD128_CFG>(p, causal, varlen, s);
        case 256: return launch_fwd_d<256, ATTN_FWD256_CFG>(p, causal, varlen, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
