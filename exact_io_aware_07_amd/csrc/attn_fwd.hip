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
// P enters the matrix product rounded to bf16; the output is divided by the
// sum of those rounded values (so the weights it applies sum to one exactly:
// a row dominated by a few keys then loses no accuracy to their rounding),
// while lse comes from the fp32 sum of the unrounded values.
// Tiles wholly above the causal boundary are never visited ("FlashAttention:
// Part 1", section 3.5).  K/V tiles are double-buffered in LDS: the global
// loads of tile t+1 are issued before tile t is computed.
//
// Split-key mode (KSPLIT, for launches with few workgroups): the NW waves of a
// workgroup own the same 32 * QB query rows and take every NW-th key tile,
// each wave loading its own tiles into its own LDS stages (no barrier in the
// loop); at the end their (max, sums, O) states are merged exactly as two
// tiles merge in the online recurrence ("Flash Attention: A Complete
// Architectural Autopsy", "The Online Softmax Recurrence") and one wave
// writes the rows.

#include "attn_tile.h"
#include "attn_launch.h"

namespace attn {

// Page size of the paged prefill's cache (as the paged decode).
constexpr int kFwdPage = 256;

// ATTN_FWD_SINGLE_STAGE=1 builds a check variant with one LDS stage: each
// tile's loads are issued only after every wave has finished the previous
// tile, so no load can overlap a read of the same stage.  Its results must
// equal the double-buffered kernel's bit for bit (same arithmetic in the same
// order); a difference would expose a race on the LDS stages.
#ifndef ATTN_FWD_SINGLE_STAGE
#define ATTN_FWD_SINGLE_STAGE 0
#endif

// K fragment reads issued ahead of the first score MFMA of a tile.
#ifndef ATTN_FWD_K_LEAD
#define ATTN_FWD_K_LEAD 8
#endif

// Packed batches of at most this many sequences run their work items longest
// sequence first (see the work-item mapping in attn_fwd_kernel).
constexpr int kLengthOrderMax = 64;

// LDS that holds the Q^T fragments a wave parks outside its registers (one
// object per instantiation that uses it).
template <int BYTES>
__device__ __forceinline__ char* q_stash() {
    __shared__ __attribute__((aligned(1024))) char buf[BYTES];
    return buf;
}

template <int D, int QB, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN, bool PAGED, bool KSPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_kernel(FwdParams p) {
    static_assert(!PAGED || VARLEN, "paged prefill packs its queries");
    static_assert(!(KSPLIT && PAGED), "split-key mode reads contiguous K/V");
    static_assert(kFwdPage % BC == 0, "key tiles must not straddle pages");
    constexpr int ROWS_W = 32 * QB;
    constexpr int BR = KSPLIT ? ROWS_W : NW * ROWS_W;  // query rows per workgroup
    constexpr int TSTEP = KSPLIT ? NW : 1;              // key tiles between a wave's tiles
    constexpr int KB = BC / 32;  // 32-key blocks per tile
    constexpr int DB = D / 32;   // 32-wide d blocks of O^T
    constexpr int KS = D / 16;   // 16-wide d steps of S^T
    // At d = 256 the Q^T and O^T registers of a 32-row wave (64 + 128) leave
    // too few for two waves per SIMD, so the second half of each lane's Q^T
    // fragments is parked in LDS and read back every tile (each lane reads
    // only what it wrote, so no barrier is involved).
    constexpr int KS_REG = (D == 256 && WPE >= 2) ? KS / 2 : KS;
    constexpr int KS_LDS = KS - KS_REG;
    // LDS reads per score MFMA group once the first ATTN_FWD_K_LEAD are out.
    constexpr int DS_GROUPS = KS * KB > ATTN_FWD_K_LEAD ? KS * KB - ATTN_FWD_K_LEAD : 1;
    constexpr int DS_PER = (KS * KB + KS_LDS * QB - ATTN_FWD_K_LEAD) / DS_GROUPS;
    static_assert(KS_LDS == 0 || DS_PER * DS_GROUPS == KS * KB + KS_LDS * QB - ATTN_FWD_K_LEAD,
                  "even LDS read schedule");
    // In split-key mode each wave loads whole tiles into stages of its own.
    using Tile = KVDirect<D, BC, KSPLIT ? 1 : NW>;
    constexpr uint32_t STAGE_BYTES = KSPLIT ? NW * Tile::BYTES : Tile::BYTES;
    // Two LDS stages as distinct objects, and a loop unrolled by two so that
    // every access names its stage statically: the compiler can then see that
    // the next tile's LDS-DMA writes never alias the reads of the current
    // tile, and does not wait for them before those reads.
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int l32 = lane & 31;
    char* const st0 = stage0 + (KSPLIT ? wave * Tile::BYTES : 0);  // this wave's stages
    char* const st1 = stage1 + (KSPLIT ? wave * Tile::BYTES : 0);
    const int lwave = KSPLIT ? 0 : wave;  // the wave's share of a tile's loads

    // Work item: heaviest query tiles first (workgroups are dealt to the 8
    // XCDs round-robin, and each XCD runs its share in launch order).
    const int BH = p.batch * p.hq;
    const int bid = blockIdx.x;
    int qt, b, hq;
    if constexpr (VARLEN) {
        // Sequences differ in length, so a block of whole sequences per XCD
        // would load the XCDs unevenly: the query heads of each work item
        // (query tile, sequence) are spread over the XCDs instead (XCD x
        // takes heads [x*hq/8, (x+1)*hq/8), which also keeps a GQA group on
        // one L2), and every XCD runs all items.
        int item;
        if ((p.hq & 7) == 0) {
            const int hpx = p.hq >> 3, x = bid & 7, kk = bid >> 3;
            item = (int)udiv_apply(kk, p.dv_hpx);
            hq = x * hpx + (kk - item * hpx);
        } else {
            item = (int)udiv_apply(bid, p.dv_bh);
            hq = bid - item * p.hq;
        }
        if (p.batch <= kLengthOrderMax) {
            // Items run longest sequence first (more keys, ties by index),
            // each sequence's query tiles last tile first.  A tile's work is
            // mostly its sequence's key prefix, so this is close to a
            // longest-first schedule, and the tiles of one sequence run
            // together while its K/V is in L2.  Every workgroup ranks the
            // sequences itself (one thread per sequence, then a wave scan of
            // the tile counts in rank order).
            __shared__ int s_len[kLengthOrderMax];
            __shared__ int s_order[kLengthOrderMax];
            __shared__ int s_first[kLengthOrderMax + 1];
            if (tid < p.batch) {
                const int kl = PAGED ? p.seqlens_k[tid] : p.cu_k[tid + 1] - p.cu_k[tid];
                s_len[tid] = kl;
            }
            __syncthreads();
            if (tid < p.batch) {
                const int mine = s_len[tid];
                int rank = 0;
                for (int o = 0; o < p.batch; ++o) {
                    const int other = s_len[o];
                    rank += (other > mine) || (other == mine && o < tid);
                }
                s_order[rank] = tid;
            }
            __syncthreads();
            if (wave == 0) {
                int tiles = 0;
                if (lane < p.batch) {
                    const int s = s_order[lane];
                    const int nq = p.cu_q[s + 1] - p.cu_q[s];
                    tiles = nq > 0 ? (nq + BR - 1) / BR : 0;
                }
                int incl = tiles;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                if (lane < p.batch) s_first[lane + 1] = incl;
                if (lane == 0) s_first[0] = 0;
            }
            __syncthreads();
            if (item >= s_first[p.batch]) {
                b = 0;
                qt = p.n_qtiles;  // past every sequence: no work
            } else {
                int lo = 0, hi = p.batch - 1;  // last rank r with s_first[r] <= item
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_first[mid] <= item) lo = mid; else hi = mid - 1;
                }
                b = s_order[lo];
                qt = (s_first[lo + 1] - s_first[lo]) - 1 - (item - s_first[lo]);
            }
        } else {
            const int ib = (int)udiv_apply(item, p.dv_batch);
            qt = p.n_qtiles - 1 - ib;
            b = item - ib * p.batch;
        }
    } else {
        // Equal-length sequences: when the (sequence, head) count is a
        // multiple of 8, all query tiles of a head run on the same XCD, so
        // that head's K/V stays in one L2.  When each XCD's share of heads is
        // a multiple of 4, the XCD runs them four heads at a time (heads 4g ..
        // 4g + 3 of its share, all their query tiles, heaviest first), so the
        // query tiles reading one K/V tile run together while it is in the L2
        // (and a GQA group of four shares one K/V head): HBM fetch per launch
        // 480 -> 284 MiB on causal MHA B=4 H=16 N=4096 and 413 -> 279 MiB on
        // causal GQA B=2 Hq=32 Hkv=8 N=8192, same time.
        int bh;
        if ((BH & 31) == 0) {
            const int hpx = BH >> 3, x = bid & 7, kk = bid >> 3;
            const int g = (int)udiv_apply(kk, p.dv_gt);  // 4 * n_qtiles items per group
            const int j = kk - g * 4 * p.n_qtiles;
            qt = p.n_qtiles - 1 - (j >> 2);
            bh = x * hpx + 4 * g + (j & 3);
        } else if ((BH & 7) == 0) {
            const int hpx = BH >> 3, x = bid & 7, kk = bid >> 3;
            const int kq = (int)udiv_apply(kk, p.dv_hpx);
            qt = p.n_qtiles - 1 - kq;
            bh = x * hpx + (kk - kq * hpx);
        } else {
            const int kq = (int)udiv_apply(bid, p.dv_bh);
            qt = p.n_qtiles - 1 - kq;
            bh = bid - kq * BH;
        }
        b = (int)udiv_apply(bh, p.dv_hq);
        hq = bh - b * p.hq;
    }
    const int kvh = (int)udiv_apply(hq, p.dv_grp);

    int q_off, k_off = 0, Nq, Nk;
    bool bad = false;  // paged: a page id out of range, or more keys than the table holds
    if constexpr (PAGED) {
        q_off = p.cu_q[b];
        Nq = p.cu_q[b + 1] - q_off;
        Nq = Nq < 0 ? 0 : Nq;
        Nk = p.seqlens_k[b];
        if (Nk < 0) {
            Nk = 0;
            bad = true;
        }
        if ((long)Nk > (long)p.max_pages * kFwdPage) {
            Nk = p.max_pages * kFwdPage;
            bad = true;
        }
    } else if constexpr (VARLEN) {
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

    // Row i (of its sequence) sees keys lo(i) .. hi(i): the bottom-right
    // causal rule and the local window (keys i + Nk - Nq - left .. i + Nk -
    // Nq + right, -1 unbounded; "Deep Dive - FlashAttention", "Causal 2.1 is
    // the decode gotcha"), clipped to the keys that exist.
    const long shift = (long)Nk - Nq;
    long roff = CAUSAL ? 0 : (1L << 40);
    if (p.wr >= 0 && p.wr < roff) roff = p.wr;
    const long loff = p.wl >= 0 ? p.wl : (1L << 40);
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        const long h = i + shift + roff;
        return (int)(h < Nk - 1 ? h : Nk - 1);
    };
    auto lo_of = [&](int i) __attribute__((always_inline)) {
        const long l = i + shift - loff;
        return (int)(l > 0 ? l : 0);
    };
    // K/V tile range: tile t covers keys [t*BC, t*BC + BC); tiles wholly
    // outside every row's range are never visited.
    const int last_row = min(q0 + BR, Nq) - 1;
    const int t_lo = lo_of(q0) / BC;
    int t_end = hi_of(last_row) < 0 ? 0 : hi_of(last_row) / BC + 1;
    if (t_end < t_lo) t_end = t_lo;

    const long kv_stride = (long)p.hkv * D;
    const uint32_t stride_b = (uint32_t)(kv_stride * 2);
    const uint16_t* kbase = p.k + ((long)k_off * p.hkv + kvh) * D;
    const uint16_t* vbase = p.v + ((long)k_off * p.hkv + kvh) * D;

    // This wave's rows and the key ranges of its first and last row.
    const int wr0 = q0 + (KSPLIT ? 0 : wave * ROWS_W);
    const bool wave_rows = wr0 < Nq;
    const int w_last_row = min(wr0 + ROWS_W, Nq) - 1;
    const int w_hi_max = hi_of(w_last_row), w_hi_min = hi_of(wr0);
    const int w_lo_min = lo_of(wr0), w_lo_max = lo_of(w_last_row);

    // Page id of key tile t (paged mode).  It is read one step before the
    // tile's loads are issued, so the table lookup never delays them.
    auto page_of = [&](int t) __attribute__((always_inline)) {
        return PAGED ? p.block_table[(long)b * p.max_pages + (t * BC) / kFwdPage] : 0;
    };
    // Loads of key tile t: contiguous K/V, or the page the block table names.
    auto issue_tile = [&](int t, int phys_v, uint32_t st) __attribute__((always_inline)) {
        const int key0 = t * BC;
        if constexpr (PAGED) {
            const int phys = __builtin_amdgcn_readfirstlane(phys_v);
            if (phys < 0 || phys >= p.num_pages) {
                bad = true;
                Tile::issue(p.k, p.v, stride_b, 0, st, lwave, lane);
            } else {
                const long row0 = (long)phys * kFwdPage + key0 % kFwdPage;
                Tile::issue(p.k + (row0 * p.hkv + kvh) * D, p.v + (row0 * p.hkv + kvh) * D, stride_b,
                            Nk - key0, st, lwave, lane);
            }
        } else {
            const long off = (long)key0 * kv_stride;
            Tile::issue(kbase + off, vbase + off, stride_b, Nk - key0, st, lwave, lane);
        }
    };

    // Q^T fragments (B operand), resident for the whole loop: steps below
    // KS_REG in registers, the rest in this wave's LDS slots (16 bytes per
    // lane and step).
    u32x4 qf[QB][KS_REG];
    char* qlds = nullptr;
    if constexpr (KS_LDS > 0) qlds = q_stash<NW * QB * KS_LDS * 1024>() + wave * (QB * KS_LDS * 1024) + lane * 16;
    auto q_frag = [&](int qb, int s) __attribute__((always_inline)) {
        if constexpr (KS_LDS > 0) {
            if (s >= KS_REG) return *reinterpret_cast<const u32x4*>(qlds + (qb * KS_LDS + s - KS_REG) * 1024);
        }
        return qf[qb][s < KS_REG ? s : 0];
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
        const uint16_t* qrow = p.q + ((long)(q_off + row) * p.hq + hq) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < Nq) z = load16(qrow + (2 * s + (lane >> 5)) * 8);
            if (s < KS_REG)
                qf[qb][s < KS_REG ? s : 0] = z;
            else if constexpr (KS_LDS > 0)
                *reinterpret_cast<u32x4*>(qlds + (qb * KS_LDS + s - KS_REG) * 1024) = z;
        }
    }

    f32x16 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.0f;
    // l_part: partial row sums of P in fp32 (for lse); lr_part: of P as
    // rounded to bf16 for the P V product (the output's divisor).
    float m_run[QB], l_part[QB], lr_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_part[qb] = 0.0f;
        lr_part[qb] = 0.0f;
    }
    const float c2 = p.scale * kLog2e;

    const int t_first = t_lo + (KSPLIT ? wave : 0);  // this wave's first tile
    int phys_next = 0;  // page id of the next tile to issue (paged mode)
    if (t_first < t_end) {
        issue_tile(t_first, page_of(t_first), lds_addr(st0));
        if (t_first + 1 < t_end) phys_next = page_of(t_first + 1);
    }
    wait_vmem();
    __syncthreads();

    auto step = [&](const int t, char* cur, char* nxt) __attribute__((always_inline)) {
        const char* ks = cur;
        const char* vs = cur + Tile::K_BYTES;
        if (!ATTN_FWD_SINGLE_STAGE && t + TSTEP < t_end) {
            issue_tile(t + TSTEP, phys_next, lds_addr(nxt));
            if (PAGED && t + 2 < t_end) phys_next = page_of(t + 2);
        }
        const int k0 = t * BC;
        const bool active = wave_rows && k0 <= w_hi_max && k0 + BC - 1 >= w_lo_min;
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
                    for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma32(a, q_frag(qb, s), sacc[kb][qb]);
                }
            }
            // Keep the K (and parked Q) fragment reads ATTN_FWD_K_LEAD MFMAs
            // ahead of their use so that LDS latency is not exposed before
            // each MFMA.
            __builtin_amdgcn_sched_group_barrier(0x100, ATTN_FWD_K_LEAD, 0);  // DS read
#pragma unroll
            for (int i = 0; i < KS * KB - ATTN_FWD_K_LEAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);       // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, DS_PER, 0);   // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, QB * ATTN_FWD_K_LEAD, 0);
            // ---- mask: only tiles crossing the diagonal or the key end ----
            const bool need_mask = (k0 + BC - 1 > w_hi_min) || (k0 < w_lo_max);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int row = wr0 + 32 * qb + l32;
                    const int hi = hi_of(row), lo = lo_of(row);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int j = k0 + score_key(kb, r, lane);
                            if (j > hi || j < lo) sacc[kb][qb][r] = -INFINITY;
                        }
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
                    lr_part[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
                }
                if (raise) m_run[qb] = m_new;
                const float shift = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
                // The tile's row sum starts from its first probability (the
                // same value as 0 + p, as p >= +0), one add fewer.
                float rs, rr = lr_part[qb];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][r], c2, -shift));
                        sacc[kb][qb][r] = e;
                        rs = (kb == 0 && r == 0) ? e : rs + e;
                    }
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        u32x4 w;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            w[j] = pack_bf16x2(sacc[kb][qb][8 * c + 2 * j], sacc[kb][qb][8 * c + 2 * j + 1]);
                        pb[kb][qb][c] = w;
                        rr = add_bf16x8(w, rr);
                    }
                }
                l_part[qb] += rs;
                lr_part[qb] = rr;
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
        if (ATTN_FWD_SINGLE_STAGE && t + TSTEP < t_end) {
            // Check variant: every wave is done with the stage before it is
            // refilled (in split-key mode only this wave reads it).
            if constexpr (!KSPLIT) __syncthreads();
            issue_tile(t + TSTEP, phys_next, lds_addr(cur));
            if (PAGED && t + 2 < t_end) phys_next = page_of(t + 2);
        }
        // The next tile's loads (this wave's share) must have landed in LDS
        // before the barrier releases other waves to read them.  In split-key
        // mode the waves run different numbers of tiles and share no stage,
        // so there is no barrier in the loop.
        wait_vmem();
        if constexpr (!KSPLIT) __syncthreads();
    };
    if constexpr (ATTN_FWD_SINGLE_STAGE) {
        for (int t = t_first; t < t_end; t += TSTEP) step(t, st0, st0);
    } else {
        for (int t = t_first; t < t_end; t += 2 * TSTEP) {
            step(t, st0, st1);
            if (t + TSTEP < t_end) step(t + TSTEP, st1, st0);
        }
    }

    if constexpr (KSPLIT) {
        // Merge the waves' states into wave 0: m = max of the shifts, each
        // wave's sums and O scaled by exp2(m_w - m).  The per-lane layout is
        // the same in every wave (same rows), so the merge is lane-wise.
        // Layout in stage0: [wave - 1][item][lane] floats, item = per qb
        // (m, l, lr, O^T registers).
        constexpr int ITEMS = QB * (3 + DB * 16);
        static_assert((NW - 1) * ITEMS * 64 * 4 <= STAGE_BYTES, "merge area fits the stages");
        float* const xs = reinterpret_cast<float*>(stage0);
        __syncthreads();  // every wave is done with its stages
        if (wave > 0) {
            float* w = xs + (wave - 1) * ITEMS * 64 + lane;
            int k = 0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                w[64 * k++] = m_run[qb];
                w[64 * k++] = l_part[qb];
                w[64 * k++] = lr_part[qb];
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) w[64 * k++] = oacc[db][qb][r];
            }
        }
        __syncthreads();
        if (wave > 0) return;
        for (int ow = 1; ow < NW; ++ow) {
            const float* w = xs + (ow - 1) * ITEMS * 64 + lane;
            int k = 0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mo = w[64 * k++];
                const float lo = w[64 * k++];
                const float lro = w[64 * k++];
                const float m = fmaxf(m_run[qb], mo);
                const float a = m_run[qb] == -INFINITY ? 0.0f : exp2f(m_run[qb] - m);
                const float bs = mo == -INFINITY ? 0.0f : exp2f(mo - m);
                l_part[qb] = l_part[qb] * a + lo * bs;
                lr_part[qb] = lr_part[qb] * a + lro * bs;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][qb][r] = oacc[db][qb][r] * a + w[64 * k++] * bs;
                m_run[qb] = m;
            }
        }
    }

    // ---- epilogue: out = O / l (bf16, round to nearest even), lse in nats ----
    const int h = lane >> 5;
    const int total_q = VARLEN ? p.cu_q[p.batch] : 0;
    if constexpr (D <= 128 && !KSPLIT && QB == 1) {
        // Output rows through LDS (the wave's own region of the stages, free
        // after the last barrier): 16-byte stores of whole rows.
        constexpr uint32_t WB = 32u * D * 2;  // bytes per wave
        static_assert((NW / 2) * WB <= STAGE_BYTES, "output staging fits the stages");
        char* const ob = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WB;
        const int row = wr0 + l32;
        const float l_tot = pair_sum(l_part[0]);
        const float lr_tot = pair_sum(lr_part[0]);
        const float inv = bad ? NAN : (l_tot > 0.0f ? 1.0f / lr_tot : 0.0f);
        f32x16 oq[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) oq[db] = oacc[db][0];
        store_rows_bf16_staged<DB>(ob, oq, inv, lane, p.out + ((long)(q_off + wr0) * p.hq + hq) * D,
                                   (long)p.hq * D, Nq - wr0);
        if (row < Nq && p.lse != nullptr && h == 0) {
            const float lse = bad ? NAN : (l_tot > 0.0f ? (m_run[0] + __log2f(l_tot)) * kLn2 : -INFINITY);
            if constexpr (VARLEN)
                p.lse[(long)hq * total_q + q_off + row] = lse;
            else
                p.lse[((long)b * p.hq + hq) * Nq + row] = lse;
        }
        return;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + 32 * qb + l32;
        const float l_tot = pair_sum(l_part[qb]);
        const float lr_tot = pair_sum(lr_part[qb]);
        if (row < Nq) {
            const float inv = bad ? NAN : (l_tot > 0.0f ? 1.0f / lr_tot : 0.0f);
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
                const float lse = bad ? NAN : (l_tot > 0.0f ? (m_run[qb] + __log2f(l_tot)) * kLn2 : -INFINITY);
                if constexpr (VARLEN)
                    p.lse[(long)hq * total_q + q_off + row] = lse;
                else
                    p.lse[((long)b * p.hq + hq) * Nq + row] = lse;
            }
        }
    }
}

template <int D, int QB, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN, bool PAGED, bool KSPLIT = false>
static hipError_t launch_fwd_cfg(const FwdParams& p0, hipStream_t stream) {
    FwdParams p = p0;
    constexpr int BR = KSPLIT ? 32 * QB : NW * 32 * QB;
    p.n_qtiles = (p.max_q + BR - 1) / BR;
    const long grid = (long)p.n_qtiles * p.batch * p.hq;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    // Divisors of the work-item mapping (see attn_udiv.h); the grid check
    // above keeps every count below 2^31.
    const int bh_all = p.batch * p.hq;
    const int per_xcd = (VARLEN ? p.hq : bh_all) >> 3;
    p.dv_hpx = udiv_make(per_xcd > 0 ? per_xcd : 1);
    p.dv_bh = udiv_make(VARLEN ? p.hq : bh_all);
    p.dv_hq = udiv_make(p.hq);
    p.dv_batch = udiv_make(p.batch);
    p.dv_grp = udiv_make(p.hkv > 0 ? p.hq / p.hkv : 1);
    p.dv_gt = udiv_make((uint32_t)(4 * p.n_qtiles));
    hipLaunchKernelGGL((attn_fwd_kernel<D, QB, BC, NW, WPE, CAUSAL, VARLEN, PAGED, KSPLIT>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

template <int D, int QB, int BC, int NW, int WPE>
static hipError_t launch_fwd_d(const FwdParams& p, bool causal, bool varlen, bool paged, hipStream_t s) {
    if (paged) {
        return causal ? launch_fwd_cfg<D, QB, BC, NW, WPE, true, true, true>(p, s)
                      : launch_fwd_cfg<D, QB, BC, NW, WPE, false, true, true>(p, s);
    }
    if (causal) {
        return varlen ? launch_fwd_cfg<D, QB, BC, NW, WPE, true, true, false>(p, s)
                      : launch_fwd_cfg<D, QB, BC, NW, WPE, true, false, false>(p, s);
    }
    return varlen ? launch_fwd_cfg<D, QB, BC, NW, WPE, false, true, false>(p, s)
                  : launch_fwd_cfg<D, QB, BC, NW, WPE, false, false, false>(p, s);
}

// Tile shapes per head dim: <QB (32-row blocks per wave), BC (keys per tile),
// NW (waves per workgroup), WPE (waves per SIMD the register budget targets)>.
#ifndef ATTN_FWD128_CFG
#define ATTN_FWD128_CFG 1, 64, 8, 2
#endif
// d = 64: one 32-row block per wave keeps a wave at 119 VGPRs, so four
// workgroups of four waves share a CU (four waves per SIMD): the same rate as
// two 64-row blocks per wave at two waves per SIMD on long sequences, and
// twice the workgroups for short ones.
#ifndef ATTN_FWD64_CFG
#define ATTN_FWD64_CFG 1, 64, 4, 4
#endif
// d = 256: eight waves at two per SIMD with half of Q^T parked in LDS (64 KiB
// of K/V stages + 64 KiB of parked Q): 930 TFLOP/s on the chunked-prefill
// workload against 710 for four waves at one per SIMD with Q^T in registers.
#ifndef ATTN_FWD256_CFG
#define ATTN_FWD256_CFG 1, 32, 8, 2
#endif

// Split-key mode: four waves share 32 query rows, each with its own stages.
template <int D, int BC>
static hipError_t launch_fwd_split(const FwdParams& p, bool causal, bool varlen, hipStream_t s) {
    if (causal)
        return varlen ? launch_fwd_cfg<D, 1, BC, 4, 2, true, true, false, true>(p, s)
                      : launch_fwd_cfg<D, 1, BC, 4, 2, true, false, false, true>(p, s);
    return varlen ? launch_fwd_cfg<D, 1, BC, 4, 2, false, true, false, true>(p, s)
                  : launch_fwd_cfg<D, 1, BC, 4, 2, false, false, false, true>(p, s);
}

// A launch whose usual grid (workgroups of `rows` query rows) fills at most
// half of the 256 compute units, with at least eight key tiles of `bc` keys
// per row and no narrow window, runs in split-key mode: four times the
// workgroups, each wave walking a quarter of the keys.
static bool use_split(const FwdParams& p, int rows, int bc) {
    const long grid = (long)((p.max_q + rows - 1) / rows) * p.batch * p.hq;
    return grid <= 128 && p.max_k >= 8 * bc && (p.wl < 0 || p.wl >= 8 * bc);
}

hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, bool varlen, bool paged, hipStream_t s) {
    switch (head_dim) {
        case 64:
            if (!paged && use_split(p, 128, 64)) return launch_fwd_split<64, 64>(p, causal, varlen, s);
            return launch_fwd_d<64, ATTN_FWD64_CFG>(p, causal, varlen, paged, s);
        case 128:
            if (!paged && use_split(p, 256, 32)) return launch_fwd_split<128, 32>(p, causal, varlen, s);
            // A narrow left window uses w + 1 of the 256 + w keys a 256-row
            // tile streams; 128-row workgroups waste half as much (measured
            // on the 4096-token causal workload: +14% at w = 512, +25% at
            // w = 64, no change at w = 1024).
            if (p.wl >= 0 && p.wl <= 512) return launch_fwd_d<128, 1, 64, 4, 2>(p, causal, varlen, paged, s);
            return launch_fwd_d<128, ATTN_FWD128_CFG>(p, causal, varlen, paged, s);
        case 256: return launch_fwd_d<256, ATTN_FWD256_CFG>(p, causal, varlen, paged, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
