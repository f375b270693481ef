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

// Waves per SIMD the split kernel's register budget targets: two when the
// query heads of a K/V head fit one 16-column block and d <= 128.
template <int D, int QB>
constexpr int dec_wpe() { return (QB == 1 && D <= 128) ? 2 : 1; }

// Tiles held in registers (in flight) per wave: two unless that would spill.
// (Three sets spill at two waves per SIMD; one set measured within 1% of two.)
template <int D, int QB>
constexpr int dec_sets() { return (D <= 128 && D * QB <= 256) ? 2 : 1; }

// Split kernel: one wave per (K/V head, chunk, request); the HPW waves of a
// workgroup take HPW adjacent K/V heads of the same (request, chunk), so the
// interleaved head segments of each cache row are read from one compute unit
// at about the same time (measured: 5-10% more HBM throughput than one head
// per workgroup, and 4-5% more than four).  The chunk is walked in tiles of 32 keys that never
// straddle a page.  S^T = K Q^T and O^T = V^T P^T run on 16x16x32 MFMAs (the g
// query heads of the K/V head are the columns, so a 16-column block wastes
// least when g is small).  K and V rows come into registers with coalesced
// 16-byte loads (each 64-lane load covers whole row segments) and are written
// to this wave's LDS region, from where the A operands are read (K directly,
// V^T with transposed reads).  NR register sets (two where the registers
// allow) hold tiles t .. t+NR-1 while tile t is computed, and tile t+NR is
// issued into tile t's set as soon as it has been written to LDS, so every
// wave keeps up to NR tiles (16 KiB each at d = 128) of reads in flight with
// no barrier.  A wave's LDS accesses execute in program order, so one LDS
// region per wave suffices: tile t+1's rows land after tile t's reads.
template <int D, int QB, int HPW>
__global__ __launch_bounds__(64 * HPW) __attribute__((amdgpu_waves_per_eu(dec_wpe<D, QB>(), dec_wpe<D, QB>())))
void attn_decode_split_kernel(DecodeParams p) {
    constexpr int BC = 32;            // keys per tile: two 16-key blocks
    constexpr int KD = D / 32;        // 32-wide d steps of S^T
    constexpr int DB = D / 16;        // 16-wide d blocks of O^T
    constexpr int CH = D / 8;         // 16-byte chunks per cache row
    constexpr int RPI = 64 / CH;      // rows per 64-lane 16-byte load
    constexpr int VI = BC / RPI;      // V loads per tile
    constexpr uint32_t VBYTES = BC * D * 2;
    static_assert(kPage % BC == 0, "tiles must not straddle pages");
    constexpr int NR = dec_sets<D, QB>();
    __shared__ __attribute__((aligned(1024))) char smem[HPW * 2 * VBYTES];

    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, G = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* const ksm = smem + wave * (2 * VBYTES);  // this wave's K tile, then V tile
    char* const vsm = ksm + VBYTES;
    const int groups = p.hkv / HPW;
    const int kvh = (blockIdx.x % groups) * HPW + wave;
    const int unit = blockIdx.x / groups;
    // Highest split index first: the last (often partial) chunks of the
    // requests, and every chunk of the short requests, come at the end of
    // the grid, where they fill the tail.
    const int split = p.n_splits - 1 - unit / p.batch;
    const int b = unit % p.batch;
    const int g = p.hq / p.hkv;
    const int hq0 = kvh * g;

    const int raw_len = p.seqlens[b];
    bool bad = raw_len < 0;
    long nk_l = bad ? 0 : (long)raw_len + p.len_add;
    long cap = (long)p.max_pages * kPage;
    if (p.len_limit > 0 && p.len_limit < cap) cap = p.len_limit;
    if (cap > 0x7fffffffL - kPage) cap = 0x7fffffffL - kPage;  // key offsets stay in int range
    if (nk_l > cap) {
        nk_l = cap;
        bad = true;
    }
    int Nk = (int)nk_l;
    const int key_begin = split * p.chunk;
    if (key_begin >= Nk && !(bad && split == 0)) return;
    const int key_end = min(Nk, key_begin + p.chunk);
    const int n_tiles = key_end > key_begin ? (key_end - key_begin + BC - 1) / BC : 0;

    const long row_stride = (long)p.hkv * D;
    const uint32_t stride_b = (uint32_t)(row_stride * 2);
    const int32_t* table = p.block_table + (long)b * p.max_pages;

    // Q^T fragments (B operand): column j of block qb is query head
    // hq0 + 16 qb + j; lane l holds its d values 32 s + 8 (l / 16) .. + 7.
    u32x4 qf[QB][KD];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = 16 * qb + l16;
        const uint16_t* qrow = p.q + ((long)b * p.hq + hq0 + j) * D;
#pragma unroll
        for (int s = 0; s < KD; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (j < g) z = load16(qrow + 32 * s + 8 * G);
            qf[qb][s] = z;
        }
    }

    f32x4 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // l_part: partial sums of P in fp32 (for lse); lr_part: of P as rounded to
    // bf16 for the P V product (the partial output's divisor, so the weights
    // it applies sum to one exactly).
    float m_run[QB], l_part[QB], lr_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_part[qb] = 0.0f;
        lr_part[qb] = 0.0f;
    }
    const float c2 = p.scale * kLog2e;

    // One tile in registers: k[i] and v[i] hold rows RPI i + l / CH, 16-byte
    // chunk l % CH.  Rows past the valid keys, and every row of a tile whose
    // page id is out of range, load as zeros.
    struct Regs {
        u32x4 k[VI];
        u32x4 v[VI];
    };
    auto load = [&](int t, Regs& R) __attribute__((always_inline)) {
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
        const uint32_t nrec = (uint32_t)nvalid * stride_b;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, nrec);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, nrec);
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const uint32_t off = (uint32_t)(RPI * i + lane / CH) * stride_b + (lane % CH) * 16;
            R.k[i] = buffer_load16_stream(rk, off);
            R.v[i] = buffer_load16_stream(rv, off);
        }
    };
    // Row-major tile in LDS; 16-byte chunk c of row r sits in slot
    // c ^ swz_v16(r), so both the 16-row K fragment reads and the transposed
    // V reads spread over all bank groups.
    auto slot = [&](uint32_t row, uint32_t c) __attribute__((always_inline)) {
        return row * (2 * D) + ((c ^ swz_v16<CH>(row)) * 16);
    };

    // Compute tile t from R; refill R with tile t + NR once it is in LDS.
    auto step = [&](int t, Regs& R) __attribute__((always_inline)) {
        const int nvalid = min(BC, key_end - (key_begin + t * BC));
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const uint32_t row = RPI * i + lane / CH, c = lane % CH;
            *reinterpret_cast<u32x4*>(ksm + slot(row, c)) = R.k[i];
            *reinterpret_cast<u32x4*>(vsm + slot(row, c)) = R.v[i];
        }
        if (t + NR < n_tiles) load(t + NR, R);
        // ---- S^T = K Q^T: two 16-key blocks --------------------------------
        // A operand of key block h, d step s: lane l reads key 16 h + l % 16,
        // d 32 s + 8 (l / 16) .. + 7 (chunk 4 s + l / 16).
        f32x4 sacc[2][QB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[h][qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KD; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(ksm + slot(16 * h + l16, 4 * s + G));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[h][qb] = mfma16(a, qf[qb][s], sacc[h][qb]);
            }
        // ---- mask the keys past the end of the chunk -------------------------
        if (nvalid < BC) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * h + 4 * G + r >= nvalid) sacc[h][qb][r] = -INFINITY;
        }
        // ---- online softmax ------------------------------------------------
        u32x4 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[h][qb][r]);
            mx = quad_max(mx);
            const float m_new = mx * c2;
            const bool raise = m_new > m_run[qb] + kRescaleThreshold;
            const bool scale_old = raise && (m_run[qb] != -INFINITY);
            if (__builtin_amdgcn_ballot_w64(scale_old)) {
                const float alpha = scale_old ? exp2f(m_run[qb] - m_new) : 1.0f;
                l_part[qb] *= alpha;
                lr_part[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
            }
            if (raise) m_run[qb] = m_new;
            const float shift = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
            float e[2][4];
            float rs = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    e[h][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[h][qb][r], c2, -shift));
                    rs += e[h][r];
                }
            l_part[qb] += rs;
            pb[qb] = u32x4{pack_bf16x2(e[0][0], e[0][1]), pack_bf16x2(e[0][2], e[0][3]),
                           pack_bf16x2(e[1][0], e[1][1]), pack_bf16x2(e[1][2], e[1][3])};
            lr_part[qb] = add_bf16x8(pb[qb], lr_part[qb]);
        }
        // ---- O^T += V^T P^T ------------------------------------------------
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const u32x4 a = read_vt16_tr<D>(vsm, db, lane);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma16(a, pb[qb], oacc[db][qb]);
        }
    };

    // NR register sets in rotation: set i holds tiles i, i + NR, i + 2 NR, ...
    Regs sets[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
        if (i < n_tiles) load(i, sets[i]);
    for (int t = 0; t < n_tiles; t += NR) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (t + i < n_tiles) step(t + i, sets[i]);
    }

    // ---- write the normalised partial and its lse ----------------------------
    const long part_row = ((long)split * p.batch + b) * p.hq + hq0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = 16 * qb + l16;
        const float L = quad_sum(l_part[qb]);
        const float Lr = quad_sum(lr_part[qb]);
        if (j < g) {
            const float inv = L > 0.0f ? 1.0f / Lr : 0.0f;
            float* orow = p.out_part + (part_row + j) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = bad ? NAN : oacc[db][qb][r] * inv;
                *reinterpret_cast<f32x4*>(orow + 16 * db + 4 * G) = w;
            }
            if (G == 0) {
                float lse = L > 0.0f ? (m_run[qb] + __log2f(L)) * kLn2 : -INFINITY;
                if (bad) lse = NAN;
                p.lse_part[part_row + j] = lse;
            }
        }
    }
}

// Sum and max over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// One workgroup (one wave) per (request, query head).  The partial rows of the
// first splits are requested before the lse reduction, so the row loads and
// the max/sum run side by side; weights of split j come from lane j.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(CombineParams p) {
    constexpr int PER = D / 64;
    constexpr int RB = 16;  // partial rows in flight
    const int bh = blockIdx.x;
    const int b = bh / p.hq;
    const int lane = threadIdx.x;
    const int raw_len = p.seqlens[b];
    const long Nk = raw_len < 0 ? -1 : (long)raw_len + p.len_add;
    const long n = Nk > 0 ? (Nk + p.chunk - 1) / p.chunk : 0;
    const bool bad = Nk < 0 || n > p.n_splits;
    const long split_stride = (long)p.batch * p.hq;
    const int nn = bad ? 0 : (int)n;
    const float* rows = p.out_part + (long)bh * D + lane;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
    // first batch of rows
    float v[RB][PER];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i) v[j][i] = j < nn ? rows[(long)j * split_stride * D + 64 * i] : 0.0f;
    float x = lane < nn ? p.lse_part[lane * split_stride + bh] : -INFINITY;
    float M = x;
    bool nan_seen = (x != x);
    for (int c = lane + 64; c < nn; c += 64) {
        const float y = p.lse_part[c * split_stride + bh];
        nan_seen |= (y != y);
        M = fmaxf(M, y);
    }
    M = wave_max(M);
    nan_seen = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
    float L = 0.0f;
    if (!bad && !nan_seen && M != -INFINITY) {
        float w = lane < nn ? __expf(x - M) : 0.0f;
        L = w;
        for (int c0 = 0; c0 < nn; c0 += 64) {
            if (c0 > 0) {
                const int c = c0 + lane;
                w = c < nn ? __expf(p.lse_part[c * split_stride + bh] - M) : 0.0f;
                L += w;
            }
            const int cnt = min(64, nn - c0);
            for (int j0 = 0; j0 < cnt; j0 += RB) {
                if (c0 > 0 || j0 > 0) {
#pragma unroll
                    for (int j = 0; j < RB; ++j)
#pragma unroll
                        for (int i = 0; i < PER; ++i)
                            v[j][i] = j0 + j < cnt ? rows[(long)(c0 + j0 + j) * split_stride * D + 64 * i] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + j));
#pragma unroll
                    for (int i = 0; i < PER; ++i) acc[i] += wj * v[j][i];
                }
            }
        }
        L = wave_sum(L);
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

// The value of feature e of a bf16 row after the rotary turn of its pair
// (features i and i + rot / 2, or 2i and 2i + 1 when interleaved): the pair
// (a, b) turns into (a cos - b sin, a sin + b cos) with the cosine and sine of
// pair index i at this position; features from rot on are unchanged.
__device__ __forceinline__ float bf16_at(const uint16_t* x, int e) {
    return __builtin_bit_cast(float, (uint32_t)x[e] << 16);
}

// Each product is rounded to float32 and then the difference or sum: the
// contraction into fused multiply-adds is switched off, so the rounding to
// bf16 that follows sees a fixed, reproducible float32 value.
__device__ __forceinline__ float rotary_feature(const uint16_t* x, int e, const float* cs, const float* sn,
                                                int rot, bool inter) {
#pragma clang fp contract(off)
    const float v = bf16_at(x, e);
    if (e >= rot) return v;
    const int half = rot >> 1;
    const bool first = inter ? (e & 1) == 0 : e < half;
    const int i = inter ? (e >> 1) : (first ? e : e - half);
    const int partner = inter ? (first ? e + 1 : e - 1) : (first ? e + half : e - half);
    const float w = bf16_at(x, partner);
    const float c = cs[i], s = sn[i];
    return first ? v * c - w * s : w * s + v * c;
}

// Append kernel: one wave per (request, row).  Rows 0 .. hkv-1 write K/V head
// `row` of the new token into the cache at position seqlens[b] (the key after
// its rotary turn, rounded to bf16; the value as given); rows hkv .. hkv+hq-1
// write query head `row - hkv` after its turn into q_rot.  A request whose
// position is negative, has no room in its table (or rotary table), or falls
// on an out-of-range page id writes nothing into the cache and NaN into its
// q_rot rows; the split kernel flags the same request and its output is NaN.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_append_kernel(AppendParams p) {
    const bool rope = p.rot_dim > 0;
    const int rows = p.hkv + (rope ? p.hq : 0);
    const int b = blockIdx.x / rows;
    const int r = blockIdx.x % rows;
    const int lane = threadIdx.x;
    const int pos = p.seqlens[b];
    bool bad = pos < 0 || (long)pos >= (long)p.max_pages * kPage || (rope && pos >= p.max_pos);
    int phys = 0;
    if (!bad) {
        phys = p.block_table[(long)b * p.max_pages + pos / kPage];
        bad = phys < 0 || phys >= p.num_pages;
    }
    const float* cs = rope && !bad ? p.rot_cos + (long)pos * (p.rot_dim >> 1) : nullptr;
    const float* sn = rope && !bad ? p.rot_sin + (long)pos * (p.rot_dim >> 1) : nullptr;
    const bool inter = p.interleaved != 0;
    if (r < p.hkv) {
        if (bad) return;
        const long src = ((long)b * p.hkv + r) * D;
        const long dst = (((long)phys * kPage + pos % kPage) * p.hkv + r) * D;
#pragma unroll
        for (int e = lane; e < D; e += 64) {
            const float kv = rope ? rotary_feature(p.k_new + src, e, cs, sn, p.rot_dim, inter)
                                  : bf16_at(p.k_new + src, e);
            p.k_cache[dst + e] = (uint16_t)(pack_bf16x2(kv, 0.0f) & 0xffffu);
            p.v_cache[dst + e] = p.v_new[src + e];
        }
    } else {
        const long row = ((long)b * p.hq + (r - p.hkv)) * D;
#pragma unroll
        for (int e = lane; e < D; e += 64) {
            const float qv = bad ? NAN : rotary_feature(p.q + row, e, cs, sn, p.rot_dim, inter);
            p.q_rot[row + e] = (uint16_t)(pack_bf16x2(qv, 0.0f) & 0xffffu);
        }
    }
}

hipError_t launch_decode_append(const AppendParams& p, int head_dim, hipStream_t s) {
    const long grid = (long)p.batch * (p.hkv + (p.rot_dim > 0 ? p.hq : 0));
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    switch (head_dim) {
        case 64:
            hipLaunchKernelGGL(attn_decode_append_kernel<64>, dim3((unsigned)grid), dim3(64), 0, s, p);
            break;
        case 128:
            hipLaunchKernelGGL(attn_decode_append_kernel<128>, dim3((unsigned)grid), dim3(64), 0, s, p);
            break;
        case 256:
            hipLaunchKernelGGL(attn_decode_append_kernel<256>, dim3((unsigned)grid), dim3(64), 0, s, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int QB, int HPW>
static hipError_t launch_split_hpw(const DecodeParams& p, hipStream_t s) {
    const long grid = (long)p.n_splits * (p.hkv / HPW) * p.batch;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_decode_split_kernel<D, QB, HPW>), dim3((unsigned)grid), dim3(64 * HPW), 0, s,
                       p);
    return hipGetLastError();
}

// Two K/V heads per workgroup when the head count allows it.
template <int D, int QB>
static hipError_t launch_split_cfg(const DecodeParams& p, hipStream_t s) {
    if (p.n_splits <= 0 || p.batch <= 0) return hipSuccess;
    return (p.hkv % 2 == 0) ? launch_split_hpw<D, QB, 2>(p, s) : launch_split_hpw<D, QB, 1>(p, s);
}

// 16-column blocks of query heads per K/V head.
template <int D>
static hipError_t launch_split_d(const DecodeParams& p, hipStream_t s) {
    const int g = p.hq / p.hkv;
    if (g <= 16) return launch_split_cfg<D, 1>(p, s);
    if (g <= 32) return launch_split_cfg<D, 2>(p, s);
    return launch_split_cfg<D, 4>(p, s);
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
