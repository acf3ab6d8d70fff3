// Steps 4-6 on gfx950: hybrid attention over (top-k or all visible compressed
// entries) U (raw window [p-S, p-1]) with one softmax and K = V ([Summary]
// 共享鍵和值向量, 短滑動窗口; [Notes] ⚠️ 注意：C128A 的因果性约束), then the
// inverse RoPE at the query position and the output store (fp32 / bf16 /
// fp8 + scales) fused as the epilogue ([Notes] Inverse RoPE 的数学原理,
// 融合 2：Inverse RoPE + FP8 Quant).
//
// Work mapping (MQA: every head shares the key rows).  A 256-thread workgroup
// serves one query (or one split of its key list); wave w owns heads
// 16w..16w+15 and keeps their q rows in registers as MFMA B operands.  Keys
// are processed in tiles of 32 gathered rows: each thread loads 4 rows x D/32
// dims (the next tile's loads are in flight while the current tile computes),
// dequantises fp8 if needed, and writes the tile to LDS twice -- row-major K
// for S^T = K.Q^T and transposed V^T for O^T = V^T.P^T -- so one HBM read of a
// row feeds both contractions.  Both are v_mfma_f32_16x16x32_bf16:
//   S^T[16 keys x 16 heads] : A = K rows (LDS), B = q (registers)
//   O^T[16 dims x 16 heads] : A = V^T rows (LDS), B = P^T (registers)
// The S^T accumulator layout (lane = head column, 4 keys per m-tile) is
// reused as the P^T operand without an LDS round trip: the key order inside
// the operand is permuted and V^T is read with the same permutation.  The
// online softmax runs in the exp2 domain with one max/sum per head column.
//
// Key addresses (top-k id -> block table -> page row) are resolved once per
// chunk of 8 tiles, one key per thread, into an LDS table, so a tile load is
// a single dependent global access.
//
// Precision variant (PREC, used for fp8 output, whose one-ULP acceptance near
// zero needs the pre-quantisation output to fp32-level accuracy): P is carried
// as P_hi + P_lo (two bf16 MFMAs), and fp8 keys are dequantised to fp32 and
// stored as two bf16 copies hi + lo, so S = K_hi.q + K_lo.q and
// O = V_hi.P_hi + V_hi.P_lo + V_lo.P_hi (~2^-16 relative).
#include "csl_kernels.hpp"

namespace csl {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;  // keys per tile
constexpr int kVtStride = kTile + 8;  // 80-byte rows: a 16-lane phase of 16-byte reads hits 64 distinct banks

template <int D>
struct Cfg {
    static constexpr int KS = D / 32;      // k-steps of S^T
    static constexpr int MT = D / 16;      // m-tiles of O^T
    static constexpr int DPT = D / 32;     // dims per loading thread
    static constexpr int KSTR = D + 8;     // K row stride (elements)
};

struct QueryInfo {
    int s;
    int64_t p;
    bool ok;
};

// (n: the same for every lane of the wave)
__device__ __forceinline__ QueryInfo query_info(const AttnArgs& a, int n) {
    QueryInfo qi;
    if (a.q_seq) {
        qi.s = a.q_seq[n];
        qi.p = a.q_pos[n];
    } else {
        int lo = 0, hi = a.num_seqs;
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (a.cu_q[mid] <= n) lo = mid;
            else hi = mid;
        }
        qi.s = lo;
        qi.p = a.q_pos_start[lo] + (n - a.cu_q[lo]);
    }
    // n is the same across the wave, so are s and p: scalar registers for them and
    // for everything derived from them (key counts, tile loop bounds)
    qi.s = __builtin_amdgcn_readfirstlane(qi.s);
    qi.p = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)((uint64_t)qi.p >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qi.p));
    qi.ok = qi.s >= 0 && qi.s < a.num_seqs && qi.p >= 0 && qi.p <= a.max_q_pos;
    return qi;
}

__device__ __forceinline__ int row_bytes(int dtype, int D) { return dtype == kFP8 ? D + D / 16 : 2 * D; }

// Address of key j of the query's list, or null if masked.
__device__ __forceinline__ const uint8_t* key_row(const AttnArgs& a, int n, int s, int64_t j, int64_t Lc,
                                                  int64_t nv_c, int64_t lo) {
    const int D = a.dim;
    if (j < Lc) {
        int64_t id = a.topk ? (int64_t)a.topk[(int64_t)n * a.k + j] : j;
        if (id < 0) return nullptr;
        if (id >= nv_c) {
            raise_error(a.err, kErrTopk);
            return nullptr;
        }
        int32_t pg = page_of(a.bt, a.max_blocks, a.comp_pages, s, id * a.comp_ratio);
        if (pg < 0) {
            raise_error(a.err, kErrPage);
            return nullptr;
        }
        int per = kBlockPositions / a.comp_ratio;
        return a.comp_rows + ((int64_t)pg * per + (id % per)) * row_bytes(a.comp_dtype, D);
    }
    int64_t t = lo + (j - Lc);
    int32_t pg = page_of(a.bt, a.max_blocks, a.swa_pages, s, t);
    if (pg < 0) {
        raise_error(a.err, kErrPage);
        return nullptr;
    }
    return a.swa_rows + ((int64_t)pg * kBlockPositions + (t & 255)) * row_bytes(a.swa_dtype, D);
}

// key_row for the keys kb + u*NT + tid (u < NU) of one thread at once: every
// top-k id is loaded before any page-table entry, so the dependent global
// loads of the NU keys overlap instead of running one key after another.
// With use_pre, `pre` holds the ids of these keys loaded earlier (top-k
// entries for j < k, else j).
template <int NU, int NT>
__device__ __forceinline__ void key_rows(const AttnArgs& a, int n, int s, int64_t kb, int64_t ke, int64_t Lc,
                                         int64_t nv_c, int64_t lo, const uint8_t* (&row)[NU], bool use_pre,
                                         const int64_t (&pre)[NU]) {
    const int tid = threadIdx.x;
    int64_t id[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int64_t j = kb + u * NT + tid;
        const bool in = j < ke && j < Lc;
        id[u] = !in ? -1 : use_pre ? pre[u] : a.topk ? (int64_t)a.topk[(int64_t)n * a.k + j] : j;
    }
    int64_t t[NU];
    int32_t pg[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int64_t j = kb + u * NT + tid;
        const bool comp = j < Lc;
        if (comp && id[u] >= nv_c) {
            raise_error(a.err, kErrTopk);
            id[u] = -1;
        }
        t[u] = j >= ke ? -1 : comp ? (id[u] >= 0 ? id[u] * a.comp_ratio : -1) : lo + (j - Lc);
        pg[u] = t[u] >= 0 ? page_of(a.bt, a.max_blocks, comp ? a.comp_pages : a.swa_pages, s, t[u]) : -1;
    }
    const int D = a.dim;
    const int per = kBlockPositions / (a.comp_ratio > 0 ? a.comp_ratio : 1);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int64_t j = kb + u * NT + tid;
        row[u] = nullptr;
        if (t[u] < 0) continue;
        if (pg[u] < 0) {
            raise_error(a.err, kErrPage);
            continue;
        }
        row[u] = j < Lc ? a.comp_rows + ((int64_t)pg[u] * per + (id[u] % per)) * row_bytes(a.comp_dtype, D)
                        : a.swa_rows + ((int64_t)pg[u] * kBlockPositions + (t[u] & 255)) * row_bytes(a.swa_dtype, D);
    }
}

// A thread's slice of 4 key rows: bf16 words, or fp8 codes + the group scale.
template <int D, int KV>
struct Slice {
    static constexpr int W = KV == kFP8 ? Cfg<D>::DPT / 4 : Cfg<D>::DPT / 2;  // 32-bit words per key
    uint32_t w[4][W];
    float scale[4];
    bool valid[4];
};

template <int D, int KV>
__device__ __forceinline__ void load_slice(Slice<D, KV>& sl, const uint8_t* const* rows, int kg, int dc) {
    constexpr int DPT = Cfg<D>::DPT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint8_t* row = rows[4 * kg + q];
        sl.valid[q] = row != nullptr;
        if constexpr (KV == kBF16) {
            if constexpr (DPT == 16) {
                u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
                if (row) {
                    v0 = *reinterpret_cast<const u32x4*>(row + dc * DPT * 2);
                    v1 = *reinterpret_cast<const u32x4*>(row + dc * DPT * 2 + 16);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    sl.w[q][c] = v0[c];
                    sl.w[q][4 + c] = v1[c];
                }
            } else {
                static_assert(DPT == 4, "dims per loading thread");
                u32x2 v = {0u, 0u};
                if (row) v = *reinterpret_cast<const u32x2*>(row + dc * DPT * 2);
                sl.w[q][0] = v[0];
                sl.w[q][1] = v[1];
            }
        } else {
            u32x4 v = {0u, 0u, 0u, 0u};
            float sc = 0.f;
            if (row) {
                v = *reinterpret_cast<const u32x4*>(row + dc * DPT);
                sc = *reinterpret_cast<const float*>(row + D + 4 * ((dc * DPT) / 64));
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) sl.w[q][c] = v[c];
            sl.scale[q] = sc;
        }
    }
}

template <int D>
__device__ __forceinline__ void write_kv(const uint32_t (&h)[4][Cfg<D>::DPT], uint16_t* Kl, uint16_t* Vt, int kg,
                                         int dc) {
    constexpr int DPT = Cfg<D>::DPT, KSTR = Cfg<D>::KSTR;
    // K rows
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint16_t* dst = Kl + (4 * kg + q) * KSTR + dc * DPT;
        if constexpr (DPT % 8 == 0) {
#pragma unroll
            for (int e = 0; e < DPT; e += 8) {
                u32x4 v;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = h[q][e + 2 * c] | (h[q][e + 2 * c + 1] << 16);
                *reinterpret_cast<u32x4*>(dst + e) = v;
            }
        } else {
            *reinterpret_cast<u32x2*>(dst) = u32x2{h[q][0] | (h[q][1] << 16), h[q][2] | (h[q][3] << 16)};
        }
    }
    // V^T rows in the order the P^T operand uses: position 8g + c holds key
    // 4g + c (c < 4) or 16 + 4g + (c - 4) (c >= 4), so a lane's 8 keys are one
    // 16-byte read.  This thread's keys 4kg..4kg+3 land at 4 adjacent positions.
    const int vpos = kg < 4 ? 8 * kg : 8 * (kg - 4) + 4;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
        u32x2 v = {h[0][e] | (h[1][e] << 16), h[2][e] | (h[3][e] << 16)};
        *reinterpret_cast<u32x2*>(Vt + (dc * DPT + e) * kVtStride + vpos) = v;
    }
}

// Write a thread's slice to LDS: K rows and V^T rows (and, with SPLITKV, the
// bf16 remainder copies).
template <int D, int KV, bool SPLITKV>
__device__ __forceinline__ void store_slice(const Slice<D, KV>& sl, uint16_t* Kl, uint16_t* Vt, uint16_t* Kl_lo,
                                            uint16_t* Vt_lo, uint32_t* valid, int kg, int dc) {
    constexpr int DPT = Cfg<D>::DPT;
    uint32_t h[4][DPT];  // bf16 bits, key q, element e
    uint32_t lo[4][SPLITKV ? DPT : 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (KV == kBF16) {
#pragma unroll
            for (int e = 0; e < DPT; ++e) h[q][e] = (sl.w[q][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        } else {
#pragma unroll
            for (int e = 0; e < DPT; ++e) {
                float v = e4m3_to_f32((sl.w[q][e >> 2] >> (8 * (e & 3))) & 0xffu) * sl.scale[q];
                h[q][e] = f32_to_bf16_bits(v);
                if constexpr (SPLITKV) lo[q][e] = f32_to_bf16_bits(v - bf16_bits_to_f32(h[q][e]));
            }
        }
    }
    write_kv<D>(h, Kl, Vt, kg, dc);
    if constexpr (SPLITKV) write_kv<D>(lo, Kl_lo, Vt_lo, kg, dc);
    if (dc == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) valid[4 * kg + q] = sl.valid[q] ? 1u : 0u;
    }
}

template <int D, int KV, bool PREC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 4)))
hybrid_attn_kernel(AttnArgs a) {
    static_assert(D == 128, "512-dim keys take hybrid_attn_mqa512_kernel; this kernel serves 128-dim keys");
    constexpr int KS = Cfg<D>::KS, MT = Cfg<D>::MT, KSTR = Cfg<D>::KSTR;
    constexpr bool SPLITKV = PREC && KV == kFP8;
    constexpr int NC = SPLITKV ? 2 : 1;
    constexpr int kChunkTiles = kThreads / kTile;  // tiles whose addresses one pass resolves
    __shared__ __attribute__((aligned(16))) uint16_t s_k[NC][kTile * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[NC][D * kVtStride];
    __shared__ const uint8_t* s_rows[kThreads];
    __shared__ uint32_t s_valid[kTile];
    __shared__ float s_rope[2][64];  // cos, sin of -p * theta^(-2j/R) for the R/2 pairs

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int kg = tid & 7, dc = tid >> 3;
    const int n = blockIdx.x % a.num_q;
    const int sp = blockIdx.x / a.num_q;

    QueryInfo qi = query_info(a, n);
    if (!qi.ok && sp == 0 && tid == 0) raise_error(a.err, (qi.s < 0 || qi.s >= a.num_seqs) ? kErrSeq : kErrPos);
    const int s = qi.s;
    const int64_t p = qi.ok ? qi.p : 0;
    const int64_t nv_c = (qi.ok && a.comp_rows) ? p / a.comp_ratio : 0;
    const int64_t Lc = a.comp_rows ? (a.topk ? (int64_t)a.k : nv_c) : 0;
    const int64_t lo = p - a.swa_window > 0 ? p - a.swa_window : 0;
    const int64_t L = qi.ok ? Lc + (p - lo) : 0;
    const int64_t n_tiles = (L + kTile - 1) / kTile;
    const int64_t tps = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int64_t t_begin = sp * tps;
    const int64_t t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;

    const int head = 16 * wave + r16;
    const bool wave_active = 16 * wave < a.n_heads;
    if (a.n_splits == 1 && tid < a.rope_dims / 2) rope_cs(-p, a.rf.inv_freq[tid], s_rope[0][tid], s_rope[1][tid]);

    // q rows as B operands: lane = head column, 8 dims per k-step
    bf16x8 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (head < a.n_heads) v = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)n * a.n_heads + head) * D + 32 * ks + 8 * g);
        qb[ks] = __builtin_bit_cast(bf16x8, v);
    }

    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    Slice<D, KV> sl;
    for (int64_t cs = t_begin; cs < t_end; cs += kChunkTiles) {
        const int64_t ce = cs + kChunkTiles < t_end ? cs + kChunkTiles : t_end;
        __syncthreads();  // the previous chunk's reads of s_rows are done
        {
            const int64_t j = cs * kTile + tid;
            s_rows[tid] = (j < ce * kTile && j < L) ? key_row(a, n, s, j, Lc, nv_c, lo) : nullptr;
        }
        __syncthreads();
        load_slice<D, KV>(sl, s_rows, kg, dc);
        for (int64_t t = cs; t < ce; ++t) {
            __syncthreads();  // the previous tile's LDS reads are done
            store_slice<D, KV, SPLITKV>(sl, s_k[0], s_vt[0], s_k[NC - 1], s_vt[NC - 1], s_valid, kg, dc);
            __syncthreads();
            if (t + 1 < ce) load_slice<D, KV>(sl, s_rows + (t + 1 - cs) * kTile, kg, dc);
            if (!wave_active) continue;

            // S^T = K . Q^T for the tile's two 16-key m-tiles
            f32x4 st[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint16_t* krow = s_k[c] + (16 * mt + r16) * KSTR + 8 * g;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
                        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], st[mt], 0, 0, 0);
                    }
                }
            }
            // online softmax over this head column (keys 16mt + 4g + i)
            float x[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s_valid[16 * mt + 4 * g + i] ? st[mt][i] * a.scale_log2 : -INFINITY;
                    x[4 * mt + i] = v;
                    tmax = fmaxf(tmax, v);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            float psum = 0.f;
            uint32_t pw[4], pl[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float p0 = exp2f(x[2 * c] - m_use), p1 = exp2f(x[2 * c + 1] - m_use);
                psum += p0 + p1;
                pw[c] = pack_bf16x2(p0, p1);
                if constexpr (PREC) {
                    pl[c] = pack_bf16x2(p0 - bf16_bits_to_f32(pw[c] & 0xffffu), p1 - bf16_bits_to_f32(pw[c] >> 16));
                }
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] *= alpha;
            }
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
            bf16x8 pbl = pb;
            if constexpr (PREC) pbl = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
            // O^T += V^T . P^T; operand slot c <-> key 4g+c (c<4), 16+4g+(c-4) (c>=4)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bf16x8 va = *reinterpret_cast<const bf16x8*>(s_vt[0] + (16 * m + r16) * kVtStride + 8 * g);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[m], 0, 0, 0);
                if constexpr (PREC) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbl, acc[m], 0, 0, 0);
                if constexpr (SPLITKV) {
                    const bf16x8 vb =
                        *reinterpret_cast<const bf16x8*>(s_vt[NC - 1] + (16 * m + r16) * kVtStride + 8 * g);
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb, acc[m], 0, 0, 0);
                }
            }
        }
    }
    __syncthreads();  // every wave passes here: s_rope is visible to the epilogue
    if (!wave_active) return;

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (head >= a.n_heads) return;

    if (a.n_splits > 1) {
        // unnormalised partial: O^T rows 16m + 4g + i of this head
        float* po = a.part_o + (((int64_t)n * a.n_splits + sp) * a.n_heads + head) * D;
#pragma unroll
        for (int m = 0; m < MT; ++m) *reinterpret_cast<f32x4*>(po + 16 * m + 4 * g) = acc[m];
        if (g == 0) {
            float* ml = a.part_ml + (((int64_t)n * a.n_splits + sp) * a.n_heads + head) * 2;
            ml[0] = m_run;
            ml[1] = l_tot;
        }
        return;
    }

    // epilogue: normalise, RoPE^-1 at p, store
    const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int rbase = D - a.rope_dims;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        acc[m] *= inv_l;
        const int d0 = 16 * m + 4 * g;
        if (d0 >= rbase) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = (d0 + 2 * c - rbase) >> 1;
                const float cs = s_rope[0][j], sn = s_rope[1][j];
                float u = acc[m][2 * c], v = acc[m][2 * c + 1];
                acc[m][2 * c] = u * cs - v * sn;
                acc[m][2 * c + 1] = u * sn + v * cs;
            }
        }
    }
    const int64_t obase = ((int64_t)n * a.n_heads + head) * D;
    if (a.out_dtype == kF32) {
        float* o = reinterpret_cast<float*>(a.out) + obase;
#pragma unroll
        for (int m = 0; m < MT; ++m) *reinterpret_cast<f32x4*>(o + 16 * m + 4 * g) = acc[m];
    } else if (a.out_dtype == kBF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + obase;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<u32x2*>(o + 16 * m + 4 * g) =
                u32x2{pack_bf16x2(acc[m][0], acc[m][1]), pack_bf16x2(acc[m][2], acc[m][3])};
    } else {
        // 64-element groups = 4 consecutive m-tiles x the 4 lanes g of this head
        uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + obase;
        float gmax[D / 64];
#pragma unroll
        for (int G = 0; G < D / 64; ++G) gmax[G] = 0.f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) gmax[m >> 2] = fmaxf(gmax[m >> 2], fabsf(acc[m][i]));
#pragma unroll
        for (int G = 0; G < D / 64; ++G) {
            float v = fmaxf(gmax[G], __shfl_xor(gmax[G], 16));
            v = fmaxf(v, __shfl_xor(v, 32));
            gmax[G] = v > 0.f ? v / 448.0f : 1.0f;  // the group's scale
            if (g == 0) a.out_scales[((int64_t)n * a.n_heads + head) * (D / 64) + G] = gmax[G];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float r = 1.0f / gmax[m >> 2];
            *reinterpret_cast<uint32_t*>(o + 16 * m + 4 * g) =
                e4m3_pack4(acc[m][0] * r, acc[m][1] * r, acc[m][2] * r, acc[m][3] * r);
        }
    }
}

// Merge the splits of (query, head), 8 dims per lane.  SHARE (many splits):
// one workgroup of NW waves per (query, head); wave w takes splits w, w + NW,
// ..., the NW running (max, sum, output) meet in LDS and wave 0 finishes, so
// that each wave's chain of dependent batches stays short.  Otherwise one wave
// per (query, head) takes every split (four heads per workgroup).
template <int D, bool SHARE, int NW = 4>
__global__ void __launch_bounds__(64 * NW) attn_combine_kernel(AttnArgs a) {
    static_assert(SHARE || NW == 4, "one wave per head: four heads per workgroup");
    __shared__ float s_o[SHARE ? NW : 1][64][8];
    __shared__ float s_ml[NW][2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hpb = SHARE ? 1 : 4;  // heads per workgroup
    const int n = blockIdx.x / ((a.n_heads + hpb - 1) / hpb);
    const int head = (blockIdx.x % ((a.n_heads + hpb - 1) / hpb)) * hpb + (SHARE ? 0 : wave);
    if (head >= a.n_heads) return;
    const int w0 = SHARE ? wave : 0, wstep = SHARE ? NW : 1;
    const bool active = 8 * lane < D;
    // the query's position (for the inverse RoPE) is loaded beside the partials
    QueryInfo qi = query_info(a, n);

    const float* ml = a.part_ml + ((int64_t)n * a.n_splits * a.n_heads + head) * 2;
    const int64_t mstride = (int64_t)a.n_heads * 2;
    const float* po = a.part_o + ((int64_t)n * a.n_splits * a.n_heads + head) * D + 8 * (active ? lane : 0);
    const int64_t pstride = (int64_t)a.n_heads * D;
    // batches of 8 of this wave's splits: all loads of a batch are issued before
    // any use; the running max M rescales what earlier batches accumulated
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float Lsum = 0.f, M = -INFINITY;
    constexpr int kB = SHARE ? 8 : 16;
    for (int sp0 = w0; sp0 < a.n_splits; sp0 += wstep * kB) {
        f32x4 v0[kB], v1[kB];
        float msp[kB], lsp[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            msp[u] = -INFINITY;
            lsp[u] = 0.f;
            v0[u] = v1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int sp = sp0 + wstep * u;
            if (sp < a.n_splits) {
                msp[u] = ml[sp * mstride];
                lsp[u] = ml[sp * mstride + 1];
                v0[u] = *reinterpret_cast<const f32x4*>(po + sp * pstride);
                v1[u] = *reinterpret_cast<const f32x4*>(po + sp * pstride + 4);
            }
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kB; ++u) Mb = fmaxf(Mb, msp[u]);
        const float Mu = Mb == -INFINITY ? 0.f : Mb;
        const float r = exp2f(M - Mu);  // 0 while nothing was accumulated
        Lsum *= r;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] *= r;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            // an empty split stored m = -inf, l = 0 and zeros: its weight is 0
            const float wsp = exp2f(msp[u] - Mu);
            Lsum = fmaf(lsp[u], wsp, Lsum);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[c] = fmaf(wsp, v0[u][c], o[c]);
                o[4 + c] = fmaf(wsp, v1[u][c], o[4 + c]);
            }
        }
        M = Mb;
    }
    if constexpr (SHARE) {
#pragma unroll
        for (int c = 0; c < 8; ++c) s_o[wave][lane][c] = o[c];
        if (lane == 0) {
            s_ml[wave][0] = M;
            s_ml[wave][1] = Lsum;
        }
        __syncthreads();
        if (wave != 0) return;
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0]);
        const float Mu = M == -INFINITY ? 0.f : M;
        Lsum = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float r = exp2f(s_ml[w][0] - Mu);  // a wave without splits holds -inf: weight 0
            Lsum = fmaf(s_ml[w][1], r, Lsum);
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = fmaf(r, s_o[w][lane][c], o[c]);
        }
    }
    const int64_t p = qi.ok ? qi.p : 0;
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    const int rbase = D - a.rope_dims;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= inv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int d = 8 * lane + 2 * c;
        if (active && d >= rbase) {  // (a lane past the row has no pair: its index would leave the table)
            float cs, sn;
            rope_cs(-p, a.rf.inv_freq[(d - rbase) >> 1], cs, sn);
            float u = o[2 * c], v = o[2 * c + 1];
            o[2 * c] = u * cs - v * sn;
            o[2 * c + 1] = u * sn + v * cs;
        }
    }
    const int64_t obase = ((int64_t)n * a.n_heads + head) * D + 8 * lane;
    if (a.out_dtype == kF32) {
        if (active) {
            float* dst = reinterpret_cast<float*>(a.out) + obase;
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
    } else if (a.out_dtype == kBF16) {
        if (active)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + obase) =
                u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                      pack_bf16x2(o[6], o[7])};
    } else {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(o[c]));
        amax = group8_max(active ? amax : 0.f);
        const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
        if (active) {
            const float r = 1.0f / scale;
            const u32x2 w = {e4m3_pack4(o[0] * r, o[1] * r, o[2] * r, o[3] * r),
                             e4m3_pack4(o[4] * r, o[5] * r, o[6] * r, o[7] * r)};
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.out) + obase) = w;
            if ((lane & 7) == 0) a.out_scales[((int64_t)n * a.n_heads + head) * (D / 64) + (lane >> 3)] = scale;
        }
    }
}


// ---------------------------------------------------------------- 512-dim bf16 keys, 32x32 tiles

// hybrid_attn_mqa512_kernel -- the path for bf16 keys of 512 dims (every
// layer of the decode and prefill workloads).  One 256-thread workgroup per
// (query, split); wave w owns heads 32 (w & 1) .. +31 and output dims
// 256 (w >> 1) .. +255.  Per tile of 32 gathered key rows:
//   * the rows are staged in LDS in their stored (row-major) layout by direct
//     global->LDS loads (each wave copies 8 rows, one 1 KiB row per
//     instruction) into a ring of 4 tiles: up to three tiles are in flight
//     while one is computed, with no registers held for them;
//   * S^T[32 keys x 32 heads] = K . Q^T on v_mfma_f32_32x32x16_bf16: A = key
//     rows from LDS, B = the wave's q rows over its 256 dims (registers); the
//     two halves of a head group are summed through LDS;
//   * online softmax per head column in the exp2 domain (v_exp_f32: weights
//     below 2^-126 of the reference flush to 0) with a lazy reference
//     max: the accumulator is rescaled only when the max grows past the
//     reference by more than 8 (so P <= 2^8), which makes rescales rare;
//   * software pipelined: the S MFMAs of the next tile are issued before the
//     softmax of the current one, so the matrix unit and the vector ALU
//     overlap within the wave (one wave per SIMD);
//   * O^T[256 dims x 32 heads] += V^T . P^T: B = P straight from the S
//     accumulator (a lane holds 16 keys of its head; they are assigned to the
//     two k-steps' slots), A = V^T read from the row-major tile with the
//     transposing LDS read ds_read_b64_tr_b16 (in each 16-lane group, output
//     lane 4b+e receives element e of the 8-byte reads of lanes b, b+4, b+8,
//     b+12: four lanes pointing at four key rows give a lane four keys of one
//     dim), so no transposed copy of the tile is written.
// With PREC (fp8 output) P is carried as P_hi + P_lo.  The epilogue and the
// split partials match hybrid_attn_kernel's.
constexpr int kT2 = 32;          // keys per tile
constexpr int kRow2 = 1040;      // LDS stride of a staged row (1024 B + 16: spreads the S-operand reads)
constexpr int kMaxKeys2 = 1024;  // key addresses resolved per pass
constexpr int kRing2 = 4;        // staged tiles: one computed, up to three in flight
// fp8 keys: 544-byte rows (512 e4m3 codes, 8 fp32 group scales) land in a
// 3-slot ring and are widened to exact bf16 codes in two bf16 tiles; the
// group scales go to a [8][32] table per tile
constexpr int kRow8 = 560;       // LDS stride of a staged fp8 row (544 B + 16)
constexpr int kFp8Ring = 3 * kT2 * kRow8;
constexpr int kFp8Bf16 = kFp8Ring;                      // offset of the two bf16 tiles
constexpr int kFp8Scales = kFp8Bf16 + 2 * kT2 * kRow2;  // offset of the two scale tables
static_assert(kFp8Scales + 2 * 8 * kT2 * 4 <= kRing2 * kT2 * kRow2, "fp8 staging fits the ring");

// Source of masked key rows (zeros: a masked key then contributes 0 * 0).
__device__ __attribute__((aligned(16))) uint8_t g_zero_kv_row[1024];

// One 1 KiB row from global memory straight into LDS: lane l's 16 bytes land
// at lds + 16 l (M0 holds the LDS address).  Issued as inline assembly so the
// compiler does not order later LDS reads behind it; the caller waits with an
// explicit vmcnt before the barrier that publishes the tile.
__device__ __forceinline__ void lds_dma_row(uint32_t lds, const uint8_t* src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)p);
}

typedef short short4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(const_cast<uint8_t*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// acc *= f for an accumulator tile held in AGPRs, in place.  Written as one
// assembly block over the 16 registers (read, multiply, write back through
// one VGPR) so that the compiler keeps no VGPR copy of the accumulator alive
// for this rarely taken path; the trailing wait states cover an MFMA that
// reads the tile next.
__device__ __forceinline__ void scale_agpr16(f32x16& acc, float f) {
    float e0 = acc[0], e1 = acc[1], e2 = acc[2], e3 = acc[3], e4 = acc[4], e5 = acc[5], e6 = acc[6], e7 = acc[7];
    float e8 = acc[8], e9 = acc[9], e10 = acc[10], e11 = acc[11], e12 = acc[12], e13 = acc[13], e14 = acc[14],
          e15 = acc[15];
    float t;
#define CSL_RS(i) "v_accvgpr_read_b32 %16, %" #i "\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %" #i ", %16\n\t"
    asm volatile(CSL_RS(0) CSL_RS(1) CSL_RS(2) CSL_RS(3) CSL_RS(4) CSL_RS(5) CSL_RS(6) CSL_RS(7) CSL_RS(8) CSL_RS(9)
                     CSL_RS(10) CSL_RS(11) CSL_RS(12) CSL_RS(13) CSL_RS(14) CSL_RS(15) "s_nop 7"
                 : "+a"(e0), "+a"(e1), "+a"(e2), "+a"(e3), "+a"(e4), "+a"(e5), "+a"(e6), "+a"(e7), "+a"(e8), "+a"(e9),
                   "+a"(e10), "+a"(e11), "+a"(e12), "+a"(e13), "+a"(e14), "+a"(e15), "=&v"(t)
                 : "v"(f));
#undef CSL_RS
    acc = f32x16{e0, e1, e2, e3, e4, e5, e6, e7, e8, e9, e10, e11, e12, e13, e14, e15};
}

template <bool PREC, bool KV8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
hybrid_attn_mqa512_kernel(AttnArgs a) {
    constexpr int D = 512;
    // bf16 keys: 4 ring slots of 32 rows.  fp8 keys: 3 slots of raw rows, 2
    // bf16 tiles, 2 scale tables (see kFp8*).  Also the epilogue's staging area.
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[kRing2 * kT2 * kRow2];
    constexpr int kSlots = KV8 ? 3 : kRing2;
    constexpr int kRowDma = KV8 ? kRow8 : kRow2;
    // where the DMA of tile tl lands, the bf16 tile S and PV read, its scale table
    auto dma_slot = [&](int tl) { return s_ring + (tl % kSlots) * (kT2 * kRowDma); };
    auto kt_of = [&](int tl) -> const uint8_t* {
        return KV8 ? s_ring + kFp8Bf16 + (tl & 1) * (kT2 * kRow2) : s_ring + (tl % kRing2) * (kT2 * kRow2);
    };
    auto sc_of = [&](int tl) { return reinterpret_cast<float*>(s_ring + kFp8Scales + (tl & 1) * (8 * kT2 * 4)); };
    __shared__ __attribute__((aligned(16))) float s_sx[4][64 * 16];  // S^T partials, one per wave
    __shared__ const uint8_t* s_rows[kMaxKeys2];
    __shared__ uint32_t s_vbits[kMaxKeys2 / 32];
    __shared__ float s_rope[2][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, h2 = lane >> 5;
    const int hg = wave & 1, dh = wave >> 1;
    const int n = blockIdx.x % a.num_q;
    const int sp = blockIdx.x / a.num_q;

    // Loads that do not depend on the query's position go first, so their
    // latencies overlap with the position lookup: the q rows and the top-k ids
    // of the first key pass (a split's key range is fixed by the host-side
    // tiles-per-split bound, not by the position).
    const int head = 32 * hg + r32;
    const bool hv = head < a.n_heads;
    // q as the B operand of S^T over the wave's 256 dims: column = head, k-step ks =
    // dims 256 dh + 16 ks + 8 h2 .. +7
    // (a missing head reads zeros from the zero row: 512 bf16, the same span)
    bf16x8 qb[16];
    {
        const uint16_t* qrow = (hv ? a.q + ((int64_t)n * a.n_heads + head) * D
                                   : reinterpret_cast<const uint16_t*>(g_zero_kv_row)) + 256 * dh + 8 * h2;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
    }
    const int64_t t_begin = a.n_splits > 1 ? (int64_t)sp * a.tiles_per_split : 0;
    constexpr int kPer = kMaxKeys2 / kThreads;
    int64_t pre_id[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t j = t_begin * kT2 + u * kThreads + tid;
        pre_id[u] = (a.topk && a.comp_rows && j < a.k) ? (int64_t)a.topk[(int64_t)n * a.k + j] : j;
    }

    QueryInfo qi = query_info(a, n);
    if (!qi.ok && sp == 0 && tid == 0) raise_error(a.err, (qi.s < 0 || qi.s >= a.num_seqs) ? kErrSeq : kErrPos);
    const int s = qi.s;
    const int64_t p = qi.ok ? qi.p : 0;
    const int64_t nv_c = (qi.ok && a.comp_rows) ? p / a.comp_ratio : 0;
    const int64_t Lc = a.comp_rows ? (a.topk ? (int64_t)a.k : nv_c) : 0;
    const int64_t lo = p - a.swa_window > 0 ? p - a.swa_window : 0;
    const int64_t L = qi.ok ? Lc + (p - lo) : 0;
    const int64_t n_tiles = (L + kT2 - 1) / kT2;
    const int64_t t_end = a.n_splits > 1 ? (t_begin + a.tiles_per_split < n_tiles ? t_begin + a.tiles_per_split : n_tiles)
                                         : n_tiles;
    const int64_t k_end = t_end * kT2 < L ? t_end * kT2 : L;
    if (a.n_splits == 1 && tid < a.rope_dims / 2) rope_cs(-p, a.rf.inv_freq[tid], s_rope[0][tid], s_rope[1][tid]);

    // An AGPR operand in inline assembly makes the compiler select the MFMAs'
    // accumulator-register form, so the output accumulator stays in AGPRs.
    asm volatile("; accumulators in AGPRs" ::"a"(0.f));
    // O^T tiles m = 0..7: value 4j + i = dim 256 dh + 32 m + 8 j + 4 h2 + i of this head
    f32x16 oacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int c = 0; c < 16; ++c) oacc[m][c] = 0.f;
    float m_ref = -INFINITY, l_run = 0.f;

    // transposed-read addresses: within 16-lane group G = lane / 16 (dims
    // 16 (G & 1) .. +15 of a 32-dim tile, key half h2 = G / 2), lane 4c + b
    // points at the key of slot c of its group (key 16 h2 + 4c + 2kk, + 1 for
    // the second read), dims +4b .. +4b+3
    const int ig = lane & 15, G = lane >> 4;
    const int tr_row = 16 * (G >> 1) + 4 * (ig >> 2);
    const int tr_col = (256 * dh + 16 * (G & 1) + 4 * (ig & 3)) * 2;  // bytes, + 64 m

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // (all 8 row addresses are read before the first copy is issued: the
    // copies' memory clobber would otherwise order each read behind them)
    auto issue_tile = [&](int tl) {
        const uint8_t* buf = dma_slot(tl);
        const uint8_t* row[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = s_rows[tl * kT2 + 8 * wave_u + i];
        if (!KV8 || lane < 34) {  // an fp8 row is 34 x 16 bytes
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_dma_row(lds_addr(buf + (8 * wave_u + i) * kRowDma), row[i] + 16 * lane);
        }
    };
    // fp8 keys: tile tl's codes widened to bf16 (e4m3 values are exact in bf16:
    // the conversion unit with scale 1) and its group scales into the table;
    // thread = (row tid / 8, 64-code group tid % 8)
    auto convert = [&](int tl) {
        const int row = tid >> 3, g = tid & 7;
        const uint8_t* src = dma_slot(tl) + row * kRow8;
        uint8_t* dst = const_cast<uint8_t*>(kt_of(tl)) + row * kRow2 + 128 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + 64 * g + 16 * q);
            u32x4 o0, o1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[c], 1.0f, false));
                const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[c], 1.0f, true));
                if (c < 2) {
                    o0[2 * c] = lo;
                    o0[2 * c + 1] = hi;
                } else {
                    o1[2 * c - 4] = lo;
                    o1[2 * c - 3] = hi;
                }
            }
            *reinterpret_cast<u32x4*>(dst + 32 * q) = o0;
            *reinterpret_cast<u32x4*>(dst + 32 * q + 16) = o1;
        }
        sc_of(tl)[g * kT2 + row] = *reinterpret_cast<const float*>(src + 512 + 4 * g);
    };
    // the wave's half of S^T for a staged tile (its 256 dims): A = key rows (LDS), B = q
    // accumulator row r = 8j + 4h + i holds key sigma(r) = 16h + 4i + j of the tile:
    // then the four keys a transposed read gathers (i = 0..3) sit 4 rows apart,
    // whose 32-byte windows fall in disjoint LDS banks
    const int s_row = 16 * ((r32 >> 2) & 1) + 4 * (r32 & 3) + (r32 >> 3);
    auto s_loads = [&](const uint8_t* kt, bf16x8 (&ka)[16]) {
        const uint8_t* krow = kt + s_row * kRow2 + 512 * dh + 16 * h2;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
    };
    // the scales of the lane's 16 keys (16 h2 + 0..15) in 64-dim group g of the row
    auto key_scales = [&](const float* sc, int g, float (&v)[16]) {
        const float* p = sc + g * kT2 + 16 * h2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p + 4 * q);
            v[4 * q] = x[0];
            v[4 * q + 1] = x[1];
            v[4 * q + 2] = x[2];
            v[4 * q + 3] = x[3];
        }
    };
    auto s_mfma = [&](const bf16x8 (&ka)[16], const float* sc) {
        f32x16 s0;
#pragma unroll
        for (int c = 0; c < 16; ++c) s0[c] = 0.f;
        if constexpr (!KV8) {
            // one accumulation chain (dependent 32x32x16 MFMAs issue back to back)
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[ks], s0, 0, 0, 0);
        } else {
            // one chain per 64-dim group over the exact codes, then the keys' group
            // scales in fp32: value c is key 16 h2 + 4 (c % 4) + c / 4
#pragma unroll
            for (int lg = 0; lg < 4; ++lg) {
                f32x16 acc;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[c] = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[4 * lg + q], qb[4 * lg + q], acc, 0, 0, 0);
                float v[16];
                key_scales(sc, 4 * dh + lg, v);
#pragma unroll
                for (int c = 0; c < 16; ++c) s0[c] = fmaf(acc[c], v[4 * (c & 3) + (c >> 2)], s0[c]);
            }
        }
        return s0;
    };
    // the two halves of a head group meet in LDS (the lanes of waves w and w ^ 2
    // hold the same (head, key) positions)
    // (layout [wave][quad][lane][4]: a quad's 16-byte accesses of 16 lanes hit distinct banks)
    float* sx_mine = s_sx[wave] + 4 * lane;
    const float* sx_other = s_sx[wave ^ 2] + 4 * lane;
    auto put_half = [&](const f32x16& h) {
#pragma unroll
        for (int c = 0; c < 16; c += 4)
            *reinterpret_cast<f32x4*>(sx_mine + 64 * c) = f32x4{h[c], h[c + 1], h[c + 2], h[c + 3]};
    };
    auto add_other = [&](f32x16& h) {
#pragma unroll
        for (int c = 0; c < 16; c += 4) {
            const f32x4 o = *reinterpret_cast<const f32x4*>(sx_other + 64 * c);
            h[c] += o[0];
            h[c + 1] += o[1];
            h[c + 2] += o[2];
            h[c + 3] += o[3];
        }
    };
    // softmax update for a tile whose S^T is in sacc (branch-free): P operands of
    // the two k-steps, and the factor of the accumulator rescale if the lane's
    // reference moved (alpha = 0 at the first move, which meets a zero accumulator)
    struct Soft {
        bf16x8 pb[2], plo[2];
        float pf[KV8 ? 16 : 1];  // fp8 keys: P in fp32, scaled per group in the PV
        float alpha;
        bool rescale;
    };
    auto softmax = [&](uint32_t vb, const f32x16& sacc) {
        Soft o;
        // value 4j + i is accumulator row 8j + 4h2 + i = key 16 h2 + 4i + j of this head column;
        // raw scores here, the (positive) logit scale enters the max and the exponent
        float x[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] = sacc[c];
        if (__builtin_amdgcn_readfirstlane(vb) != 0xffffffffu) {
            // a masked key in this tile (ragged end, unused top-k slot)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((vb >> (16 * h2 + 4 * i + j)) & 1u)) x[4 * j + i] = -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int c = 0; c < 16; ++c) tmax = fmaxf(tmax, x[c]);
        {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        tmax *= a.scale_log2;
        // lazy reference: moves only when the max passes it by more than 8
        const bool move = tmax > m_ref + 8.0f;
        const float alpha = __builtin_amdgcn_exp2f(move ? m_ref - tmax : 0.f);
        o.alpha = alpha;
        o.rescale = move && m_ref != -INFINITY;
        l_run *= alpha;
        m_ref = move ? tmax : m_ref;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float psum = 0.f;
        uint32_t pw[8], pl[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(x[2 * c], a.scale_log2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(x[2 * c + 1], a.scale_log2, -m_use));
            psum += p0 + p1;
            if constexpr (KV8) {
                o.pf[2 * c] = p0;
                o.pf[2 * c + 1] = p1;
            }
            pw[c] = pack_bf16x2(p0, p1);
            if constexpr (PREC)
                pl[c] = pack_bf16x2(p0 - bf16_bits_to_f32(pw[c] & 0xffffu), p1 - bf16_bits_to_f32(pw[c] >> 16));
        }
        l_run += psum;
        // k-step kk takes values j = 2kk (slots 8 h2 + 0..3) and j = 2kk+1 (slots 8 h2 + 4..7):
        // slot 8 h2 + 4u + i is key 16 h2 + 4i + 2kk + u
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            o.pb[kk] = __builtin_bit_cast(bf16x8, u32x4{pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]});
            o.plo[kk] = o.pb[kk];
            if constexpr (PREC)
                o.plo[kk] = __builtin_bit_cast(bf16x8, u32x4{pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2], pl[4 * kk + 3]});
        }
        return o;
    };
    // O^T += V^T . P^T for a staged tile (A = V^T by transposed LDS reads)
    auto pv = [&](const Soft& sm, const uint8_t* kt, const float* sc) {
        if (__ballot(sm.rescale)) {
#pragma unroll
            for (int m = 0; m < 8; ++m) scale_agpr16(oacc[m], sm.alpha);
        }
        if constexpr (KV8) {
            // V = codes x group scale: the scale of key j in group g moves onto
            // P (B operand element e of k-step kk is key 16 h2 + 4 (e % 4) + 2 kk + e / 4),
            // m-tiles 2 lg, 2 lg + 1 are the wave's group lg
#pragma unroll
            for (int lg = 0; lg < 4; ++lg) {
                float v[16];
                key_scales(sc, 4 * dh + lg, v);
                bf16x8 va[2][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int mm = 0; mm < 2; ++mm) {
                        const uint8_t* base = kt + (tr_row + 2 * kk) * kRow2 + tr_col + 64 * (2 * lg + mm);
                        const u32x2 v0 = lds_read_tr16(base);
                        const u32x2 v1 = lds_read_tr16(base + kRow2);
                        va[mm][kk] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
                    }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float x2[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * e2 + h;
                            x2[h] = sm.pf[8 * kk + e] * v[4 * (e & 3) + 2 * kk + (e >> 2)];
                        }
                        hw[e2] = pack_bf16x2(x2[0], x2[1]);
                        if constexpr (PREC)
                            lw[e2] = pack_bf16x2(x2[0] - bf16_bits_to_f32(hw[e2] & 0xffffu),
                                                 x2[1] - bf16_bits_to_f32(hw[e2] >> 16));
                    }
                    const bf16x8 pbh = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
#pragma unroll
                    for (int mm = 0; mm < 2; ++mm)
                        oacc[2 * lg + mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mm][kk], pbh, oacc[2 * lg + mm], 0, 0, 0);
                    if constexpr (PREC) {
                        const bf16x8 pbl = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
                        for (int mm = 0; mm < 2; ++mm)
                            oacc[2 * lg + mm] =
                                __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mm][kk], pbl, oacc[2 * lg + mm], 0, 0, 0);
                    }
                }
            }
            return;
        }
        bf16x8 va[8][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint8_t* base = kt + (tr_row + 2 * kk) * kRow2 + tr_col + 64 * m;
                const u32x2 v0 = lds_read_tr16(base);
                const u32x2 v1 = lds_read_tr16(base + kRow2);
                va[m][kk] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
            }
        // consecutive MFMAs go to different accumulators (no back-to-back dependences)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int m = 0; m < 8; ++m) oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m][kk], sm.pb[kk], oacc[m], 0, 0, 0);
            if constexpr (PREC) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m][kk], sm.plo[kk], oacc[m], 0, 0, 0);
            }
        }
        // transposed reads run 4 MFMAs ahead: 8 reads, then (MFMA, 2 reads) x 12, then the rest
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, PREC ? 2 : 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PREC ? 8 : 4, 0);
    };
    // S of the next tile overlapped with the softmax of the current one: the 16
    // operand reads first, then each MFMA followed by a share of the softmax's
    // vector instructions
    auto s_next_softmax = [&](const uint8_t* kt_next, const float* sc_next, uint32_t vb, const f32x16& sacc,
                              f32x16& s_out) {
        bf16x8 ka[16];
        s_loads(kt_next, ka);
        const Soft sm = softmax(vb, sacc);
        s_out = s_mfma(ka, sc_next);
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        return sm;
    };

    for (int64_t kb = t_begin * kT2; kb < k_end; kb += kMaxKeys2) {
        const int64_t ke = kb + kMaxKeys2 < k_end ? kb + kMaxKeys2 : k_end;
        const int ntl = __builtin_amdgcn_readfirstlane((int)((ke - kb + kT2 - 1) / kT2));  // (uniform)
        const bool first = kb == t_begin * kT2;
        if (!first) __syncthreads();  // the previous pass is done with s_rows and the tiles
        {
            const uint8_t* rr[kPer];
            key_rows<kPer, kThreads>(a, n, s, kb, ke, Lc, nv_c, lo, rr, first, pre_id);
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int i = u * kThreads + tid;
                if (u * kThreads >= ntl * kT2) break;  // uniform
                if (i < ntl * kT2) s_rows[i] = rr[u] ? rr[u] : g_zero_kv_row;  // a masked key copies the zero row
                const uint64_t bits = __ballot(rr[u] != nullptr);
                const int t0 = (u * kThreads + 64 * wave) / kT2;
                if (lane == 0 && t0 < ntl) s_vbits[t0] = (uint32_t)bits;
                if (lane == 0 && t0 + 1 < ntl) s_vbits[t0 + 1] = (uint32_t)(bits >> 32);
            }
        }
        __syncthreads();
        for (int t = 0; t < 3 && t < ntl; ++t) issue_tile(t);
        // tile 0 (at most tiles 1 and 2 pending), then S of tile 0
        if (ntl >= 3) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (ntl == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if constexpr (KV8) {
            convert(0);
            __syncthreads();
        }
        f32x16 s_cur;
        {
            bf16x8 ka[16];
            s_loads(kt_of(0), ka);
            s_cur = s_mfma(ka, sc_of(0));
        }
        put_half(s_cur);
        __syncthreads();
        add_other(s_cur);
        // iteration t: the S MFMAs of tile t+1 interleaved with the softmax of
        // tile t; then O += V^T P^T for tile t; the S halves of tile t+1 meet
        // after the PV.  Ring: tile t (PV), t+1 (S), t+2 and t+3 in flight.
        for (int t = 0; t + 1 < ntl; ++t) {
            if (t + 2 < ntl) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile t+1 complete; every wave is past tile t-1 (buffer t+3) and its S exchange
            if (t + 3 < ntl) issue_tile(t + 3);
            if constexpr (KV8) {
                convert(t + 1);  // (its bf16 tile held tile t-1, done with before the barrier above)
                __syncthreads();
            }
            f32x16 s_next;
            const Soft sm = s_next_softmax(kt_of(t + 1), sc_of(t + 1), s_vbits[t], s_cur, s_next);
            pv(sm, kt_of(t), sc_of(t));
            put_half(s_next);
            __syncthreads();
            add_other(s_next);
            s_cur = s_next;
        }
        pv(softmax(s_vbits[ntl - 1], s_cur), kt_of(ntl - 1), sc_of(ntl - 1));
    }

    const float l_tot = sum_xor32(l_run);
    if (a.n_splits > 1) {
        if (!hv) return;
        // unnormalised partial relative to m_ref: dims 256 dh + 32 m + 8 j + 4 h2 .. +3 of this head
        // (bf16 keys: non-temporal stores, which measured faster; the fp8-key
        // launches measured slightly faster with ordinary stores)
        float* po = a.part_o + (((int64_t)n * a.n_splits + sp) * a.n_heads + head) * D + 256 * dh + 4 * h2;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {oacc[m][4 * j], oacc[m][4 * j + 1], oacc[m][4 * j + 2], oacc[m][4 * j + 3]};
                if constexpr (KV8) *reinterpret_cast<f32x4*>(po + 32 * m + 8 * j) = v;
                else __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(po + 32 * m + 8 * j));
            }
        if (h2 == 0 && dh == 0) {
            float* ml = a.part_ml + (((int64_t)n * a.n_splits + sp) * a.n_heads + head) * 2;
            ml[0] = m_ref;
            ml[1] = l_tot;
        }
        return;
    }

    // epilogue.  The accumulator is read once: RoPE^-1 at p on the raw values of
    // the rotated dims (pairs are adjacent values i = 0,1 / 2,3; the rotation
    // commutes with the 1/l scaling), then 1/l and the conversion.  For fp8 the
    // 1/l cancels inside each 64-dim group: code = e4m3(v * 448 / amax(v)),
    // scale = amax(v) / l / 448.  The converted rows are staged in the (now
    // idle) tile ring in output order, padded against bank conflicts, and the
    // query's output leaves with contiguous 16-byte stores.
    const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int rbase = D - a.rope_dims;
    const int esz = a.out_dtype == kF32 ? 4 : a.out_dtype == kBF16 ? 2 : 1;
    const int rstride = D * esz + 16;
    uint8_t* stage = s_ring;
    // RoPE^-1 in place on a 32-dim tile m: skipped (uniformly) below the rotated
    // tail; inside it each pair takes its cos/sin or (1, 0) by a select, so no
    // lane-dependent branch splits the wave
    auto rope_tile = [&](float (&v)[16], int m) {
        const int t0 = 256 * dh + 32 * m;
        if (t0 + 32 <= rbase) return;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int d = t0 + 8 * j + 4 * h2 + 2 * c;
                const bool rot = d >= rbase;
                const int pj = rot ? (d - rbase) >> 1 : 0;
                const float cr = s_rope[0][pj], sr = s_rope[1][pj];
                const float cs = rot ? cr : 1.f, sn = rot ? sr : 0.f;
                const float u = v[4 * j + 2 * c], w = v[4 * j + 2 * c + 1];
                v[4 * j + 2 * c] = u * cs - w * sn;
                v[4 * j + 2 * c + 1] = u * sn + w * cs;
            }
    };
    __syncthreads();  // every wave is done with the ring
    uint8_t* srow = stage + head * rstride;
    if (a.out_dtype == kFP8) {
        // 64-dim groups: tiles m = 2 g4, 2 g4 + 1 of the wave's 256 dims, halves h2 = 0, 1
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            float v0[16], v1[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                v0[c] = oacc[2 * g4][c];
                v1[c] = oacc[2 * g4 + 1][c];
            }
            rope_tile(v0, 2 * g4);
            rope_tile(v1, 2 * g4 + 1);
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fmaxf(fabsf(v0[c]), fabsf(v1[c])));
            {
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
                amax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
            }
            const float gmax = amax * inv_l;
            const float scale = gmax > 0.f ? gmax / 448.0f : 1.0f;
            const float r = gmax > 0.f ? 448.0f / amax : 0.f;
            if (h2 == 0 && hv) a.out_scales[((int64_t)n * a.n_heads + head) * (D / 64) + 4 * dh + g4] = scale;
            // NaN or infinity anywhere in the wave's group makes the sum of v * 0 a NaN:
            // only then does the conversion need its per-value NaN handling
            float nz = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) nz = fmaf(v1[c], 0.f, fmaf(v0[c], 0.f, nz));
            const bool finite = __ballot(nz != nz) == 0;
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const float* v = mm ? v1 : v0;
                const int m = 2 * g4 + mm;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint32_t*>(srow + 256 * dh + 32 * m + 8 * j + 4 * h2) = e4m3_pack4_finite(
                        v[4 * j] * r, v[4 * j + 1] * r, v[4 * j + 2] * r, v[4 * j + 3] * r);
            }
            if (__builtin_expect(!finite, 0)) {  // rare: the codes again, with the per-value NaN handling
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const float* v = mm ? v1 : v0;
                    const int m = 2 * g4 + mm;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<uint32_t*>(srow + 256 * dh + 32 * m + 8 * j + 4 * h2) =
                            e4m3_pack4(v[4 * j] * r, v[4 * j + 1] * r, v[4 * j + 2] * r, v[4 * j + 3] * r);
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            float v[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) v[c] = oacc[m][c];
            rope_tile(v, m);
#pragma unroll
            for (int c = 0; c < 16; ++c) v[c] *= inv_l;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 256 * dh + 32 * m + 8 * j + 4 * h2;
                if (a.out_dtype == kF32)
                    *reinterpret_cast<f32x4*>(srow + 4 * d0) = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
                else
                    *reinterpret_cast<u32x2*>(srow + 2 * d0) =
                        u32x2{pack_bf16x2(v[4 * j], v[4 * j + 1]), pack_bf16x2(v[4 * j + 2], v[4 * j + 3])};
            }
        }
    }
    __syncthreads();
    // the query's n_heads rows (contiguous in the output) in 16-byte chunks
    const int rchunks = D * esz / 16;
    const int nchunks = a.n_heads * rchunks;
    uint8_t* out = reinterpret_cast<uint8_t*>(a.out) + (int64_t)n * a.n_heads * D * esz;
    for (int c = tid; c < nchunks; c += kThreads) {
        const int h = c / rchunks, off = (c - h * rchunks) * 16;
        *reinterpret_cast<u32x4*>(out + (int64_t)c * 16) = *reinterpret_cast<const u32x4*>(stage + h * rstride + off);
    }
}


}  // namespace

template <int D, int KV>
void launch_prec(const AttnArgs& a, dim3 grid, hipStream_t st, const LaunchEvents& ev) {
    if (a.out_dtype == kFP8) launch_kernel(ev, true, true, hybrid_attn_kernel<D, KV, true>, grid, dim3(kThreads), st, a);
    else launch_kernel(ev, true, true, hybrid_attn_kernel<D, KV, false>, grid, dim3(kThreads), st, a);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0) return hipSuccess;
    dim3 grid((unsigned)((int64_t)a.num_q * a.n_splits));
    const int kv = a.comp_rows ? a.comp_dtype : a.swa_dtype;
    if (a.dim == 512 && kv == kBF16) {
        if (a.out_dtype == kFP8) launch_kernel(ev, true, true, hybrid_attn_mqa512_kernel<true, false>, grid, dim3(kThreads), st, a);
        else launch_kernel(ev, true, true, hybrid_attn_mqa512_kernel<false, false>, grid, dim3(kThreads), st, a);
        return hipGetLastError();
    }
    if (a.dim == 512 && kv == kFP8) {
        if (a.out_dtype == kFP8) launch_kernel(ev, true, true, hybrid_attn_mqa512_kernel<true, true>, grid, dim3(kThreads), st, a);
        else launch_kernel(ev, true, true, hybrid_attn_mqa512_kernel<false, true>, grid, dim3(kThreads), st, a);
        return hipGetLastError();
    }
    // 128-dim keys (bf16 only: fp8 rows need dim % 256 == 0): the generic kernel
    if (a.dim == 128 && kv == kBF16) launch_prec<128, kBF16>(a, grid, st, ev);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0 || a.n_splits <= 1) return hipSuccess;
    // up to 16 splits: one batch per wave, four heads per workgroup; more: the
    // split list shared by the four waves of a (query, head) workgroup.  The
    // shared form also takes 5..16 splits when the four-heads form would fill
    // fewer than 256 workgroups: there more, shorter workgroups are faster.
    const bool share = a.n_splits > 16 || (a.n_splits > 4 && (int64_t)a.num_q * ((a.n_heads + 3) / 4) < 256);
    const dim3 grid((unsigned)((int64_t)a.num_q * (share ? a.n_heads : (a.n_heads + 3) / 4)));
    if (a.dim == 512) {
        // more than 64 splits: sixteen waves share them (a few batches per wave); 33..64: eight
        // waves, so that each takes one batch of at most 8
        if (a.n_splits > 64) launch_kernel(ev, true, true, attn_combine_kernel<512, true, 16>, grid, dim3(1024), st, a);
        else if (a.n_splits > 32) launch_kernel(ev, true, true, attn_combine_kernel<512, true, 8>, grid, dim3(512), st, a);
        else if (share) launch_kernel(ev, true, true, attn_combine_kernel<512, true>, grid, dim3(kThreads), st, a);
        else launch_kernel(ev, true, true, attn_combine_kernel<512, false>, grid, dim3(kThreads), st, a);
    } else if (a.dim == 128) {
        if (share) launch_kernel(ev, true, true, attn_combine_kernel<128, true>, grid, dim3(kThreads), st, a);
        else launch_kernel(ev, true, true, attn_combine_kernel<128, false>, grid, dim3(kThreads), st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace csl
