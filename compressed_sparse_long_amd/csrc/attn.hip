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
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, D == 512 ? 1 : 4)))
hybrid_attn_kernel(AttnArgs a) {
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
            uint32_t code = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) code |= f32_to_e4m3(acc[m][i] / gmax[m >> 2]) << (8 * i);
            *reinterpret_cast<uint32_t*>(o + 16 * m + 4 * g) = code;
        }
    }
}

// Merge the splits of one (query, head): one wave, 8 dims per lane.
template <int D>
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x / ((a.n_heads + 3) / 4);
    const int head = (blockIdx.x % ((a.n_heads + 3) / 4)) * 4 + wave;
    if (head >= a.n_heads) return;
    const bool active = 8 * lane < D;
    QueryInfo qi = query_info(a, n);
    const int64_t p = qi.ok ? qi.p : 0;

    const float* ml = a.part_ml + ((int64_t)n * a.n_splits * a.n_heads + head) * 2;
    const int64_t mstride = (int64_t)a.n_heads * 2;
    const float* po = a.part_o + ((int64_t)n * a.n_splits * a.n_heads + head) * D + 8 * (active ? lane : 0);
    const int64_t pstride = (int64_t)a.n_heads * D;
    // one pass, batches of 16 splits: all loads of a batch are issued before
    // any use; the running max M rescales what earlier batches accumulated
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float Lsum = 0.f, M = -INFINITY;
    constexpr int kB = 16;
    for (int sp0 = 0; sp0 < a.n_splits; sp0 += kB) {
        f32x4 v0[kB], v1[kB];
        float msp[kB], lsp[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            msp[u] = -INFINITY;
            lsp[u] = 0.f;
            v0[u] = v1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sp0 + u < a.n_splits) {
                const int sp = sp0 + u;
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
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    const int rbase = D - a.rope_dims;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= inv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int d = 8 * lane + 2 * c;
        if (d >= rbase) {
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
            u32x2 w = {0u, 0u};
#pragma unroll
            for (int c = 0; c < 8; ++c) w[c >> 2] |= f32_to_e4m3(o[c] / scale) << (8 * (c & 3));
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.out) + obase) = w;
            if ((lane & 7) == 0) a.out_scales[((int64_t)n * a.n_heads + head) * (D / 64) + (lane >> 3)] = scale;
        }
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
    if (a.dim == 512 && kv == kBF16) launch_prec<512, kBF16>(a, grid, st, ev);
    else if (a.dim == 512 && kv == kFP8) launch_prec<512, kFP8>(a, grid, st, ev);
    else if (a.dim == 128 && kv == kBF16) launch_prec<128, kBF16>(a, grid, st, ev);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0 || a.n_splits <= 1) return hipSuccess;
    dim3 grid((unsigned)((int64_t)a.num_q * ((a.n_heads + 3) / 4)));
    if (a.dim == 512) launch_kernel(ev, true, true, attn_combine_kernel<512>, grid, dim3(kThreads), st, a);
    else if (a.dim == 128) launch_kernel(ev, true, true, attn_combine_kernel<128>, grid, dim3(kThreads), st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace csl
