// Steps 2-3 on gfx950: DSA indexer scores and causal top-k ([Summary]
// DeepSeek V4 注意力架構: DSA; [Notes] 压缩参数细节: k = 512 for c4a).
//
// index_score_kernel -- the HBM stream of the decode step.  A workgroup
// (4 waves) scores 256 consecutive entries of one query; each wave owns one
// 64-entry page.  The head-batched contraction qI[16 heads x d] . K^T[d x 16
// entries] is one v_mfma_f32_16x16x32_bf16 per 32 dims per 16 entries: the A
// operand holds the query's heads (rows), the B operand the entries (columns),
// both loaded straight from HBM in the MFMA lane layout (a lane reads 16
// contiguous bytes of one row).  ReLU, the per-head weight and the sum over
// heads are fused on the accumulators (4 heads in-lane, then 2 cross-lane
// xor steps), and each wave stores its 64 fp32 scores with one coalesced
// 256-byte write.  Grid: x = 256-entry chunk (fastest), y = query, with the
// chunk count a multiple of 8 so a chunk maps to the same XCD for every query.
//
// topk_select_kernel -- one 1024-thread workgroup per query: an exact radix
// select of the k-th largest score key (11/11/10-bit rounds, LDS histograms),
// then an order-preserving pass in which each wave owns a contiguous range of
// ids and emits the selected ids in ascending order with ballots; ties at the
// k-th score go to the lower ids.
#include "csl_kernels.hpp"

namespace csl {

namespace {

__device__ __forceinline__ bool query_ok(const IndexArgs& a, int n, int& s, int64_t& p) {
    s = a.q_seq[n];
    p = a.q_pos[n];
    return s >= 0 && s < a.num_seqs && p >= 0 && p <= a.max_q_pos;
}

__device__ __forceinline__ int64_t visible(const IndexArgs& a, int64_t p) {
    int64_t nv = p >> 2;
    return nv < a.stride ? nv : a.stride;
}

template <int DI>
__global__ void __launch_bounds__(256) index_score_kernel(IndexArgs a) {
    constexpr int KS = DI / 32;
    const int n = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int s;
    int64_t p;
    if (!query_ok(a, n, s, p)) {
        if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(a.err, (s < 0 || s >= a.num_seqs) ? kErrSeq : kErrPos);
        return;
    }
    const int64_t nv = visible(a, p);
    const int64_t e0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
    if (e0 >= nv) return;
    float* out = a.scores + (int64_t)n * a.stride + e0;
    const int32_t pg = page_of(a.bt, a.max_blocks, a.num_pages, s, e0 * 4);
    if (pg < 0) {
        if (lane == 0) raise_error(a.err, kErrPage);
        if (e0 + lane < nv) out[lane] = -INFINITY;
        return;
    }
    const uint8_t* base = a.rows + (int64_t)pg * 64 * (DI * 2);

    // B operands: the wave's 64 entries as 4 tiles of 16, issued first
    bf16x8 kb[4][KS];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kb[t][ks] = *reinterpret_cast<const bf16x8*>(base + (16 * t + r16) * (DI * 2) + (32 * ks + 8 * g) * 2);

    // A operands: the query's heads (rows beyond n_heads are zero)
    bf16x8 qa[KS];
    const bool hv = r16 < a.n_heads;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (hv) v = *reinterpret_cast<const u32x4*>(a.q_idx + ((int64_t)n * a.n_heads + r16) * DI + 32 * ks + 8 * g);
        qa[ks] = __builtin_bit_cast(bf16x8, v);
    }
    float wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int h = 4 * g + i;
        wv[i] = h < a.n_heads ? a.w[(int64_t)n * a.n_heads + h] : 0.f;
    }

    float sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb[t][ks], acc, 0, 0, 0);
        // acc[i] = <q_head(4g+i), key(16t + r16)>
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[i], fmaxf(acc[i], 0.f), v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        sc[t] = v;
    }
    // lane l stores entry e0 + l, i.e. tile g, column r16
    float mine = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
    if (e0 + lane < nv) out[lane] = mine;
}

// Order-preserving 32-bit key of an fp32 score (+0 and -0 share one key).
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive scan of one uint32 per thread over the workgroup; also returns the total.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        uint32_t c = s_wave[w];
        before += w < wave ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Keys of a query's scores: in LDS, or read from global memory.
struct LdsKeys {
    const uint32_t* k;
    __device__ __forceinline__ uint32_t operator()(int64_t e) const { return k[e]; }
};
struct GlobalKeys {
    const float* sc;
    __device__ __forceinline__ uint32_t operator()(int64_t e) const { return score_key(sc[e]); }
};

// Exact radix select (11/11/10-bit rounds) of the `want`-th largest key among
// keys [0, n) of `key_at`; returns the key, and in *rem how many copies of it
// are taken.  LDS histograms; every thread of the workgroup must call it.
template <typename Keys>
__device__ uint32_t radix_select(const Keys& key_at, int64_t n, uint32_t want, uint32_t* rem_out, uint32_t* s_hist,
                                 uint32_t* s_wave, uint32_t* s_sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, rem = want;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
        const int sh = shifts[r], nb = 1 << widths[r];
        for (int b = tid; b < 2048; b += kSelThreads) s_hist[b] = 0;
        __syncthreads();
        for (int64_t e = tid; e < n; e += kSelThreads) {
            uint32_t key = key_at(e);
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns the two bins nb-1-2t and nb-2-2t (counted from the top)
        const int hi = nb - 1 - 2 * tid;
        uint32_t c_hi = hi >= 0 ? s_hist[hi] : 0u;
        uint32_t c_lo = hi - 1 >= 0 ? s_hist[hi - 1] : 0u;
        uint32_t tot;
        uint32_t above = block_excl_scan(c_hi + c_lo, s_wave, tot);
        if (hi >= 0) {
            if (above < rem && rem <= above + c_hi) {
                s_sel[0] = prefix | ((uint32_t)hi << sh);
                s_sel[1] = rem - above;
            } else if (hi - 1 >= 0 && above + c_hi < rem && rem <= above + c_hi + c_lo) {
                s_sel[0] = prefix | ((uint32_t)(hi - 1) << sh);
                s_sel[1] = rem - above - c_hi;
            }
        }
        __syncthreads();
        prefix = s_sel[0];
        rem = s_sel[1];
        pmask |= (uint32_t)(nb - 1) << sh;
        __syncthreads();
    }
    *rem_out = rem;
    return prefix;
}

// Emit the ids of keys > T, plus the first `rem` ids (by id) of keys == T, in
// ascending id order.  Wave w owns ids [w*seg, (w+1)*seg).
template <typename Keys>
__device__ void emit_ordered(const Keys& key_at, int64_t nv, uint32_t T, uint32_t rem, int k, int32_t* out,
                             uint32_t (*s_cnt)[kSelWaves]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t seg = ((nv + kSelWaves - 1) / kSelWaves + 63) & ~(int64_t)63;
    const int64_t lo = (int64_t)wave * seg;
    const int64_t hi = lo + seg < nv ? lo + seg : nv;
    uint32_t n_gt = 0, n_eq = 0;
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        bool in = e < hi;
        uint32_t key = in ? key_at(e) : 0u;
        n_gt += __popcll(__ballot(in && key > T));
        n_eq += __popcll(__ballot(in && key == T));
    }
    if (lane == 0) {
        s_cnt[0][wave] = n_gt;
        s_cnt[1][wave] = n_eq;
    }
    __syncthreads();
    uint32_t out_pos = 0, eq_seen = 0;
    for (int w = 0; w < wave; ++w) {
        uint32_t eq_w = s_cnt[1][w];
        uint32_t take_eq = eq_seen >= rem ? 0u : (eq_w < rem - eq_seen ? eq_w : rem - eq_seen);
        out_pos += s_cnt[0][w] + take_eq;
        eq_seen += eq_w;
    }
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        bool in = e < hi;
        uint32_t key = in ? key_at(e) : 0u;
        bool gt = in && key > T, eq = in && key == T;
        uint64_t eqm = __ballot(eq);
        uint32_t eq_rank = eq_seen + __popcll(eqm & lanemask_lt(lane));
        bool sel = gt || (eq && eq_rank < rem);
        uint64_t selm = __ballot(sel);
        const uint32_t dst = out_pos + __popcll(selm & lanemask_lt(lane));
        if (sel && dst < (uint32_t)k) out[dst] = (int32_t)e;
        out_pos += __popcll(selm);
        eq_seen += __popcll(eqm);
    }
}

constexpr int kRegKeys = 32;                     // keys per thread held in registers
constexpr int kRegMax = kRegKeys * kSelThreads;  // 32768 candidates
constexpr int kCandCap = 4096;                   // boundary-bin candidates kept in LDS
constexpr int kRankCap = kSelThreads;            // candidates ranked directly

// Exact radix select (11/11/10-bit rounds) over register-resident keys: the
// `want`-th largest of the valid keys; *rem = copies of it that are taken.
__device__ uint32_t radix_select_regs(const uint32_t (&key)[32], int nmine, uint32_t want, uint32_t* rem_out,
                                      uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, rem = want;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
        const int sh = shifts[r], nb = 1 << widths[r];
        for (int b = tid; b < 2048; b += kSelThreads) s_hist[b] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i < nmine && (key[i] & pmask) == prefix) atomicAdd(&s_hist[(key[i] >> sh) & (nb - 1)], 1u);
        __syncthreads();
        const int hi = nb - 1 - 2 * tid;
        uint32_t c_hi = hi >= 0 ? s_hist[hi] : 0u;
        uint32_t c_lo = hi - 1 >= 0 ? s_hist[hi - 1] : 0u;
        uint32_t tot;
        uint32_t above = block_excl_scan(c_hi + c_lo, s_wave, tot);
        if (hi >= 0) {
            if (above < rem && rem <= above + c_hi) {
                s_sel[0] = prefix | ((uint32_t)hi << sh);
                s_sel[1] = rem - above;
            } else if (hi - 1 >= 0 && above + c_hi < rem && rem <= above + c_hi + c_lo) {
                s_sel[0] = prefix | ((uint32_t)(hi - 1) << sh);
                s_sel[1] = rem - above - c_hi;
            }
        }
        __syncthreads();
        prefix = s_sel[0];
        rem = s_sel[1];
        pmask |= (uint32_t)(nb - 1) << sh;
        __syncthreads();
    }
    *rem_out = rem;
    return prefix;
}

// Register-resident select for nv <= 32768.  Thread t holds the 32 keys of ids
// [32t, 32t+32), so ids stay ordered by thread and every compaction is one
// block-wide exclusive scan of per-thread counts:
//  1. a 2048-bin histogram of the keys inside a window of 2^24 key units
//     below the largest key (two octaves of fp32 score below the maximum;
//     keys under the window are not counted), scanned from the top: the bin b
//     that holds the k-th key and `want` = its rank inside b.  Bins of 2^13
//     key units keep b small.  If fewer than k keys fall in the window, an
//     exact 3-round radix select over all keys is used instead;
//  2. b's keys are compacted to LDS and the k-th key T is the candidate with
//     #(> T) < want <= #(>= T);
//  3. ids with key > T, then the first `rem` ids with key == T, are written in
//     ascending order through one scan of packed (count_gt, count_eq).
__device__ void select_registers(const float* sc, int64_t nv, int k, int32_t* out, float* kth, uint32_t* s_hist,
                                 uint32_t* s_wave, uint32_t* s_sel, uint32_t* s_cand) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t e0 = (int64_t)tid * kRegKeys;
    uint32_t key[kRegKeys];
    if (e0 + kRegKeys <= nv) {
        const float4* p4 = reinterpret_cast<const float4*>(sc + e0);
#pragma unroll
        for (int i = 0; i < kRegKeys / 4; ++i) {
            const float4 v = p4[i];
            key[4 * i] = score_key(v.x);
            key[4 * i + 1] = score_key(v.y);
            key[4 * i + 2] = score_key(v.z);
            key[4 * i + 3] = score_key(v.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i) key[i] = e0 + i < nv ? score_key(sc[e0 + i]) : 0u;
    }
    const int nmine = (int)(nv - e0 < 0 ? 0 : (nv - e0 < kRegKeys ? nv - e0 : kRegKeys));

    // the largest key, and the histogram zeroed under the same barrier
    uint32_t kmax = 0u;
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) kmax = i < nmine ? max(kmax, key[i]) : kmax;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    if (lane == 0) s_sel[8 + wave] = kmax;
    for (int b = tid; b < 2048; b += kSelThreads) s_hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) kmax = max(kmax, s_sel[8 + w]);
    constexpr uint32_t kWin = (1u << 24) - 1u;
    const uint32_t lo = kmax > kWin ? kmax - kWin : 0u;
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i)
        if (i < nmine && key[i] >= lo) atomicAdd(&s_hist[(key[i] - lo) >> 13], 1u);
    __syncthreads();
    const int hb = 2047 - 2 * tid;  // this thread's two bins, from the top
    const uint32_t c_hi = s_hist[hb], c_lo = s_hist[hb - 1];
    uint32_t tot;
    const uint32_t above = block_excl_scan(c_hi + c_lo, s_wave, tot);
    if (above < (uint32_t)k && (uint32_t)k <= above + c_hi) {
        s_sel[0] = hb;
        s_sel[1] = k - above;
        s_sel[2] = c_hi;
    } else if (above + c_hi < (uint32_t)k && (uint32_t)k <= above + c_hi + c_lo) {
        s_sel[0] = hb - 1;
        s_sel[1] = k - above - c_hi;
        s_sel[2] = c_lo;
    }
    __syncthreads();

    uint32_t T, rem;
    if (tot >= (uint32_t)k && s_sel[2] <= (uint32_t)kCandCap) {
        const uint32_t bsel = s_sel[0], want = s_sel[1], cnt = s_sel[2];
        auto in_bin = [&](uint32_t kk) { return kk >= lo && ((kk - lo) >> 13) == bsel; };
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i) mine += (i < nmine && in_bin(key[i])) ? 1u : 0u;
        uint32_t off = block_excl_scan(mine, s_wave, tot);
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i)
            if (i < nmine && in_bin(key[i])) s_cand[off++] = key[i];
        __syncthreads();
        if (cnt <= (uint32_t)kRankCap) {
            if ((uint32_t)tid < cnt) {
                const uint32_t kc = s_cand[tid];
                uint32_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < cnt; ++j) {
                    const uint32_t kj = s_cand[j];
                    gt += kj > kc ? 1u : 0u;
                    ge += kj >= kc ? 1u : 0u;
                }
                if (gt < want && want <= ge) {  // every copy of T writes the same values
                    s_sel[4] = kc;
                    s_sel[5] = want - gt;
                }
            }
            __syncthreads();
            T = s_sel[4];
            rem = s_sel[5];
        } else {
            T = radix_select(LdsKeys{s_cand}, (int64_t)cnt, want, &rem, s_hist, s_wave, s_sel + 4);
        }
    } else {
        T = radix_select_regs(key, nmine, (uint32_t)k, &rem, s_hist, s_wave, s_sel + 4);
    }

    // 3. ordered emission: one scan of packed (count_gt | count_eq << 16)
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
        ngt += (i < nmine && key[i] > T) ? 1u : 0u;
        neq += (i < nmine && key[i] == T) ? 1u : 0u;
    }
    const uint32_t pre = block_excl_scan(ngt | (neq << 16), s_wave, tot);
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xffffu) + (eq_before < rem ? eq_before : rem);
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
        if (i >= nmine) break;
        bool sel = key[i] > T;
        if (key[i] == T) {
            sel = eq_before < rem;
            ++eq_before;
        }
        if (sel) {
            if (pos < (uint32_t)k) out[pos] = (int32_t)(e0 + i);
            ++pos;
        }
    }
    if (tid == 0 && kth) *kth = key_score(T);
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(IndexArgs a) {
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_cnt[2][kSelWaves];
    __shared__ uint32_t s_sel[8 + kSelWaves];
    __shared__ float s_min[kSelWaves];

    const int n = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;  // the score kernel reports bad queries
    const float* sc = a.scores + (int64_t)n * a.stride;
    int32_t* out = a.topk + (int64_t)n * a.k;
    const int k = a.k;
    float* kth = a.kth ? a.kth + n : nullptr;

    if (nv <= k) {
        for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
        if (kth) {
            float m = INFINITY;
            for (int64_t e = tid; e < nv; e += kSelThreads) m = fminf(m, sc[e]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m = fminf(m, __shfl_xor(m, o));
            if (lane == 0) s_min[wave] = m;
            __syncthreads();
            if (tid == 0) {
                float r = INFINITY;
                for (int w = 0; w < kSelWaves; ++w) r = fminf(r, s_min[w]);
                *kth = nv > 0 ? r : -INFINITY;
            }
        }
        return;
    }
    if (nv <= kRegMax) {
        select_registers(sc, nv, k, out, kth, s_hist, s_wave, s_sel, s_cand);
    } else {
        uint32_t rem;
        const uint32_t T = radix_select(GlobalKeys{sc}, nv, (uint32_t)k, &rem, s_hist, s_wave, s_sel);
        emit_ordered(GlobalKeys{sc}, nv, T, rem, k, out, s_cnt);
        if (tid == 0 && kth) *kth = key_score(T);
    }
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t st) {
    if (a.num_q <= 0) return hipSuccess;
    dim3 grid((unsigned)(a.stride / 256), (unsigned)a.num_q);
    switch (a.dim) {
        case 32: hipLaunchKernelGGL(index_score_kernel<32>, grid, dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL(index_score_kernel<64>, grid, dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL(index_score_kernel<128>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_topk_select(const IndexArgs& a, hipStream_t st) {
    if (a.num_q <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)a.num_q), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace csl
