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

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(IndexArgs a) {
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_cnt[2][kSelWaves];
    __shared__ uint32_t s_prefix, s_rem;
    __shared__ float s_min[kSelWaves];

    const int n = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int s;
    int64_t p;
    int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;  // the score kernel reports bad queries
    const float* sc = a.scores + (int64_t)n * a.stride;
    int32_t* out = a.topk + (int64_t)n * a.k;
    const int k = a.k;

    if (nv <= k) {
        for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
        if (a.kth) {
            float m = INFINITY;
            for (int64_t e = tid; e < nv; e += kSelThreads) m = fminf(m, sc[e]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m = fminf(m, __shfl_xor(m, o));
            if (lane == 0) s_min[wave] = m;
            __syncthreads();
            if (tid == 0) {
                float r = INFINITY;
                for (int w = 0; w < kSelWaves; ++w) r = fminf(r, s_min[w]);
                a.kth[n] = nv > 0 ? r : -INFINITY;
            }
        }
        return;
    }

    // radix select of the k-th largest key: rounds of 11, 11 and 10 bits
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
        const int sh = shifts[r], nb = 1 << widths[r];
        for (int b = tid; b < 2048; b += kSelThreads) s_hist[b] = 0;
        __syncthreads();
        for (int64_t e = tid; e < nv; e += kSelThreads) {
            uint32_t key = score_key(sc[e]);
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
                s_prefix = prefix | ((uint32_t)hi << sh);
                s_rem = rem - above;
            } else if (hi - 1 >= 0 && above + c_hi < rem && rem <= above + c_hi + c_lo) {
                s_prefix = prefix | ((uint32_t)(hi - 1) << sh);
                s_rem = rem - above - c_hi;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        rem = s_rem;
        pmask |= (uint32_t)(nb - 1) << sh;
        __syncthreads();
    }
    const uint32_t T = prefix;  // the k-th largest key; `rem` copies of it are taken

    // each wave owns ids [w*seg, (w+1)*seg); count keys > T and == T per wave
    const int64_t seg = ((nv + kSelWaves - 1) / kSelWaves + 63) & ~(int64_t)63;
    const int64_t lo = (int64_t)wave * seg;
    const int64_t hi = lo + seg < nv ? lo + seg : nv;
    uint32_t n_gt = 0, n_eq = 0;
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        uint32_t key = e < hi ? score_key(sc[e]) : 0u;
        bool in = e < hi;
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
    // ordered emission
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        bool in = e < hi;
        uint32_t key = in ? score_key(sc[e]) : 0u;
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
    if (tid == 0 && a.kth) a.kth[n] = key_score(T);
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
