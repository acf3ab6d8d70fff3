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

// 64-entry units per wave in the score kernel (the score row stride is a
// multiple of 2048 = 8 waves' worth of units, so every launch divides evenly).
constexpr int kScoreUnits = 4;

__device__ __forceinline__ bool query_ok(const IndexArgs& a, int n, int& s, int64_t& p) {
    s = a.q_seq[n];
    p = a.q_pos[n];
    return s >= 0 && s < a.num_seqs && p >= 0 && p <= a.max_q_pos;
}

__device__ __forceinline__ int64_t visible(const IndexArgs& a, int64_t p) {
    int64_t nv = p >> 2;
    return nv < a.stride ? nv : a.stride;
}

template <int DI, int U>
__global__ void __launch_bounds__(256) index_score_kernel(IndexArgs a) {
    constexpr int KS = DI / 32;          // MFMA k-steps per row
    constexpr int RB = DI * 2;           // index row bytes
    constexpr int CPR = RB / 16;         // 16-byte chunks per row
    constexpr int NLD = CPR;             // 1 KiB loads per 64-row unit
    constexpr int LROW = RB + 16;        // padded LDS row (spreads the banks of the MFMA-layout reads)
    __shared__ __attribute__((aligned(16))) uint8_t s_unit[4][64 * LROW];
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
    // the wave's U consecutive 64-entry units; unit u is block u of the sequence
    const int64_t u0 = ((int64_t)blockIdx.x * 4 + wave) * U;
    if (u0 * 64 >= nv) return;
    int32_t mypg = 0;  // lane j < U: page of unit u0 + j (-1 unmapped)
    if (lane < U && (u0 + lane) * 64 < nv) mypg = page_of(a.bt, a.max_blocks, a.num_pages, s, (u0 + lane) * 256);

    // A unit (64 rows) streams in with contiguous 1 KiB loads (lane l takes
    // chunk l % CPR of row l / CPR), non-temporal since every row is read once
    // per step; it then passes through the wave's own LDS slice to reach the
    // MFMA operand layout, whose direct loads (16 rows x 64 B per instruction)
    // stream measurably slower.  The next unit is in flight meanwhile.  An
    // unmapped or invisible unit reads page 0 (always allocated); its scores
    // are not used.
    u32x4 ld[NLD];
    auto issue = [&](int j) {
        const int32_t pg = __shfl(mypg, j);
        const u32x4* base = reinterpret_cast<const u32x4*>(a.rows + (int64_t)(pg < 0 ? 0 : pg) * 64 * RB);
#pragma unroll
        for (int q = 0; q < NLD; ++q) ld[q] = __builtin_nontemporal_load(base + q * 64 + lane);
    };
    issue(0);

    // A operands: the query's heads (rows beyond n_heads are zero); head weights
    bf16x8 qa[KS];
    const bool hv = r16 < a.n_heads;
    const uint16_t* qrow = a.q_idx + ((int64_t)n * a.n_heads + (hv ? r16 : 0)) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g);
        if (!hv) v = u32x4{0u, 0u, 0u, 0u};
        qa[ks] = __builtin_bit_cast(bf16x8, v);
    }
    float wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        const float x = a.w[(int64_t)n * a.n_heads + (h < a.n_heads ? h : 0)];
        wv[i] = h < a.n_heads ? x : 0.f;
    }

    uint8_t* su = s_unit[wave];
    constexpr int RPL = 64 / CPR;  // rows per 1 KiB load
#pragma unroll
    for (int j = 0; j < U; ++j) {
        // this unit into LDS (in-order LDS ops of one wave: the reads of the
        // previous unit have been issued before these writes)
#pragma unroll
        for (int q = 0; q < NLD; ++q)
            *reinterpret_cast<u32x4*>(su + (q * RPL + lane / CPR) * LROW + (lane % CPR) * 16) = ld[q];
        if (j + 1 < U) issue(j + 1);
        float sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kb = *reinterpret_cast<const bf16x8*>(su + (16 * t + r16) * LROW + (4 * ks + g) * 16);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, acc, 0, 0, 0);
            }
            // acc[i] = <q_head(4g+i), key(16t + r16)>
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaf(wv[i], fmaxf(acc[i], 0.f), v);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            sc[t] = v;
        }
        const int64_t e0 = (u0 + j) * 64;
        if (e0 >= nv) break;
        const int32_t pg = __shfl(mypg, j);
        // lane l stores entry e0 + l, i.e. tile g, column r16
        float mine = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
        if (pg < 0) {
            if (lane == 0) raise_error(a.err, kErrPage);
            mine = -INFINITY;
        }
        if (e0 + lane < nv) a.scores[(int64_t)n * a.stride + e0 + lane] = mine;
    }
}

// Order-preserving 32-bit key of an fp32 score (+0 and -0 share one key).
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Exclusive scan of one uint32 per thread over an NT-thread workgroup; also returns the total.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
    constexpr int NW = NT / 64;
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
    for (int w = 0; w < NW; ++w) {
        uint32_t c = s_wave[w];
        before += w < wave ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// Scan of a 2048-bin histogram from the top: the bin holding the `want`-th
// largest key and the rank of that key inside the bin.  Every thread calls it;
// the result lands in s_sel[0] (bin), s_sel[1] (rank), s_sel[2] (bin count),
// and the histogram total is returned.
template <int NT>
__device__ uint32_t find_bin(const uint32_t* s_hist, uint32_t want, int nbins, uint32_t* s_wave, uint32_t* s_sel) {
    constexpr int PER = 2048 / NT;  // bins per thread (2 for 1024 threads, 8 for 256)
    const int tid = threadIdx.x;
    const int top = nbins - 1 - PER * tid;  // this thread's bins top, top-1, ..., from the top
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = top - i >= 0 ? s_hist[top - i] : 0u;
        sum += c[i];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(sum, s_wave, tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (top - i >= 0 && above < want && want <= above + c[i]) {
            s_sel[0] = top - i;
            s_sel[1] = want - above;
            s_sel[2] = c[i];
        }
        above += c[i];
    }
    __syncthreads();
    return tot;
}

// Keys of a query's scores read from global memory.
struct GlobalKeys {
    const float* sc;
    __device__ __forceinline__ uint32_t operator()(int64_t e) const { return score_key(sc[e]); }
};
struct LdsKeys {
    const uint32_t* k;
    __device__ __forceinline__ uint32_t operator()(int64_t e) const { return k[e]; }
};

// Exact radix select (11/11/10-bit rounds) of the `want`-th largest among keys
// [0, n) of `key_at`; *rem = copies of it that are taken.
template <int NT, typename Keys>
__device__ uint32_t radix_select(const Keys& key_at, int64_t n, uint32_t want, uint32_t* rem_out, uint32_t* s_hist,
                                 uint32_t* s_wave, uint32_t* s_sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, rem = want;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
        const int sh = shifts[r], nb = 1 << widths[r];
        for (int b = tid; b < 2048; b += NT) s_hist[b] = 0;
        __syncthreads();
        for (int64_t e = tid; e < n; e += NT) {
            uint32_t key = key_at(e);
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_bin<NT>(s_hist, rem, nb, s_wave, s_sel);
        prefix |= s_sel[0] << sh;
        rem = s_sel[1];
        pmask |= (uint32_t)(nb - 1) << sh;
        __syncthreads();
    }
    *rem_out = rem;
    return prefix;
}

// The same over register-resident keys (slot i of a thread valid iff bit i of vmask).
template <int NT, int KPT>
__device__ __forceinline__ uint32_t radix_select_regs(const uint32_t (&key)[KPT], uint32_t vmask, uint32_t want, uint32_t* rem_out,
                                      uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, rem = want;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
        const int sh = shifts[r], nb = 1 << widths[r];
        for (int b = tid; b < 2048; b += NT) s_hist[b] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (((vmask >> i) & 1u) && (key[i] & pmask) == prefix) atomicAdd(&s_hist[(key[i] >> sh) & (nb - 1)], 1u);
        __syncthreads();
        find_bin<NT>(s_hist, rem, nb, s_wave, s_sel);
        prefix |= s_sel[0] << sh;
        rem = s_sel[1];
        pmask |= (uint32_t)(nb - 1) << sh;
        __syncthreads();
    }
    *rem_out = rem;
    return prefix;
}

constexpr int kCandCap = 4096;  // boundary-bin keys kept in LDS

// Exact selection over register-resident keys (slot i valid iff bit i of vmask;
// at least `want` valid keys in the workgroup): returns the `want`-th largest
// key T and *rem, the number of its copies inside the top `want`.
//  1. a 2048-bin histogram of the keys inside a window of 2^24 key units below
//     the largest key (two octaves of fp32 score below the maximum; keys under
//     the window are not counted, so crowded low bins cost nothing), scanned
//     from the top: the bin b that holds the want-th key and its rank in b;
//  2. b's keys (a few: bins are 2^13 key units wide) are compacted to LDS and T
//     is the one with #(> T) < rank <= #(>= T).
// If fewer than `want` keys fall in the window, or b is crowded, an exact
// 3-round radix select over all keys is used instead.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t block_select(const uint32_t (&key)[KPT], uint32_t vmask, uint32_t want, uint32_t* rem_out,
                                 uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel, uint32_t* s_cand) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kmax = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) kmax = ((vmask >> i) & 1u) ? max(kmax, key[i]) : kmax;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    if (lane == 0) s_sel[8 + wave] = kmax;
    for (int b = tid; b < 2048; b += NT) s_hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) kmax = max(kmax, s_sel[8 + w]);
    constexpr uint32_t kWin = (1u << 24) - 1u;
    const uint32_t lo = kmax > kWin ? kmax - kWin : 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (((vmask >> i) & 1u) && key[i] >= lo) atomicAdd(&s_hist[(key[i] - lo) >> 13], 1u);
    __syncthreads();
    const uint32_t tot = find_bin<NT>(s_hist, want, 2048, s_wave, s_sel);
    if (tot >= want && s_sel[2] <= (uint32_t)kCandCap) {
        const uint32_t bsel = s_sel[0], rank = s_sel[1], cnt = s_sel[2];
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            mine += (((vmask >> i) & 1u) && key[i] >= lo && ((key[i] - lo) >> 13) == bsel) ? 1u : 0u;
        uint32_t t2;
        uint32_t off = block_excl_scan<NT>(mine, s_wave, t2);
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (((vmask >> i) & 1u) && key[i] >= lo && ((key[i] - lo) >> 13) == bsel) s_cand[off++] = key[i];
        __syncthreads();
        if (cnt <= (uint32_t)NT) {
            if ((uint32_t)tid < cnt) {
                const uint32_t kc = s_cand[tid];
                uint32_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < cnt; ++j) {
                    const uint32_t kj = s_cand[j];
                    gt += kj > kc ? 1u : 0u;
                    ge += kj >= kc ? 1u : 0u;
                }
                if (gt < rank && rank <= ge) {  // every copy of T writes the same values
                    s_sel[4] = kc;
                    s_sel[5] = rank - gt;
                }
            }
            __syncthreads();
            *rem_out = s_sel[5];
            const uint32_t T = s_sel[4];
            __syncthreads();
            return T;
        }
        return radix_select<NT>(LdsKeys{s_cand}, (int64_t)cnt, rank, rem_out, s_hist, s_wave, s_sel + 4);
    }
    return radix_select_regs<NT, KPT>(key, vmask, want, rem_out, s_hist, s_wave, s_sel + 4);
}

// Emit, in slot order (ids ascending by thread, then slot), the ids of keys > T
// and of the first `rem` keys == T.  `ids(i)` gives slot i's id.  Writes
// positions < k only.  Returns (through s_sel[6]) the id of the last taken copy
// of T (the k-th element).
template <int NT, int KPT, typename Ids>
__device__ __forceinline__ void emit_selected(const uint32_t (&key)[KPT], uint32_t vmask, uint32_t T, uint32_t rem, int k,
                              const Ids& ids, int32_t* out, uint32_t* s_wave, uint32_t* s_sel, bool write) {
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool v = (vmask >> i) & 1u;
        ngt += (v && key[i] > T) ? 1u : 0u;
        neq += (v && key[i] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan<NT>(ngt | (neq << 16), s_wave, tot);
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xffffu) + (eq_before < rem ? eq_before : rem);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (!((vmask >> i) & 1u)) continue;
        bool sel = key[i] > T;
        if (key[i] == T) {
            sel = eq_before < rem;
            if (eq_before + 1 == rem) s_sel[6] = (uint32_t)ids(i);
            ++eq_before;
        }
        if (sel) {
            if (write && pos < (uint32_t)k) out[pos] = ids(i);
            ++pos;
        }
    }
}

// ---------------------------------------------------------------- single-pass select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRegKeys = 32;                     // keys per thread held in registers
constexpr int kRegMax = kRegKeys * kSelThreads;  // 32768 candidates

// Full select for one query by one 1024-thread workgroup: thread t holds the
// scores of ids [32t, 32t+32) in registers (nv <= 32768), else the keys are
// read from global memory in radix rounds.  Used when the two-stage select
// does not apply or its check fails.
__device__ __forceinline__ void select_full(const float* sc, int64_t nv, int k, int32_t* out, float* kth, uint32_t* s_hist,
                            uint32_t* s_wave, uint32_t* s_sel, uint32_t* s_cand) {
    const int tid = threadIdx.x;
    if (nv <= kRegMax) {
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
        const int64_t nm = nv - e0 < 0 ? 0 : (nv - e0 < kRegKeys ? nv - e0 : kRegKeys);
        const uint32_t vmask = nm >= 32 ? 0xffffffffu : ((1u << nm) - 1u);
        uint32_t rem;
        const uint32_t T = block_select<kSelThreads, kRegKeys>(key, vmask, (uint32_t)k, &rem, s_hist, s_wave, s_sel,
                                                               s_cand);
        emit_selected<kSelThreads, kRegKeys>(key, vmask, T, rem, k, [&](int i) { return (int32_t)(e0 + i); }, out,
                                             s_wave, s_sel, true);
        if (tid == 0 && kth) *kth = key_score(T);
        return;
    }
    // long lists: radix rounds and an ordered emission over global memory;
    // wave w owns ids [w*seg, (w+1)*seg)
    uint32_t rem;
    const uint32_t T = radix_select<kSelThreads>(GlobalKeys{sc}, nv, (uint32_t)k, &rem, s_hist, s_wave, s_sel);
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t seg = ((nv + kSelWaves - 1) / kSelWaves + 63) & ~(int64_t)63;
    const int64_t lo = (int64_t)wave * seg;
    const int64_t hi = lo + seg < nv ? lo + seg : nv;
    uint32_t n_gt = 0, n_eq = 0;
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        const bool in = e < hi;
        const uint32_t key = in ? score_key(sc[e]) : 0u;
        n_gt += __popcll(__ballot(in && key > T));
        n_eq += __popcll(__ballot(in && key == T));
    }
    uint32_t* s_cnt = s_cand;  // [2][kSelWaves]
    if (lane == 0) {
        s_cnt[wave] = n_gt;
        s_cnt[kSelWaves + wave] = n_eq;
    }
    __syncthreads();
    uint32_t out_pos = 0, eq_seen = 0;
    for (int w = 0; w < wave; ++w) {
        const uint32_t eq_w = s_cnt[kSelWaves + w];
        const uint32_t take_eq = eq_seen >= rem ? 0u : (eq_w < rem - eq_seen ? eq_w : rem - eq_seen);
        out_pos += s_cnt[w] + take_eq;
        eq_seen += eq_w;
    }
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        const bool in = e < hi;
        const uint32_t key = in ? score_key(sc[e]) : 0u;
        const bool gt = in && key > T, eq = in && key == T;
        const uint64_t eqm = __ballot(eq);
        const uint32_t eq_rank = eq_seen + __popcll(eqm & lanemask_lt(lane));
        const bool sel = gt || (eq && eq_rank < rem);
        const uint64_t selm = __ballot(sel);
        const uint32_t dst = out_pos + __popcll(selm & lanemask_lt(lane));
        if (sel && dst < (uint32_t)k) out[dst] = (int32_t)e;
        out_pos += __popcll(selm);
        eq_seen += __popcll(eqm);
    }
    if (tid == 0 && kth) *kth = key_score(T);
}

// Fewer visible entries than k: all of them, then -1; kth = the smallest score.
__device__ void select_all(const float* sc, int64_t nv, int k, int32_t* out, float* kth, float* s_min) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x / 64;
    for (int j = tid; j < k; j += blockDim.x) out[j] = j < nv ? j : -1;
    if (!kth) return;
    float m = INFINITY;
    for (int64_t e = tid; e < nv; e += blockDim.x) m = fminf(m, sc[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fminf(m, __shfl_xor(m, o));
    if (lane == 0) s_min[wave] = m;
    __syncthreads();
    if (tid == 0) {
        float r = INFINITY;
        for (int w = 0; w < nw; ++w) r = fminf(r, s_min[w]);
        *kth = nv > 0 ? r : -INFINITY;
    }
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(IndexArgs a) {
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_sel[8 + kSelWaves];
    __shared__ float s_min[kSelWaves];
    const int n = blockIdx.x;
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;  // the score kernel reports bad queries
    const float* sc = a.scores + (int64_t)n * a.stride;
    int32_t* out = a.topk + (int64_t)n * a.k;
    float* kth = a.kth ? a.kth + n : nullptr;
    if (nv <= a.k) select_all(sc, nv, a.k, out, kth, s_min);
    else select_full(sc, nv, a.k, out, kth, s_hist, s_wave, s_sel, s_cand);
}

// ---------------------------------------------------------------- two-stage select

constexpr int kChunk = 2048;        // ids per first-stage workgroup
constexpr int kLocalThreads = 256;  // 8 ids per thread
constexpr int kMergeSlots = 8;      // candidates per thread in the second stage (8192 per query)

// Stage 1: one 256-thread workgroup per (query, chunk of 2048 ids): the chunk's
// first `kl` ids in (score desc, id asc) order -- its local top-kl, written in
// ascending id order -- and the (kl+1)-th, whose position the merge checks.
__global__ void __launch_bounds__(kLocalThreads) topk_local_kernel(IndexArgs a) {
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[kLocalThreads / 64];
    __shared__ uint32_t s_sel[8 + kLocalThreads / 64];
    const int n = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;
    const int64_t base = (int64_t)blk * kChunk;
    if (base >= nv || nv <= a.k) return;  // the merge reads chunks below nv only
    const float* sc = a.scores + (int64_t)n * a.stride + base;
    const int64_t nvalid = nv - base < kChunk ? nv - base : kChunk;
    const int kl = a.kl;
    uint2* cand = a.cand + ((int64_t)n * a.nchunks + blk) * kl;
    const int64_t e0 = (int64_t)tid * 8;
    uint32_t key[8];
    uint32_t vmask = 0;
    if (e0 + 8 <= nvalid) {
        const float4 v0 = reinterpret_cast<const float4*>(sc + e0)[0];
        const float4 v1 = reinterpret_cast<const float4*>(sc + e0)[1];
        key[0] = score_key(v0.x); key[1] = score_key(v0.y); key[2] = score_key(v0.z); key[3] = score_key(v0.w);
        key[4] = score_key(v1.x); key[5] = score_key(v1.y); key[6] = score_key(v1.z); key[7] = score_key(v1.w);
        vmask = 0xffu;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            key[i] = e0 + i < nvalid ? score_key(sc[e0 + i]) : 0u;
            vmask |= (e0 + i < nvalid ? 1u : 0u) << i;
        }
    }
    if (nvalid <= kl) {
        // every id is a candidate; no (kl+1)-th element
        uint32_t tot;
        uint32_t pos = block_excl_scan<kLocalThreads>((uint32_t)__popc(vmask), s_wave, tot);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((vmask >> i) & 1u) cand[pos++] = make_uint2(key[i], (uint32_t)(base + e0 + i));
        for (int j = (int)tot + tid; j < kl; j += kLocalThreads) cand[j] = make_uint2(0u, 0xffffffffu);
        if (tid == 0) a.c_next[(int64_t)n * a.nchunks + blk] = make_uint2(0u, 0xffffffffu);
        return;
    }
    uint32_t rem;
    const uint32_t T = block_select<kLocalThreads, 8>(key, vmask, (uint32_t)kl + 1, &rem, s_hist, s_wave, s_sel, s_cand);
    // the top kl+1 = keys > T and the first `rem` copies of T; its last copy of T
    // (id order) is the (kl+1)-th element and is not a candidate
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool v = (vmask >> i) & 1u;
        ngt += (v && key[i] > T) ? 1u : 0u;
        neq += (v && key[i] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan<kLocalThreads>(ngt | (neq << 16), s_wave, tot);
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xffffu) + (eq_before < rem - 1 ? eq_before : rem - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!((vmask >> i) & 1u)) continue;
        bool sel = key[i] > T;
        if (key[i] == T) {
            sel = eq_before + 1 < rem;
            if (eq_before + 1 == rem) a.c_next[(int64_t)n * a.nchunks + blk] = make_uint2(T, (uint32_t)(base + e0 + i));
            ++eq_before;
        }
        if (sel) {
            if (pos < (uint32_t)kl) cand[pos] = make_uint2(key[i], (uint32_t)(base + e0 + i));
            ++pos;
        }
    }
}

// Stage 2: one 1024-thread workgroup per query.  The chunks' candidate lists,
// concatenated, are in ascending id order; thread t holds slots [8t, 8t+8).
// The top k of the candidates (score desc, id asc) is exact when every chunk's
// (kl+1)-th element comes after the k-th selected element in that order: every
// id outside the candidates then comes after it too.  Otherwise (or when the
// lists do not fit) the full select runs on the scores.
__global__ void __launch_bounds__(kSelThreads) topk_merge_kernel(IndexArgs a) {
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_sel[8 + kSelWaves];
    __shared__ float s_min[kSelWaves];
    __shared__ uint32_t s_fail;
    const int n = blockIdx.x, tid = threadIdx.x;
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;
    const float* sc = a.scores + (int64_t)n * a.stride;
    int32_t* out = a.topk + (int64_t)n * a.k;
    float* kth = a.kth ? a.kth + n : nullptr;
    if (nv <= a.k) {
        select_all(sc, nv, a.k, out, kth, s_min);
        return;
    }
    const int nch = (int)((nv + kChunk - 1) / kChunk);
    const int64_t nslots = (int64_t)nch * a.kl;
    // A chunk of L visible ids yields min(L, kl) candidates; with fewer than k
    // in all, the candidates cannot hold the top k (short rows, few chunks).
    const int64_t ncand = (nv / kChunk) * a.kl + (int64_t)min<int64_t>(a.kl, nv % kChunk);
    if (nslots > (int64_t)kMergeSlots * kSelThreads || ncand < a.k) {
        select_full(sc, nv, a.k, out, kth, s_hist, s_wave, s_sel, s_cand);
        return;
    }
    const uint2* cand = a.cand + (int64_t)n * a.nchunks * a.kl;
    uint32_t key[kMergeSlots], id[kMergeSlots], vmask = 0;
#pragma unroll
    for (int i = 0; i < kMergeSlots; ++i) {
        const int64_t f = (int64_t)tid * kMergeSlots + i;
        uint2 c = make_uint2(0u, 0xffffffffu);
        if (f < nslots) c = cand[f];
        key[i] = c.x;
        id[i] = c.y;
        vmask |= (c.y != 0xffffffffu ? 1u : 0u) << i;
    }
    if (tid == 0) s_fail = 0;
    uint32_t rem;
    const uint32_t T = block_select<kSelThreads, kMergeSlots>(key, vmask, (uint32_t)a.k, &rem, s_hist, s_wave, s_sel,
                                                             s_cand);
    // the k-th element's id (s_sel[6]) from a counting pass, then the check
    emit_selected<kSelThreads, kMergeSlots>(key, vmask, T, rem, a.k, [&](int i) { return (int32_t)id[i]; }, out,
                                            s_wave, s_sel, false);
    __syncthreads();
    const uint32_t idk = s_sel[6];
    for (int c = tid; c < nch; c += kSelThreads) {
        const uint2 nx = a.c_next[(int64_t)n * a.nchunks + c];
        if (nx.y != 0xffffffffu && !(nx.x < T || (nx.x == T && nx.y > idk))) s_fail = 1;
    }
    __syncthreads();
    if (s_fail) {
        select_full(sc, nv, a.k, out, kth, s_hist, s_wave, s_sel, s_cand);
        return;
    }
    emit_selected<kSelThreads, kMergeSlots>(key, vmask, T, rem, a.k, [&](int i) { return (int32_t)id[i]; }, out,
                                            s_wave, s_sel, true);
    if (tid == 0 && kth) *kth = key_score(T);
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0) return hipSuccess;
    constexpr int U = kScoreUnits;
    dim3 grid((unsigned)(a.stride / (256 * U)), (unsigned)a.num_q);
    switch (a.dim) {
        case 32: launch_kernel(ev, true, true, index_score_kernel<32, U>, grid, dim3(256), st, a); break;
        case 64: launch_kernel(ev, true, true, index_score_kernel<64, U>, grid, dim3(256), st, a); break;
        case 128: launch_kernel(ev, true, true, index_score_kernel<128, U>, grid, dim3(256), st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_topk_select(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0) return hipSuccess;
    if (a.kl > 0) {
        launch_kernel(ev, true, false, topk_local_kernel, dim3((unsigned)a.nchunks, (unsigned)a.num_q),
                      dim3(kLocalThreads), st, a);
        launch_kernel(ev, false, true, topk_merge_kernel, dim3((unsigned)a.num_q), dim3(kSelThreads), st, a);
    } else {
        launch_kernel(ev, true, true, topk_select_kernel, dim3((unsigned)a.num_q), dim3(kSelThreads), st, a);
    }
    return hipGetLastError();
}

}  // namespace csl
