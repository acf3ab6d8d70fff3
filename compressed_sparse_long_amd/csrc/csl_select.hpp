// Exact top-k selection by one workgroup (shared by the indexer's select
// kernels and the decode attention kernel that merges first-stage
// candidates in its prologue): order-preserving score keys, block scans,
// histogram + radix selection over register-resident or global keys, and
// the ordered emission of the selected ids.  Outputs go through a functor
// out(position, id), so a caller can write the global top-k array, a
// workgroup's LDS slice of it, or both.
#pragma once
#include "csl_kernels.hpp"

namespace csl {
namespace {

// Writes selected ids to a global array.
struct GlobalOut {
    int32_t* p;
    __device__ __forceinline__ void operator()(uint32_t pos, int32_t id) const { p[pos] = id; }
};

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
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_scan_add(v);
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
__device__ __forceinline__ uint32_t find_bin(const uint32_t* s_hist, uint32_t want, int nbins, uint32_t* s_wave, uint32_t* s_sel) {
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
__device__ __forceinline__ uint32_t radix_select(const Keys& key_at, int64_t n, uint32_t want, uint32_t* rem_out, uint32_t* s_hist,
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

// An NB-bin histogram in LDS scanned from the top by one wave: the bin that
// holds the rank-th largest counted key, the rank inside that bin and its
// count (valid if total >= rank).  Lane l sums bins NB-1-PER*l downwards; the
// hit lane's PER bins are then spread over lanes for a second scan.  A packed
// histogram holds two 16-bit counts per word (counts below 65536).
struct BinPick {
    uint32_t bin, rank, cnt, total;
};
// Count of bin b in a histogram of NB bins, plain (one word per bin) or
// packed (bins 2w and 2w+1 in the low and high halves of word w).
template <bool PACKED>
__device__ __forceinline__ uint32_t hist_bin(const uint32_t* hist, int b) {
    if constexpr (PACKED) return (hist[b >> 1] >> (16 * (b & 1))) & 0xffffu;
    else return hist[b];
}
template <int NB, bool PACKED = false>
__device__ __forceinline__ BinPick wave_find_bin(const uint32_t* hist, uint32_t rank) {
    constexpr int PER = NB >= 64 ? NB / 64 : 1;
    constexpr int WPER = PACKED ? PER / 2 : PER;  // words per lane
    const int lane = threadIdx.x & 63;
    const int top = NB - 1 - PER * lane;
    uint32_t sum = 0;
    if constexpr (WPER >= 4) {
        const int w0 = PACKED ? (top + 1 - PER) >> 1 : top + 1 - PER;
#pragma unroll
        for (int v = 0; v < WPER / 4; ++v) {
            const u32x4 h = *reinterpret_cast<const u32x4*>(hist + w0 + 4 * v);
            sum += PACKED ? (h[0] & 0xffffu) + (h[0] >> 16) + (h[1] & 0xffffu) + (h[1] >> 16) + (h[2] & 0xffffu) +
                                (h[2] >> 16) + (h[3] & 0xffffu) + (h[3] >> 16)
                          : h[0] + h[1] + h[2] + h[3];
        }
    } else {
        static_assert(PER == 1, "bins per lane: 1 or a multiple of 4 words");
        sum = top >= 0 ? hist_bin<PACKED>(hist, top) : 0u;
    }
    const uint32_t incl = wave_scan_add(sum);
    BinPick r = {0u, 0u, 0u, lane_value(incl, 63)};
    if (r.total < rank) return r;
    const uint32_t above = incl - sum;
    const int L = __builtin_ctzll(__ballot(above < rank && rank <= incl));
    const uint32_t above_l = lane_value(above, L);
    if constexpr (PER == 1) {
        r.bin = (uint32_t)(NB - 1 - L);
        r.rank = rank - above_l;
        r.cnt = lane_value(sum, L);
    } else {
        const int top_l = NB - 1 - PER * L;
        const uint32_t c = lane < PER ? hist_bin<PACKED>(hist, top_l - lane) : 0u;
        const uint32_t in2 = wave_scan_add(c) + above_l;
        const int J = __builtin_ctzll(__ballot(lane < PER && in2 - c < rank && rank <= in2));
        r.bin = (uint32_t)(top_l - J);
        r.cnt = lane_value(c, J);
        r.rank = rank - (lane_value(in2, J) - r.cnt);
    }
    return r;
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The rank-th largest of cn <= 64 keys in LDS, by one wave (lane j ranks key j
// against all): T, and *rem = its copies among the top `rank`.
__device__ __forceinline__ void pairwise_rank(const uint32_t* cbuf, uint32_t cn, uint32_t rank, uint32_t& T,
                                              uint32_t& rem) {
    const int lane = threadIdx.x & 63;
    uint32_t kc = 0, gt = 0, ge = 0;
    if ((uint32_t)lane < cn) {
        kc = cbuf[lane];
        for (uint32_t j = 0; j < cn; ++j) {
            const uint32_t kj = cbuf[j];
            gt += kj > kc ? 1u : 0u;
            ge += kj >= kc ? 1u : 0u;
        }
    }
    const int L = __builtin_ctzll(__ballot((uint32_t)lane < cn && gt < rank && rank <= ge));
    T = lane_value(kc, L);
    rem = rank - lane_value(gt, L);
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
// With WAVE_PICK every wave scans the histogram itself and, when b holds at
// most 64 keys, ranks them itself, so that common case takes three workgroup
// barriers instead of ten: shorter for a lone workgroup on a CU, dearer where
// many share one (the repeated scans cost more than the barriers save).  A
// crowded b goes through workgroup scans; if fewer than `want` keys fall in
// the window, an exact 3-round radix select over all keys is used instead.
// s_hist must be 16-byte aligned.
template <int NT, int KPT, bool WAVE_PICK = false, int CAP = kCandCap>
__device__ __forceinline__ uint32_t block_select(const uint32_t (&key)[KPT], uint32_t vmask, uint32_t want, uint32_t* rem_out,
                                 uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel, uint32_t* s_cand) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kmax = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) kmax = ((vmask >> i) & 1u) ? max(kmax, key[i]) : kmax;
    kmax = wave_max_u32(kmax);
    if (lane == 0) s_sel[8 + wave] = kmax;
    if (tid == 0) s_sel[3] = 0u;  // compaction count
    for (int b = tid; b < 512; b += NT) reinterpret_cast<u32x4*>(s_hist)[b] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) kmax = max(kmax, s_sel[8 + w]);
    constexpr uint32_t kWin = (1u << 24) - 1u;
    const uint32_t lo = kmax > kWin ? kmax - kWin : 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (((vmask >> i) & 1u) && key[i] >= lo) atomicAdd(&s_hist[(key[i] - lo) >> 13], 1u);
    __syncthreads();
    // the same pick in every wave (every wave reads the same histogram)
    const BinPick bp = WAVE_PICK ? wave_find_bin<2048>(s_hist, want) : BinPick{0u, 0u, 0u, 0u};
    if (WAVE_PICK && bp.total >= want && bp.cnt <= 64u) {
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (((vmask >> i) & 1u) && key[i] >= lo && ((key[i] - lo) >> 13) == bp.bin)
                s_cand[atomicAdd(&s_sel[3], 1u)] = key[i];
        __syncthreads();
        uint32_t T, rem;
        pairwise_rank(s_cand, bp.cnt, bp.rank, T, rem);
        *rem_out = rem;
        return T;
    }
    const uint32_t tot = find_bin<NT>(s_hist, want, 2048, s_wave, s_sel);
    if (tot >= want && s_sel[2] <= (uint32_t)CAP) {
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
template <int NT, int KPT, typename Ids, typename Out>
__device__ __forceinline__ void emit_selected(const uint32_t (&key)[KPT], uint32_t vmask, uint32_t T, uint32_t rem, int k,
                              const Ids& ids, const Out& out, uint32_t* s_wave, uint32_t* s_sel, bool write) {
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
            if (write && pos < (uint32_t)k) out(pos, ids(i));
            ++pos;
        }
    }
}

// ---------------------------------------------------------------- single-pass select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRegKeys = 32;                     // keys per thread held in registers

// Full select for one query by one NT-thread workgroup: thread t holds the
// scores of ids [32t, 32t+32) in registers (nv <= 32*NT), else the keys are
// read from global memory in radix rounds.  Used when the two-stage select
// does not apply or its check fails.
template <int NT, typename Out>
__device__ __forceinline__ void select_full(const float* sc, int64_t nv, int k, const Out& out, float* kth, uint32_t* s_hist,
                            uint32_t* s_wave, uint32_t* s_sel, uint32_t* s_cand) {
    const int tid = threadIdx.x;
    if (nv <= (int64_t)kRegKeys * NT) {
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
        const uint32_t T = block_select<NT, kRegKeys>(key, vmask, (uint32_t)k, &rem, s_hist, s_wave, s_sel,
                                                               s_cand);
        emit_selected<NT, kRegKeys>(key, vmask, T, rem, k, [&](int i) { return (int32_t)(e0 + i); }, out,
                                             s_wave, s_sel, true);
        if (tid == 0 && kth) *kth = key_score(T);
        return;
    }
    // long lists: radix rounds and an ordered emission over global memory;
    // wave w owns ids [w*seg, (w+1)*seg)
    uint32_t rem;
    const uint32_t T = radix_select<NT>(GlobalKeys{sc}, nv, (uint32_t)k, &rem, s_hist, s_wave, s_sel);
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int NW = NT / 64;
    const int64_t seg = ((nv + NW - 1) / NW + 63) & ~(int64_t)63;
    const int64_t lo = (int64_t)wave * seg;
    const int64_t hi = lo + seg < nv ? lo + seg : nv;
    uint32_t n_gt = 0, n_eq = 0;
    for (int64_t e = lo + lane; e - lane < hi; e += 64) {
        const bool in = e < hi;
        const uint32_t key = in ? score_key(sc[e]) : 0u;
        n_gt += __popcll(__ballot(in && key > T));
        n_eq += __popcll(__ballot(in && key == T));
    }
    uint32_t* s_cnt = s_cand;  // [2][NW]
    if (lane == 0) {
        s_cnt[wave] = n_gt;
        s_cnt[NW + wave] = n_eq;
    }
    __syncthreads();
    uint32_t out_pos = 0, eq_seen = 0;
    for (int w = 0; w < wave; ++w) {
        const uint32_t eq_w = s_cnt[NW + w];
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
        if (sel && dst < (uint32_t)k) out(dst, (int32_t)e);
        out_pos += __popcll(selm);
        eq_seen += __popcll(eqm);
    }
    if (tid == 0 && kth) *kth = key_score(T);
}

// Fewer visible entries than k: all of them, then -1; kth = the smallest score.
template <typename Out>
__device__ __forceinline__ void select_all(const float* sc, int64_t nv, int k, const Out& out, float* kth, float* s_min) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x / 64;
    for (int j = tid; j < k; j += blockDim.x) out((uint32_t)j, j < nv ? j : -1);
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

// ---- single-wave selection: no workgroup barriers.  A wave's LDS operations
// execute in issue order, so after this point a lane reads what any lane of the
// wave wrote before it; the fence keeps the compiler from moving them across.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Emit of a first-stage chunk for slots of 64 consecutive ids (slot i of lane
// l is id base + 64 (slot0 + i) + l), given T, rem, and the counts of keys > T
// and == T among the chunk's ids before the first slot: candidates are the
// keys > T and the first rem - 1 copies of T in id order, each at its rank in
// id order among the candidates; the rem-th copy of T is the (kl+1)-th element.
template <int NS>
__device__ __forceinline__ void emit_first_stage(const uint32_t (&key)[NS], uint32_t vmask, int64_t base, int slot0,
                                                 uint32_t T, uint32_t rem, uint32_t gt_before, uint32_t eq_before,
                                                 int kl, uint2* cand, uint2* cnext) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const bool v = (vmask >> i) & 1u;
        const bool gt = v && key[i] > T, eq = v && key[i] == T;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        const uint32_t e = eq_before + lanes_below(me);
        const uint32_t pos = gt_before + lanes_below(mg) + (e < rem - 1 ? e : rem - 1);
        const uint32_t id = (uint32_t)(base + 64 * (slot0 + i) + lane);
        if ((gt || (eq && e + 1 < rem)) && pos < (uint32_t)kl) cand[pos] = make_uint2(key[i], id);
        if (eq && e + 1 == rem) *cnext = make_uint2(T, id);
        gt_before += (uint32_t)__popcll(mg);
        eq_before += (uint32_t)__popcll(me);
    }
}

// The want-th largest of a wave's keys (NK per lane, slot i valid iff bit i of
// vmask), by one wave.  Radix rounds over rel = key - lo, counting only keys
// >= lo: with WINDOW, lo = max - (2^24 - 1) (two octaves of fp32 score below
// the maximum; digits at bits 13..23, 2..12, 0..1), else lo = 0 (bits 21..31,
// 10..20, 0..9).  Each round histograms its digit in `hist` (1024 words of
// LDS: 2048 bins of 16 bits, two to a word, as a wave holds at most 2048 keys)
// and finds the bin of the rank; once that bin holds at most 64 keys they are
// compacted to `cbuf` (64 words) and ranked pairwise.  Returns false (uniform)
// if fewer than `want` keys are >= lo; else T and *rem, the number of copies
// of T inside the top `want`.
template <bool WINDOW, int NK = 16>
__device__ __forceinline__ bool wave_select(const uint32_t (&key)[NK], uint32_t vmask, uint32_t want, uint32_t lo,
                                            uint32_t* hist, uint32_t* cbuf, uint32_t& T, uint32_t& rem) {
    static_assert(NK <= 32, "slot masks are 32 bits");
    static_assert(NK * 64 < 65536, "bin counts fit 16 bits");
    const int lane = threadIdx.x & 63;
    uint32_t rel[NK], in = 0;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        rel[i] = key[i] - lo;
        in |= (((vmask >> i) & 1u) && key[i] >= lo ? 1u : 0u) << i;
    }
    uint32_t prefix = 0, pmask = 0, rank = want;
    auto matches = [&](int i) { return ((in >> i) & 1u) && (rel[i] & pmask) == prefix; };
    auto build = [&](int sh, int nb) {
        for (int w = 4 * lane; w < nb / 2; w += 256) *reinterpret_cast<u32x4*>(hist + w) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NK; ++i)
            if (matches(i)) {
                const uint32_t bin = (rel[i] >> sh) & (uint32_t)(nb - 1);
                atomicAdd(&hist[bin >> 1], 1u << (16 * (bin & 1u)));
            }
        wave_lds_sync();
    };
    auto take = [&](const BinPick& b, int sh, int nb) {
        prefix |= b.bin << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        rank = b.rank;
    };
    // the bin's keys (at most 64) ranked pairwise
    auto finish = [&](uint32_t cn) {
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < NK; ++i) mine += matches(i) ? 1u : 0u;
        uint32_t off = wave_scan_add(mine) - mine;
#pragma unroll
        for (int i = 0; i < NK; ++i)
            if (matches(i)) {
                if (off < 64u) cbuf[off] = rel[i];
                ++off;
            }
        wave_lds_sync();
        pairwise_rank(cbuf, cn, rank, T, rem);
        T += lo;
        wave_lds_sync();
    };
    constexpr int kSh0 = WINDOW ? 13 : 21, kSh1 = WINDOW ? 2 : 10;
    build(kSh0, 2048);
    BinPick b = wave_find_bin<2048, true>(hist, rank);
    if (b.total < rank) return false;
    take(b, kSh0, 2048);
    if (b.cnt <= 64u) {
        finish(b.cnt);
        return true;
    }
    build(kSh1, 2048);
    b = wave_find_bin<2048, true>(hist, rank);
    take(b, kSh1, 2048);
    if (b.cnt <= 64u) {
        finish(b.cnt);
        return true;
    }
    constexpr int kNb2 = WINDOW ? 4 : 1024;
    build(0, kNb2);
    b = wave_find_bin<kNb2, true>(hist, rank);
    take(b, 0, kNb2);
    T = prefix + lo;
    rem = rank;
    wave_lds_sync();
    return true;
}


// ---------------------------------------------------------------- merge of first-stage candidates

constexpr int kChunk = 1024;  // ids per first-stage chunk (one workgroup of the decode score kernel)

// A query's first-stage output: for each 1024-id chunk, its first kl ids in
// (score desc, id asc) order, written in ascending id order ((key, id) pairs,
// id 0xffffffff = empty), and the chunk's (kl+1)-th element; and the full
// score row for the fallback.
struct MergeIn {
    const uint2* cand;   // [nchunks][kl]
    const uint2* cnext;  // [nchunks]
    const float* sc;     // [nv] scores
    int64_t nv;          // visible ids
    int kl, k;
};
// The candidate slots a merge thread holds (KPT of them) and the (kl+1)-th
// element of chunk `thread`, loaded before the query's visible count is known.
template <int KPT>
struct CandRegs {
    uint2 c[KPT];
    uint2 nx;
};
// Thread t loads slots [KPT t, KPT t + KPT) of the first nslots_max and chunk t's
// next element if t < nch_max; slots past the query's chunks are masked by the merge.
template <int KPT>
__device__ __forceinline__ void cand_load(const MergeIn& in, int64_t nslots_max, int nch_max, CandRegs<KPT>& r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int64_t f = (int64_t)tid * KPT + i;
        r.c[i] = make_uint2(0u, 0xffffffffu);
        if (f < nslots_max) r.c[i] = in.cand[f];
    }
    r.nx = make_uint2(0u, 0xffffffffu);
    if (tid < nch_max) r.nx = in.cnext[tid];
}

// LDS of one merge: hist[2048], cand[kCandCap], wave[NT/64], sel[8 + NT/64], min[NT/64], fail[1].
struct MergeLds {
    uint32_t* hist;
    uint32_t* cand;
    uint32_t* wave;
    uint32_t* sel;
    float* min;
    uint32_t* fail;
};

// The top k of a query by one NT-thread workgroup from its first-stage
// candidates (thread t holds slots [KPT t, KPT t + KPT) of the concatenated
// lists, which are in ascending id order).  The top k of the candidates
// (score desc, id asc) is exact when every chunk's (kl+1)-th element comes
// after the k-th selected element in that order: every id outside the
// candidates then comes after it too.  Otherwise, or when the candidates
// cannot hold k ids, the full select runs on the score row and overwrites
// every output position.  Fewer than k visible ids: all of them, then -1.
// Every thread calls it; out(pos, id) receives each position 0..k-1 (a
// position may be written twice when the fallback runs); kth (nullable) the
// k-th score.
template <int NT, int KPT, bool WAVE_PICK, typename Out>
__device__ __forceinline__ void merge_candidates(const MergeIn& in, const CandRegs<KPT>& r, const Out& out, float* kth,
                                                 const MergeLds& m) {
    const int tid = threadIdx.x;
    const int64_t nv = in.nv;
    if (nv <= in.k) {
        select_all(in.sc, nv, in.k, out, kth, m.min);
        return;
    }
    const int nch = (int)((nv + kChunk - 1) / kChunk);
    const int64_t nslots = (int64_t)nch * in.kl;
    // a chunk of L visible ids yields min(L, kl) candidates
    const int64_t ncand = (nv / kChunk) * in.kl + (int64_t)min<int64_t>(in.kl, nv % kChunk);
    if (nslots > (int64_t)KPT * NT || ncand < in.k) {
        select_full<NT>(in.sc, nv, in.k, out, kth, m.hist, m.wave, m.sel, m.cand);
        return;
    }
    // the chunks' (kl+1)-th elements, fetched beside the candidates
    const uint2 nx = tid < nch ? r.nx : make_uint2(0u, 0xffffffffu);
    uint32_t key[KPT], id[KPT], vmask = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int64_t f = (int64_t)tid * KPT + i;
        uint2 c = make_uint2(0u, 0xffffffffu);
        if (f < nslots) c = r.c[i];
        key[i] = c.x;
        id[i] = c.y;
        vmask |= (c.y != 0xffffffffu ? 1u : 0u) << i;
    }
    if (tid == 0) *m.fail = 0;
    uint32_t rem;
    const uint32_t T = block_select<NT, KPT, WAVE_PICK>(key, vmask, (uint32_t)in.k, &rem, m.hist, m.wave, m.sel, m.cand);
    // emit, and learn the k-th element's id (sel[6]) for the check
    emit_selected<NT, KPT>(key, vmask, T, rem, in.k, [&](int i) { return (int32_t)id[i]; }, out, m.wave, m.sel, true);
    __syncthreads();
    const uint32_t idk = m.sel[6];
    bool bad = nx.y != 0xffffffffu && !(nx.x < T || (nx.x == T && nx.y > idk));
    for (int c = tid + NT; c < nch; c += NT) {
        const uint2 x = in.cnext[c];
        bad |= x.y != 0xffffffffu && !(x.x < T || (x.x == T && x.y > idk));
    }
    if (bad) *m.fail = 1;
    __syncthreads();
    if (*m.fail) {
        select_full<NT>(in.sc, nv, in.k, out, kth, m.hist, m.wave, m.sel, m.cand);
        return;
    }
    if (tid == 0 && kth) *kth = key_score(T);
}

}  // namespace
}  // namespace csl
