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
#include "csl_insert.hpp"
#include "csl_select.hpp"

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


__device__ __forceinline__ void select_query(const IndexArgs& a, const int n) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_sel[8 + kSelWaves];
    __shared__ float s_min[kSelWaves];
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;  // the score kernel reports bad queries
    const float* sc = a.scores + (int64_t)n * a.stride;
    int32_t* out = a.topk + (int64_t)n * a.k;
    float* kth = a.kth ? a.kth + n : nullptr;
    if (nv <= a.k) select_all(sc, nv, a.k, GlobalOut{out}, kth, s_min);
    else select_full<kSelThreads>(sc, nv, a.k, GlobalOut{out}, kth, s_hist, s_wave, s_sel, s_cand);
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(IndexArgs a) { select_query(a, blockIdx.x); }

// ---------------------------------------------------------------- two-stage select

// ---------------------------------------------------------------- scores (+ first stage)

// index_score_kernel<DI, U, LOCAL> -- the HBM stream of the decode step.  A
// workgroup (4 waves) scores 4*U*64 consecutive entries of one query; a wave
// streams U consecutive 64-entry units (one paged block each).  A unit comes
// in with contiguous 1 KiB loads (lane l takes chunk l % CPR of row l / CPR),
// non-temporal since every row is read once per step, then passes through
// the wave's own LDS slice to reach the MFMA operand layout, whose direct
// loads (16 rows x 64 B per instruction) stream measurably slower.  The next
// unit is in flight meanwhile.  qI[16 heads x d] . K^T[d x 16 entries] is one
// v_mfma_f32_16x16x32_bf16 per 32 dims; ReLU, the head weight and the head
// sum are fused on the accumulators (4 heads in-lane, 2 cross-lane steps).
// An unmapped or invisible unit reads page 0 (always allocated) and its
// scores are not used; an unmapped unit scores -inf and is flagged.
//
// With LOCAL (U = 4: a workgroup = one 1024-entry chunk), the workgroup then
// reuses its LDS for the first stage of the top-k: the chunk's first kl ids in
// (score desc, id asc) order -- written in ascending id order -- and the
// (kl+1)-th, whose position the merge checks.
constexpr int kMergeSlots = 8;      // candidates per merge thread

// First stage of the two-stage top-k over one 1024-id chunk of query n, by one
// wave whose lane l holds the keys of ids base + 16 l .. +15 (ids at or past
// base + nvalid are invalid): the chunk's first kl ids in (score desc, id asc)
// order, written in ascending id order, and the (kl+1)-th, whose position the
// merge checks (none if nvalid <= kl).  hist / cbuf: LDS of 1024 and 64 words
// that only this wave uses.
__device__ __forceinline__ void wave_first_stage(const IndexArgs& a, int n, int blk, const uint32_t (&key)[16],
                                                 int64_t base, int nvalid, uint32_t* hist, uint32_t* cbuf) {
    const int lane = threadIdx.x & 63;
    const int kl = a.kl;
    uint2* cand = a.cand + ((int64_t)n * a.nchunks + blk) * kl;
    uint2* cnext = a.c_next + (int64_t)n * a.nchunks + blk;
    const int e0 = 16 * lane;
    const uint32_t vmask = e0 >= nvalid ? 0u : (nvalid - e0 >= 16 ? 0xffffu : (1u << (nvalid - e0)) - 1u);
    if (nvalid <= kl) {
        // every id is a candidate; no (kl+1)-th element
        const uint32_t cntv = (uint32_t)__popc(vmask);
        uint32_t pos = wave_scan_add(cntv) - cntv;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((vmask >> i) & 1u) cand[pos++] = make_uint2(key[i], (uint32_t)(base + e0 + i));
        for (int j = nvalid + lane; j < kl; j += 64) cand[j] = make_uint2(0u, 0xffffffffu);
        if (lane == 0) *cnext = make_uint2(0u, 0xffffffffu);
        return;
    }
    const uint32_t want = (uint32_t)kl + 1;
    uint32_t kmax = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) kmax = ((vmask >> i) & 1u) ? max(kmax, key[i]) : kmax;
    kmax = wave_max_u32(kmax);
    constexpr uint32_t kWin = (1u << 24) - 1u;
    uint32_t T = 0, rem = 0;
    if (!wave_select<true>(key, vmask, want, kmax > kWin ? kmax - kWin : 0u, hist, cbuf, T, rem))
        wave_select<false>(key, vmask, want, 0u, hist, cbuf, T, rem);
    // the top kl+1 = keys > T and the first `rem` copies of T; its last copy
    // of T (id order) is the (kl+1)-th element and is not a candidate
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const bool v = (vmask >> i) & 1u;
        ngt += (v && key[i] > T) ? 1u : 0u;
        neq += (v && key[i] == T) ? 1u : 0u;
    }
    const uint32_t packed = ngt | (neq << 16);
    const uint32_t pre = wave_scan_add(packed) - packed;
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xffffu) + (eq_before < rem - 1 ? eq_before : rem - 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (!((vmask >> i) & 1u)) continue;
        bool sel = key[i] > T;
        if (key[i] == T) {
            sel = eq_before + 1 < rem;
            if (eq_before + 1 == rem) *cnext = make_uint2(T, (uint32_t)(base + e0 + i));
            ++eq_before;
        }
        if (sel) {
            if (pos < (uint32_t)kl) cand[pos] = make_uint2(key[i], (uint32_t)(base + e0 + i));
            ++pos;
        }
    }
}

// Stand-alone first stage (after the query-blocked score kernel): each wave
// takes one (query, chunk), keys read from the score row; no barriers.
__global__ void __launch_bounds__(256) topk_local_kernel(IndexArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[4][1024];
    __shared__ uint32_t s_cbuf[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.y, blk = blockIdx.x * 4 + wave;
    if (blk >= a.nchunks) return;
    int s;
    int64_t p;
    const int64_t nv = query_ok(a, n, s, p) ? visible(a, p) : 0;
    const int64_t base = (int64_t)blk * kChunk;
    if (base >= nv || nv <= a.k) return;  // uniform over the wave; the merge reads chunks below nv only
    const int nvalid = (int)(nv - base < kChunk ? nv - base : kChunk);
    const float* sc = a.scores + (int64_t)n * a.stride + base + 16 * lane;
    uint32_t key[16];
    if (16 * lane + 16 <= nvalid) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 x = reinterpret_cast<const float4*>(sc)[v];
            key[4 * v] = score_key(x.x);
            key[4 * v + 1] = score_key(x.y);
            key[4 * v + 2] = score_key(x.z);
            key[4 * v + 3] = score_key(x.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) key[i] = 16 * lane + i < nvalid ? score_key(sc[i]) : 0u;
    }
    wave_first_stage(a, n, blk, key, base, nvalid, s_hist[wave], s_cbuf[wave]);
}

// LDS of one score workgroup (also the insert body's, when inserts ride in the launch).
template <int DI>
constexpr int score_smem_bytes() {
    constexpr int kUnitBytes = 4 * 64 * (DI * 2 + 16);
    constexpr int kSelBytes = (kChunk + 2048 + 64 + 8) * 4;
    return kUnitBytes > kSelBytes ? kUnitBytes : kSelBytes;
}

// The score workgroup (chunk bx of query n).  Every thread calls it.
template <int DI, int U, bool LOCAL, bool FP4>
__device__ __forceinline__ void score_block(const IndexArgs& a, const int bx, const int n, uint8_t* s_mem) {
    constexpr int KS = DI / 32;          // MFMA k-steps per row
    constexpr int RB = DI * 2;           // bf16 row bytes (the LDS layout)
    constexpr int RBG = FP4 ? DI / 2 + DI / 32 : RB;  // stored row bytes
    static_assert(!FP4 || DI == 128, "fp4 index rows are 128 wide");
    constexpr int CPR = RB / 16;         // 16-byte chunks per row
    constexpr int NLD = CPR;             // 1 KiB loads per 64-row unit
    constexpr int LROW = RB + 16;        // padded LDS row (spreads the banks of the MFMA-layout reads)
    static_assert(!LOCAL || 4 * U * 64 == kChunk, "a first-stage chunk is one workgroup");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int s;
    int64_t p;
    if (!query_ok(a, n, s, p)) {
        if (bx == 0 && tid == 0) raise_error(a.err, (s < 0 || s >= a.num_seqs) ? kErrSeq : kErrPos);
        return;
    }
    const int64_t nv = visible(a, p);
    const int64_t wg0 = (int64_t)bx * 4 * U * 64;  // first entry of the workgroup
    if (wg0 >= nv) return;                                   // uniform over the workgroup
    // the wave's U consecutive 64-entry units; unit u is block u of the sequence
    const int64_t u0 = ((int64_t)bx * 4 + wave) * U;
    float mine_u[U];
#pragma unroll
    for (int j = 0; j < U; ++j) mine_u[j] = -INFINITY;
    if (u0 * 64 < nv) {
        int32_t mypg = 0;  // lane j < U: page of unit u0 + j (-1 unmapped)
        if (lane < U && (u0 + lane) * 64 < nv) mypg = page_of(a.bt, a.max_blocks, a.num_pages, s, (u0 + lane) * 256);
        // bf16: contiguous 1 KiB loads; fp4: lane l takes row l (64 code bytes, 4 scale bytes)
        u32x4 ld[FP4 ? 4 : NLD];
        uint32_t lds4 = 0;
        auto issue = [&](int j) {
            const int32_t pg = __shfl(mypg, j);
            if constexpr (FP4) {
                const uint8_t* r = a.rows + (int64_t)(pg < 0 ? 0 : pg) * 64 * RBG + lane * RBG;
#pragma unroll
                for (int q = 0; q < 4; ++q) ld[q] = load16_a4(r + 16 * q);
                lds4 = *reinterpret_cast<const uint32_t*>(r + 64);
            } else {
                const u32x4* base = reinterpret_cast<const u32x4*>(a.rows + (int64_t)(pg < 0 ? 0 : pg) * 64 * RB);
#pragma unroll
                for (int q = 0; q < NLD; ++q) ld[q] = __builtin_nontemporal_load(base + q * 64 + lane);
            }
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

        uint8_t* su = s_mem + wave * 64 * LROW;
        constexpr int RPL = 64 / CPR;  // rows per 1 KiB load
#pragma unroll
        for (int j = 0; j < U; ++j) {
            // this unit into LDS (in-order LDS ops of one wave: the reads of the
            // previous unit have been issued before these writes)
            if constexpr (FP4) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    uint32_t w[16];
                    mxfp4_to_bf16(ld[b], (lds4 >> (8 * b)) & 255u, w);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<u32x4*>(su + lane * LROW + 64 * b + 16 * i) =
                            u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                }
            } else {
#pragma unroll
                for (int q = 0; q < NLD; ++q)
                    *reinterpret_cast<u32x4*>(su + (q * RPL + lane / CPR) * LROW + (lane % CPR) * 16) = ld[q];
            }
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
                v = sum_xor16(v);
                v = sum_xor32(v);
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
            mine_u[j] = mine;
            if (e0 + lane < nv) a.scores[(int64_t)n * a.stride + e0 + lane] = mine;
        }
    }
    if constexpr (LOCAL) {
        if (nv <= a.k) return;  // uniform: the merge takes every visible id
        // ---- first stage of the top-k over this chunk (ids wg0 + 64 (wave U + j) + lane):
        // the four waves histogram the window below the chunk's largest key
        // (as wave_select's first round), find the bin of the (kl+1)-th key,
        // gather that bin's keys, rank them pairwise (every wave alike), and
        // each emits its own ids
        const int kl = a.kl;
        const int nvalid = (int)(nv - wg0 < kChunk ? nv - wg0 : kChunk);
        uint2* cand = a.cand + ((int64_t)n * a.nchunks + bx) * kl;
        uint2* cnext = a.c_next + (int64_t)n * a.nchunks + bx;
        uint32_t kw[U], vmask = 0, kmax = 0u;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            kw[j] = score_key(mine_u[j]);
            const bool v = (wave * U + j) * 64 + lane < nvalid;
            vmask |= (v ? 1u : 0u) << j;
            if (v) kmax = max(kmax, kw[j]);
        }
        kmax = wave_max_u32(kmax);
        uint32_t* s_keys = reinterpret_cast<uint32_t*>(s_mem);  // [kChunk], id order
        uint32_t* s_hist = s_keys + kChunk;                     // [2048]
        uint32_t* s_cbuf = s_hist + 2048;                       // [64]
        uint32_t* s_w = s_cbuf + 64;                            // [4] wave maxima, then counts; [4] gather count
        __syncthreads();  // every wave is done with its unit slice
        if (nvalid <= kl) {
            // every id is a candidate; no (kl+1)-th element
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int e = (wave * U + j) * 64 + lane;
                if (e < nvalid) cand[e] = make_uint2(kw[j], (uint32_t)(wg0 + e));
            }
            for (int j = nvalid + tid; j < kl; j += 256) cand[j] = make_uint2(0u, 0xffffffffu);
            if (tid == 0) *cnext = make_uint2(0u, 0xffffffffu);
            return;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) s_keys[(wave * U + j) * 64 + lane] = kw[j];
        reinterpret_cast<u32x4*>(s_hist)[tid] = u32x4{0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4*>(s_hist)[256 + tid] = u32x4{0u, 0u, 0u, 0u};
        if (lane == 0) s_w[wave] = kmax;
        if (tid == 0) s_w[4] = 0u;
        __syncthreads();
        kmax = max(max(s_w[0], s_w[1]), max(s_w[2], s_w[3]));
        constexpr uint32_t kWin = (1u << 24) - 1u;
        const uint32_t lo = kmax > kWin ? kmax - kWin : 0u;
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (((vmask >> j) & 1u) && kw[j] >= lo) atomicAdd(&s_hist[(kw[j] - lo) >> 13], 1u);
        __syncthreads();
        const uint32_t want = (uint32_t)kl + 1;
        const BinPick b = wave_find_bin<2048>(s_hist, want);
        uint32_t T, rem;
        if (b.total < want || b.cnt > 64u) {
            // the window holds fewer than kl+1 keys or a crowded bin: wave 0
            // runs the single-wave selection over the chunk (after every
            // wave has read the histogram it reuses)
            __syncthreads();
            if (wave != 0) return;
            uint32_t key[16];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 kv = reinterpret_cast<const uint4*>(s_keys)[4 * lane + v];
                key[4 * v] = kv.x;
                key[4 * v + 1] = kv.y;
                key[4 * v + 2] = kv.z;
                key[4 * v + 3] = kv.w;
            }
            wave_first_stage(a, n, bx, key, wg0, nvalid, s_hist, s_cbuf);
            return;
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (((vmask >> j) & 1u) && kw[j] >= lo && ((kw[j] - lo) >> 13) == b.bin)
                s_cbuf[atomicAdd(&s_w[4], 1u) & 63u] = kw[j];
        __syncthreads();
        pairwise_rank(s_cbuf, b.cnt, b.rank, T, rem);
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const bool v = (vmask >> j) & 1u;
            ngt += (uint32_t)__popcll(__ballot(v && kw[j] > T));
            neq += (uint32_t)__popcll(__ballot(v && kw[j] == T));
        }
        if (lane == 0) s_w[wave] = ngt | (neq << 16);  // the maxima there were read before the histogram
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += s_w[w];
        emit_first_stage<U>(kw, vmask, wg0, wave * U, T, rem, before & 0xffffu, before >> 16, kl, cand, cnext);
    }
}

template <int DI, int U, bool LOCAL, bool FP4 = false>
__global__ void __launch_bounds__(256) index_score_kernel(IndexArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[score_smem_bytes<DI>()];
    score_block<DI, U, LOCAL, FP4>(a, blockIdx.x, blockIdx.y, s_mem);
}

// The decode score launch with the step's writes riding in it: rows y < num_q
// of the grid are score workgroups; the rows after them take, in order, one
// (new token, pool) insert per workgroup, then the query-side rows (four per
// workgroup).  They are dispatched after every score workgroup, so they run
// while the stream's last workgroups drain.  The writes touch positions the
// step's queries do not read (the queries at p see entries and raw tokens
// below p), so the scores are the same as without them.
template <int DI, int U, bool LOCAL, bool FP4 = false>
__global__ void __launch_bounds__(256) index_score_insert_kernel(IndexArgs a, CompressArgs c, QSideArgs q) {
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[score_smem_bytes<DI>()];
    static_assert(sizeof(InsertSmem) <= score_smem_bytes<DI>(), "the insert body fits the score workgroup's LDS");
    if ((int)blockIdx.y < a.num_q) {
        score_block<DI, U, LOCAL, FP4>(a, blockIdx.x, blockIdx.y, s_mem);
        return;
    }
    const int64_t i = ((int64_t)blockIdx.y - a.num_q) * gridDim.x + blockIdx.x;
    const int64_t n_ins = (int64_t)c.total_new * c.n_jobs;
    const int64_t n_qb = q.n_items > 0 ? (q.n_items + 3) / 4 : 0;
    if (i < n_ins) insert_block(c, (int)(i / c.total_new), (int)(i % c.total_new), *reinterpret_cast<InsertSmem*>(s_mem));
    else if (i < n_ins + n_qb) qside_block<1>(q, i - n_ins);
}

// index_score_tiled_kernel<DI, QW> -- scores for many queries (prefill chunks).
// A workgroup takes a block of 4*QW queries and one 1024-entry chunk.  The
// chunk's pages of the queries' sequence stream once through double-buffered
// LDS (contiguous 16-byte loads by all 256 threads; pages are reused by every
// query block, so the loads are cached).  Each wave contracts its QW queries,
// two at a time, against every staged page with v_mfma_f32_32x32x16_bf16:
// A = 32 rows = 2 queries x 16 heads (registers), B = 32 entries (LDS), so one
// LDS read of an operand feeds QW/2 MFMAs and one page load 4*QW queries.  In
// the 32x32 accumulator a lane holds 8 heads of each of the two queries for
// its entry column: ReLU, head weight and the in-lane sum, then one 32-lane
// swap completes the head sum.  Score rows stream out (non-temporal stores).
// Queries of another sequence inside the block are taken in further passes
// over the chunk, one per sequence.
constexpr int kTiledQW = 4;           // queries per wave (4 waves per workgroup; even)
constexpr int kTiledMinQueries = 64;  // calls with at least this many queries use the tiled kernel

template <int DI, int QW, bool FP4 = false>
__global__ void __launch_bounds__(256) index_score_tiled_kernel(IndexArgs a) {
    constexpr int kTiledQ = 4 * QW;       // queries per workgroup
    constexpr int PP = QW / 2;            // query pairs per wave
    constexpr int KS = DI / 16, RB = DI * 2, CPR = RB / 16, LROW = RB + 16;
    constexpr int RBG = FP4 ? DI / 2 + DI / 32 : RB;  // stored row bytes
    constexpr int UNIT = 64 * RBG;        // bytes of a 64-entry page
    constexpr int LPT = FP4 ? 1 : UNIT / 16 / 256;  // 16-byte loads per thread per page
    static_assert(QW % 2 == 0, "queries go to the MFMA in pairs");
    static_assert(FP4 || (LPT >= 1 && UNIT == LPT * 16 * 256), "a page is a whole number of workgroup loads");
    static_assert(!FP4 || DI == 128, "fp4 index rows are 128 wide: thread = (row, 32-element block)");
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2][64 * LROW];
    __shared__ int32_t s_qs[kTiledQ];
    __shared__ int64_t s_qnv[kTiledQ];
    __shared__ int32_t s_pg[kChunk / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, h2 = lane >> 5;
    const int blk = blockIdx.x;
    const int64_t c0 = (int64_t)blk * kChunk;
    const int q0 = blockIdx.y * kTiledQ;
    if (tid < kTiledQ) {
        const int n = q0 + tid;
        int s = -1;
        int64_t p = 0, nv = 0;
        if (n < a.num_q) {
            if (query_ok(a, n, s, p)) {
                nv = visible(a, p);
            } else {
                if (blk == 0) raise_error(a.err, (s < 0 || s >= a.num_seqs) ? kErrSeq : kErrPos);
                s = -1;
            }
        }
        s_qs[tid] = s;
        s_qnv[tid] = nv;
    }
    __syncthreads();

    // A operands of the wave's query pairs: row r32 = query 2pp + r32/16, head
    // r32 % 16 (rows beyond n_heads or of invalid queries are zero); dims
    // 16 ks + 8 h2 .. +7.  Head weights of the lane's accumulator rows: value
    // 4j + i of the 32x32 accumulator is row 8j + 4 h2 + i.
    bf16x8 qa[PP][KS];
    float wv[PP][16];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
        const int qi = QW * wave + 2 * pp + (r32 >> 4);
        const int n = q0 + qi;
        const bool qv = n < a.num_q && s_qs[qi] >= 0;
        const int nn = qv ? n : 0;
        const int hd = r32 & 15;
        const bool hv = qv && hd < a.n_heads;
        const uint16_t* qrow = a.q_idx + ((int64_t)nn * a.n_heads + (hd < a.n_heads ? hd : 0)) * DI;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h2);
            if (!hv) v = u32x4{0u, 0u, 0u, 0u};
            qa[pp][ks] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * j + 4 * h2 + i;  // query 2pp + row/16, head row % 16
                const int qj = QW * wave + 2 * pp + (row >> 4);
                const int nj = q0 + qj;
                const int h = row & 15;
                const bool ok = nj < a.num_q && s_qs[qj] >= 0 && h < a.n_heads;
                const float x = a.w[(int64_t)(ok ? nj : 0) * a.n_heads + (ok ? h : 0)];
                wv[pp][4 * j + i] = ok ? x : 0.f;
            }
    }
    int64_t nvl[PP];  // visible entries of the query this lane stores, per pair
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) nvl[pp] = s_qnv[QW * wave + 2 * pp + h2];

    uint32_t done = 0;  // queries handled (the same in every thread)
    for (;;) {
        // the next sequence: the first query not handled whose visible range reaches this chunk
        int sg = -1;
        int64_t nvmax = 0;
        uint32_t gmask = 0;
        for (int i = 0; i < kTiledQ; ++i) {
            if ((done >> i) & 1u) continue;
            const int si = s_qs[i];
            const int64_t nvi = s_qnv[i];
            if (si < 0 || nvi <= c0) {
                done |= 1u << i;
                continue;
            }
            if (sg < 0) sg = si;
            if (si == sg) {
                gmask |= 1u << i;
                nvmax = nvi > nvmax ? nvi : nvmax;
            }
        }
        if (sg < 0) break;
        done |= gmask;
        const int64_t ce = c0 + kChunk < nvmax ? c0 + kChunk : nvmax;
        const int npages = (int)((ce - c0 + 63) / 64);
        __syncthreads();  // the previous pass's reads of s_pg and s_k are done
        if (tid < npages) s_pg[tid] = page_of(a.bt, a.max_blocks, a.num_pages, sg, (c0 + 64 * tid) * 4);
        __syncthreads();
        const int32_t pgl = lane < npages ? s_pg[lane] : -1;  // lane j: page j of the pass (read with readlane)
        u32x4 st[2][LPT];
        uint32_t st_e8[2] = {0u, 0u};  // fp4: the scale byte of the thread's block
        auto load_page = [&](int j, int b) {
            const int32_t pg = __builtin_amdgcn_readlane(pgl, j);
            if constexpr (FP4) {
                // thread = (row tid / 4, 32-element block tid % 4)
                const uint8_t* r = a.rows + (int64_t)(pg < 0 ? 0 : pg) * UNIT + (tid >> 2) * RBG;
                st[b][0] = load16_a4(r + 16 * (tid & 3));
                st_e8[b] = r[DI / 2 + (tid & 3)];
            } else {
                const u32x4* base = reinterpret_cast<const u32x4*>(a.rows + (int64_t)(pg < 0 ? 0 : pg) * UNIT);
#pragma unroll
                for (int q = 0; q < LPT; ++q) st[b][q] = base[q * 256 + tid];
            }
        };
        auto store_page = [&](int lb, int b) {
            if constexpr (FP4) {
                uint32_t w[16];
                mxfp4_to_bf16(st[b][0], st_e8[b], w);
                uint8_t* dst = s_k[lb] + (tid >> 2) * LROW + 64 * (tid & 3);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4*>(dst + 16 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            } else {
#pragma unroll
                for (int q = 0; q < LPT; ++q) {
                    const int c = q * 256 + tid;  // 16-byte chunk of the page
                    *reinterpret_cast<u32x4*>(s_k[lb] + (c / CPR) * LROW + (c % CPR) * 16) = st[b][q];
                }
            }
        };
        load_page(0, 0);
        if (npages > 1) load_page(1, 1);
        store_page(0, 0);
        __syncthreads();
        // page j: registers st[j & 1] then LDS s_k[j & 1]; two pages' loads in flight
        auto body = [&](int j, int b) {
            if (j + 2 < npages) load_page(j + 2, b);
            const uint8_t* sk = s_k[b];
            const int64_t e0 = c0 + 64 * j;
            const int32_t pg = __builtin_amdgcn_readlane(pgl, j);
            if (pg < 0 && lane == 0 && ((gmask >> (QW * wave)) & ((1u << QW) - 1u))) raise_error(a.err, kErrPage);
            float mine[PP][2];  // the lane's score: query 2pp + h2, entry e0 + 32 t + r32
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x16 acc[PP];
#pragma unroll
                for (int pp = 0; pp < PP; ++pp)
#pragma unroll
                    for (int c = 0; c < 16; ++c) acc[pp][c] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 kb =
                        *reinterpret_cast<const bf16x8*>(sk + (32 * t + r32) * LROW + (16 * ks + 8 * h2) * 2);
#pragma unroll
                    for (int pp = 0; pp < PP; ++pp)
                        acc[pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[pp][ks], kb, acc[pp], 0, 0, 0);
                }
#pragma unroll
                for (int pp = 0; pp < PP; ++pp) {
                    float va = 0.f, vb = 0.f;  // the pair's first and second query
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        va = fmaf(wv[pp][c], __builtin_amdgcn_fmed3f(acc[pp][c], 0.f, FLT_MAX), va);
                        vb = fmaf(wv[pp][8 + c], __builtin_amdgcn_fmed3f(acc[pp][8 + c], 0.f, FLT_MAX), vb);
                    }
                    va = sum_xor32(va);
                    vb = sum_xor32(vb);
                    mine[pp][t] = h2 == 0 ? va : vb;
                }
            }
            // the next page into LDS before this page's scores go out: its wait for the page's
            // loads (a count of outstanding memory operations) then does not include the stores
            if (j + 1 < npages) store_page(b ^ 1, b ^ 1);
#pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
                const int qi = QW * wave + 2 * pp + h2;
                const bool store = (gmask >> qi) & 1u;
                float* row = a.scores + (int64_t)(q0 + qi) * a.stride + e0 + r32;
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (store && e0 + 32 * t + r32 < nvl[pp])
                        __builtin_nontemporal_store(pg < 0 ? -INFINITY : mine[pp][t], row + 32 * t);
            }
            __syncthreads();
        };
        for (int j = 0; j < npages; j += 2) {
            body(j, 0);
            if (j + 1 < npages) body(j + 1, 1);
        }
    }
}

// Stage 2: one NT-thread workgroup per query (merge_candidates, 8*NT
// candidate slots), the full select on the score row when the candidates do
// not decide the result.
template <int NT>
__device__ __forceinline__ void merge_query(const IndexArgs& a, const int n) {
    constexpr int NW = NT / 64;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
    __shared__ uint32_t s_cand[kCandCap];
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_sel[8 + NW];
    __shared__ float s_min[NW];
    __shared__ uint32_t s_fail;
    int s;
    int64_t p;
    MergeIn in;
    in.nv = query_ok(a, n, s, p) ? visible(a, p) : 0;
    in.sc = a.scores + (int64_t)n * a.stride;
    in.cand = a.cand + (int64_t)n * a.nchunks * a.kl;
    in.cnext = a.c_next + (int64_t)n * a.nchunks;
    in.kl = a.kl;
    in.k = a.k;
    const MergeLds m = {s_hist, s_cand, s_wave, s_sel, s_min, &s_fail};
    CandRegs<kMergeSlots> cr;
    if (in.nv > in.k) {
        const int nch = (int)((in.nv + kChunk - 1) / kChunk);
        cand_load(in, (int64_t)nch * in.kl, nch, cr);
    }
    merge_candidates<NT, kMergeSlots, false>(in, cr, GlobalOut{a.topk + (int64_t)n * a.k}, a.kth ? a.kth + n : nullptr,
                                             m);
}

// The 256-thread merge serves calls with many queries (a prefill chunk: one
// workgroup per query): the compiler is held to six waves per SIMD instead of
// the four its register use allows, at the price of some spills (0.050 -> 0.040
// ms on an 8192-query chunk).
template <int NT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 ? 6 : 1, 8)))
topk_merge_kernel(IndexArgs a) {
    merge_query<NT>(a, blockIdx.x);
}

// The select with the inserts of the same step in its grid: workgroups past
// num_q each insert one (new token, pool) with their first 256 threads (the
// other waves end at once; a barrier waits only for the waves still running).
// The select reads only the score workspace, so the inserts cannot change
// what the queries select, and they fill the CUs that the few select
// workgroups leave idle.  MERGE: the two-stage merge, else the full select.
template <int NT, bool MERGE>
__global__ void __launch_bounds__(NT) topk_select_insert_kernel(IndexArgs a, CompressArgs c, QSideArgs q) {
    if ((int)blockIdx.x >= a.num_q) {
        if (threadIdx.x >= 256) return;
        const int64_t i = (int64_t)blockIdx.x - a.num_q, n_ins = (int64_t)c.total_new * c.n_jobs;
        if (i < n_ins) {
            __shared__ InsertSmem sm;
            insert_block(c, (int)(i / c.total_new), (int)(i % c.total_new), sm);
        } else {
            qside_block<1>(q, i - n_ins);  // one row per wave: decode-sized batches
        }
        return;
    }
    if constexpr (MERGE) merge_query<NT>(a, blockIdx.x);
    else select_query(a, blockIdx.x);
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0) return hipSuccess;
    if (a.tiled) {
        constexpr int QW = kTiledQW;
        dim3 grid((unsigned)(a.stride / kChunk), (unsigned)((a.num_q + 4 * QW - 1) / (4 * QW)));
        if (a.fp4) {
            if (a.dim != 128) return hipErrorInvalidValue;
            launch_kernel(ev, true, true, index_score_tiled_kernel<128, QW, true>, grid, dim3(256), st, a);
            return hipGetLastError();
        }
        switch (a.dim) {
            case 32: launch_kernel(ev, true, true, index_score_tiled_kernel<32, QW>, grid, dim3(256), st, a); break;
            case 64: launch_kernel(ev, true, true, index_score_tiled_kernel<64, QW>, grid, dim3(256), st, a); break;
            case 128: launch_kernel(ev, true, true, index_score_tiled_kernel<128, QW>, grid, dim3(256), st, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    constexpr int U = kScoreUnits;
    dim3 grid((unsigned)(a.stride / (256 * U)), (unsigned)a.num_q);
    const bool local = a.kl > 0;
    if (a.fp4) {
        if (a.dim != 128) return hipErrorInvalidValue;
        if (local) launch_kernel(ev, true, true, index_score_kernel<128, U, true, true>, grid, dim3(256), st, a);
        else launch_kernel(ev, true, true, index_score_kernel<128, U, false, true>, grid, dim3(256), st, a);
        return hipGetLastError();
    }
    switch (a.dim) {
        case 32:
            if (local) launch_kernel(ev, true, true, index_score_kernel<32, U, true>, grid, dim3(256), st, a);
            else launch_kernel(ev, true, true, index_score_kernel<32, U, false>, grid, dim3(256), st, a);
            break;
        case 64:
            if (local) launch_kernel(ev, true, true, index_score_kernel<64, U, true>, grid, dim3(256), st, a);
            else launch_kernel(ev, true, true, index_score_kernel<64, U, false>, grid, dim3(256), st, a);
            break;
        case 128:
            if (local) launch_kernel(ev, true, true, index_score_kernel<128, U, true>, grid, dim3(256), st, a);
            else launch_kernel(ev, true, true, index_score_kernel<128, U, false>, grid, dim3(256), st, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The decode score kernel with the step's inserts and query-side rows as
// extra grid rows (launch_index_score's decode path otherwise).
template <int DI, bool LOCAL, bool FP4>
void launch_score_insert(const IndexArgs& a, const CompressArgs& c, const QSideArgs& q, dim3 grid, hipStream_t st,
                         const LaunchEvents& ev) {
    launch_kernel(ev, true, true, index_score_insert_kernel<DI, kScoreUnits, LOCAL, FP4>, grid, dim3(256), st, a, c, q);
}

hipError_t launch_index_score_insert(const IndexArgs& a, const CompressArgs& c, const QSideArgs& q, hipStream_t st,
                                     const LaunchEvents& ev) {
    const int64_t n_ins = (int64_t)c.total_new * c.n_jobs;
    const int64_t n_qb = q.n_items > 0 ? (q.n_items + 3) / 4 : 0;
    if (a.num_q <= 0 || a.tiled || n_ins + n_qb <= 0) {
        // nothing rides along (or the query-blocked kernel scores): separate launches
        hipError_t e = launch_index_score(a, st, ev);
        if (e == hipSuccess) e = launch_compress(c, st);
        if (e == hipSuccess) e = launch_qside(q, st);
        return e;
    }
    const int64_t gx = a.stride / (256 * kScoreUnits);
    const int64_t rows = (n_ins + n_qb + gx - 1) / gx;
    if (a.num_q + rows > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)(a.num_q + rows));
    const bool local = a.kl > 0;
    if (a.fp4) {
        if (a.dim != 128) return hipErrorInvalidValue;
        if (local) launch_score_insert<128, true, true>(a, c, q, grid, st, ev);
        else launch_score_insert<128, false, true>(a, c, q, grid, st, ev);
        return hipGetLastError();
    }
    switch (a.dim) {
        case 32:
            if (local) launch_score_insert<32, true, false>(a, c, q, grid, st, ev);
            else launch_score_insert<32, false, false>(a, c, q, grid, st, ev);
            break;
        case 64:
            if (local) launch_score_insert<64, true, false>(a, c, q, grid, st, ev);
            else launch_score_insert<64, false, false>(a, c, q, grid, st, ev);
            break;
        case 128:
            if (local) launch_score_insert<128, true, false>(a, c, q, grid, st, ev);
            else launch_score_insert<128, false, false>(a, c, q, grid, st, ev);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// With a first stage (kl > 0): the decode score kernel has already written each
// chunk's candidates (the tiled one has not: the stand-alone first stage runs),
// then the merge; otherwise one full select per query.
hipError_t launch_topk_select(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.num_q <= 0) return hipSuccess;
    if (a.kl > 0) {
        if (a.tiled)
            launch_kernel(ev, true, false, topk_local_kernel, dim3((unsigned)((a.nchunks + 3) / 4), (unsigned)a.num_q),
                          dim3(256), st, a);
        if ((int64_t)a.nchunks * a.kl <= (int64_t)kMergeSlots * 256)
            launch_kernel(ev, !a.tiled, true, topk_merge_kernel<256>, dim3((unsigned)a.num_q), dim3(256), st, a);
        else if ((int64_t)a.nchunks * a.kl <= (int64_t)kMergeSlots * 512)
            launch_kernel(ev, !a.tiled, true, topk_merge_kernel<512>, dim3((unsigned)a.num_q), dim3(512), st, a);
        else
            launch_kernel(ev, !a.tiled, true, topk_merge_kernel<kSelThreads>, dim3((unsigned)a.num_q),
                          dim3(kSelThreads), st, a);
    } else {
        launch_kernel(ev, true, true, topk_select_kernel, dim3((unsigned)a.num_q), dim3(kSelThreads), st, a);
    }
    return hipGetLastError();
}

// The select with the inserts and the query-side rows riding in its last
// launch (one workgroup per token and pool, then one per four query-side rows,
// after the queries' workgroups).
hipError_t launch_topk_select_insert(const IndexArgs& a, const CompressArgs& c, const QSideArgs& q, hipStream_t st,
                                     const LaunchEvents& ev) {
    const int64_t n_ins = (int64_t)c.total_new * c.n_jobs;
    const int64_t n_qb = q.n_items > 0 ? (q.n_items + 3) / 4 : 0;
    if (a.num_q <= 0 || n_ins + n_qb <= 0 || a.num_q + n_ins + n_qb > 0x7fffffff) {
        hipError_t e = launch_topk_select(a, st, ev);
        if (e == hipSuccess) e = launch_compress(c, st);
        if (e == hipSuccess) e = launch_qside(q, st);
        return e;
    }
    const dim3 grid((unsigned)(a.num_q + n_ins + n_qb));
    if (a.kl > 0) {
        if (a.tiled)
            launch_kernel(ev, true, false, topk_local_kernel, dim3((unsigned)((a.nchunks + 3) / 4), (unsigned)a.num_q),
                          dim3(256), st, a);
        if ((int64_t)a.nchunks * a.kl <= (int64_t)kMergeSlots * 256)
            launch_kernel(ev, !a.tiled, true, topk_select_insert_kernel<256, true>, grid, dim3(256), st, a, c, q);
        else if ((int64_t)a.nchunks * a.kl <= (int64_t)kMergeSlots * 512)
            launch_kernel(ev, !a.tiled, true, topk_select_insert_kernel<512, true>, grid, dim3(512), st, a, c, q);
        else
            launch_kernel(ev, !a.tiled, true, topk_select_insert_kernel<kSelThreads, true>, grid, dim3(kSelThreads), st,
                          a, c, q);
    } else {
        launch_kernel(ev, true, true, topk_select_insert_kernel<kSelThreads, false>, grid, dim3(kSelThreads), st, a, c,
                      q);
    }
    return hipGetLastError();
}

bool index_use_tiled(int num_q) { return num_q >= kTiledMinQueries; }

}  // namespace csl
