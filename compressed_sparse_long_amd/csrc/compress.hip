// Step 1 on gfx950: token-axis compressor + RMSNorm + RoPE + paged insert,
// one fused kernel ([Notes] 融合 1：Compressor + RMSNorm + RoPE + Cache Insert;
// windows from [Notes] 数学附录精要: C4A / C128A 的精确位置范围), plus the
// raw-window insert (ratio 1: RoPE at the token, no norm; [Notes] 融合 3).
//
// Work mapping.  Several pools of a layer (raw window, c4a main, c4a index,
// c128a main) are filled by one launch: grid.y picks the pool (job), grid.x
// the new token -- the horizontal fusion of independent per-pool work.  One
// 256-thread workgroup per (token, pool).  For ratio > 1, wave 0 appends the
// token to the compressor state; if the token closes an entry, the four waves
// split the window's tokens, the weighted partial sums meet in LDS and wave 0
// normalises, rotates and stores the row.  For ratio 1, wave 0 rotates and
// stores the token's row.  A lane owns 8 consecutive dims (one 16-byte
// load/store per row), so a wave covers a row of up to 512 dims and RoPE pairs
// never straddle lanes.  Elementwise and HBM-bound: no MFMA.
#include "csl_insert.hpp"

namespace csl {

namespace {

__global__ void __launch_bounds__(kThreads) compress_insert_kernel(CompressArgs args) {
    __shared__ InsertSmem sm;
    insert_block(args, blockIdx.y, blockIdx.x, sm);
}

// ---------------------------------------------------------------- query side

// Sequence s of new token j and its position t = start_pos[s] + (j - cu[s]).
// Lane i reads (cu[i], cu[i+1], start_pos[i]) for 64 sequences per step, all in
// one round of loads; the lane whose range holds j is found by ballot and its
// values are broadcast.  Wave-uniform.  A j outside every range (cu not
// covering it) gives the last sequence.
__device__ __forceinline__ void token_seq_pos(const int32_t* __restrict__ cu, const int64_t* __restrict__ start,
                                              int num_seqs, int j, int& s_out, int64_t& t_out) {
    const int lane = threadIdx.x & 63;
    for (int b = 0; b < num_seqs; b += 64) {
        const int i = b + lane;
        int lo = 0, hi = 0;
        int64_t st = 0;
        if (i < num_seqs) {
            lo = cu[i];
            hi = cu[i + 1];
            st = start[i];
        }
        const uint64_t m = __ballot(i < num_seqs && lo <= j && j < hi);
        if (m) {
            const int l = __ffsll((unsigned long long)m) - 1;
            const uint32_t st_lo = lane_value((uint32_t)st, l), st_hi = lane_value((uint32_t)(st >> 32), l);
            s_out = b + l;
            t_out = (int64_t)(((uint64_t)st_hi << 32) | st_lo) + (j - (int)lane_value((uint32_t)lo, l));
            return;
        }
    }
    s_out = num_seqs - 1;
    t_out = start[s_out] + (j - cu[s_out]);
}

// The step before attention ([Notes] 融合 3：Q Norm + KV RoPE + K Insert;
// [Summary] Kernel 融合): every query head of a new token is RMS-normed and
// rotated at the token's position, and the token's raw key is rotated and
// inserted into the ratio-1 pool.  Work items are the flattened rows
// [total_new*n_heads Q rows | total_new K rows]; wave w of workgroup b owns the
// kQItems consecutive items from (4b + w) * kQItems and branches per item on
// its kind, with no communication between waves (the pages' one-warp-per-head
// dispatch).  A wave issues the loads of all its items first, so each lane has
// kQItems 16-byte reads in flight.  When the token changes (the Q rows of a
// token are consecutive) the wave finds its position and each of the first
// R/2 lanes takes the cos/sin of one rotated pair, which the lanes holding
// the rotated dims then read across the wave.  q_out is written with
// non-temporal stores (it is read by a later kernel, not this one).
// HBM-bound: read q and x, write q_out and the key row.  ITEMS trades latency
// (short per-wave chains for a few tokens) against bytes in flight per wave.
template <int kQItems>
__global__ void __launch_bounds__(kThreads) q_norm_rope_insert_kernel(QSideArgs a) {
    // the wave index through readfirstlane: item indices, kinds and row bases are scalar
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = a.dim;
    const bool active = lane * 8 < D;
    const int64_t g0 = ((int64_t)blockIdx.x * 4 + wave) * kQItems;
    if (g0 >= a.n_items) return;

    u32x4 raw[kQItems];  // bf16 pairs, unpacked when the item is processed
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
        const int64_t g = g0 + u;
        raw[u] = u32x4{0, 0, 0, 0};
        if (g < a.n_items && active) {
            const uint16_t* src = g < a.n_q_rows ? a.q + g * D : a.x + (g - a.n_q_rows) * D;
            raw[u] = *reinterpret_cast<const u32x4*>(src + 8 * lane);
        }
    }
    float gn[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) gn[c] = (a.gain && active) ? a.gain[8 * lane + c] : 1.0f;

    const int base = D - a.rope_dims;
    int64_t cur_j = -1, t = 0;
    int cur_s = 0;
    float cs[4], sn[4];
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
        const int64_t g = g0 + u;
        if (g >= a.n_items) break;  // wave-uniform
        const bool is_q = g < a.n_q_rows;
        const int64_t j = is_q ? g / a.n_heads : g - a.n_q_rows;
        if (j != cur_j) {  // wave-uniform: the token's position and its rotation
            cur_j = j;
            token_seq_pos(a.cu_new, a.start_pos, a.num_seqs, (int)j, cur_s, t);
            float pc = 1.f, ps = 0.f;
            if (lane < (a.rope_dims >> 1)) rope_cs(t, a.rf.inv_freq[lane], pc, ps);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int d = 8 * lane + 2 * c;
                const bool rot = active && d >= base;
                const int src = rot ? (d - base) >> 1 : 0;
                const float c0 = __shfl(pc, src), s0 = __shfl(ps, src);
                cs[c] = rot ? c0 : 1.f;
                sn[c] = rot ? s0 : 0.f;
            }
        }
        float w[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            w[2 * c] = __uint_as_float(raw[u][c] << 16);
            w[2 * c + 1] = __uint_as_float(raw[u][c] & 0xffff0000u);
        }
        if (is_q) {
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) ss = fmaf(w[c], w[c], ss);
            ss = wave_allsum(ss);
            const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
            for (int c = 0; c < 8; ++c) w[c] = w[c] * inv * gn[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float x0 = w[2 * c], x1 = w[2 * c + 1];
            w[2 * c] = x0 * cs[c] - x1 * sn[c];
            w[2 * c + 1] = x0 * sn[c] + x1 * cs[c];
        }
        if (is_q) {
            if (active) {
                u32x4 o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(w[2 * c], w[2 * c + 1]);
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.q_out + g * D + 8 * lane));
            }
        } else {
            const int32_t pg = page_of(a.bt, a.max_blocks, a.num_pages, cur_s, t);
            if (pg < 0) {
                if (lane == 0) raise_error(a.err, (t < 0 || (t >> 8) >= a.max_blocks) ? kErrPos : kErrPage);
                continue;
            }
            uint8_t* row = a.rows + ((int64_t)pg * kBlockPositions + (t & 255)) * a.row_bytes;
            store8(row, a.dtype, D, lane, active, w);
        }
    }
}

}  // namespace

constexpr int64_t kQSideBig = 16384, kQSideMid = 4096;

// Rows per wave: 4 once the launch has enough rows to keep every SIMD busy
// at 4 per wave, else fewer rows per wave and more waves.
int qside_items(int64_t n_items) { return n_items >= kQSideBig ? 4 : (n_items >= kQSideMid ? 2 : 1); }

hipError_t launch_qside(const QSideArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.n_items <= 0) return hipSuccess;
    const int items = qside_items(a.n_items);
    const int64_t waves = (a.n_items + items - 1) / items;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (items == 4) launch_kernel(ev, true, true, q_norm_rope_insert_kernel<4>, grid, dim3(kThreads), st, a);
    else if (items == 2) launch_kernel(ev, true, true, q_norm_rope_insert_kernel<2>, grid, dim3(kThreads), st, a);
    else launch_kernel(ev, true, true, q_norm_rope_insert_kernel<1>, grid, dim3(kThreads), st, a);
    return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st, const LaunchEvents& ev) {
    if (a.total_new <= 0 || a.n_jobs <= 0) return hipSuccess;
    launch_kernel(ev, true, true, compress_insert_kernel, dim3((unsigned)a.total_new, (unsigned)a.n_jobs),
                  dim3(kThreads), st, a);
    return hipGetLastError();
}

}  // namespace csl
