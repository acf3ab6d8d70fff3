// The insert of one new token into one pool (the ratio-1 raw-window row, or the
// compressor state and any entry the token closes), and the query-side rows
// (per-head Q norm + RoPE, raw-key RoPE + insert), shared by their stand-alone
// launches and the top-k launch that carries them beside its select.
// Pages: [Notes] 融合 1：Compressor + RMSNorm + RoPE + Cache Insert; windows
// from [Notes] 数学附录精要: C4A / C128A 的精确位置范围; raw rows per [Notes]
// 融合 3.  See compress.hip for the work mapping.
#pragma once
#include "csl_kernels.hpp"

namespace csl {
namespace {

constexpr int kThreads = 256;

// Sequence s with cu[s] <= j < cu[s+1]: the wave reads 64 boundaries per step
// in parallel and counts the ones <= j (cu is non-decreasing).  Wave-uniform.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int num_seqs, int j) {
    const int lane = threadIdx.x & 63;
    int s = -1;
    for (int base = 1; base <= num_seqs; base += 64) {
        const int i = base + lane;
        const bool le = i <= num_seqs && cu[i] <= j;
        s += (int)__popcll(__ballot(le));
        if (!__ballot(i <= num_seqs && !le)) continue;
        break;
    }
    s += 1;
    return s < num_seqs ? s : num_seqs - 1;
}

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        v[2 * c] = __uint_as_float(r[c] << 16);
        v[2 * c + 1] = __uint_as_float(r[c] & 0xffff0000u);
    }
}

// Rotate the lane's 8 dims [d0, d0+8) at position `pos` (pairs in the last R dims).
// `active` = the lane owns dims (d0 < dim): a lane past the row rotates nothing,
// so every frequency index stays below rope_dims / 2.
__device__ __forceinline__ void rope8(float* v, int d0, int dim, int rope_dims, const RopeFreqs& rf, int64_t pos,
                                      bool active) {
    int base = dim - rope_dims;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        int d = d0 + 2 * c;
        if (active && d >= base) {
            float cs, sn;
            rope_cs(pos, rf.inv_freq[(d - base) >> 1], cs, sn);
            float a = v[2 * c], b = v[2 * c + 1];
            v[2 * c] = a * cs - b * sn;
            v[2 * c + 1] = a * sn + b * cs;
        }
    }
}

// Store the lane's 8 values of a row; every lane of the wave must call this
// (fp8 reduces the group amax across 8 lanes, fp4 the block max across 4).  `active` = lane owns dims.
__device__ __forceinline__ void store8(uint8_t* row, int dtype, int dim, int lane, bool active, const float* v) {
    if (dtype == kBF16) {
        if (active) {
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(v[2 * c], v[2 * c + 1]);
            *reinterpret_cast<u32x4*>(row + 16 * lane) = o;
        }
        return;
    }
    if (dtype == kFP4) {
        // MXFP4: the 32-element block is 4 lanes.  Scale 2^(floor(log2 amax) - 2)
        // as an E8M0 byte; each element scaled by a power of two (exact) and
        // rounded to E2M1 by counting the midpoints it passes (a tie sits at
        // the even code: strict at 0.25, 1.25, 2.5, 5; inclusive at 0.75,
        // 1.75, 3.5), saturating at 6.
        float bmax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) bmax = fmaxf(bmax, fabsf(v[c]));
        bmax = active ? bmax : 0.f;
        bmax = fmaxf(bmax, __shfl_xor(bmax, 1));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 2));
        int sh = bmax > 0.f ? __builtin_amdgcn_frexp_expf(bmax) - 3 : -127;
        sh = sh < -127 ? -127 : (sh > 127 ? 127 : sh);
        if (active) {
            uint32_t word = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float q = __builtin_amdgcn_ldexpf(v[c], -sh);
                const float r = fabsf(q);
                const uint32_t code = (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) +
                                      (uint32_t)(r >= 1.75f) + (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) +
                                      (uint32_t)(r > 5.0f);
                word |= (code | ((__float_as_uint(q) >> 28) & 8u)) << (4 * c);
            }
            *reinterpret_cast<uint32_t*>(row + 4 * lane) = word;
            if ((lane & 3) == 0) row[dim / 2 + (lane >> 2)] = (uint8_t)(sh + 127);
        }
        return;
    }
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[c]));
    amax = group8_max(active ? amax : 0.f);
    float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    if (active) {
        const float r = 1.0f / scale;
        const u32x2 o = {e4m3_pack4(v[0] * r, v[1] * r, v[2] * r, v[3] * r),
                         e4m3_pack4(v[4] * r, v[5] * r, v[6] * r, v[7] * r)};
        *reinterpret_cast<u32x2*>(row + 8 * lane) = o;
        if ((lane & 7) == 0) *reinterpret_cast<float*>(row + dim + 4 * (lane >> 3)) = scale;
    }
}

// LDS of one insert workgroup.
struct InsertSmem {
    float w[kThreads];
    const uint16_t* ptr[kThreads];
    float red[4][512];
    float tmp[8];
};

// Token j of job `jb` (one 256-thread workgroup): the whole insert of that
// token into that pool.  Every thread of the workgroup calls it.
__device__ __forceinline__ void insert_block(const CompressArgs& args, int jb, int j, InsertSmem& sm) {
    const CompressJob& a = args.job[jb];
    const RopeFreqs& rf = args.rf[jb];
    float* s_w = sm.w;
    const uint16_t** s_ptr = sm.ptr;
    float (*s_red)[512] = sm.red;
    float* s_tmp = sm.tmp;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.dim;
    const bool active = lane * 8 < D;

    if (a.ratio == 1) {
        if (wave != 0) return;
        int s = find_seq(args.cu_new, args.num_seqs, j);
        int64_t t = args.start_pos[s] + (j - args.cu_new[s]);
        int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, t);
        if (pg < 0) {
            if (lane == 0) raise_error(args.err, (t < 0 || (t >> 8) >= args.max_blocks) ? kErrPos : kErrPage);
            return;
        }
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (active) load8(a.x + (int64_t)j * D + 8 * lane, v);
        rope8(v, 8 * lane, D, a.rope_dims, rf, t, active);
        uint8_t* row = a.rows + ((int64_t)pg * kBlockPositions + (t & 255)) * a.row_bytes;
        store8(row, a.dtype, D, lane, active, v);
        return;
    }

    const int s = find_seq(args.cu_new, args.num_seqs, j);
    const int64_t start = args.start_pos[s];
    const int cbase = args.cu_new[s];
    const int64_t t = start + (j - cbase);
    const int r = a.ratio, W = a.coff * a.ratio;

    // 1. append the token to the compressor state
    if (wave == 0) {
        int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, t);
        if (pg < 0) {
            if (lane == 0) raise_error(args.err, (t < 0 || (t >> 8) >= args.max_blocks) ? kErrPos : kErrPage);
        } else {
            int64_t tok = (int64_t)pg * kBlockPositions + (t & 255);
            if (active)
                *reinterpret_cast<u32x4*>(a.state_x + tok * D + 8 * lane) =
                    *reinterpret_cast<const u32x4*>(a.x + (int64_t)j * D + 8 * lane);
            if (lane < a.coff) a.state_logits[tok * a.coff + lane] = a.logits[(int64_t)j * a.coff + lane];
        }
    }
    if ((t + 1) % r != 0) return;  // uniform across the workgroup
    const int64_t i = (t + 1) / r - 1;

    // 2. window weights: thread k owns window slot k
    float lg = -INFINITY;
    const uint16_t* ptr = nullptr;
    if (tid < W) {
        int64_t tk = (int64_t)r * (i + 1) - W + tid;
        int col = tid / r;
        if (tk >= start) {
            int64_t jj = cbase + (tk - start);
            lg = a.logits[jj * a.coff + col];
            ptr = a.x + jj * D;
        } else if (tk >= 0) {
            int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, tk);
            if (pg < 0) {
                raise_error(args.err, kErrPage);
            } else {
                int64_t tok = (int64_t)pg * kBlockPositions + (tk & 255);
                lg = a.state_logits[tok * a.coff + col];
                ptr = a.state_x + tok * D;
            }
        }
    }
    float m = wave_max(lg);
    if (lane == 0) s_tmp[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_tmp[0], s_tmp[1]), fmaxf(s_tmp[2], s_tmp[3]));
    float e = ptr ? __expf(lg - m) : 0.f;
    float den = wave_sum(e);
    __syncthreads();
    if (lane == 0) s_tmp[4 + wave] = den;
    s_w[tid] = e;
    s_ptr[tid] = ptr;
    __syncthreads();
    den = s_tmp[4] + s_tmp[5] + s_tmp[6] + s_tmp[7];
    const float inv_den = den > 0.f ? 1.0f / den : 0.f;

    // 3. weighted sum: wave w takes window slots w, w+4, w+8, ...
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) {
#pragma unroll 4
        for (int k = wave; k < W; k += 4) {
            const uint16_t* p = s_ptr[k];
            if (!p) continue;
            float wk = s_w[k] * inv_den;
            float v[8];
            load8(p + 8 * lane, v);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = fmaf(wk, v[c], acc[c]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) s_red[wave][8 * lane + c] = acc[c];
    }
    __syncthreads();
    if (wave != 0) return;

    // 4. RMSNorm, RoPE at r*i, store
    float u[8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        int d = 8 * lane + c;
        u[c] = active ? (s_red[0][d] + s_red[1][d]) + (s_red[2][d] + s_red[3][d]) : 0.f;
        ss = fmaf(u[c], u[c], ss);
    }
    ss = wave_sum(ss);
    float inv = 1.0f / sqrtf(ss / (float)D + args.eps);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float g = (a.gain && active) ? a.gain[8 * lane + c] : 1.0f;
        u[c] = u[c] * inv * g;
    }
    rope8(u, 8 * lane, D, a.rope_dims, rf, (int64_t)r * i, active);
    int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, (int64_t)r * i);
    if (pg < 0) {
        if (lane == 0) raise_error(args.err, kErrPage);
        return;
    }
    const int per_page = kBlockPositions / r;
    uint8_t* row = a.rows + ((int64_t)pg * per_page + (i % per_page)) * a.row_bytes;
    store8(row, a.dtype, D, lane, active, u);
}


// Windows of at most this many tokens (raw rows and c4a) are inserted by one wave.
constexpr int kWaveWindow = 64;

// The same insert as insert_block for a pool whose window holds at most
// kWaveWindow tokens, by one wave with no LDS and no barrier, in the same
// arithmetic order (lane k holds window slot k as thread k does there; the
// weighted sum keeps four partial sums over the slots k = w mod 4 and adds
// them as (0 + 1) + (2 + 3)), so the rows are bit-identical.  The token's row
// and logits are requested before its sequence and page are known.
__device__ __forceinline__ void insert_wave(const CompressArgs& args, int jb, int j) {
    const CompressJob& a = args.job[jb];
    const RopeFreqs& rf = args.rf[jb];
    const int lane = threadIdx.x & 63;
    const int D = a.dim;
    const bool active = lane * 8 < D;
    u32x4 xr = {0u, 0u, 0u, 0u};
    if (active) xr = *reinterpret_cast<const u32x4*>(a.x + (int64_t)j * D + 8 * lane);
    const float lgj = a.ratio > 1 && lane < a.coff ? a.logits[(int64_t)j * a.coff + lane] : 0.f;
    const int s = find_seq(args.cu_new, args.num_seqs, j);
    const int64_t start = args.start_pos[s];
    const int cbase = args.cu_new[s];
    const int64_t t = start + (j - cbase);
    const int32_t pgt = page_of(args.bt, args.max_blocks, a.num_pages, s, t);
    if (a.ratio == 1) {
        if (pgt < 0) {
            if (lane == 0) raise_error(args.err, (t < 0 || (t >> 8) >= args.max_blocks) ? kErrPos : kErrPage);
            return;
        }
        float v[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[2 * c] = __uint_as_float(xr[c] << 16);
            v[2 * c + 1] = __uint_as_float(xr[c] & 0xffff0000u);
        }
        rope8(v, 8 * lane, D, a.rope_dims, rf, t, active);
        uint8_t* row = a.rows + ((int64_t)pgt * kBlockPositions + (t & 255)) * a.row_bytes;
        store8(row, a.dtype, D, lane, active, v);
        return;
    }

    // 1. append the token to the compressor state
    if (pgt < 0) {
        if (lane == 0) raise_error(args.err, (t < 0 || (t >> 8) >= args.max_blocks) ? kErrPos : kErrPage);
    } else {
        const int64_t tok = (int64_t)pgt * kBlockPositions + (t & 255);
        if (active) *reinterpret_cast<u32x4*>(a.state_x + tok * D + 8 * lane) = xr;
        if (lane < a.coff) a.state_logits[tok * a.coff + lane] = lgj;
    }
    const int r = a.ratio, W = a.coff * a.ratio;
    if ((t + 1) % r != 0) return;  // uniform across the wave
    const int64_t i = (t + 1) / r - 1;

    // 2. window weights: lane k owns window slot k
    float lg = -INFINITY;
    const uint16_t* ptr = nullptr;
    if (lane < W) {
        const int64_t tk = (int64_t)r * (i + 1) - W + lane;
        const int col = lane / r;
        if (tk >= start) {
            const int64_t jj = cbase + (tk - start);
            lg = a.logits[jj * a.coff + col];
            ptr = a.x + jj * D;
        } else if (tk >= 0) {
            const int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, tk);
            if (pg < 0) {
                raise_error(args.err, kErrPage);
            } else {
                const int64_t tok = (int64_t)pg * kBlockPositions + (tk & 255);
                lg = a.state_logits[tok * a.coff + col];
                ptr = a.state_x + tok * D;
            }
        }
    }
    const float m = wave_max(lg);
    const float e = ptr ? __expf(lg - m) : 0.f;
    const float den = wave_sum(e);
    const float inv_den = den > 0.f ? 1.0f / den : 0.f;

    // 3. weighted sum
    float acc[4][8];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[w][c] = 0.f;
    const uint64_t pv = reinterpret_cast<uint64_t>(ptr);
    for (int k0 = 0; k0 < W; k0 += 4) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int k = k0 + w;
            if (k >= W) break;
            const uint64_t pk = ((uint64_t)lane_value((uint32_t)(pv >> 32), k) << 32) | lane_value((uint32_t)pv, k);
            if (!pk) continue;
            const float wk = __uint_as_float(lane_value(__float_as_uint(e), k)) * inv_den;
            if (active) {
                float v[8];
                load8(reinterpret_cast<const uint16_t*>(pk) + 8 * lane, v);
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[w][c] = fmaf(wk, v[c], acc[w][c]);
            }
        }
    }

    // 4. RMSNorm, RoPE at r*i, store
    float u[8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u[c] = active ? (acc[0][c] + acc[1][c]) + (acc[2][c] + acc[3][c]) : 0.f;
        ss = fmaf(u[c], u[c], ss);
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + args.eps);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float g = (a.gain && active) ? a.gain[8 * lane + c] : 1.0f;
        u[c] = u[c] * inv * g;
    }
    rope8(u, 8 * lane, D, a.rope_dims, rf, (int64_t)r * i, active);
    const int32_t pg = page_of(args.bt, args.max_blocks, a.num_pages, s, (int64_t)r * i);
    if (pg < 0) {
        if (lane == 0) raise_error(args.err, kErrPage);
        return;
    }
    const int per_page = kBlockPositions / r;
    uint8_t* row = a.rows + ((int64_t)pg * per_page + (i % per_page)) * a.row_bytes;
    store8(row, a.dtype, D, lane, active, u);
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
// HBM-bound: read q and x, write q_out and the key row.  kQItems trades latency
// (short per-wave chains for a few tokens) against bytes in flight per wave.
// Workgroup blk (256 threads) of the flattened rows; no barriers.
template <int kQItems>
__device__ __forceinline__ void qside_block(const QSideArgs& a, int64_t blk) {
    // the wave index through readfirstlane: item indices, kinds and row bases are scalar
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = a.dim;
    const bool active = lane * 8 < D;
    const int64_t g0 = (blk * 4 + wave) * kQItems;
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
}  // namespace csl
