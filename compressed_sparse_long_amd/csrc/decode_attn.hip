// Steps 4-6 for decode queries on gfx950, 512-dim bf16 or fp8 keys: hybrid attention
// over (top-k or every visible compressed entry) U raw window [p-S, p-1] with
// one softmax and K = V ([Summary] 共享鍵和值向量, 短滑動窗口; [Notes] ⚠️ 注意：
// C128A 的因果性约束), inverse RoPE at the query position and the output store
// (fp32 / bf16 / fp8 + scales) as the epilogue ([Notes] Inverse RoPE 的数学原理,
// 融合 2：Inverse RoPE + FP8 Quant).  Optionally the launch first merges the
// indexer's first-stage candidates into the top-k ([Summary] DeepSeek V4 注意力
// 架構: DSA), so that index scores -> top-k -> attention is two launches.
//
// Why this shape.  A decode step has few queries (16 in the 128K workload),
// each with 640 keys of 1 KiB, and one workgroup gathers random rows at only
// ~85 GB/s, so a query's keys are split over several workgroups.  With all 64
// heads in one workgroup a split's fp32 partial (64 x 512 x 4 B) is larger
// than the keys it read; so a workgroup takes 16 heads (one MFMA column
// block) and a contiguous share of the key list, and its partial is 32 KiB.
// Kernel boundaries and agent-scope fences each cost microseconds here, so
// the splits are merged inside the launch: every split writes its partial
// with device-coherent stores, waits for them, and counts itself in on an
// arrival counter; the last of a (query, head group) reads the others'
// partials with device-coherent loads and finishes the output.  Nothing
// waits on another workgroup.
//
// Work mapping.  Workgroup = (query n, head group hg of 16 heads, split sp of
// `per` keys); the G head groups of one (n, sp) get block indices equal mod 8
// so that their shared key rows meet in one L2.  Wave w owns output dims
// 128w .. 128w+127 and the same slice of every dot product.  32-key tiles
// are staged by direct global->LDS loads in a 4-slot ring (every slot filled
// before the loop) and taken two per pass, one softmax over the pair; per tile:
//   * S^T[32 keys x 16 heads] over the wave's 128 dims on
//     v_mfma_f32_16x16x32_bf16 (A = key rows, LDS; B = the wave's q slice,
//     registers); the four waves' partial sums meet in LDS and every wave
//     adds them in the same order, so all hold the same S;
//   * online softmax per head in the exp2 domain with a lazy reference max
//     (rescale only when the max passes it by more than 8);
//   * O^T[128 dims x 16 heads] += V^T . P^T: B = P straight from the S
//     accumulator, A = V^T by transposing LDS reads (ds_read_b64_tr_b16) of
//     the row-major tile.  Accumulator row a of S^T m-tile mt holds the key
//     in LDS row 16 mt + 4 (a % 4) + a / 4 of the tile, which is the key
//     order the transposed reads produce, and keeps both the S operand reads
//     and the transposed reads free of bank conflicts (1040-byte rows).
// fp8 keys (544-byte rows: 512 e4m3 codes, then one fp32 scale per 64-dim
// group) are staged as stored, six slots deep, and widened to their exact
// bf16 values on the way to the MFMAs (the conversion unit with scale 1); the
// V^T operands come from 8-bit transposing reads.  S runs one MFMA chain per
// 64-dim group and adds the chains times the keys' group scales in fp32; in
// P.V the group scale of each key moves onto P, so V needs no rounding.
#include "csl_insert.hpp"
#include "csl_select.hpp"

namespace csl {

namespace {

constexpr int kDT = 256;           // threads per workgroup (4 waves)
constexpr int kDTile = 32;         // keys per tile
constexpr int kDRow = 1040;        // LDS stride of a staged 1 KiB row (260 words: 4 banks apart)
constexpr int kDRing = 4;          // ring slots: one computed, up to three in flight
// fp8 keys: 544-byte rows (512 e4m3 codes, then the 8 fp32 scales of the 64-dim groups)
constexpr int kDRowBytes8 = 544;
constexpr int kDRow8 = 560;        // LDS stride of a staged fp8 row (140 words)
constexpr int kDRing8 = 6;         // ring slots for fp8 rows: one computed, up to five in flight
constexpr int kDBt = 2048;         // block-table entries staged in LDS (contexts up to 512K positions)
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer descriptor word 3 (untyped dword access)
constexpr int kSc1 = 16;                      // cache policy: device scope (coherent across the XCDs' L2s)

// Source of masked key rows (zeros) and of q rows of heads past n_heads.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row512[1024];

__device__ __forceinline__ void dma_row(uint32_t lds, const uint8_t* src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)p);
}

// eight e4m3 codes (bytes of w, in order) to their exact bf16 values
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
    return __builtin_bit_cast(bf16x8, o);
}

// transposing 8-bit LDS read: in each 16-lane group, lane j receives byte j % 8 of the
// 8-byte words read by lanes 2c + j / 8 (c = 0..7) of the group
typedef int int2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 tr8_read(const uint8_t* p) {
    const int2v v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2v*)(const_cast<uint8_t*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// tiles of n 8-load issues each may stay in flight (n <= 6)
__device__ __forceinline__ void wait_tiles(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    }
}

typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 tr_read(const uint8_t* p) {
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(const_cast<uint8_t*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Writes the merged top-k: every position to the global row (when this
// workgroup is the writer) and positions [lo, lo + cnt) to the workgroup's LDS slice.
struct SliceOut {
    int32_t* g;
    int32_t* lds;
    uint32_t lo, cnt;
    __device__ __forceinline__ void operator()(uint32_t pos, int32_t id) const {
        if (g) g[pos] = id;
        if (pos - lo < cnt) lds[pos - lo] = id;
    }
};

// Workgroups past the attention's take one (new token, pool) insert each of
// `c` (the fused call's index-pool inserts: this launch never reads index rows).
// MERGE: 0 = ids given (or dense); 1 = the workgroup merges the first-stage
// candidates, 8 slots per thread (up to kDecodeMergeSlots).
template <bool PREC, int MERGE, bool KV8>
__global__ void __launch_bounds__(kDT) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_attn_kernel(DecodeArgs d, CompressArgs c) {
    constexpr int D = 512;
    constexpr int ROW = KV8 ? kDRow8 : kDRow;           // LDS stride of a staged row
    constexpr int RING = KV8 ? kDRing8 : kDRing;        // ring slots
    constexpr int RB = KV8 ? kDRowBytes8 : 2 * D;       // stored row bytes
    constexpr int KMAX = kDecodeMaxSplitKeys;           // keys of one split
    constexpr int KR = (KMAX + kDT - 1) / kDT;          // rounds of address resolution (one thread per key)
    constexpr int kBtPer = kDBt / kDT;  // block-table entries staged per thread
    const AttnArgs& a = d.at;
    // ring of staged key tiles; before the first tile it holds the merge's
    // scratch, after the last one the epilogue's staging
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[RING * kDTile * ROW];
    static_assert(sizeof(InsertSmem) <= sizeof(s_ring), "the insert body fits the ring");
    const int64_t n_attn = ((int64_t)a.num_q * d.S + 7) / 8 * 8 * d.G;
    if ((int64_t)blockIdx.x >= n_attn) {
        const int64_t i = (int64_t)blockIdx.x - n_attn;
        if (i < (int64_t)c.total_new * c.n_jobs)
            insert_block(c, (int)(i / c.total_new), (int)(i % c.total_new), *reinterpret_cast<InsertSmem*>(s_ring));
        return;
    }
    __shared__ __attribute__((aligned(16))) f32x4 s_sx[2][4][2][64];  // S^T partials: [tile of the pair][wave][m-tile]
    __shared__ const uint8_t* s_rows[KMAX];
    __shared__ uint32_t s_vbits[KMAX / 32];
    __shared__ int32_t s_ids[MERGE ? KMAX : 1];
    __shared__ int32_t s_bt[kDBt];
    __shared__ float s_rope[2][64];
    __shared__ uint32_t s_flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    // block -> (n, hg, sp); blocks 8G b .. 8G b + 8G - 1 hold pairs (n, sp) = 8b .. 8b + 7, head group
    // by block / 8 within that range
    const int B8 = 8 * d.G;
    const int ublk = blockIdx.x / B8, rem = blockIdx.x - ublk * B8;
    const int hg = rem >> 3;
    const int u = ublk * 8 + (rem & 7);
    const int n = u / d.S, sp = u - n * d.S;
    if (n >= a.num_q) return;  // padding of the last block of eight pairs

    const int head = 16 * hg + r16;
    const bool hv = head < a.n_heads;
    const int64_t kb = (int64_t)sp * d.per;

    // every load that needs only n first, in one round trip: the query's sequence and
    // position, the wave's q slice, and the given ids or the first-stage candidates
    const int s_raw = a.q_seq[n];
    const int64_t p_raw = a.q_pos[n];
    // the inverse-RoPE frequency of the pair this thread rotates in the epilogue
    const bool rope_lane = tid < a.rope_dims / 2;
    const double inv_freq = rope_lane ? a.rf.inv_freq[tid] : 0.0;
    // q slice of the wave as the B operand of S^T: column = head, k-step ks = dims 128 wave + 32 ks + 8 g .. +7
    bf16x8 qb[4];
    {
        const uint16_t* qrow = (hv ? a.q + ((int64_t)n * a.n_heads + head) * D
                                   : reinterpret_cast<const uint16_t*>(g_zero_row512)) + 128 * wave + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }
    int32_t pre_id[KR];
#pragma unroll
    for (int u = 0; u < KR; ++u) {
        const int j = u * kDT + tid;
        pre_id[u] = -1;
        if (!MERGE && a.topk && j < d.per && kb + j < a.k) pre_id[u] = a.topk[(int64_t)n * a.k + kb + j];
    }
    MergeIn in;
    in.sc = d.scores + (int64_t)n * d.stride;
    in.cand = d.cand + (int64_t)n * d.nchunks * d.kl;
    in.cnext = d.c_next + (int64_t)n * d.nchunks;
    in.kl = d.kl;
    in.k = a.k;
    CandRegs<8> cr;
    if (MERGE) cand_load(in, (int64_t)d.nchunks * d.kl, d.nchunks, cr);

    // the query (wave-uniform)
    int s = __builtin_amdgcn_readfirstlane(s_raw);
    const int64_t p_in = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)((uint64_t)p_raw >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p_raw));
    const bool ok = s >= 0 && s < a.num_seqs && p_in >= 0 && p_in <= a.max_q_pos;
    if (!ok && hg == 0 && sp == 0 && tid == 0) raise_error(a.err, (s < 0 || s >= a.num_seqs) ? kErrSeq : kErrPos);
    if (!ok) s = 0;
    const int64_t p = ok ? p_in : 0;
    const int64_t nv_c = (ok && a.comp_rows) ? p / a.comp_ratio : 0;
    const int64_t Lc = a.comp_rows ? (a.topk || MERGE ? (int64_t)a.k : nv_c) : 0;
    const int64_t lo = p - a.swa_window > 0 ? p - a.swa_window : 0;
    const int64_t L = ok ? Lc + (p - lo) : 0;
    const int64_t ke = kb + d.per < L ? kb + d.per : L;
    const int64_t kce = ke < Lc ? ke : Lc;
    const int nk = ke > kb ? (int)(ke - kb) : 0;     // keys of this split
    const int nkc = kce > kb ? (int)(kce - kb) : 0;  // of them compressed
    in.nv = ok ? (p >> 2 < d.stride ? p >> 2 : d.stride) : 0;

    const int64_t nbt64 = ok ? ((p + 255) >> 8 < (int64_t)a.max_blocks ? (p + 255) >> 8 : (int64_t)a.max_blocks) : 0;
    const bool staged = nbt64 <= kDBt;
    int32_t btv[kBtPer];
    {
        const int32_t* btrow = a.bt + (int64_t)s * a.max_blocks;
#pragma unroll
        for (int i = 0; i < kBtPer; ++i) {
            const int b = i * kDT + tid;
            btv[i] = (staged && b < (int)nbt64) ? btrow[b] : -1;
        }
    }

    if constexpr (MERGE > 0) {
        // the top-k of the query from the first-stage candidates: every workgroup of the query
        // runs the same deterministic merge; (hg 0, split 0) writes the top-k row and kth
        uint32_t* sm = reinterpret_cast<uint32_t*>(s_ring);
        const MergeLds m = {sm, sm + 2048, sm + 2048 + kCandCap, sm + 2048 + kCandCap + 4,
                            reinterpret_cast<float*>(sm + 2048 + kCandCap + 16), sm + 2048 + kCandCap + 20};
        const bool writer = hg == 0 && sp == 0;
        const SliceOut out = {writer ? d.topk_out + (int64_t)n * a.k : nullptr, s_ids, (uint32_t)kb, (uint32_t)nkc};
        float* kthp = writer && d.kth ? d.kth + n : nullptr;
        if (in.nv <= a.k) select_all(in.sc, in.nv, a.k, out, kthp, m.min);
        else merge_candidates<kDT, 8, true>(in, cr, out, kthp, m);  // one workgroup per CU: per-wave picks
    }
    // the block-table row lands after the merge, which does not need it
#pragma unroll
    for (int i = 0; i < kBtPer; ++i)
        if (i * kDT + tid < (int)nbt64 && staged) s_bt[i * kDT + tid] = btv[i];
    __syncthreads();  // s_bt, s_ids, s_rope; the merge is done with the ring

    // the split's key rows: in round u thread t resolves key kb + 256 u + t
#pragma unroll
    for (int u = 0; u < KR; ++u) {
        const int jj = u * kDT + tid;
        if (u * kDT >= nk) break;  // (uniform)
        const uint8_t* row = nullptr;
        if (jj < nk) {
            const int64_t j = kb + jj;
            int32_t pg = -1;
            int64_t slot = 0;
            const uint8_t* base = nullptr;
            int per_page = 0, np = 0;
            int64_t blk = -1;
            if (j < Lc) {
                const int64_t id = MERGE ? (int64_t)s_ids[jj] : (a.topk ? (int64_t)pre_id[u] : j);
                if (id >= nv_c) raise_error(a.err, kErrTopk);
                if (id >= 0 && id < nv_c) {
                    per_page = kBlockPositions / a.comp_ratio;  // 64 or 2: a power of two
                    blk = id >> (31 - __builtin_clz((unsigned)per_page));
                    slot = id & (per_page - 1);
                    base = a.comp_rows;
                    np = a.comp_pages;
                }
            } else {
                const int64_t t = lo + (j - Lc);
                blk = t >> 8;
                slot = t & 255;
                per_page = kBlockPositions;
                base = a.swa_rows;
                np = a.swa_pages;
            }
            if (blk >= 0) {
                pg = blk < a.max_blocks ? (staged ? s_bt[blk] : a.bt[(int64_t)s * a.max_blocks + blk]) : -1;
                if (pg < 0 || pg >= np) raise_error(a.err, kErrPage);
                else row = base + ((int64_t)pg * per_page + slot) * RB;
            }
        }
        // every row of the round's tiles gets an address (masked keys copy the zero row)
        if (jj < KMAX) s_rows[jj] = row ? row : g_zero_row512;
        const uint64_t bits = __ballot(row != nullptr);
        const int vw = (u * kDT + 64 * wave) / 32;
        if (lane == 0 && vw < KMAX / 32) s_vbits[vw] = (uint32_t)bits;
        if (lane == 0 && vw + 1 < KMAX / 32) s_vbits[vw + 1] = (uint32_t)(bits >> 32);
    }
    __syncthreads();

    const int ntl = __builtin_amdgcn_readfirstlane((nk + kDTile - 1) / kDTile);
    auto tile = [&](int t) { return s_ring + (t % RING) * (kDTile * ROW); };
    auto issue = [&](int t) {
        uint8_t* slot = s_ring + (t % RING) * (kDTile * ROW);
        const uint8_t* src[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) src[i] = s_rows[t * kDTile + 8 * wave + i];
        if (!KV8 || lane < kDRowBytes8 / 16) {  // an fp8 row is 34 x 16 bytes
#pragma unroll
            for (int i = 0; i < 8; ++i) dma_row(lds_off(slot + (8 * wave + i) * ROW), src[i] + 16 * lane);
        }
    };
    // the q loads retire here: the compiler's own wait for them would otherwise sit
    // inside the tile loop and, counting the tiles' loads too, drain every tile in flight
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qb[ks]));
    double inv_freq_r = inv_freq;  // (likewise the frequency, used after the issue)
    asm volatile("" : "+v"(inv_freq_r));
    // every ring slot is filled before the loop; a pair of tiles frees two slots
    int issued = ntl < RING ? ntl : RING;
    for (int t = 0; t < issued; ++t) issue(t);
    // the epilogue's inverse-RoPE angles while the first tiles are in flight
    if (rope_lane) rope_cs(-p, inv_freq_r, s_rope[0][tid], s_rope[1][tid]);

    f32x4 oacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_run = 0.f;

    // S operand row of this lane (accumulator row r16 of an m-tile) and the
    // transposed-read row.  bf16 keys: k-slot group g of the PV reads LDS rows
    // 4 i + g (+ 16 for slots 4..7), and accumulator row a of m-tile mt is the
    // key in LDS row 16 mt + 4 (a % 4) + a / 4.  fp8 keys: lane L of the PV's
    // 8-bit transposed read takes row L / 2 (so lane 16 g + r gets keys 8 g .. 8 g + 7
    // of dim r), and accumulator row a of m-tile mt is the key in LDS row
    // 8 (a / 4) + 4 mt + a % 4: softmax value 4 mt + i of a lane is key 8 g + 4 mt + i.
    const int s_row = KV8 ? 8 * (r16 >> 2) + (r16 & 3) : 4 * (r16 & 3) + (r16 >> 2);  // + 4 mt (fp8) / 16 mt
    const int tr_row = 4 * (r16 >> 2) + g;
    const int tr_col = (128 * wave + 4 * (r16 & 3)) * 2;  // bytes, + 32 per m-tile of 16 dims
    auto key_bit = [&](int mt, int i) { return KV8 ? 8 * g + 4 * mt + i : 16 * mt + 4 * i + g; };

    // the wave's S^T partial of tile t (two 16-key m-tiles over its 128 dims): operand reads, then MFMAs.
    // fp8 keys: codes widened to bf16 on the way; one MFMA chain per 64-dim group (k-steps 0, 1 and
    // 2, 3), each times its keys' group scale (the lane's keys: rows 8 g + 4 mt + i)
    struct SOps {
        bf16x8 av[2][4];
        float s0[2][4], s1[2][4];
    };
    auto s_reads = [&](int t, SOps& o) {
        const uint8_t* kt = tile(t);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            if constexpr (KV8) {
                const uint8_t* ka = kt + (s_row + 4 * mt) * ROW + 128 * wave + 8 * g;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) o.av[mt][ks] = fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(ka + 32 * ks));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float2 v = *reinterpret_cast<const float2*>(kt + (8 * g + 4 * mt + i) * ROW + 512 + 8 * wave);
                    o.s0[mt][i] = v.x;
                    o.s1[mt][i] = v.y;
                }
            } else {
                const uint8_t* ka = kt + (16 * mt + s_row) * ROW + (128 * wave + 8 * g) * 2;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) o.av[mt][ks] = *reinterpret_cast<const bf16x8*>(ka + 64 * ks);
            }
        }
    };
    auto s_mfma = [&](const SOps& o, f32x4 (&sa)[2]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sa[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (KV8) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.av[mt][0], qb[0], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.av[mt][2], qb[2], c1, 0, 0, 0);
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.av[mt][1], qb[1], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.av[mt][3], qb[3], c1, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) sa[mt][i] = fmaf(c0[i], o.s0[mt][i], c1[i] * o.s1[mt][i]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sa[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.av[mt][ks], qb[ks], sa[mt], 0, 0, 0);
        }
    };

    // iteration i takes tiles t = 2i and t + 1 (when there is one): both S^T partials, one
    // barrier to meet the four waves' partials, one softmax over the pair's keys, both P.V
    // products.  Two tiles per pass halve the passes' dependent chains (LDS round trips,
    // barriers, the cross-lane max), which bound the loop at one wave per SIMD.
    for (int t = 0; t < ntl; t += 2) {
        const bool two = t + 1 < ntl;  // (uniform)
        const int tl = two ? t + 1 : t;
        // tiles t .. tl have landed: the loads of the tiles issued after them may still be in flight
        wait_tiles(issued - (tl + 1));
        __syncthreads();  // the pair is visible; every wave is done with the slots and the S partials before it
        while (issued < ntl && issued < t + RING) issue(issued++);  // the slots the previous pair freed
        {
            SOps so0, so1;
            f32x4 sa0[2], sa1[2];
            s_reads(t, so0);
            if (two) s_reads(t + 1, so1);
            s_mfma(so0, sa0);
            if (two) s_mfma(so1, sa1);
            s_sx[0][wave][0][lane] = sa0[0];
            s_sx[0][wave][1][lane] = sa0[1];
            if (two) {
                s_sx[1][wave][0][lane] = sa1[0];
                s_sx[1][wave][1][lane] = sa1[1];
            }
        }
        __syncthreads();  // the four waves' S^T partials of the pair
        f32x4 sf[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                sf[h][mt] = (h == 0 || two)
                                ? ((s_sx[h][0][mt][lane] + s_sx[h][1][mt][lane]) + s_sx[h][2][mt][lane]) + s_sx[h][3][mt][lane]
                                : f32x4{0.f, 0.f, 0.f, 0.f};

        // softmax over the pair: value 8 h + (mt, i) is the key in LDS row key_bit(mt, i) of tile t + h
        const uint32_t vb0 = s_vbits[t], vb1 = two ? s_vbits[t + 1] : 0u;
        float x[16];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            const int h = cc >> 3, mt = (cc >> 2) & 1, i = cc & 3;
            const uint32_t vb = h ? vb1 : vb0;
            x[cc] = ((vb >> key_bit(mt, i)) & 1u) ? sf[h][mt][i] : -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) tmax = fmaxf(tmax, x[cc]);
        tmax = max_xor32(max_xor16(tmax)) * a.scale_log2;
        const bool move = tmax > m_ref + 8.0f;
        const float alpha = __builtin_amdgcn_exp2f(move ? m_ref - tmax : 0.f);
        const bool rescale = move && m_ref != -INFINITY;
        l_run *= alpha;
        m_ref = move ? tmax : m_ref;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float pf[16];
        float psum = 0.f;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            pf[cc] = __builtin_amdgcn_exp2f(fmaf(x[cc], a.scale_log2, -m_use));
            psum += pf[cc];
        }
        l_run += psum;
        if (__ballot(rescale)) {
#pragma unroll
            for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h == 1 && !two) break;  // (uniform)
            const uint8_t* kt = tile(t + h);
            // the P operands of tile t + h (hi and, for fp8 output, lo parts); fp8 keys: one per
            // 64-dim group of the wave, P times the key's group scale (V = codes x scale),
            // element cc = key 8 g + cc
            bf16x8 pb[2], plo[2];
            {
                float sc[2][8];
                if constexpr (KV8) {
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) {
                        const float2 v = *reinterpret_cast<const float2*>(kt + (8 * g + cc) * ROW + 512 + 8 * wave);
                        sc[0][cc] = v.x;
                        sc[1][cc] = v.y;
                    }
                }
#pragma unroll
                for (int gp = 0; gp < (KV8 ? 2 : 1); ++gp) {
                    uint32_t pw[4], pl[4];
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) {
                        const float q0 = pf[8 * h + 2 * cc], q1 = pf[8 * h + 2 * cc + 1];
                        const float p0 = KV8 ? q0 * sc[gp][2 * cc] : q0;
                        const float p1 = KV8 ? q1 * sc[gp][2 * cc + 1] : q1;
                        pw[cc] = pack_bf16x2(p0, p1);
                        if constexpr (PREC)
                            pl[cc] = pack_bf16x2(p0 - bf16_bits_to_f32(pw[cc] & 0xffffu), p1 - bf16_bits_to_f32(pw[cc] >> 16));
                    }
                    pb[gp] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
                    plo[gp] = pb[gp];
                    if constexpr (PREC) plo[gp] = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
                }
                if constexpr (!KV8) {
                    pb[1] = pb[0];
                    plo[1] = plo[0];
                }
            }
            // O^T += V^T . P^T over the wave's 8 m-tiles of 16 dims
            bf16x8 va[8];
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) {
                if constexpr (KV8) {
                    va[mm] = fp8x8_to_bf16(tr8_read(kt + (lane >> 1) * ROW + 128 * wave + 16 * mm + 8 * (lane & 1)));
                } else {
                    const uint8_t* b0 = kt + tr_row * ROW + tr_col + 32 * mm;
                    const u32x2 v0 = tr_read(b0), v1 = tr_read(b0 + 16 * ROW);
                    va[mm] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
                }
            }
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) {
                // m-tiles 0..3 are the wave's first 64-dim group, 4..7 its second
                oacc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mm], pb[mm >> 2], oacc[mm], 0, 0, 0);
                if constexpr (PREC) oacc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mm], plo[mm >> 2], oacc[mm], 0, 0, 0);
            }
        }
    }
    // the head's sum over its four lanes (every wave holds the same softmax)
    float l_tot = sum_xor16(l_run);
    l_tot = sum_xor32(l_tot);

    const int S = d.S;
    bool last = true;
    uint32_t* cnt = d.cnt + (int64_t)n * d.G + hg;
    if (S > 1) {
        const int64_t H = a.n_heads;
        if (!d.combine) {
            // partials for attn_combine_kernel: [n][S][H][D] fp32 and [n][S][H][2]
            if (hv) {
                float* po = a.part_o + (((int64_t)n * S + sp) * H + head) * D + 128 * wave + 4 * g;
#pragma unroll
                for (int mm = 0; mm < 8; ++mm) __builtin_nontemporal_store(oacc[mm], reinterpret_cast<f32x4*>(po + 16 * mm));
                if (wave == 0 && g == 0) {
                    float* ml = a.part_ml + (((int64_t)n * S + sp) * H + head) * 2;
                    ml[0] = m_ref;
                    ml[1] = l_tot;
                }
            }
            return;
        }
        // this split's partial with device-scope stores (coherent across the XCDs' L2s), relative
        // to the group's base: split x, head row h, dim c at ((x H + h) D + c) * 4 bytes
        float* gbase_o = a.part_o + ((int64_t)n * S * H + 16 * hg) * D;
        float* gbase_ml = a.part_ml + ((int64_t)n * S * H + 16 * hg) * 2;
        const int rec_o = (int)((((int64_t)S - 1) * H + 16) * D * 4);
        const int rec_ml = (int)((((int64_t)S - 1) * H + 16) * 2 * 4);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(gbase_o, 0, rec_o, kBufDword3);
        const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(gbase_ml, 0, rec_ml, kBufDword3);
        const int row_o = ((sp * (int)H + r16) * D + 128 * wave + 4 * g) * 4;
        if (hv) {
#pragma unroll
            for (int mm = 0; mm < 8; ++mm)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oacc[mm]), ro, row_o + 64 * mm, 0, kSc1);
            if (wave == 0 && g == 0)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m_ref), __float_as_uint(l_tot)}, rml,
                                                      (sp * (int)H + r16) * 8, 0, kSc1);
        }
        // the stores are complete (visible device-wide) before the arrival is counted
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) s_flag = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_flag != (uint32_t)(S - 1)) return;  // another split finishes this (query, head group)
        // last arriver: every other split has stored and counted; merge with device-scope loads,
        // the splits in split order (this one's from registers) so that the result does not
        // depend on which split arrived last; an empty split (m = -inf) weighs 0.  Loads of
        // absent splits use an offset past the buffer's end (they return 0), so every load is
        // issued unconditionally and a batch's loads are all in flight together.
        constexpr int kOob = 0x7ffffff0;
        float msx[kDecodeMaxCombine], lsx[kDecodeMaxCombine];
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < kDecodeMaxCombine; ++x) {
            const bool other = x < S && x != sp && hv;
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rml, other ? (x * (int)H + r16) * 8 : kOob, 0, kSc1);
            msx[x] = x == sp ? m_ref : (x < S && hv ? __uint_as_float(v[0]) : -INFINITY);
            lsx[x] = x == sp ? l_tot : __uint_as_float(v[1]);
            M = fmaxf(M, msx[x]);
        }
        const float Mu = M == -INFINITY ? 0.f : M;
        f32x4 acc[8];
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        constexpr int kBatch = 4;
#pragma unroll
        for (int x0 = 0; x0 < kDecodeMaxCombine; x0 += kBatch) {
            if (x0 >= S) break;
            f32x4 v[kBatch][8];
#pragma unroll
            for (int xb = 0; xb < kBatch; ++xb) {
                const int x = x0 + xb;
                const bool other = x < S && x != sp && hv;
                const int rx = other ? ((x * (int)H + r16) * D + 128 * wave + 4 * g) * 4 : kOob;
#pragma unroll
                for (int mm = 0; mm < 8; ++mm)
                    v[xb][mm] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, other ? rx + 64 * mm : kOob, 0, kSc1));
            }
#pragma unroll
            for (int xb = 0; xb < kBatch; ++xb) {
                const int x = x0 + xb;
                if (x >= S) break;
                const float wx = __builtin_amdgcn_exp2f(msx[x] - Mu);
                lsum = fmaf(lsx[x], wx, lsum);
#pragma unroll
                for (int mm = 0; mm < 8; ++mm)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        acc[mm][cc] = fmaf(wx, x == sp ? oacc[mm][cc] : v[xb][mm][cc], acc[mm][cc]);
            }
        }
        l_tot = lsum;
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) oacc[mm] = acc[mm];
        last = true;
    }

    // epilogue: RoPE^-1 at p on the raw values of the rotated dims (pairs are
    // adjacent values of a lane; the rotation commutes with the 1/l scaling),
    // then 1/l and the conversion; for fp8 the 1/l cancels inside each 64-dim
    // group: code = e4m3(v * 448 / amax(v)), scale = amax(v) / l / 448.  The
    // group's rows are staged in the idle ring and leave in contiguous 16-byte stores.
    const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int rbase = D - a.rope_dims;
    const int esz = a.out_dtype == kF32 ? 4 : a.out_dtype == kBF16 ? 2 : 1;
    const int rstride = D * esz + 16;
    __syncthreads();  // every wave is done with the ring
    uint8_t* srow = s_ring + r16 * rstride;
    float v[8][4];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
        const int d0 = 128 * wave + 16 * mm + 4 * g;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) v[mm][cc] = oacc[mm][cc];
        if (128 * wave + 16 * mm + 16 > rbase) {  // (uniform) a tile with rotated dims
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int dd = d0 + 2 * cc;
                const bool rot = dd >= rbase;
                const int pj = rot ? (dd - rbase) >> 1 : 0;
                const float cs = rot ? s_rope[0][pj] : 1.f, sn = rot ? s_rope[1][pj] : 0.f;
                const float x0 = v[mm][2 * cc], x1 = v[mm][2 * cc + 1];
                v[mm][2 * cc] = x0 * cs - x1 * sn;
                v[mm][2 * cc + 1] = x0 * sn + x1 * cs;
            }
        }
    }
    if (a.out_dtype == kFP8) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {  // 64-dim groups: m-tiles 4 gp .. 4 gp + 3
            float amax = 0.f, nz = 0.f;
#pragma unroll
            for (int mm = 4 * gp; mm < 4 * gp + 4; ++mm)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    amax = fmaxf(amax, fabsf(v[mm][cc]));
                    nz = fmaf(v[mm][cc], 0.f, nz);  // NaN or infinity anywhere makes this a NaN
                }
            amax = max_xor32(max_xor16(amax));
            const float gmax = amax * inv_l;
            const float scale = gmax > 0.f ? gmax / 448.0f : 1.0f;
            const float r = gmax > 0.f ? 448.0f / amax : 0.f;
            if (g == 0 && hv) a.out_scales[((int64_t)n * a.n_heads + head) * (D / 64) + 2 * wave + gp] = scale;
            const bool finite = __ballot(nz != nz) == 0;
#pragma unroll
            for (int mm = 4 * gp; mm < 4 * gp + 4; ++mm) {
                const int d0 = 128 * wave + 16 * mm + 4 * g;
                *reinterpret_cast<uint32_t*>(srow + d0) =
                    finite ? e4m3_pack4_finite(v[mm][0] * r, v[mm][1] * r, v[mm][2] * r, v[mm][3] * r)
                           : e4m3_pack4(v[mm][0] * r, v[mm][1] * r, v[mm][2] * r, v[mm][3] * r);
            }
        }
    } else {
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) {
            const int d0 = 128 * wave + 16 * mm + 4 * g;
            const float y0 = v[mm][0] * inv_l, y1 = v[mm][1] * inv_l, y2 = v[mm][2] * inv_l, y3 = v[mm][3] * inv_l;
            if (a.out_dtype == kF32) *reinterpret_cast<f32x4*>(srow + 4 * d0) = f32x4{y0, y1, y2, y3};
            else *reinterpret_cast<u32x2*>(srow + 2 * d0) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        }
    }
    __syncthreads();
    // the group's head rows (contiguous in the output) in 16-byte chunks
    const int nrows = a.n_heads - 16 * hg < 16 ? a.n_heads - 16 * hg : 16;
    const int rchunks = D * esz / 16;
    uint8_t* out = reinterpret_cast<uint8_t*>(a.out) + ((int64_t)n * a.n_heads + 16 * hg) * D * esz;
    for (int cc = tid; cc < nrows * rchunks; cc += kDT) {
        const int h = cc / rchunks, off = (cc - h * rchunks) * 16;
        *reinterpret_cast<u32x4*>(out + (int64_t)cc * 16) = *reinterpret_cast<const u32x4*>(s_ring + h * rstride + off);
    }
    // the group's counter back to zero for the next call (last, so nothing above waits for it)
    if (S > 1 && last && tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_decode_attn(const DecodeArgs& d, const CompressArgs& c, hipStream_t st, const LaunchEvents& ev) {
    const AttnArgs& a = d.at;
    if (a.num_q <= 0) return hipSuccess;
    if (a.dim != 512) return hipErrorInvalidValue;
    const int64_t pairs = (int64_t)a.num_q * d.S;
    const int64_t n_ins = c.total_new > 0 ? (int64_t)c.total_new * c.n_jobs : 0;
    if ((pairs + 7) / 8 * 8 * d.G + n_ins > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((pairs + 7) / 8 * 8 * d.G + n_ins));
    const bool prec = a.out_dtype == kFP8;
    const bool kv8 = a.swa_dtype == kFP8;
    if (kv8 != (a.comp_rows ? a.comp_dtype == kFP8 : kv8) || (!kv8 && a.swa_dtype != kBF16)) return hipErrorInvalidValue;
    const int64_t slots = (int64_t)d.nchunks * d.kl;
    if (d.cand != nullptr && slots > kDecodeMergeSlots) return hipErrorInvalidValue;
    static_assert(kDecodeMergeSlots == 8 * kDT, "one merge slot group of 8 per thread");
    const int merge = d.cand == nullptr ? 0 : 1;
    auto go = [&](auto kern) { launch_kernel(ev, true, true, kern, grid, dim3(kDT), st, d, c); };
#define CSL_DECODE_VARIANT(P, M, K) \
    if (prec == P && merge == M && kv8 == K) go(decode_attn_kernel<P, M, K>);
    CSL_DECODE_VARIANT(false, 0, false) CSL_DECODE_VARIANT(true, 0, false)
    CSL_DECODE_VARIANT(false, 1, false) CSL_DECODE_VARIANT(true, 1, false)
    CSL_DECODE_VARIANT(false, 0, true) CSL_DECODE_VARIANT(true, 0, true)
    CSL_DECODE_VARIANT(false, 1, true) CSL_DECODE_VARIANT(true, 1, true)
#undef CSL_DECODE_VARIANT
    return hipGetLastError();
}

}  // namespace csl
