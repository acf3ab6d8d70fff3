/*
 * csl.h -- C ABI of the MI355X (gfx950) hybrid compressed-attention library.
 *
 * The library computes the data-parallel hot path of DeepSeek-V4-style
 * hybrid compressed attention on a shared-K/V latent cache, as described in
 *   [Notes]   "DeepSeek V4 in vLLM 技术博客详尽笔记"
 *   [Summary] "vLLM DeepSeek V4 支援：高效長上下文注意力"
 * in four calls: compress_insert, index_topk, hybrid_attn_decode and
 * hybrid_attn_prefill, over caches paged in blocks of 256 native positions,
 * plus the query-side step before them (q_norm_rope_insert).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE memory unless marked "host".  The caller owns every
 *    buffer; the library allocates no device memory.  Scratch space is the
 *    caller's `ws`, sized by the matching *_workspace() query.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronises.
 *  - Arguments are validated on the host before anything is launched; a call
 *    that returns an error has launched nothing.  The message of the last
 *    failure on the calling thread is csl_last_error().
 *  - Data errors that only the device can see (an unmapped page inside a range
 *    a call must read or write, a top-k id that is not visible to its query, a
 *    position beyond the block table, a sequence index out of range) do not
 *    fault: the affected key/row is skipped (masked) and a bit is set in a
 *    sticky per-device error word, read and cleared by
 *    csl_read_device_error().
 *  - Calls that share buffers on one stream are ordered; calls on different
 *    streams that write the same pool pages race.
 *
 * Layout of a pool (one page per 256 native positions of a sequence; every
 * pool of a layer is indexed by the same block table, [Notes]
 * 解决方案一：统一逻辑块大小):
 *   rows          [num_pages][256/ratio][row_bytes]
 *                 bf16 row: dim x bf16                       (row_bytes = 2*dim)
 *                 fp8 row : dim x e4m3fn codes, then dim/64 x fp32 scales
 *                                                            (row_bytes = dim + dim/16)
 *   state_x       [num_pages][256][dim] bf16      (ratio > 1: raw tokens, the
 *   state_logits  [num_pages][256][coff] fp32      compressor state kept like
 *                 sliding-window KV, [Notes] 解决方案二：压缩器状态滑动窗口化)
 * Entry i of a ratio-r pool of sequence s lives in page
 * block_table[s][(i*r)/256], row i mod (256/r); raw token t (ratio 1) in page
 * block_table[s][t/256], row t mod 256.
 */
#ifndef CSL_H
#define CSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* csl_stream_t; /* a hipStream_t */

typedef enum {
    CSL_OK = 0,
    CSL_EINVAL = -1,       /* bad argument (NULL, out of range, inconsistent descriptor) */
    CSL_ERANGE = -2,       /* a size beyond what the kernels support */
    CSL_EALIGN = -3,       /* a pointer not aligned to 16 bytes */
    CSL_EWORKSPACE = -4,   /* workspace smaller than the *_workspace() query */
    CSL_EHIP = -5,         /* the HIP runtime reported an error (text in csl_last_error) */
    CSL_EUNSUPPORTED = -6  /* a valid combination the library does not implement */
} csl_status;

/* Row formats.  CSL_FP8_E4M3 rows: dim e4m3fn codes, then dim/64 fp32 scales
 * (amax/448 per 64 elements).  CSL_MXFP4 rows (index pools, dim 128): dim/2
 * bytes of E2M1 codes (element 2i in the low nibble of byte i), then dim/32
 * E8M0 bytes, the scale 2^(e-127) of each 32-element block -- the OCP MX
 * "MXFP4" format, our reading of the fp4 indexer cache ([Summary] 將索引器
 * 快取使用 fp4; [Notes] FP4 Indexer).  The block scale is
 * 2^(floor(log2 amax) - 2); elements round to nearest even and saturate at 6. */
typedef enum { CSL_F32 = 0, CSL_BF16 = 1, CSL_FP8_E4M3 = 2, CSL_MXFP4 = 3 } csl_dtype;

/* Device error bits (csl_read_device_error). */
#define CSL_DEVERR_UNMAPPED_PAGE 0x1u /* a needed page is -1 or >= num_pages: row skipped */
#define CSL_DEVERR_TOPK_ID 0x2u       /* a top-k id >= the query's visible count: key skipped */
#define CSL_DEVERR_POSITION 0x4u      /* a position < 0, > max_q_pos, or beyond max_blocks*256 */
#define CSL_DEVERR_SEQ 0x8u           /* a sequence index outside [0, num_seqs) */

typedef struct {
    int32_t ratio;      /* 1 = raw sliding-window keys, 4 = c4a, 128 = c128a */
    int32_t coff;       /* logits per token: window = coff*ratio tokens (c4a: 2, c128a: 1, raw: 1) */
    int32_t dim;        /* row width D (512 for the shared latent, 128 for index keys) */
    int32_t rope_dims;  /* rotated tail R of each row (even, <= dim, <= 128; 0 = none) */
    double rope_theta;  /* RoPE base (10000) */
    int32_t dtype;      /* CSL_BF16, CSL_FP8_E4M3, or CSL_MXFP4 (index pools only) */
    int32_t num_pages;
    void* rows;          /* [num_pages][256/ratio][row_bytes] */
    void* state_x;       /* [num_pages][256][dim] bf16; required iff ratio > 1 */
    float* state_logits; /* [num_pages][256][coff];   required iff ratio > 1 */
} csl_pool;

typedef struct {
    const int32_t* block_table; /* [num_seqs][max_blocks] page ids, -1 = unmapped */
    int32_t num_seqs;
    int32_t max_blocks;
} csl_pages;

/* Bytes of one stored row of `dim` elements in `dtype` (0 if unsupported). */
size_t csl_row_bytes(int32_t dim, int32_t dtype);

/*
 * Step 1 -- compressor + RMSNorm + RoPE + paged insert ([Notes] 融合 1：
 * Compressor + RMSNorm + RoPE + Cache Insert; window definitions in [Notes]
 * 数学附录精要: C4A / C128A 的精确位置范围).
 *
 * Sequence s receives tokens x[cu_new[s] .. cu_new[s+1]) at native positions
 * start_pos[s], start_pos[s]+1, ...
 *  - ratio 1: row t = RoPE(x_t, t), no norm (the raw-window keys, [Notes]
 *    融合 3：Q Norm + KV RoPE + K Insert).  logits and gain must be NULL.
 *  - ratio r > 1, coff c, window W = c*r: every token (x_t and its c logits)
 *    is written to the state; each entry i whose last token r(i+1)-1 arrives
 *    in the call is computed:  w = softmax over the window's logits (slot k of
 *    the window takes logit column k/r of token r(i+1)-W+k; tokens before
 *    position 0 are left out), u = sum_k w_k x_k, y = u / sqrt(mean(u^2)+eps)
 *    * gain, y = RoPE(y, r*i), stored as a bf16 or fp8 row.  Window tokens
 *    before start_pos[s] are read from the state, so a sequence can be fed in
 *    any chunking with identical results.
 * x: [total_new][dim] bf16; logits: [total_new][coff] fp32; gain: [dim] fp32
 * or NULL (unit gain).  start_pos: [num_seqs] int64; cu_new: [num_seqs+1]
 * int32 with cu_new[num_seqs] == total_new (host value).
 * Limits: dim % 8 == 0, dim <= 512 (fp8: dim % 256 == 0).
 */
csl_status csl_compress_insert(const csl_pool* pool /* host */, const csl_pages* pages /* host */,
                               const int64_t* start_pos, const int32_t* cu_new, int32_t total_new,
                               const uint16_t* x, const float* logits, const float* gain, float eps,
                               csl_stream_t stream);

/*
 * Step 1, several pools of a layer in one launch (the horizontal fusion of
 * independent per-pool inserts): the same batch of new tokens (start_pos,
 * cu_new, total_new) goes into every job's pool, each with its own x, logits
 * and gain, with exactly the semantics of csl_compress_insert per job.
 * 1 <= n_jobs <= 4; jobs (host array) must target different pools.
 */
typedef struct {
    const csl_pool* pool; /* host */
    const uint16_t* x;    /* [total_new][pool->dim] bf16 */
    const float* logits;  /* [total_new][pool->coff] fp32; NULL iff pool->ratio == 1 */
    const float* gain;    /* [pool->dim] fp32 or NULL (unit gain); NULL for ratio 1 */
} csl_insert_job;
csl_status csl_compress_insert_multi(int32_t n_jobs, const csl_insert_job* jobs /* host */,
                                     const csl_pages* pages /* host */, const int64_t* start_pos,
                                     const int32_t* cu_new, int32_t total_new, float eps, csl_stream_t stream);

/*
 * The query side of a step, fused with the raw-key insert ([Notes] 融合 3：
 * Q Norm + KV RoPE + K Insert; [Summary] Kernel 融合: queries and raw window
 * keys prepared in one kernel).  For new token j of sequence s, at position
 * t = start_pos[s] + (j - cu_new[s]):
 *  - every head h: y = q[j][h] / sqrt(mean(q[j][h]^2) + eps) * q_gain (an
 *    RMSNorm over the head's dim entries; q_gain [dim] fp32 shared by all
 *    heads, NULL = unit gain), then y = RoPE(y, t) with swa's rope_dims and
 *    rope_theta, stored as bf16 in q_out[j][h] -- the already normed and
 *    rotated q that the attention calls take;
 *  - raw key row t of `swa` = RoPE(x_j, t), exactly as csl_compress_insert
 *    does for a ratio-1 pool.
 * q, q_out: [total_new][n_heads][swa->dim] bf16; q_out may be q itself (in
 * place) but must not overlap it otherwise.  x: [total_new][swa->dim] bf16.
 * start_pos, cu_new as in csl_compress_insert.  swa: ratio 1, bf16 or fp8
 * rows.  Limits: 1 <= n_heads <= 1024.  An unmapped page skips that key row
 * (device error bit); the queries are written regardless.
 */
csl_status csl_q_norm_rope_insert(const csl_pool* swa /* host */, const csl_pages* pages /* host */,
                                  const int64_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                  const uint16_t* x, const uint16_t* q, int32_t n_heads, const float* q_gain,
                                  float eps, uint16_t* q_out, csl_stream_t stream);

/*
 * Steps 2-3 -- DSA indexer scores and causal top-k ([Summary] DeepSeek V4
 * 注意力架構: DSA keeps only the top-k compressed tokens; [Notes] 压缩参数细节:
 * k = 512 on c4a layers).
 *
 * For query n (sequence q_seq[n], position q_pos[n] = p) the candidates are
 * the index entries i with 4(i+1) <= p (an entry is visible once its last
 * token precedes the query, [Notes] 数学附录精要: 因果性条件).  Score:
 *     sigma(n,i) = sum_h w[n][h] * max(0, <q_idx[n][h], index_row_i>)
 * in fp32 from bf16 inputs.  topk[n] receives the k best ids (ties: lower
 * id first) in ascending order, padded with -1 when fewer than k are
 * visible; kth_score[n] (nullable) the score of the weakest selected id
 * (-inf if none).
 * index_pool: ratio 4, dim 32/64/128, bf16 rows, or dim 128 CSL_MXFP4 rows
 * (scored as their bf16 values: every E2M1 value times 2^k is exact in bf16).  q_idx: [num_q][n_heads]
 * [dim] bf16; w: [num_q][n_heads] fp32; topk: [num_q][k] int32;
 * n_heads <= 16; 1 <= k <= 2048; every q_pos <= max_q_pos (host bound that
 * sizes the grid).
 * Workspace (device, caller-owned, contents undefined on entry and exit):
 * one fp32 score row per query (max_q_pos/4 rounded up to 2048 entries) plus,
 * when the two-stage select is used (more than k visible entries and at most
 * 8192 first-stage candidates per query), 8-byte (key, id) candidates for
 * each 1024-entry chunk.  csl_index_topk_workspace() gives the exact size.
 */
size_t csl_index_topk_workspace(int32_t num_q, int64_t max_q_pos, int32_t k);
csl_status csl_index_topk(const csl_pool* index_pool /* host */, const csl_pages* pages /* host */,
                          int32_t num_q, const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos,
                          const uint16_t* q_idx, const float* w, int32_t n_heads, int32_t k, int32_t* topk,
                          float* kth_score, void* ws, size_t ws_bytes, csl_stream_t stream);

/* The query side of a step, for csl_index_topk_insert: the arguments of
 * csl_q_norm_rope_insert that the inserts do not share. */
typedef struct {
    const csl_pool* swa; /* host: ratio-1 pool that receives RoPE(x_t, t) */
    const uint16_t* x;   /* [total_new][swa->dim] bf16 */
    const uint16_t* q;   /* [total_new][n_heads][swa->dim] bf16, before the norm */
    int32_t n_heads;
    const float* q_gain; /* [swa->dim] fp32 or NULL (unit gain) */
    uint16_t* q_out;     /* may equal q */
} csl_qside_job;

/*
 * Steps 1-3 of a decode step with the writes of the step overlapped with the
 * indexer ([Notes] 优化二：多 CUDA 流并行: the indexer branch runs beside the
 * main KV compression and the raw-window insert; [Summary] 多串流分割; the
 * query side, [Notes] 融合 3).  Exactly csl_index_topk, then
 * csl_compress_insert_multi (if n_jobs > 0), then csl_q_norm_rope_insert (if
 * qside is not NULL) on `stream`, with the same arguments and results: the
 * writes run after the index scores are computed, as extra workgroups of the
 * top-k selection's last launch, whose few workgroups leave most of the GPU
 * idle.  Validation covers every part before anything is launched.
 * 0 <= n_jobs <= 4 (0 only with qside); no job may target qside->swa.
 */
csl_status csl_index_topk_insert(const csl_pool* index_pool /* host */, const csl_pages* pages /* host */,
                                 int32_t num_q, const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos,
                                 const uint16_t* q_idx, const float* w, int32_t n_heads, int32_t k, int32_t* topk,
                                 float* kth_score, void* ws, size_t ws_bytes, int32_t n_jobs,
                                 const csl_insert_job* jobs /* host */, const int64_t* start_pos,
                                 const int32_t* cu_new, int32_t total_new, float eps,
                                 const csl_qside_job* qside /* host, nullable */, csl_stream_t stream);

/*
 * Steps 4-6 -- hybrid attention, inverse RoPE, optional fp8 output.
 *
 * Query n (sequence s, position p) attends with ONE softmax over
 *   - compressed entries: topk[n][0..k) of `comp` (c4a; -1 = none), or, when
 *     topk is NULL, every visible entry i with r(i+1) <= p (c128a, [Notes]
 *     压缩参数细节 "全注意力"); comp may be NULL (window only);
 *   - raw tokens max(0, p - swa_window) .. p-1 of `swa` (ratio-1 pool;
 *     [Notes] ⚠️ 注意：C128A 的因果性约束),
 * with K = V = the stored row ([Summary] 共享鍵和值向量) and logits
 * softmax_scale * <q[n][h], K>.  Each head's output o is rotated back,
 * o = RoPE^-1(o, p) on the last rope_dims dims ([Notes] Inverse RoPE 的数学
 * 原理), and stored ([Notes] 融合 2：Inverse RoPE + FP8 Quant):
 *   CSL_F32 / CSL_BF16: out [num_q][n_heads][dim];
 *   CSL_FP8_E4M3: out [num_q][n_heads][dim] e4m3fn codes and out_scales
 *   [num_q][n_heads][dim/64] fp32, scale = amax/448 per 64 elements.
 * An empty key set gives 0.  q: [num_q][n_heads][dim] bf16, already normed
 * and rotated at p.  Limits: dim in {128, 512}, n_heads <= 64, softmax_scale
 * finite and > 0 (else CSL_EINVAL), rope_dims and rope_theta taken from `swa`
 * (comp must match).
 *
 * decode:  queries listed one by one (q_seq, q_pos: [num_q]); long key sets
 *          are split across workgroups and merged (needs ws).
 * prefill: queries of sequence s are cu_q[s] .. cu_q[s+1]-1 at positions
 *          q_pos_start[s], q_pos_start[s]+1, ...; one workgroup per query.
 *
 * Decode workspace (device, caller-owned; csl_hybrid_attn_workspace() bytes,
 * 0 = none needed and ws may be NULL): the first 16 KiB hold arrival counters
 * of the splits and MUST BE ZERO before the first call that uses this ws
 * (e.g. allocate it zero-filled); every call that completes leaves them zero
 * again, so a ws can be reused by any later decode call, on one stream at a
 * time.  The rest holds split partials (contents undefined on entry and exit).
 */
size_t csl_hybrid_attn_workspace(int32_t num_q, int32_t n_heads, int32_t dim, int32_t comp_ratio, int32_t k,
                                 int32_t swa_window, int64_t max_q_pos);
csl_status csl_hybrid_attn_decode(const csl_pool* comp /* host, nullable */, const csl_pool* swa /* host */,
                                  const csl_pages* pages /* host */, int32_t num_q, const int32_t* q_seq,
                                  const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q, int32_t n_heads,
                                  const int32_t* topk, int32_t k, int32_t swa_window, float softmax_scale,
                                  int32_t out_dtype, void* out, float* out_scales, void* ws, size_t ws_bytes,
                                  csl_stream_t stream);
/*
 * A decode step's attention with the step's inserts riding along ([Notes]
 * 优化二：多 CUDA 流并行: the writes of a step overlap its reads): the
 * results of csl_compress_insert_multi(n_jobs, jobs, pages, start_pos,
 * cu_new, total_new, eps) followed by csl_hybrid_attn_decode(comp, swa, ...),
 * provided that no query reads what the inserts write: every inserted token's
 * position is at least the position of each query of its sequence (a decode
 * step inserts the token at the query's own position, and a query at p reads
 * raw tokens below p and compressed entries that close below p).  Otherwise
 * the results are undefined.  For 512-dim bf16 or fp8 keys the inserts run as
 * extra workgroups of the attention launch (one launch for a dense c128a
 * step); for other keys they run in a launch of their own first.  Arguments,
 * limits and workspace as for the two calls (1 <= n_jobs <= 4); validation
 * covers both before anything is launched.
 */
csl_status csl_hybrid_attn_decode_insert(const csl_pool* comp /* host, nullable */, const csl_pool* swa /* host */,
                                         const csl_pages* pages /* host */, int32_t num_q, const int32_t* q_seq,
                                         const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q,
                                         int32_t n_heads, const int32_t* topk, int32_t k, int32_t swa_window,
                                         float softmax_scale, int32_t out_dtype, void* out, float* out_scales,
                                         int32_t n_jobs, const csl_insert_job* jobs /* host */,
                                         const int64_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                         float eps, void* ws, size_t ws_bytes, csl_stream_t stream);
csl_status csl_hybrid_attn_prefill(const csl_pool* comp /* host, nullable */, const csl_pool* swa /* host */,
                                   const csl_pages* pages /* host */, const int32_t* cu_q,
                                   const int64_t* q_pos_start, int32_t total_q, int64_t max_q_pos,
                                   const uint16_t* q, int32_t n_heads, const int32_t* topk, int32_t k,
                                   int32_t swa_window, float softmax_scale, int32_t out_dtype, void* out,
                                   float* out_scales, csl_stream_t stream);

/*
 * Steps 1-6 of a c4a decode step in two launches ([Summary] DeepSeek V4 注意力
 * 架構: the indexer's top-k feeds the sparse attention; [Notes] 优化二：多 CUDA
 * 流并行 for the writes that ride along): exactly csl_index_topk_insert(
 * index_pool, ..., topk, kth_score, ..., n_jobs, jobs, ..., qside), then
 * csl_hybrid_attn_decode(comp, swa, ..., topk, k, ...), with the same
 * arguments and results (topk and kth_score are written as by the indexer).
 * The first launch scores the index entries (with each 1024-entry chunk's
 * first-stage candidates) and carries the inserts and query-side rows; the
 * second merges each query's candidates into its top-k and runs the
 * attention, splits merged in the launch.
 * comp: ratio 4, dim 512, bf16 or fp8 rows; swa: ratio 1,
 * the same dim and dtype.  ws: csl_index_attn_decode_workspace() bytes, its
 * first 16 KiB zero before the first use and left zero (as for
 * csl_hybrid_attn_decode).  0 <= n_jobs <= 4.
 */
size_t csl_index_attn_decode_workspace(int32_t num_q, int32_t n_heads, int64_t max_q_pos, int32_t k,
                                       int32_t swa_window);
csl_status csl_index_attn_decode(const csl_pool* index_pool /* host */, const csl_pool* comp /* host */,
                                 const csl_pool* swa /* host */, const csl_pages* pages /* host */, int32_t num_q,
                                 const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos,
                                 const uint16_t* q_idx, const float* w, int32_t n_idx_heads, int32_t k, int32_t* topk,
                                 float* kth_score, const uint16_t* q, int32_t n_heads, int32_t swa_window,
                                 float softmax_scale, int32_t out_dtype, void* out, float* out_scales, int32_t n_jobs,
                                 const csl_insert_job* jobs /* host */, const int64_t* start_pos,
                                 const int32_t* cu_new, int32_t total_new, float eps,
                                 const csl_qside_job* qside /* host, nullable */, void* ws, size_t ws_bytes,
                                 csl_stream_t stream);

/*
 * csl_index_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus ws, ws_bytes),
 * kernels and results as csl_index_attn_decode; its scratch is a static device
 * array of 64 MiB in the library, one copy per device, held until the process
 * ends.  A call whose csl_index_attn_decode_workspace() exceeds 64 MiB returns
 * CSL_ERANGE and launches nothing (16 queries of 64 heads fit up to 1M
 * positions).  The first call on a device also launches, on `stream`, the
 * clearing of the scratch's arrival counters.  The library allocates nothing
 * in this call.  Every call on one device shares that device's scratch: calls
 * that overlap on one device (different streams, or different host threads
 * without ordering) race and give undefined results.
 */
csl_status csl_index_attn_decode_noalloc(const csl_pool* index_pool /* host */, const csl_pool* comp /* host */,
                                         const csl_pool* swa /* host */, const csl_pages* pages /* host */,
                                         int32_t num_q, const int32_t* q_seq, const int64_t* q_pos,
                                         int64_t max_q_pos, const uint16_t* q_idx, const float* w,
                                         int32_t n_idx_heads, int32_t k, int32_t* topk, float* kth_score,
                                         const uint16_t* q, int32_t n_heads, int32_t swa_window,
                                         float softmax_scale, int32_t out_dtype, void* out, float* out_scales,
                                         int32_t n_jobs, const csl_insert_job* jobs /* host */,
                                         const int64_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                         float eps, const csl_qside_job* qside /* host, nullable */,
                                         csl_stream_t stream);

/* Message of the last failing call on the calling thread ("" if none). */
const char* csl_last_error(void);

/* Synchronises the current device, returns its sticky CSL_DEVERR_* word in
 * *flags (host) and clears it.  For tests and debugging. */
csl_status csl_read_device_error(uint32_t* flags);

/* Kernel timers: when enabled for a kernel id, every launch of that kernel
 * (at most 65536 between reads) goes through hipExtLaunchKernel with a HIP
 * event pair that the runtime stamps with the kernel's own start and end
 * (for CSL_KERNEL_TOPK_SELECT: from the first of its kernels to the last),
 * on the launch stream and with no extra queue packets.  csl_timer_read
 * synchronises the device, returns the summed durations (ms) and the launch
 * count, and resets.  Kernel ids: */
#define CSL_KERNEL_COMPRESS 0
#define CSL_KERNEL_INDEX_SCORE 1
#define CSL_KERNEL_TOPK_SELECT 2
#define CSL_KERNEL_ATTN 3
#define CSL_KERNEL_ATTN_COMBINE 4
#define CSL_KERNEL_QSIDE 5
csl_status csl_timer_enable(int32_t kernel_id, int32_t on);
csl_status csl_timer_read(int32_t kernel_id, double* total_ms /* host */, int64_t* launches /* host */);

#ifdef __cplusplus
}
#endif
#endif
