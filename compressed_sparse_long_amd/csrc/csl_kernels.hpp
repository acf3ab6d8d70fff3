// Argument blocks and launchers of the gfx950 kernels (host + device).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csl_device.hpp"

namespace csl {

struct CompressJob {
    uint8_t* rows;
    uint16_t* state_x;
    float* state_logits;
    const uint16_t* x;
    const float* logits;
    const float* gain;
    int ratio, coff, dim, rope_dims, dtype, num_pages, row_bytes;
};

constexpr int kMaxInsertJobs = 4;

struct CompressArgs {
    CompressJob job[kMaxInsertJobs];
    RopeFreqs rf[kMaxInsertJobs];
    const int32_t* bt;
    const int64_t* start_pos;
    const int32_t* cu_new;
    uint32_t* err;
    int n_jobs, num_seqs, max_blocks, total_new;
    float eps;
};

// Query side: per-head Q RMSNorm + Q RoPE and the raw-key RoPE + insert of
// the same new tokens, one launch.
struct QSideArgs {
    const uint16_t* q;  // [total_new][n_heads][dim] bf16
    uint16_t* q_out;    // same shape; may equal q
    const uint16_t* x;  // [total_new][dim] bf16 raw keys
    const float* gain;  // [dim] or null
    uint8_t* rows;      // ratio-1 pool rows
    const int32_t* bt;
    const int64_t* start_pos;
    const int32_t* cu_new;
    uint32_t* err;
    int64_t n_q_rows;  // total_new * n_heads
    int64_t n_items;   // n_q_rows + total_new
    int n_heads, dim, rope_dims, dtype, num_pages, row_bytes, num_seqs, max_blocks;
    float eps;
    RopeFreqs rf;
};

struct IndexArgs {
    const uint8_t* rows;  // ratio-4 index pool: bf16 rows, or MXFP4 rows (fp4 = 1, dim 128: 68 bytes)
    const int32_t* bt;
    const int32_t* q_seq;
    const int64_t* q_pos;
    const uint16_t* q_idx;  // [num_q][n_heads][dim]
    const float* w;         // [num_q][n_heads]
    float* scores;          // [num_q][stride]
    int32_t* topk;          // [num_q][k]
    float* kth;             // [num_q] or null
    uint2* cand;            // [num_q][nchunks][kl] (key, id) first-stage candidates
    uint2* c_next;          // [num_q][nchunks] (key, id) of each chunk's (kl+1)-th element
    uint32_t* err;
    int64_t max_q_pos;
    int64_t stride;  // entries per query row of `scores` (multiple of 2048)
    int num_q, n_heads, dim, k, num_pages, num_seqs, max_blocks;
    int nchunks;     // stride / 1024 (first-stage chunks)
    int kl;          // first-stage candidates per chunk (0: single-pass select)
    int tiled;       // query-blocked score kernel (many queries) instead of one query per row
    int fp4;         // index rows are MXFP4
};

struct AttnArgs {
    const uint8_t* comp_rows;  // null = no compressed keys
    const uint8_t* swa_rows;
    const int32_t* bt;
    const int32_t* q_seq;        // decode: [num_q]; null in prefill
    const int64_t* q_pos;        // decode: [num_q]; null in prefill
    const int32_t* cu_q;         // prefill: [num_seqs+1]
    const int64_t* q_pos_start;  // prefill: [num_seqs]
    const uint16_t* q;
    const int32_t* topk;  // null = dense over visible entries
    void* out;
    float* out_scales;
    float* part_o;   // [num_q][n_splits][n_heads][dim]
    float* part_ml;  // [num_q][n_splits][n_heads][2]
    uint32_t* err;
    int64_t max_q_pos;
    int num_q, n_heads, dim, rope_dims, k, swa_window, comp_ratio, comp_dtype, swa_dtype, out_dtype;
    int comp_pages, swa_pages, num_seqs, max_blocks, n_splits;
    int64_t tiles_per_split;  // n_splits > 1: 32-key tiles of each split (from the longest possible key list)
    float scale_log2;  // softmax_scale * log2(e)
    RopeFreqs rf;
};

// Decode attention over 512-dim bf16 or fp8 keys (decode_attn_kernel): the attention
// arguments plus the work split and, when the launch also merges the
// indexer's first-stage candidates, where they are.
constexpr int kDecodeMaxSplitKeys = 256;  // keys of one split (8 tiles of 32)
constexpr int kDecodeMaxCombine = 8;      // splits merged in the launch by the last arriver
constexpr int kDecodeCounters = 4096;     // arrival counters at the start of the workspace (16 KiB)
constexpr int kDecodeMergeSlots = 2048;   // first-stage candidate slots one attention workgroup merges
struct DecodeArgs {
    AttnArgs at;
    int G;        // head groups of 16
    int S;        // key splits per (query, head group)
    int per;      // keys per split (multiple of 32, <= kDecodeMaxSplitKeys)
    int combine;  // S > 1: 1 = the last-arriving split merges (counters), 0 = partials for attn_combine_kernel
    uint32_t* cnt;  // [num_q * G] arrival counters, zero on entry and left zero
    // merge of first-stage candidates (the fused index + attention call); null cand = ids from at.topk
    const uint2* cand;    // [num_q][nchunks][kl]
    const uint2* c_next;  // [num_q][nchunks]
    const float* scores;  // [num_q][stride]
    int64_t stride;
    int nchunks, kl;
    int32_t* topk_out;  // [num_q][k] the merged top-k
    float* kth;         // [num_q] or null
};

// Events of a timed launch.  A launcher hands `start` to the first kernel it
// starts and `stop` to the last; the runtime stamps them with those kernels'
// own begin and end times (no marker packets in the queue), so the interval
// is the kernels' run time.  Both null: an untimed launch.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Which events of the current timed call were handed to a kernel (bit 0:
// start, bit 1: stop), so that the caller can record the ones no kernel took.
extern thread_local unsigned g_events_used;

template <typename F, typename... Args>
inline void launch_kernel(const LaunchEvents& ev, bool first, bool last, F kernel, dim3 grid, dim3 block,
                          hipStream_t st, Args... args) {
    hipEvent_t b = first ? ev.start : nullptr, e = last ? ev.stop : nullptr;
    if (b || e) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, b, e, 0, args...);
        g_events_used |= (b ? 1u : 0u) | (e ? 2u : 0u);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st, const LaunchEvents& ev = {});
hipError_t launch_qside(const QSideArgs& a, hipStream_t st, const LaunchEvents& ev = {});
hipError_t launch_index_score(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev = {});
hipError_t launch_index_score_insert(const IndexArgs& a, const CompressArgs& c, const QSideArgs& q, hipStream_t st,
                                     const LaunchEvents& ev = {});
hipError_t launch_topk_select(const IndexArgs& a, hipStream_t st, const LaunchEvents& ev = {});
hipError_t launch_topk_select_insert(const IndexArgs& a, const CompressArgs& c, const QSideArgs& q, hipStream_t st,
                                     const LaunchEvents& ev = {});
bool index_use_tiled(int num_q);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st, const LaunchEvents& ev = {});
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st, const LaunchEvents& ev = {});
// c: inserts riding as extra workgroups (c.total_new = 0: none)
hipError_t launch_decode_attn(const DecodeArgs& d, const CompressArgs& c, hipStream_t st, const LaunchEvents& ev = {});

}  // namespace csl
