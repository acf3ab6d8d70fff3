// Host side of the C ABI (include/csl.h): argument validation, workspace
// sizing, launch configuration, the sticky device error word and the
// optional per-kernel event timers.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "csl.h"
#include "csl_kernels.hpp"

__device__ uint32_t csl_device_error_word;

namespace csl {
thread_local unsigned g_events_used = 0;
}

namespace {

using namespace csl;

thread_local std::string g_err;

csl_status fail(csl_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

csl_status hip_fail(hipError_t e, const char* what) {
    return fail(CSL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;

csl_status device_error_ptr(uint32_t** out) {
    static uint32_t* ptrs[kMaxDevices] = {};
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CSL_EUNSUPPORTED, "device id %d beyond %d", dev, kMaxDevices);
    hipError_t se = hipSuccess;
    std::call_once(once[dev], [&] {
        se = hipGetSymbolAddress(reinterpret_cast<void**>(&ptrs[dev]), HIP_SYMBOL(csl_device_error_word));
    });
    if (se != hipSuccess) return hip_fail(se, "hipGetSymbolAddress(error word)");
    if (!ptrs[dev]) return fail(CSL_EHIP, "error word of device %d is unavailable", dev);
    *out = ptrs[dev];
    return CSL_OK;
}

// ---------------------------------------------------------------- static scratch

// Scratch of the no-allocation fused decode call: one copy per device, held
// until the process ends, shared by every such call on that device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

__global__ void zero_words_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of `scratch` on the current device (the host-side name is
// only a stand-in), taken once per device.  The first call on a device also
// clears the arrival counters at the start of the scratch (on `st`, before the
// caller's launches); every call that completes leaves them zero again.
csl_status static_scratch(hipStream_t st, void** out) {
    static void* ptrs[kMaxDevices] = {};
    static hipError_t errs[kMaxDevices] = {};
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CSL_EUNSUPPORTED, "device id %d beyond %d", dev, kMaxDevices);
    std::call_once(once[dev], [&] {
        void* ptr = nullptr;
        hipError_t se = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
        if (se == hipSuccess && ptr) {
            constexpr int words = kDecodeCounters;
            hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                               static_cast<uint32_t*>(ptr), words);
            se = hipGetLastError();
        }
        errs[dev] = se;
        if (se == hipSuccess) ptrs[dev] = ptr;
    });
    if (errs[dev] != hipSuccess) return hip_fail(errs[dev], "static scratch set-up");
    if (!ptrs[dev]) return fail(CSL_EHIP, "static scratch of device %d is unavailable", dev);
    *out = ptrs[dev];
    return CSL_OK;
}

// ---------------------------------------------------------------- timers

struct Timer {
    std::atomic<bool> on{false};
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
    size_t used = 0;
};
constexpr int kNumKernels = 6;
constexpr size_t kMaxTimed = 65536;
Timer g_timer[kNumKernels];
std::mutex g_timer_mu;

// Runs launch(ev).  With the kernel's timer off (the normal case) no lock is
// taken and no events are used.  With it on, the call takes the next event
// pair; an event that no kernel took (a call that launched nothing, or fewer
// kernels than the pair assumed) is recorded on the stream right away, so
// every handed-out pair holds a valid interval.
template <typename F>
hipError_t timed(int kid, hipStream_t st, F&& launch) {
    Timer& t = g_timer[kid];
    if (!t.on.load(std::memory_order_relaxed)) return launch(LaunchEvents{});
    hipEvent_t b = nullptr, e = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_timer_mu);
        if (t.on && t.used < kMaxTimed) {
            if (t.used == t.ev.size()) {
                hipEvent_t x, y;
                if (hipEventCreate(&x) == hipSuccess && hipEventCreate(&y) == hipSuccess) t.ev.push_back({x, y});
            }
            if (t.used < t.ev.size()) {
                b = t.ev[t.used].first;
                e = t.ev[t.used].second;
                ++t.used;
            }
        }
    }
    LaunchEvents ev;
    ev.start = b;
    ev.stop = e;
    g_events_used = 0;
    hipError_t r = launch(ev);
    if (b && !(g_events_used & 1u)) (void)hipEventRecord(b, st);
    if (e && !(g_events_used & 2u)) (void)hipEventRecord(e, st);
    return r;
}

// ---------------------------------------------------------------- validation

size_t row_bytes_of(int dim, int dtype) {
    if (dim <= 0) return 0;
    if (dtype == CSL_BF16) return 2 * (size_t)dim;
    if (dtype == CSL_FP8_E4M3) return (dim % 256 == 0) ? (size_t)dim + dim / 16 : 0;
    if (dtype == CSL_MXFP4) return (dim % 32 == 0) ? (size_t)dim / 2 + dim / 32 : 0;
    if (dtype == CSL_F32) return 4 * (size_t)dim;
    return 0;
}

csl_status check_pages(const csl_pages* pg) {
    if (!pg || !pg->block_table) return fail(CSL_EINVAL, "pages or block_table is NULL");
    if (pg->num_seqs <= 0 || pg->max_blocks <= 0)
        return fail(CSL_EINVAL, "num_seqs (%d) and max_blocks (%d) must be > 0", pg->num_seqs, pg->max_blocks);
    return CSL_OK;
}

csl_status check_pool(const csl_pool* P, const char* name) {
    if (!P) return fail(CSL_EINVAL, "%s pool is NULL", name);
    if (!P->rows) return fail(CSL_EINVAL, "%s.rows is NULL", name);
    if (P->ratio != 1 && P->ratio != 4 && P->ratio != 128)
        return fail(CSL_EINVAL, "%s.ratio = %d, expected 1, 4 or 128", name, P->ratio);
    if (P->coff < 1 || P->coff > 2 || (P->ratio == 1 && P->coff != 1))
        return fail(CSL_EINVAL, "%s.coff = %d invalid for ratio %d", name, P->coff, P->ratio);
    if (P->dim < 8 || P->dim > 512 || P->dim % 8)
        return fail(CSL_ERANGE, "%s.dim = %d, expected a multiple of 8 in [8, 512]", name, P->dim);
    if (P->rope_dims < 0 || P->rope_dims > P->dim || P->rope_dims % 4 || P->rope_dims > 128)
        return fail(CSL_EINVAL, "%s.rope_dims = %d, expected a multiple of 4 in [0, min(dim, 128)]", name,
                    P->rope_dims);
    if (P->rope_dims > 0 && !(P->rope_theta > 0.0)) return fail(CSL_EINVAL, "%s.rope_theta must be > 0", name);
    if (P->dtype != CSL_BF16 && P->dtype != CSL_FP8_E4M3 && P->dtype != CSL_MXFP4)
        return fail(CSL_EINVAL, "%s.dtype = %d, expected CSL_BF16, CSL_FP8_E4M3 or CSL_MXFP4", name, P->dtype);
    if (P->dtype == CSL_FP8_E4M3 && P->dim % 256)
        return fail(CSL_EUNSUPPORTED, "%s: fp8 rows need dim %% 256 == 0 (got %d)", name, P->dim);
    if (P->dtype == CSL_MXFP4 && P->dim != 128)
        return fail(CSL_EUNSUPPORTED, "%s: fp4 rows need dim 128 (got %d)", name, P->dim);
    if (P->num_pages <= 0) return fail(CSL_EINVAL, "%s.num_pages must be > 0", name);
    if (!aligned16(P->rows)) return fail(CSL_EALIGN, "%s.rows is not 16-byte aligned", name);
    if (P->ratio > 1) {
        if (P->state_x && !aligned16(P->state_x)) return fail(CSL_EALIGN, "%s.state_x is not 16-byte aligned", name);
    }
    return CSL_OK;
}

RopeFreqs make_freqs(int rope_dims, double theta) {
    RopeFreqs rf;
    for (int j = 0; j < 64; ++j)
        rf.inv_freq[j] = (j < rope_dims / 2) ? std::pow(theta, -2.0 * j / (double)rope_dims) : 0.0;
    return rf;
}

int64_t index_stride(int64_t max_q_pos) {
    int64_t nv = max_q_pos / 4;
    if (nv < 1) nv = 1;
    return (nv + 2047) / 2048 * 2048;
}

// First-stage candidates per 1024-id chunk for the two-stage top-k (the score
// kernel's workgroup selects them): the expected share of the top k in a chunk
// plus five standard deviations (a chunk holding more only costs the exact
// fallback), at most 8192 per query; 0 = single-pass select.
constexpr int kIndexChunk = 1024;

int index_local_k(int64_t max_q_pos, int k) {
    const int64_t nv = max_q_pos / 4;
    if (nv <= k) return 0;
    const double expect = (double)k * kIndexChunk / (double)nv;
    int kl = (int)std::ceil((expect + 5.0 * std::sqrt(expect) + 4.0) / 8.0) * 8;
    kl = kl < 16 ? 16 : (kl > kIndexChunk ? kIndexChunk : kl);
    const int64_t nchunks = index_stride(max_q_pos) / kIndexChunk;
    return nchunks * kl <= 8192 ? kl : 0;
}

// 32-key tiles of the longest key list any query at or below max_q_pos can have.
int64_t decode_tiles(int comp_ratio, int k, int swa_window, int64_t max_q_pos) {
    int64_t keys = (int64_t)(swa_window < max_q_pos ? swa_window : max_q_pos);
    if (comp_ratio > 0) keys += k > 0 ? k : max_q_pos / comp_ratio;
    return (keys + 31) / 32;
}

// Splits of a decode launch.  Every split writes a heads x dim fp32 partial
// that the merge reads back, so splits take several 32-key tiles: 4 for bf16
// keys, 2 for fp8 keys (whose tiles cost more: the codes are widened in LDS).
// A launch that would then hold fewer than 32 workgroups halves the tiles per
// split until it does not (down to one), and there are at most 512 / num_q
// splits.
int decode_splits(int num_q, int comp_ratio, int k, int swa_window, int64_t max_q_pos, bool fp8_keys) {
    const int64_t tiles = decode_tiles(comp_ratio, k, swa_window, max_q_pos);
    int64_t tps = fp8_keys ? 2 : 4;
    int64_t cap = tiles / tps > 1 ? tiles / tps : 1;
    while (tps > 1 && (int64_t)num_q * cap < 32) {
        tps /= 2;
        cap = tiles / tps > 1 ? tiles / tps : 1;
    }
    const int64_t want = (512 + num_q - 1) / (num_q > 0 ? num_q : 1);
    int64_t sp = want < cap ? want : cap;
    if (sp > 1024) sp = 1024;
    return (int)(sp > 1 ? sp : 1);
}

// Decode attention on 512-dim bf16 or fp8 keys (decode_attn_kernel): G head groups of
// 16; the key list (rounded up to 32-key tiles) split so that the launch holds
// about 256 workgroups but no split has fewer than about four tiles, two passes
// of the loop's tile pairs (the last arriving split reads every other split's
// partial, so short splits cost more there than they save in the tile loop: the
// 8-query c128a step took 18.6 us with six two-tile splits, 15.4 with four
// three-tile ones, 14.5 with three of four, 15.3 with two of six), with 32..256
// keys per split; at most 8 splits are merged inside the launch by the
// last arriving split (more, or more than kDecodeCounters (query, head group)
// pairs: partials for the combine kernel).
// (Fewer, longer splits measured slower: eight fp8 splits of 1040 keys for the
// 1M c128a layer took the step from 72 to 115 us.)
struct DecodePlan {
    int G, S, per, combine;
};
DecodePlan decode_plan(int num_q, int n_heads, int comp_ratio, int k, int swa_window, int64_t max_q_pos) {
    DecodePlan pl;
    pl.G = (n_heads + 15) / 16;
    const int64_t keys = decode_tiles(comp_ratio, k, swa_window, max_q_pos) * 32;
    const int64_t groups = (int64_t)(num_q > 0 ? num_q : 1) * pl.G;
    int64_t want = 256 / groups > 1 ? 256 / groups : 1;
    const int64_t by_tiles = (keys / 32 + 3) / 4;
    if (by_tiles >= 1 && by_tiles < want) want = by_tiles;
    auto round32 = [](int64_t x) { return (x + 31) / 32 * 32; };
    int64_t per = round32((keys + want - 1) / want);
    per = per < 32 ? 32 : (per > kDecodeMaxSplitKeys ? kDecodeMaxSplitKeys : per);
    int64_t S = keys > 0 ? (keys + per - 1) / per : 1;
    if (S > kDecodeMaxCombine && keys <= (int64_t)kDecodeMaxCombine * kDecodeMaxSplitKeys) {
        per = round32((keys + kDecodeMaxCombine - 1) / kDecodeMaxCombine);
        S = (keys + per - 1) / per;
    }
    pl.per = (int)per;
    pl.S = (int)(S > 1 ? S : 1);
    pl.combine = pl.S > 1 && pl.S <= kDecodeMaxCombine && groups <= kDecodeCounters;
    return pl;
}

constexpr size_t kCounterBytes = (size_t)kDecodeCounters * sizeof(uint32_t);  // zero-on-entry block at ws offset 0

// Bytes of split partials ([num_q][splits][n_heads][dim] fp32 and [..][2]).
size_t partial_bytes(int num_q, int splits, int n_heads, int dim) {
    return splits > 1 ? (size_t)num_q * splits * n_heads * ((size_t)dim + 2) * sizeof(float) : 0;
}

// Whether the decode call runs decode_attn_kernel (512-dim bf16 or fp8 keys).
bool use_decode_kernel(int dim, int key_dtype) { return dim == 512 && (key_dtype == CSL_BF16 || key_dtype == CSL_FP8_E4M3); }

// Workspace of a decode attention call: the counter block, then the partials
// of the larger of the paths the key type could take (the key type is not an
// argument of the query); 0 when no path needs partials.
size_t attn_ws_bytes(int32_t num_q, int32_t n_heads, int32_t dim, int32_t comp_ratio, int32_t k, int32_t swa_window,
                     int64_t max_q_pos) {
    if (num_q <= 0 || n_heads <= 0 || dim <= 0) return 0;
    const int sp8 = decode_splits(num_q, comp_ratio, k, swa_window, max_q_pos, true);
    const int sp16 = decode_splits(num_q, comp_ratio, k, swa_window, max_q_pos, false);
    size_t need = partial_bytes(num_q, sp8 > sp16 ? sp8 : sp16, n_heads, dim);
    if (dim == 512) {
        const DecodePlan pl = decode_plan(num_q, n_heads, comp_ratio, k, swa_window, max_q_pos);
        const size_t b = partial_bytes(num_q, pl.S, n_heads, dim);
        need = b > need ? b : need;
    }
    return need > 0 ? kCounterBytes + need : 0;
}

csl_status check_attn_common(const csl_pool* comp, const csl_pool* swa, const csl_pages* pages, int n_heads,
                             const int32_t* topk, int k, int swa_window, int out_dtype, const void* out,
                             const float* out_scales, const uint16_t* q, int64_t max_q_pos, float softmax_scale) {
    csl_status st;
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(CSL_EINVAL, "softmax_scale must be finite and > 0");
    if ((st = check_pages(pages))) return st;
    if ((st = check_pool(swa, "swa"))) return st;
    if (swa->ratio != 1) return fail(CSL_EINVAL, "swa.ratio must be 1 (raw window keys)");
    if (swa->dim != 128 && swa->dim != 512) return fail(CSL_EUNSUPPORTED, "attention dim %d (supported: 128, 512)", swa->dim);
    if (comp) {
        if ((st = check_pool(comp, "comp"))) return st;
        if (comp->ratio == 1) return fail(CSL_EINVAL, "comp.ratio must be 4 or 128");
        if (comp->dim != swa->dim || comp->rope_dims != swa->rope_dims || comp->rope_theta != swa->rope_theta)
            return fail(CSL_EINVAL, "comp and swa pools differ in dim / rope_dims / rope_theta");
        if (comp->dtype != swa->dtype) return fail(CSL_EUNSUPPORTED, "comp and swa pools must share one dtype");
    } else if (topk) {
        return fail(CSL_EINVAL, "topk given without a compressed pool");
    }
    if (swa->dtype == CSL_FP8_E4M3 && swa->dim != 512) return fail(CSL_EUNSUPPORTED, "fp8 keys need dim 512");
    if (swa->dtype == CSL_MXFP4) return fail(CSL_EUNSUPPORTED, "fp4 rows are for index pools; attention keys are bf16 or fp8");
    if (n_heads < 1 || n_heads > 64) return fail(CSL_ERANGE, "n_heads = %d, supported 1..64", n_heads);
    if (topk && (k < 1 || k > 65536)) return fail(CSL_ERANGE, "k = %d out of range", k);
    if (swa_window < 0) return fail(CSL_EINVAL, "swa_window < 0");
    if (max_q_pos < 0) return fail(CSL_EINVAL, "max_q_pos < 0");
    if (max_q_pos >= (int64_t)pages->max_blocks * 256 + 1)
        return fail(CSL_ERANGE, "max_q_pos %lld beyond the block table (%d blocks)", (long long)max_q_pos,
                    pages->max_blocks);
    if (out_dtype != CSL_F32 && out_dtype != CSL_BF16 && out_dtype != CSL_FP8_E4M3)
        return fail(CSL_EINVAL, "out_dtype = %d", out_dtype);
    if (!out || !q) return fail(CSL_EINVAL, "q or out is NULL");
    if (out_dtype == CSL_FP8_E4M3 && !out_scales) return fail(CSL_EINVAL, "fp8 output needs out_scales");
    if (!aligned16(q) || !aligned16(out)) return fail(CSL_EALIGN, "q and out must be 16-byte aligned");
    return CSL_OK;
}

void fill_attn(AttnArgs& a, const csl_pool* comp, const csl_pool* swa, const csl_pages* pages, int n_heads,
               const int32_t* topk, int k, int swa_window, float softmax_scale, int out_dtype, void* out,
               float* out_scales, const uint16_t* q, int64_t max_q_pos, uint32_t* err) {
    a.comp_rows = comp ? static_cast<const uint8_t*>(comp->rows) : nullptr;
    a.swa_rows = static_cast<const uint8_t*>(swa->rows);
    a.bt = pages->block_table;
    a.q = q;
    a.topk = topk;
    a.out = out;
    a.out_scales = out_scales;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.err = err;
    a.max_q_pos = max_q_pos;
    a.n_heads = n_heads;
    a.dim = swa->dim;
    a.rope_dims = swa->rope_dims;
    a.k = topk ? k : 0;
    a.swa_window = swa_window;
    a.comp_ratio = comp ? comp->ratio : 1;
    a.comp_dtype = comp ? comp->dtype : swa->dtype;
    a.swa_dtype = swa->dtype;
    a.out_dtype = out_dtype;
    a.comp_pages = comp ? comp->num_pages : 0;
    a.swa_pages = swa->num_pages;
    a.num_seqs = pages->num_seqs;
    a.max_blocks = pages->max_blocks;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.rf = make_freqs(swa->rope_dims, swa->rope_theta);
}

}  // namespace

extern "C" {

size_t csl_row_bytes(int32_t dim, int32_t dtype) { return row_bytes_of(dim, dtype); }

const char* csl_last_error(void) { return g_err.c_str(); }

csl_status csl_read_device_error(uint32_t* flags) {
    if (!flags) return fail(CSL_EINVAL, "flags is NULL");
    uint32_t* p = nullptr;
    csl_status st = device_error_ptr(&p);
    if (st) return st;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    e = hipMemcpy(flags, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    uint32_t zero = 0;
    e = hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clear error word)");
    return CSL_OK;
}

csl_status csl_timer_enable(int32_t kid, int32_t on) {
    if (kid < 0 || kid >= kNumKernels) return fail(CSL_EINVAL, "kernel id %d", kid);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_timer[kid].on = on != 0;
    return CSL_OK;
}

csl_status csl_timer_read(int32_t kid, double* total_ms, int64_t* launches) {
    if (kid < 0 || kid >= kNumKernels || !total_ms || !launches) return fail(CSL_EINVAL, "bad timer read");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    std::lock_guard<std::mutex> lk(g_timer_mu);
    Timer& t = g_timer[kid];
    double sum = 0.0;
    const size_t used = t.used;
    t.used = 0;  // reset even if a query below fails, so later reads start clean
    for (size_t i = 0; i < used; ++i) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, t.ev[i].first, t.ev[i].second);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        sum += ms;
    }
    *total_ms = sum;
    *launches = (int64_t)used;
    return CSL_OK;
}

// Validates an insert batch and fills its kernel arguments (a.total_new = 0:
// nothing to launch).  Launches nothing.
csl_status prepare_inserts(int32_t n_jobs, const csl_insert_job* jobs, const csl_pages* pages, const int64_t* start_pos,
                           const int32_t* cu_new, int32_t total_new, float eps, CompressArgs& a) {
    csl_status st;
    if (n_jobs < 1 || n_jobs > kMaxInsertJobs) return fail(CSL_ERANGE, "n_jobs = %d, supported 1..%d", n_jobs, kMaxInsertJobs);
    if (!jobs) return fail(CSL_EINVAL, "jobs is NULL");
    if ((st = check_pages(pages))) return st;
    if (total_new < 0) return fail(CSL_EINVAL, "total_new < 0");
    if (!start_pos || !cu_new) return fail(CSL_EINVAL, "start_pos or cu_new is NULL");
    if (!(eps >= 0.f)) return fail(CSL_EINVAL, "eps must be >= 0");
    a.total_new = 0;
    a.n_jobs = n_jobs;
    for (int i = 0; i < n_jobs; ++i) {
        const csl_pool* pool = jobs[i].pool;
        if ((st = check_pool(pool, "pool"))) return st;
        if (total_new > 0 && !jobs[i].x) return fail(CSL_EINVAL, "job %d: x is NULL", i);
        if (jobs[i].x && !aligned16(jobs[i].x)) return fail(CSL_EALIGN, "job %d: x is not 16-byte aligned", i);
        if (pool->ratio == 1) {
            if (jobs[i].logits || jobs[i].gain)
                return fail(CSL_EINVAL, "job %d: ratio-1 (raw window) inserts take no logits and no gain", i);
        } else {
            if (!pool->state_x || !pool->state_logits)
                return fail(CSL_EINVAL, "job %d: ratio > 1 needs the compressor state", i);
            if (total_new > 0 && !jobs[i].logits) return fail(CSL_EINVAL, "job %d: logits is NULL", i);
        }
        CompressJob& J = a.job[i];
        J.rows = static_cast<uint8_t*>(pool->rows);
        J.state_x = static_cast<uint16_t*>(pool->state_x);
        J.state_logits = pool->state_logits;
        J.x = jobs[i].x;
        J.logits = jobs[i].logits;
        J.gain = jobs[i].gain;
        J.ratio = pool->ratio;
        J.coff = pool->coff;
        J.dim = pool->dim;
        J.rope_dims = pool->rope_dims;
        J.dtype = pool->dtype;
        J.num_pages = pool->num_pages;
        J.row_bytes = (int)row_bytes_of(pool->dim, pool->dtype);
        a.rf[i] = make_freqs(pool->rope_dims, pool->rope_theta);
    }
    if (total_new == 0) return CSL_OK;
    a.bt = pages->block_table;
    a.start_pos = start_pos;
    a.cu_new = cu_new;
    a.err = nullptr;  // set by the caller once every check has passed
    a.num_seqs = pages->num_seqs;
    a.max_blocks = pages->max_blocks;
    a.total_new = total_new;
    a.eps = eps;
    return CSL_OK;
}

csl_status csl_compress_insert_multi(int32_t n_jobs, const csl_insert_job* jobs, const csl_pages* pages,
                                     const int64_t* start_pos, const int32_t* cu_new, int32_t total_new, float eps,
                                     csl_stream_t stream) {
    CompressArgs a;
    csl_status st = prepare_inserts(n_jobs, jobs, pages, start_pos, cu_new, total_new, eps, a);
    if (st || a.total_new == 0) return st;
    if ((st = device_error_ptr(&a.err))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(CSL_KERNEL_COMPRESS, s, [&](const LaunchEvents& ev) { return launch_compress(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "compress_insert launch");
    return CSL_OK;
}

csl_status csl_compress_insert(const csl_pool* pool, const csl_pages* pages, const int64_t* start_pos,
                               const int32_t* cu_new, int32_t total_new, const uint16_t* x, const float* logits,
                               const float* gain, float eps, csl_stream_t stream) {
    csl_insert_job job = {pool, x, logits, gain};
    return csl_compress_insert_multi(1, &job, pages, start_pos, cu_new, total_new, eps, stream);
}

// Validates a query-side batch and fills its kernel arguments (a.n_items = 0:
// nothing to launch; a.err set by the caller).  Launches nothing.
csl_status prepare_qside(const csl_pool* swa, const csl_pages* pages, const int64_t* start_pos, const int32_t* cu_new,
                         int32_t total_new, const uint16_t* x, const uint16_t* q, int32_t n_heads, const float* q_gain,
                         float eps, uint16_t* q_out, QSideArgs& a) {
    csl_status st;
    a.n_items = 0;
    if ((st = check_pool(swa, "swa"))) return st;
    if ((st = check_pages(pages))) return st;
    if (swa->ratio != 1) return fail(CSL_EINVAL, "swa.ratio must be 1 (raw window keys)");
    if (swa->dtype == CSL_MXFP4) return fail(CSL_EUNSUPPORTED, "raw window keys are bf16 or fp8, not fp4");
    if (n_heads < 1 || n_heads > 1024) return fail(CSL_ERANGE, "n_heads = %d, supported 1..1024", n_heads);
    if (total_new < 0) return fail(CSL_EINVAL, "total_new < 0");
    if (!(eps >= 0.f)) return fail(CSL_EINVAL, "eps must be >= 0");
    if (!start_pos || !cu_new) return fail(CSL_EINVAL, "start_pos or cu_new is NULL");
    if (total_new == 0) return CSL_OK;
    if (!x || !q || !q_out) return fail(CSL_EINVAL, "x, q or q_out is NULL");
    if (!aligned16(x) || !aligned16(q) || !aligned16(q_out)) return fail(CSL_EALIGN, "x, q and q_out must be 16-byte aligned");
    const int64_t n_q_rows = (int64_t)total_new * n_heads;
    const int64_t n_items = n_q_rows + total_new;
    if ((n_items + 15) / 16 > 0x7fffffff) return fail(CSL_ERANGE, "total_new * (n_heads + 1) too large");
    if (q_out != q) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(q), b0 = reinterpret_cast<uintptr_t>(q_out);
        const uintptr_t len = (uintptr_t)n_q_rows * swa->dim * 2;
        if (a0 < b0 + len && b0 < a0 + len) return fail(CSL_EINVAL, "q_out overlaps q without being equal to it");
    }
    a.q = q;
    a.q_out = q_out;
    a.x = x;
    a.gain = q_gain;
    a.rows = static_cast<uint8_t*>(swa->rows);
    a.bt = pages->block_table;
    a.start_pos = start_pos;
    a.cu_new = cu_new;
    a.err = nullptr;
    a.n_q_rows = n_q_rows;
    a.n_items = n_items;
    a.n_heads = n_heads;
    a.dim = swa->dim;
    a.rope_dims = swa->rope_dims;
    a.dtype = swa->dtype;
    a.num_pages = swa->num_pages;
    a.row_bytes = (int)row_bytes_of(swa->dim, swa->dtype);
    a.num_seqs = pages->num_seqs;
    a.max_blocks = pages->max_blocks;
    a.eps = eps;
    a.rf = make_freqs(swa->rope_dims, swa->rope_theta);
    return CSL_OK;
}

csl_status csl_q_norm_rope_insert(const csl_pool* swa, const csl_pages* pages, const int64_t* start_pos,
                                  const int32_t* cu_new, int32_t total_new, const uint16_t* x, const uint16_t* q,
                                  int32_t n_heads, const float* q_gain, float eps, uint16_t* q_out,
                                  csl_stream_t stream) {
    QSideArgs a;
    csl_status st = prepare_qside(swa, pages, start_pos, cu_new, total_new, x, q, n_heads, q_gain, eps, q_out, a);
    if (st || a.n_items == 0) return st;
    if ((st = device_error_ptr(&a.err))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(CSL_KERNEL_QSIDE, s, [&](const LaunchEvents& ev) { return launch_qside(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "q_norm_rope_insert launch");
    return CSL_OK;
}

size_t csl_index_topk_workspace(int32_t num_q, int64_t max_q_pos, int32_t k) {
    if (num_q <= 0 || max_q_pos < 0 || k < 1) return 0;
    const int64_t stride = index_stride(max_q_pos), nchunks = stride / kIndexChunk;
    const int kl = index_local_k(max_q_pos, k);
    return (size_t)num_q * ((size_t)stride * sizeof(float) + (kl > 0 ? (size_t)nchunks * (kl + 1) * 8 : 0));
}

// Validates an indexer call and fills its kernel arguments (a.num_q = 0:
// nothing to launch).  Launches nothing.
csl_status prepare_index(const csl_pool* index_pool, const csl_pages* pages, int32_t num_q, const int32_t* q_seq,
                         const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q_idx, const float* w,
                         int32_t n_heads, int32_t k, int32_t* topk, float* kth_score, void* ws, size_t ws_bytes,
                         IndexArgs& a) {
    csl_status st;
    a.num_q = 0;
    if ((st = check_pool(index_pool, "index"))) return st;
    if ((st = check_pages(pages))) return st;
    if (index_pool->ratio != 4) return fail(CSL_EUNSUPPORTED, "the indexer runs on ratio-4 (c4a) pools only");
    if (index_pool->dtype != CSL_BF16 && index_pool->dtype != CSL_MXFP4)
        return fail(CSL_EUNSUPPORTED, "index rows must be bf16 or fp4");
    if (index_pool->dim != 32 && index_pool->dim != 64 && index_pool->dim != 128)
        return fail(CSL_EUNSUPPORTED, "index dim %d (supported: 32, 64, 128)", index_pool->dim);
    if (n_heads < 1 || n_heads > 16) return fail(CSL_ERANGE, "index n_heads = %d, supported 1..16", n_heads);
    if (k < 1 || k > 2048) return fail(CSL_ERANGE, "k = %d, supported 1..2048", k);
    if (num_q < 0 || num_q > 65535) return fail(CSL_ERANGE, "num_q = %d, supported 0..65535", num_q);
    if (max_q_pos < 0) return fail(CSL_EINVAL, "max_q_pos < 0");
    if (max_q_pos >= (int64_t)pages->max_blocks * 256 + 1)
        return fail(CSL_ERANGE, "max_q_pos beyond the block table");
    if (num_q == 0) return CSL_OK;
    if (!q_seq || !q_pos || !q_idx || !w || !topk) return fail(CSL_EINVAL, "a required pointer is NULL");
    if (!aligned16(q_idx)) return fail(CSL_EALIGN, "q_idx is not 16-byte aligned");
    size_t need = csl_index_topk_workspace(num_q, max_q_pos, k);
    if (!ws || ws_bytes < need) return fail(CSL_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned16(ws)) return fail(CSL_EALIGN, "ws is not 16-byte aligned");
    a.rows = static_cast<const uint8_t*>(index_pool->rows);
    a.bt = pages->block_table;
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.q_idx = q_idx;
    a.w = w;
    a.scores = static_cast<float*>(ws);
    a.topk = topk;
    a.kth = kth_score;
    a.err = nullptr;  // set by the caller once every check has passed
    a.max_q_pos = max_q_pos;
    a.stride = index_stride(max_q_pos);
    a.nchunks = (int)(a.stride / kIndexChunk);
    a.kl = index_local_k(max_q_pos, k);
    a.tiled = index_use_tiled(num_q) ? 1 : 0;
    a.fp4 = index_pool->dtype == CSL_MXFP4 ? 1 : 0;
    a.cand = reinterpret_cast<uint2*>(a.scores + (size_t)num_q * a.stride);
    a.c_next = a.cand + (size_t)num_q * a.nchunks * a.kl;
    a.num_q = num_q;
    a.n_heads = n_heads;
    a.dim = index_pool->dim;
    a.k = k;
    a.num_pages = index_pool->num_pages;
    a.num_seqs = pages->num_seqs;
    a.max_blocks = pages->max_blocks;
    return CSL_OK;
}

csl_status csl_index_topk(const csl_pool* index_pool, const csl_pages* pages, int32_t num_q, const int32_t* q_seq,
                          const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q_idx, const float* w,
                          int32_t n_heads, int32_t k, int32_t* topk, float* kth_score, void* ws, size_t ws_bytes,
                          csl_stream_t stream) {
    IndexArgs a;
    csl_status st = prepare_index(index_pool, pages, num_q, q_seq, q_pos, max_q_pos, q_idx, w, n_heads, k, topk,
                                  kth_score, ws, ws_bytes, a);
    if (st || a.num_q == 0) return st;
    if ((st = device_error_ptr(&a.err))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(CSL_KERNEL_INDEX_SCORE, s, [&](const LaunchEvents& ev) { return launch_index_score(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "index_score launch");
    e = timed(CSL_KERNEL_TOPK_SELECT, s, [&](const LaunchEvents& ev) { return launch_topk_select(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "topk_select launch");
    return CSL_OK;
}

csl_status csl_index_topk_insert(const csl_pool* index_pool, const csl_pages* pages, int32_t num_q,
                                 const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q_idx,
                                 const float* w, int32_t n_heads, int32_t k, int32_t* topk, float* kth_score,
                                 void* ws, size_t ws_bytes, int32_t n_jobs, const csl_insert_job* jobs,
                                 const int64_t* start_pos, const int32_t* cu_new, int32_t total_new, float eps,
                                 const csl_qside_job* qside, csl_stream_t stream) {
    IndexArgs a;
    CompressArgs c;
    QSideArgs q;
    csl_status st = prepare_index(index_pool, pages, num_q, q_seq, q_pos, max_q_pos, q_idx, w, n_heads, k, topk,
                                  kth_score, ws, ws_bytes, a);
    if (st) return st;
    c.total_new = 0;
    c.n_jobs = 0;
    if (n_jobs != 0 || !qside) {
        if ((st = prepare_inserts(n_jobs, jobs, pages, start_pos, cu_new, total_new, eps, c))) return st;
    }
    q.n_items = 0;
    if (qside && (st = prepare_qside(qside->swa, pages, start_pos, cu_new, total_new, qside->x, qside->q,
                                     qside->n_heads, qside->q_gain, eps, qside->q_out, q)))
        return st;
    if (qside) {
        for (int i = 0; i < n_jobs; ++i)
            if (jobs[i].pool->rows == qside->swa->rows)
                return fail(CSL_EINVAL, "job %d inserts into the query side's raw pool", i);
    }
    if (a.num_q == 0 && c.total_new == 0 && q.n_items == 0) return CSL_OK;
    uint32_t* err = nullptr;
    if ((st = device_error_ptr(&err))) return st;
    a.err = err;
    c.err = err;
    q.err = err;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (a.num_q > 0) {
        e = timed(CSL_KERNEL_INDEX_SCORE, s, [&](const LaunchEvents& ev) { return launch_index_score(a, s, ev); });
        if (e != hipSuccess) return hip_fail(e, "index_score launch");
    }
    if (c.total_new == 0 && q.n_items == 0) {
        if (a.num_q > 0) e = timed(CSL_KERNEL_TOPK_SELECT, s, [&](const LaunchEvents& ev) { return launch_topk_select(a, s, ev); });
    } else {
        e = timed(CSL_KERNEL_TOPK_SELECT, s, [&](const LaunchEvents& ev) { return launch_topk_select_insert(a, c, q, s, ev); });
    }
    if (e != hipSuccess) return hip_fail(e, "topk_select / insert launch");
    return CSL_OK;
}

size_t csl_hybrid_attn_workspace(int32_t num_q, int32_t n_heads, int32_t dim, int32_t comp_ratio, int32_t k,
                                 int32_t swa_window, int64_t max_q_pos) {
    return attn_ws_bytes(num_q, n_heads, dim, comp_ratio, k, swa_window, max_q_pos);
}

}  // extern "C"

namespace {

// csl_hybrid_attn_decode, and with `ins` (inserts prepared by prepare_inserts,
// total_new > 0) csl_hybrid_attn_decode_insert: on decode_attn_kernel the
// inserts run as extra workgroups of the attention launch, otherwise in a
// launch of their own before it.  Validation precedes every launch.
csl_status hybrid_decode(const csl_pool* comp, const csl_pool* swa, const csl_pages* pages, int32_t num_q,
                         const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q,
                         int32_t n_heads, const int32_t* topk, int32_t k, int32_t swa_window, float softmax_scale,
                         int32_t out_dtype, void* out, float* out_scales, void* ws, size_t ws_bytes,
                         CompressArgs* ins, csl_stream_t stream) {
    if (num_q == 0 && !ins) return CSL_OK;
    csl_status st;
    hipError_t e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto inserts_alone = [&]() -> csl_status {
        if (!ins) return CSL_OK;
        e = timed(CSL_KERNEL_COMPRESS, s, [&](const LaunchEvents& ev) { return launch_compress(*ins, s, ev); });
        return e == hipSuccess ? CSL_OK : hip_fail(e, "compress_insert launch");
    };
    uint32_t* err = nullptr;
    if (num_q == 0) {
        if ((st = device_error_ptr(&err))) return st;
        ins->err = err;
        return inserts_alone();
    }
    if ((st = check_attn_common(comp, swa, pages, n_heads, topk, k, swa_window, out_dtype, out, out_scales, q,
                                max_q_pos, softmax_scale)))
        return st;
    if (!q_seq || !q_pos) return fail(CSL_EINVAL, "q_seq or q_pos is NULL");
    const int cr = comp ? comp->ratio : 0;
    const int kk = topk ? k : 0;
    size_t need = csl_hybrid_attn_workspace(num_q, n_heads, swa->dim, cr, kk, swa_window, max_q_pos);
    if (need > 0 && (!ws || ws_bytes < need)) return fail(CSL_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (need > 0 && !aligned16(ws)) return fail(CSL_EALIGN, "ws is not 16-byte aligned");
    if ((st = device_error_ptr(&err))) return st;
    if (ins) ins->err = err;
    AttnArgs a;
    fill_attn(a, comp, swa, pages, n_heads, topk, k, swa_window, softmax_scale, out_dtype, out, out_scales, q,
              max_q_pos, err);
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.cu_q = nullptr;
    a.q_pos_start = nullptr;
    a.num_q = num_q;
    float* part = need > 0 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
    if (use_decode_kernel(swa->dim, swa->dtype)) {
        const DecodePlan pl = decode_plan(num_q, n_heads, cr, kk, swa_window, max_q_pos);
        if ((int64_t)(num_q * (int64_t)pl.S + 7) / 8 * 8 * pl.G > 0x7fffffff) return fail(CSL_ERANGE, "grid too large");
        DecodeArgs d;
        d.at = a;
        d.G = pl.G;
        d.S = pl.S;
        d.per = pl.per;
        d.combine = pl.combine;
        d.cnt = static_cast<uint32_t*>(ws);
        d.cand = nullptr;
        d.c_next = nullptr;
        d.scores = nullptr;
        d.stride = 0;
        d.nchunks = 0;
        d.kl = 0;
        d.topk_out = nullptr;
        d.kth = nullptr;
        d.at.n_splits = pl.S;
        if (pl.S > 1) {
            d.at.part_o = part;
            d.at.part_ml = part + (size_t)num_q * pl.S * n_heads * swa->dim;
        }
        CompressArgs none;
        none.total_new = 0;
        none.n_jobs = 0;
        const CompressArgs& ride = ins ? *ins : none;
        e = timed(CSL_KERNEL_ATTN, s, [&](const LaunchEvents& ev) { return launch_decode_attn(d, ride, s, ev); });
        if (e != hipSuccess) return hip_fail(e, "decode_attn launch");
        if (pl.S > 1 && !pl.combine) {
            e = timed(CSL_KERNEL_ATTN_COMBINE, s, [&](const LaunchEvents& ev) { return launch_attn_combine(d.at, s, ev); });
            if (e != hipSuccess) return hip_fail(e, "attn_combine launch");
        }
        return CSL_OK;
    }
    const int sp = decode_splits(num_q, cr, kk, swa_window, max_q_pos, swa->dtype == CSL_FP8_E4M3);
    if ((int64_t)num_q * sp > 0x7fffffff) return fail(CSL_ERANGE, "grid too large");
    if ((st = inserts_alone())) return st;
    a.n_splits = sp;
    a.tiles_per_split = (decode_tiles(cr, kk, swa_window, max_q_pos) + sp - 1) / sp;
    if (sp > 1) {
        a.part_o = part;
        a.part_ml = a.part_o + (size_t)num_q * sp * n_heads * swa->dim;
    }
    e = timed(CSL_KERNEL_ATTN, s, [&](const LaunchEvents& ev) { return launch_attn(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "hybrid_attn launch");
    if (sp > 1) {
        e = timed(CSL_KERNEL_ATTN_COMBINE, s, [&](const LaunchEvents& ev) { return launch_attn_combine(a, s, ev); });
        if (e != hipSuccess) return hip_fail(e, "attn_combine launch");
    }
    return CSL_OK;
}

}  // namespace

extern "C" {

csl_status csl_hybrid_attn_decode(const csl_pool* comp, const csl_pool* swa, const csl_pages* pages, int32_t num_q,
                                  const int32_t* q_seq, const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q,
                                  int32_t n_heads, const int32_t* topk, int32_t k, int32_t swa_window,
                                  float softmax_scale, int32_t out_dtype, void* out, float* out_scales, void* ws,
                                  size_t ws_bytes, csl_stream_t stream) {
    if (num_q < 0) return fail(CSL_EINVAL, "num_q < 0");
    return hybrid_decode(comp, swa, pages, num_q, q_seq, q_pos, max_q_pos, q, n_heads, topk, k, swa_window,
                         softmax_scale, out_dtype, out, out_scales, ws, ws_bytes, nullptr, stream);
}

csl_status csl_hybrid_attn_decode_insert(const csl_pool* comp, const csl_pool* swa, const csl_pages* pages,
                                         int32_t num_q, const int32_t* q_seq, const int64_t* q_pos,
                                         int64_t max_q_pos, const uint16_t* q, int32_t n_heads, const int32_t* topk,
                                         int32_t k, int32_t swa_window, float softmax_scale, int32_t out_dtype,
                                         void* out, float* out_scales, int32_t n_jobs, const csl_insert_job* jobs,
                                         const int64_t* start_pos, const int32_t* cu_new, int32_t total_new,
                                         float eps, void* ws, size_t ws_bytes, csl_stream_t stream) {
    if (num_q < 0) return fail(CSL_EINVAL, "num_q < 0");
    CompressArgs c;
    csl_status st = prepare_inserts(n_jobs, jobs, pages, start_pos, cu_new, total_new, eps, c);
    if (st) return st;
    return hybrid_decode(comp, swa, pages, num_q, q_seq, q_pos, max_q_pos, q, n_heads, topk, k, swa_window,
                         softmax_scale, out_dtype, out, out_scales, ws, ws_bytes, c.total_new > 0 ? &c : nullptr,
                         stream);
}

// Workspace of csl_index_attn_decode: [counters | attention partials | index scores and candidates].
size_t fused_attn_part(int32_t num_q, int32_t n_heads, int64_t max_q_pos, int32_t k, int32_t swa_window) {
    const DecodePlan pl = decode_plan(num_q, n_heads, 4, k, swa_window, max_q_pos);
    return kCounterBytes + (partial_bytes(num_q, pl.S, n_heads, 512) + 255) / 256 * 256;
}

size_t csl_index_attn_decode_workspace(int32_t num_q, int32_t n_heads, int64_t max_q_pos, int32_t k,
                                       int32_t swa_window) {
    if (num_q <= 0 || n_heads <= 0 || max_q_pos < 0 || k < 1) return 0;
    return fused_attn_part(num_q, n_heads, max_q_pos, k, swa_window) + csl_index_topk_workspace(num_q, max_q_pos, k);
}

csl_status csl_index_attn_decode(const csl_pool* index_pool, const csl_pool* comp, const csl_pool* swa,
                                 const csl_pages* pages, int32_t num_q, const int32_t* q_seq, const int64_t* q_pos,
                                 int64_t max_q_pos, const uint16_t* q_idx, const float* w, int32_t n_idx_heads,
                                 int32_t k, int32_t* topk, float* kth_score, const uint16_t* q, int32_t n_heads,
                                 int32_t swa_window, float softmax_scale, int32_t out_dtype, void* out,
                                 float* out_scales, int32_t n_jobs, const csl_insert_job* jobs,
                                 const int64_t* start_pos, const int32_t* cu_new, int32_t total_new, float eps,
                                 const csl_qside_job* qside, void* ws, size_t ws_bytes, csl_stream_t stream) {
    csl_status st;
    if (num_q < 0) return fail(CSL_EINVAL, "num_q < 0");
    if (!comp) return fail(CSL_EINVAL, "the fused decode call needs the compressed pool");
    if ((st = check_attn_common(comp, swa, pages, n_heads, topk, k, swa_window, out_dtype, out, out_scales, q,
                                max_q_pos, softmax_scale)))
        return st;
    if (comp->ratio != 4) return fail(CSL_EINVAL, "comp.ratio must be 4: the indexer selects c4a entries");
    if (!use_decode_kernel(swa->dim, swa->dtype))
        return fail(CSL_EUNSUPPORTED, "the fused decode call takes 512-dim bf16 or fp8 keys");
    if (!topk) return fail(CSL_EINVAL, "topk is NULL");
    const size_t need = csl_index_attn_decode_workspace(num_q, n_heads, max_q_pos, k, swa_window);
    if (num_q > 0 && (!ws || ws_bytes < need)) return fail(CSL_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (ws && !aligned16(ws)) return fail(CSL_EALIGN, "ws is not 16-byte aligned");
    const size_t attn_part = num_q > 0 ? fused_attn_part(num_q, n_heads, max_q_pos, k, swa_window) : 0;
    IndexArgs ia;
    CompressArgs c;
    QSideArgs qa;
    if ((st = prepare_index(index_pool, pages, num_q, q_seq, q_pos, max_q_pos, q_idx, w, n_idx_heads, k, topk,
                            kth_score, num_q > 0 ? static_cast<uint8_t*>(ws) + attn_part : nullptr,
                            num_q > 0 ? ws_bytes - attn_part : 0, ia)))
        return st;
    c.total_new = 0;
    c.n_jobs = 0;
    if (n_jobs != 0) {
        if ((st = prepare_inserts(n_jobs, jobs, pages, start_pos, cu_new, total_new, eps, c))) return st;
    }
    // inserts into the index pool ride in the attention launch, which never reads index rows;
    // the others (raw window, main) ride in the score launch, which reads only index rows
    CompressArgs ci;
    ci.total_new = 0;
    ci.n_jobs = 0;
    if (c.total_new > 0) {
        ci = c;
        int nk = 0, ni = 0;
        for (int i = 0; i < c.n_jobs; ++i) {
            const bool to_index = jobs[i].pool->rows == index_pool->rows;
            CompressArgs& dst = to_index ? ci : c;
            int& m = to_index ? ni : nk;
            dst.job[m] = c.job[i];
            dst.rf[m] = c.rf[i];
            ++m;
        }
        c.n_jobs = nk;
        ci.n_jobs = ni;
        if (nk == 0) c.total_new = 0;
        if (ni == 0) ci.total_new = 0;
        if (ia.num_q == 0 && ni > 0) {  // no attention launch to carry them
            for (int i = 0; i < ni; ++i) {
                c.job[c.n_jobs] = ci.job[i];
                c.rf[c.n_jobs] = ci.rf[i];
                ++c.n_jobs;
            }
            c.total_new = ci.total_new;
            ci.total_new = 0;
            ci.n_jobs = 0;
        }
    }
    qa.n_items = 0;
    if (qside && (st = prepare_qside(qside->swa, pages, start_pos, cu_new, total_new, qside->x, qside->q,
                                     qside->n_heads, qside->q_gain, eps, qside->q_out, qa)))
        return st;
    if (qside) {
        for (int i = 0; i < n_jobs; ++i)
            if (jobs[i].pool->rows == qside->swa->rows)
                return fail(CSL_EINVAL, "job %d inserts into the query side's raw pool", i);
    }
    if (ia.num_q == 0 && c.total_new == 0 && ci.total_new == 0 && qa.n_items == 0) return CSL_OK;
    uint32_t* err = nullptr;
    if ((st = device_error_ptr(&err))) return st;
    ia.err = err;
    c.err = err;
    ci.err = err;
    qa.err = err;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(CSL_KERNEL_INDEX_SCORE, s, [&](const LaunchEvents& ev) {
        return launch_index_score_insert(ia, c, qa, s, ev);
    });
    if (e != hipSuccess) return hip_fail(e, "index_score launch");
    if (ia.num_q == 0) return CSL_OK;
    // the attention launch merges up to 2048 candidate slots per query (8 per thread); every
    // workgroup of a query repeats the merge, which past that size costs more than the select
    // launch (1M positions, 4096 slots: 29.3 us fused against 8.9 + 15.4 us)
    const bool merge = ia.kl > 0 && !ia.tiled && (int64_t)ia.nchunks * ia.kl <= kDecodeMergeSlots;
    if (!merge) {
        // no first-stage candidates (short rows or many queries) or too many: the select launch,
        // then attention on its ids
        e = timed(CSL_KERNEL_TOPK_SELECT, s, [&](const LaunchEvents& ev) { return launch_topk_select(ia, s, ev); });
        if (e != hipSuccess) return hip_fail(e, "topk_select launch");
    }
    AttnArgs a;
    fill_attn(a, comp, swa, pages, n_heads, topk, k, swa_window, softmax_scale, out_dtype, out, out_scales, q,
              max_q_pos, err);
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.cu_q = nullptr;
    a.q_pos_start = nullptr;
    a.num_q = num_q;
    const DecodePlan pl = decode_plan(num_q, n_heads, 4, k, swa_window, max_q_pos);
    DecodeArgs d;
    d.at = a;
    d.G = pl.G;
    d.S = pl.S;
    d.per = pl.per;
    d.combine = pl.combine;
    d.cnt = static_cast<uint32_t*>(ws);
    d.cand = merge ? ia.cand : nullptr;
    d.c_next = ia.c_next;
    d.scores = ia.scores;
    d.stride = ia.stride;
    d.nchunks = ia.nchunks;
    d.kl = ia.kl;
    d.topk_out = topk;
    d.kth = kth_score;
    if (merge) d.at.topk = nullptr;  // the ids come from the merge in the launch
    d.at.n_splits = pl.S;
    if (pl.S > 1) {
        float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes);
        d.at.part_o = part;
        d.at.part_ml = part + (size_t)num_q * pl.S * n_heads * 512;
    }
    e = timed(CSL_KERNEL_ATTN, s, [&](const LaunchEvents& ev) { return launch_decode_attn(d, ci, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "decode_attn launch");
    if (pl.S > 1 && !pl.combine) {
        e = timed(CSL_KERNEL_ATTN_COMBINE, s, [&](const LaunchEvents& ev) { return launch_attn_combine(d.at, s, ev); });
        if (e != hipSuccess) return hip_fail(e, "attn_combine launch");
    }
    return CSL_OK;
}

csl_status csl_index_attn_decode_noalloc(const csl_pool* index_pool, const csl_pool* comp, const csl_pool* swa,
                                         const csl_pages* pages, int32_t num_q, const int32_t* q_seq,
                                         const int64_t* q_pos, int64_t max_q_pos, const uint16_t* q_idx,
                                         const float* w, int32_t n_idx_heads, int32_t k, int32_t* topk,
                                         float* kth_score, const uint16_t* q, int32_t n_heads, int32_t swa_window,
                                         float softmax_scale, int32_t out_dtype, void* out, float* out_scales,
                                         int32_t n_jobs, const csl_insert_job* jobs, const int64_t* start_pos,
                                         const int32_t* cu_new, int32_t total_new, float eps,
                                         const csl_qside_job* qside, csl_stream_t stream) {
    if (num_q < 0) return fail(CSL_EINVAL, "num_q < 0");
    const size_t need = csl_index_attn_decode_workspace(num_q, n_heads, max_q_pos, k, swa_window);
    if (need > kStaticScratchBytes)
        return fail(CSL_ERANGE, "the call needs %zu bytes of scratch, the static scratch holds %zu", need,
                    kStaticScratchBytes);
    void* ws = nullptr;
    csl_status st;
    if ((st = static_scratch(static_cast<hipStream_t>(stream), &ws))) return st;
    return csl_index_attn_decode(index_pool, comp, swa, pages, num_q, q_seq, q_pos, max_q_pos, q_idx, w, n_idx_heads,
                                 k, topk, kth_score, q, n_heads, swa_window, softmax_scale, out_dtype, out,
                                 out_scales, n_jobs, jobs, start_pos, cu_new, total_new, eps, qside, ws,
                                 kStaticScratchBytes, stream);
}

csl_status csl_hybrid_attn_prefill(const csl_pool* comp, const csl_pool* swa, const csl_pages* pages,
                                   const int32_t* cu_q, const int64_t* q_pos_start, int32_t total_q,
                                   int64_t max_q_pos, const uint16_t* q, int32_t n_heads, const int32_t* topk,
                                   int32_t k, int32_t swa_window, float softmax_scale, int32_t out_dtype, void* out,
                                   float* out_scales, csl_stream_t stream) {
    if (total_q < 0) return fail(CSL_EINVAL, "total_q < 0");
    if (total_q == 0) return CSL_OK;
    csl_status st = check_attn_common(comp, swa, pages, n_heads, topk, k, swa_window, out_dtype, out, out_scales, q,
                                      max_q_pos, softmax_scale);
    if (st) return st;
    if (!cu_q || !q_pos_start) return fail(CSL_EINVAL, "cu_q or q_pos_start is NULL");
    uint32_t* err = nullptr;
    if ((st = device_error_ptr(&err))) return st;
    AttnArgs a;
    fill_attn(a, comp, swa, pages, n_heads, topk, k, swa_window, softmax_scale, out_dtype, out, out_scales, q,
              max_q_pos, err);
    a.q_seq = nullptr;
    a.q_pos = nullptr;
    a.cu_q = cu_q;
    a.q_pos_start = q_pos_start;
    a.num_q = total_q;
    a.n_splits = 1;
    a.tiles_per_split = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(CSL_KERNEL_ATTN, s, [&](const LaunchEvents& ev) { return launch_attn(a, s, ev); });
    if (e != hipSuccess) return hip_fail(e, "hybrid_attn launch");
    return CSL_OK;
}

}  // extern "C"
