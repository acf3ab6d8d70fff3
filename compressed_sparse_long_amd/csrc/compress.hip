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
// stores the token's row.  The stand-alone launch gives pools whose window
// holds at most 64 tokens (raw rows, c4a) one wave per token instead, four
// tokens to a workgroup, with the same arithmetic: the per-token work is a
// few dependent memory round trips, and a quarter of the workgroups carry it.
// A lane owns 8 consecutive dims (one 16-byte
// load/store per row), so a wave covers a row of up to 512 dims and RoPE pairs
// never straddle lanes.  Elementwise and HBM-bound: no MFMA.
#include "csl_insert.hpp"

namespace csl {

namespace {

// Which jobs take a wave per token and which a workgroup per token.
struct InsertSplit {
    int n_wave, n_block;
    int wave_job[kMaxInsertJobs], block_job[kMaxInsertJobs];
};

// grid.x: groups of four tokens; grid.y: one row per wave-per-token job, then
// four rows per workgroup-per-token job (token 4 x + row % 4).
__global__ void __launch_bounds__(kThreads) compress_insert_kernel(CompressArgs args, InsertSplit sp) {
    __shared__ InsertSmem sm;
    const int y = blockIdx.y;
    if (y < sp.n_wave) {
        const int64_t j = 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
        if (j < args.total_new) insert_wave(args, sp.wave_job[y], (int)j);
        return;
    }
    const int yb = y - sp.n_wave;
    const int64_t j = 4 * (int64_t)blockIdx.x + (yb & 3);
    if (j < args.total_new) insert_block(args, sp.block_job[yb >> 2], (int)j, sm);
}

template <int kQItems>
__global__ void __launch_bounds__(kThreads) q_norm_rope_insert_kernel(QSideArgs a) {
    qside_block<kQItems>(a, blockIdx.x);
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
    InsertSplit sp;
    sp.n_wave = sp.n_block = 0;
    for (int i = 0; i < a.n_jobs; ++i) {
        const CompressJob& J = a.job[i];
        if (J.ratio == 1 || J.coff * J.ratio <= kWaveWindow) sp.wave_job[sp.n_wave++] = i;
        else sp.block_job[sp.n_block++] = i;
    }
    launch_kernel(ev, true, true, compress_insert_kernel,
                  dim3((unsigned)((a.total_new + 3) / 4), (unsigned)(sp.n_wave + 4 * sp.n_block)), dim3(kThreads), st,
                  a, sp);
    return hipGetLastError();
}

}  // namespace csl
