/*
 * csl_oracle.c -- plain CPU oracle for hybrid compressed attention on a
 * shared-K/V latent cache (c4a / c128a compression, DSA top-k, a 128-token
 * raw sliding window, one softmax, inverse RoPE, optional fp8).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product library
 * (compressed_sparse_long_amd) never calls it, and the two share no source:
 * no headers, codecs, tables or helpers.
 *
 * Style: scalar loops in the order the pages state the method, fp64
 * arithmetic throughout, rounding to a storage format (bf16, e4m3) only where
 * a cache row or an output is stored.  OpenMP runs independent queries (or
 * independent sequences) in parallel and changes no arithmetic.
 *
 * Pages cited (title, then the section named at each use):
 *   [Notes]   "DeepSeek V4 in vLLM 技术博客详尽笔记"
 *   [Summary] "vLLM DeepSeek V4 支援：高效長上下文注意力"
 *   [Serving] "DeepSeek-V4服务：百万token上下文成为推理系统难题"
 *
 * Where the pages leave a step open or garble it, this file takes the
 * plainest reading the rest supports, named at the code that uses it:
 *   R1  compressed entry i (ratio r) is visible to a query at p iff its last
 *       token is before p: r(i+1) <= p.  (The appendix's "4i < p" / "128i < p"
 *       would let a query see tokens >= p, which the C128A note forbids.)
 *   R2  the raw window is tokens max(0, p-S) .. p-1; a query does not see its
 *       own token.
 *   R3  c4a entry i covers [4i-4, 4i+3] and is rotated at 4i (T/4 entries).
 *   R4  window positions before token 0 are left out of the softmax.
 *   R5  each token carries `coff` logits; window slot k uses column k / r;
 *       the weights are the softmax over the window's logits.
 *   R6  RMSNorm over all dims, eps 1e-6, optional gain, on compressed entries.
 *   R7  RoPE rotates adjacent pairs of the last rope_dims dims by
 *       pos * theta^(-2j/rope_dims); angles in fp64.
 *   R8  the inverse rotation uses the query's position p.
 *   R9  V is the stored (rotated) row itself (K = V).
 *   R10 raw window rows are RoPE(x_t, t), with no norm.
 *   R12 logits are softmax_scale * <q, K>; no sink, no bias.
 *   R13 one softmax over the union of compressed and raw keys.
 *   R14 sigma = sum_h w_h * ReLU(<q_h, k>), no 1/sqrt(d).
 *   R15 top-k ties go to the lower index; fewer than k candidates -> all of
 *       them and -1 padding; ids are emitted in ascending order.
 *   R17 fp8 = OCP e4m3fn, round-to-nearest-even, saturating at 448; one fp32
 *       scale = amax/448 per 64 elements (1 when amax = 0).
 *   R21 the query-side norm is an RMSNorm per head over its dim entries
 *       (eps 1e-6, one optional gain vector shared by the heads); the query
 *       is then rotated at its own token's position with the raw pool's RoPE.
 *   R20 fp4 index rows = OCP MX "MXFP4": blocks of 32 elements share one
 *       E8M0 scale 2^(floor(log2 amax) - 2); elements are E2M1, rounded to
 *       nearest even, saturating at 6; an all-zero block has scale code 0.
 *       The rounding decisions are taken on the fp32 value (the kernel's
 *       precision).
 * Pinned by tests/test_oracle_*.py; numeric values of the full path beyond
 * those pins are "parity unpinned": the pages print no worked example.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_FP8 = 2, O_FP4 = 3 };
#define O_BLOCK 256 /* native positions per logical block, [Notes] 解决方案一：统一逻辑块大小 */

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* Nearest value with `sig` significant bits and exponent >= emin, ties to
 * even (IEEE 754 roundTiesToEven; nearbyint in the default rounding mode). */
static double round_to_format(double v, int sig, int emin)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(fabs(v), &e); /* |v| = m * 2^e, m in [0.5, 1) */
    int ex = e - 1;
    if (ex < emin) ex = emin;
    double quantum = ldexp(1.0, ex - (sig - 1));
    return nearbyint(v / quantum) * quantum;
}

static double bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* bfloat16: 8 significant bits, fp32's exponent range. */
static uint16_t f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    double r = round_to_format(v, 8, -126);
    float f = (float)r; /* exact: r is a bf16 value (or overflows to inf) */
    if (fabs(r) > 3.3895313892515355e38) f = (float)(r > 0 ? INFINITY : -INFINITY);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* OCP 8-bit float E4M3 ("e4m3fn"): bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448. */
static double e4m3_to_f64(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to nearest even, saturating to +-448. */
static uint8_t f64_to_e4m3(double v)
{
    if (isnan(v)) return 0x7F;
    uint8_t s = signbit(v) ? 0x80 : 0;
    double r = fabs(round_to_format(v, 4, -6));
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return s;
    if (r < ldexp(1.0, -6)) return s | (uint8_t)(r / ldexp(1.0, -9));
    int e;
    double m = frexp(r, &e); /* r = m * 2^e, m in [0.5,1) -> r = (2m) * 2^(e-1) */
    int ex = e - 1;
    int mant = (int)((2.0 * m - 1.0) * 8.0);
    return s | (uint8_t)(((ex + 7) << 3) | mant);
}

/* OCP 4-bit float E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent 0 is subnormal (0 or 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static double e2m1_to_f64(int c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* The E2M1 code nearest to v: searched over the eight magnitudes, ties to the
 * even code (mantissa bit 0), anything at or past 6 saturating to 6. */
static int f64_to_e2m1(double v)
{
    int s = signbit(v) ? 8 : 0;
    double r = fabs(v), bd = r;
    int best = 0;
    for (int c = 1; c < 8; c++) {
        double d = fabs(r - e2m1_to_f64(c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return s | best;
}

/* One 32-element MXFP4 block: 16 code bytes (element 2i in the low nibble of
 * byte i) and the E8M0 scale code (value 2^(code - 127)). */
static void mxfp4_block(const double* y, uint8_t* codes, uint8_t* scale)
{
    float v[32];
    double amax = 0.0;
    for (int i = 0; i < 32; i++) {
        v[i] = (float)y[i];
        if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
    }
    memset(codes, 0, 16);
    if (amax == 0.0) {
        *scale = 0;
        return;
    }
    int e;
    frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
    int sh = (e - 1) - 2;
    if (sh < -127) sh = -127;
    if (sh > 127) sh = 127;
    *scale = (uint8_t)(sh + 127);
    for (int i = 0; i < 32; i++) codes[i / 2] |= (uint8_t)(f64_to_e2m1(ldexp((double)v[i], -sh)) << (4 * (i & 1)));
}

/* Bytes of one stored row: bf16 = 2 per element; fp8 = one code per
 * element followed by one fp32 scale per 64 elements; fp4 = a nibble per
 * element followed by one E8M0 byte per 32 elements; f32 = 4 per element. */
int64_t csl_oracle_row_bytes(int dim, int dtype)
{
    if (dtype == O_BF16) return 2 * (int64_t)dim;
    if (dtype == O_FP8) return (int64_t)dim + 4 * (int64_t)(dim / 64);
    if (dtype == O_FP4) return (int64_t)dim / 2 + (int64_t)(dim / 32);
    return 4 * (int64_t)dim;
}

/* Quantise one 64-element group: scale = fp32(amax / 448) (1 when amax = 0),
 * code = e4m3(y / scale).  Returns the scale. */
static float fp8_group(const double* y, uint8_t* codes)
{
    double amax = 0.0;
    for (int i = 0; i < 64; i++)
        if (fabs(y[i]) > amax) amax = fabs(y[i]);
    float scale = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    for (int i = 0; i < 64; i++) codes[i] = f64_to_e4m3(y[i] / (double)scale);
    return scale;
}

static void store_row(uint8_t* dst, const double* y, int dim, int dtype)
{
    if (dtype == O_BF16) {
        uint16_t* d = (uint16_t*)dst;
        for (int i = 0; i < dim; i++) d[i] = f64_to_bf16(y[i]);
    } else if (dtype == O_FP8) {
        float* scales = (float*)(dst + dim);
        for (int g = 0; g < dim / 64; g++) {
            float sc = fp8_group(y + 64 * g, dst + 64 * g);
            memcpy(&scales[g], &sc, 4);
        }
    } else if (dtype == O_FP4) {
        for (int b = 0; b < dim / 32; b++) mxfp4_block(y + 32 * b, dst + 16 * b, dst + dim / 2 + b);
    } else {
        float* d = (float*)dst;
        for (int i = 0; i < dim; i++) d[i] = (float)y[i];
    }
}

static void load_row(const uint8_t* src, double* y, int dim, int dtype)
{
    if (dtype == O_BF16) {
        const uint16_t* s = (const uint16_t*)src;
        for (int i = 0; i < dim; i++) y[i] = bf16_to_f64(s[i]);
    } else if (dtype == O_FP8) {
        for (int g = 0; g < dim / 64; g++) {
            float sc;
            memcpy(&sc, src + dim + 4 * g, 4);
            for (int i = 0; i < 64; i++) y[64 * g + i] = e4m3_to_f64(src[64 * g + i]) * (double)sc;
        }
    } else if (dtype == O_FP4) {
        for (int i = 0; i < dim; i++)
            y[i] = ldexp(e2m1_to_f64((src[i / 2] >> (4 * (i & 1))) & 15), (int)src[dim / 2 + i / 32] - 127);
    } else {
        const float* s = (const float*)src;
        for (int i = 0; i < dim; i++) y[i] = s[i];
    }
}

double csl_oracle_bf16_to_f64(uint16_t h) { return bf16_to_f64(h); }
uint16_t csl_oracle_f64_to_bf16(double v) { return f64_to_bf16(v); }
double csl_oracle_e4m3_to_f64(uint8_t c) { return e4m3_to_f64(c); }
uint8_t csl_oracle_f64_to_e4m3(double v) { return f64_to_e4m3(v); }
double csl_oracle_e2m1_to_f64(int c) { return e2m1_to_f64(c); }
int csl_oracle_f64_to_e2m1(double v) { return f64_to_e2m1(v); }
void csl_oracle_mxfp4_block(const double* y, uint8_t* codes, uint8_t* scale) { mxfp4_block(y, codes, scale); }

/* ------------------------------------------------------------------ */
/* RoPE                                                                */
/* ------------------------------------------------------------------ */

/* Rotate the last `rope_dims` entries of v, as adjacent pairs, by the angle
 * pos * theta^(-2j/rope_dims) for pair j (R7: interleaved pairs in the tail;
 * angles in fp64 from the exact integer position).  RoPE^-1(v, p) is this
 * with pos = -p.  [Notes] Inverse RoPE 的数学原理; [Notes] 数学附录精要. */
static void rope(double* v, int dim, int rope_dims, double theta, double pos)
{
    int base = dim - rope_dims;
    for (int j = 0; j < rope_dims / 2; j++) {
        double freq = pow(theta, -2.0 * j / (double)rope_dims);
        double phi = pos * freq;
        double c = cos(phi), s = sin(phi);
        double a = v[base + 2 * j], b = v[base + 2 * j + 1];
        v[base + 2 * j] = a * c - b * s;
        v[base + 2 * j + 1] = a * s + b * c;
    }
}

void csl_oracle_rope(double* v, int dim, int rope_dims, double theta, int64_t pos)
{
    rope(v, dim, rope_dims, theta, (double)pos);
}

/* ------------------------------------------------------------------ */
/* Paged cache                                                         */
/* ------------------------------------------------------------------ */

/* A pool: one page per 256 native positions of a sequence, shared block
 * table for every pool ([Notes] 解决方案一：统一逻辑块大小: a c4a block holds
 * 256/4 = 64 entries, a c128a block 256/128 = 2).  rows: [pages][256/ratio]
 * [row_bytes].  Compressor state, stored like sliding-window KV of raw
 * tokens ([Notes] 解决方案二：压缩器状态滑动窗口化): state_x [pages][256][dim]
 * bf16 and state_logits [pages][256][coff] fp32. */
typedef struct {
    int32_t ratio, coff, dim, rope_dims;
    double rope_theta;
    int32_t dtype, num_pages;
    uint8_t* rows;
    uint16_t* state_x;
    float* state_logits;
} csl_oracle_pool;

/* Page of native position t of sequence s, or -1 if unmapped. */
static int64_t page_of(const int32_t* bt, int max_blocks, int s, int64_t t, int num_pages)
{
    if (t < 0) return -1;
    int64_t b = t / O_BLOCK;
    if (b >= max_blocks) return -1;
    int32_t pg = bt[(int64_t)s * max_blocks + b];
    if (pg < 0 || pg >= num_pages) return -1;
    return pg;
}

/* Row of compressed entry i (ratio r): page of native position r*i, row
 * i mod (256/r).  For r = 1 this is raw token i. */
static uint8_t* entry_row(const csl_oracle_pool* P, const int32_t* bt, int max_blocks, int s, int64_t i)
{
    int per_page = O_BLOCK / P->ratio;
    int64_t pg = page_of(bt, max_blocks, s, i * P->ratio, P->num_pages);
    if (pg < 0) return NULL;
    return P->rows + ((size_t)pg * per_page + (size_t)(i % per_page)) * (size_t)csl_oracle_row_bytes(P->dim, P->dtype);
}

/* ------------------------------------------------------------------ */
/* Step 1: compressor + RMSNorm + RoPE + insert                        */
/* ------------------------------------------------------------------ */

/* Entry i of a pool with ratio r and overlap factor c covers the W = c*r
 * native tokens r(i+1)-W .. r(i+1)-1: for c4a (r=4, c=2) that is
 * [4i-4, 4i+3], for c128a (r=128, c=1) [128i, 128i+127] ([Notes] 数学附录精要:
 * C4A 的精确位置范围 / C128A 的精确位置范围).  Window position k takes the
 * logit column floor(k/r) of its token (R5), weights are the softmax over the
 * window's logits, tokens at negative positions are left out of the softmax
 * (R4).  u = sum_k w_k x_k; y = u / sqrt(mean(u^2) + eps) * gain (R6);
 * then RoPE at position r*i; then the store.  The entry exists once its last
 * token has arrived.  Returns the number of unmapped pages met. */
/* The entry from its window: xr[k] = token r(i+1)-W+k (NULL = masked: a
 * negative position or an unmapped page), lg[k] = that token's logit in
 * column floor(k/r). */
static void entry_from_window(const csl_oracle_pool* P, int64_t i, const uint16_t* const* xr, const double* lg,
                              const float* gain, double eps, double* y)
{
    int W = P->coff * P->ratio, D = P->dim;
    double mx = -INFINITY;
    for (int k = 0; k < W; k++)
        if (xr[k] && lg[k] > mx) mx = lg[k];
    double den = 0.0;
    for (int k = 0; k < W; k++)
        if (xr[k]) den += exp(lg[k] - mx);
    for (int d = 0; d < D; d++) y[d] = 0.0;
    for (int k = 0; k < W && den > 0.0; k++) {
        if (!xr[k]) continue;
        double wk = exp(lg[k] - mx) / den;
        for (int d = 0; d < D; d++) y[d] += wk * bf16_to_f64(xr[k][d]);
    }
    double ms = 0.0;
    for (int d = 0; d < D; d++) ms += y[d] * y[d];
    ms /= D;
    double inv = 1.0 / sqrt(ms + eps);
    for (int d = 0; d < D; d++) y[d] = y[d] * inv * (gain ? (double)gain[d] : 1.0);
    rope(y, D, P->rope_dims, P->rope_theta, (double)((int64_t)P->ratio * i));
}

/* Entry i of sequence s, its window read from the compressor state.
 * Returns the number of unmapped pages met. */
static int compress_entry(const csl_oracle_pool* P, const int32_t* bt, int max_blocks, int s,
                          int64_t i, const float* gain, double eps, double* y)
{
    int r = P->ratio, W = P->coff * P->ratio, D = P->dim;
    double* lg = (double*)malloc(sizeof(double) * W);
    const uint16_t** xr = (const uint16_t**)malloc(sizeof(void*) * W);
    int faults = 0;
    for (int k = 0; k < W; k++) {
        int64_t t = (int64_t)r * (i + 1) - W + k;
        xr[k] = NULL;
        lg[k] = 0.0;
        if (t < 0) continue;                       /* before the sequence: masked */
        int64_t pg = page_of(bt, max_blocks, s, t, P->num_pages);
        if (pg < 0) { faults++; continue; }
        size_t tok = (size_t)pg * O_BLOCK + (size_t)(t % O_BLOCK);
        xr[k] = P->state_x + tok * (size_t)D;
        lg[k] = P->state_logits[tok * (size_t)P->coff + (size_t)(k / r)];
    }
    entry_from_window(P, i, xr, lg, gain, eps, y);
    free(lg);
    free(xr);
    return faults;
}

/* Rows one by one from explicit windows, with no pool state: for each n,
 * entry ids[n] of a pool shaped like P from x_win[n] = its W = coff*ratio
 * window tokens r(i+1)-W .. r(i+1)-1 ([W][dim] bf16; rows at negative
 * positions are ignored) and logits_win[n] = those tokens' logits
 * ([W][coff] fp32; NULL for ratio 1).  Ratio 1: row = RoPE(x_i, i), no norm.
 * out[n] receives the stored row (P->dtype).  The same arithmetic as
 * csl_oracle_compress_insert, for checking sampled entries of a large cache. */
void csl_oracle_compress_rows(const csl_oracle_pool* P, int n, const int64_t* ids, const uint16_t* x_win,
                              const float* logits_win, const float* gain, double eps, uint8_t* out)
{
    int r = P->ratio, W = P->coff * P->ratio, D = P->dim;
    size_t rb = csl_oracle_row_bytes(D, P->dtype);
#pragma omp parallel for schedule(dynamic)
    for (int m = 0; m < n; m++) {
        double* y = (double*)malloc(sizeof(double) * D);
        const uint16_t* xw = x_win + (size_t)m * W * D;
        int64_t i = ids[m];
        if (r == 1) {
            for (int d = 0; d < D; d++) y[d] = bf16_to_f64(xw[d]);
            rope(y, D, P->rope_dims, P->rope_theta, (double)i);
        } else {
            double* lg = (double*)malloc(sizeof(double) * W);
            const uint16_t** xr = (const uint16_t**)malloc(sizeof(void*) * W);
            for (int k = 0; k < W; k++) {
                int64_t t = (int64_t)r * (i + 1) - W + k;
                xr[k] = t < 0 ? NULL : xw + (size_t)k * D;
                lg[k] = t < 0 ? 0.0 : (double)logits_win[((size_t)m * W + k) * P->coff + (size_t)(k / r)];
            }
            entry_from_window(P, i, xr, lg, gain, eps, y);
            free(lg);
            free(xr);
        }
        store_row(out + (size_t)m * rb, y, D, P->dtype);
        free(y);
    }
}

/* compress_insert over a batch of chunks: sequence s receives tokens
 * x[cu_new[s] .. cu_new[s+1]) at native positions start_pos[s] + j.
 *  - ratio 1 (raw sliding-window keys): row t = RoPE(x_t, t), no norm (R10;
 *    [Notes] 融合 3：Q Norm + KV RoPE + K Insert).
 *  - ratio > 1: every token goes into the compressor state; each entry whose
 *    last token arrives in the chunk is computed from the state and stored.
 * Returns the number of faults (unmapped pages, missing state). */
int csl_oracle_compress_insert(const csl_oracle_pool* P, const int32_t* bt, int num_seqs, int max_blocks,
                               const int64_t* start_pos, const int32_t* cu_new, const uint16_t* x,
                               const float* logits, const float* gain, double eps)
{
    int faults = 0;
    int D = P->dim;
#pragma omp parallel for schedule(dynamic) reduction(+ : faults)
    for (int s = 0; s < num_seqs; s++) {
        double* y = (double*)malloc(sizeof(double) * D);
        for (int j = cu_new[s]; j < cu_new[s + 1]; j++) {
            int64_t t = start_pos[s] + (j - cu_new[s]);
            const uint16_t* xj = x + (size_t)j * D;
            if (P->ratio == 1) {
                for (int d = 0; d < D; d++) y[d] = bf16_to_f64(xj[d]);
                rope(y, D, P->rope_dims, P->rope_theta, (double)t);
                uint8_t* row = entry_row(P, bt, max_blocks, s, t);
                if (!row) { faults++; continue; }
                store_row(row, y, D, P->dtype);
                continue;
            }
            int64_t pg = page_of(bt, max_blocks, s, t, P->num_pages);
            if (pg < 0 || !P->state_x || !P->state_logits) { faults++; continue; }
            size_t tok = (size_t)pg * O_BLOCK + (size_t)(t % O_BLOCK);
            memcpy(P->state_x + tok * (size_t)D, xj, sizeof(uint16_t) * (size_t)D);
            for (int c = 0; c < P->coff; c++)
                P->state_logits[tok * (size_t)P->coff + c] = logits[(size_t)j * P->coff + c];
            if ((t + 1) % P->ratio != 0) continue;
            int64_t i = (t + 1) / P->ratio - 1;
            faults += compress_entry(P, bt, max_blocks, s, i, gain, eps, y);
            uint8_t* row = entry_row(P, bt, max_blocks, s, i);
            if (!row) { faults++; continue; }
            store_row(row, y, D, P->dtype);
        }
        free(y);
    }
    return faults;
}

/* ------------------------------------------------------------------ */
/* Query side: Q RMSNorm + Q RoPE beside the raw-key RoPE + insert     */
/* ------------------------------------------------------------------ */

/* The step just before attention, which the pages fuse into one kernel
 * ([Notes] 融合 3：Q Norm + KV RoPE + K Insert; [Summary] Kernel 融合):
 * for new token j of sequence s, at position t = start_pos[s] + (j - cu_new[s]),
 *   - every query head h (R21): y = q[j][h] / sqrt(mean(q[j][h]^2) + eps)
 *     * gain, an RMSNorm over the head's dim entries with one gain vector
 *     shared by all heads (unit when NULL); then y = RoPE(y, t) with the raw
 *     pool's rope_dims and theta (queries and keys rotate alike, so the logit
 *     depends on the query-key distance); stored as bf16 in q_out[j][h];
 *   - the raw key row t = RoPE(x_j, t), exactly the ratio-1 insert above.
 * q, q_out: [total][n_heads][dim] bf16, total = cu_new[num_seqs].  Returns
 * the number of unmapped pages met by the insert (the queries are written
 * regardless). */
int csl_oracle_q_norm_rope_insert(const csl_oracle_pool* swa, const int32_t* bt, int num_seqs, int max_blocks,
                                  const int64_t* start_pos, const int32_t* cu_new, const uint16_t* x,
                                  const uint16_t* q, int n_heads, const float* gain, double eps, uint16_t* q_out)
{
    int D = swa->dim;
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < num_seqs; s++) {
        double* y = (double*)malloc(sizeof(double) * D);
        for (int j = cu_new[s]; j < cu_new[s + 1]; j++) {
            int64_t t = start_pos[s] + (j - cu_new[s]);
            for (int h = 0; h < n_heads; h++) {
                size_t off = ((size_t)j * n_heads + h) * (size_t)D;
                double ms = 0.0;
                for (int d = 0; d < D; d++) {
                    y[d] = bf16_to_f64(q[off + d]);
                    ms += y[d] * y[d];
                }
                ms /= D;
                double inv = 1.0 / sqrt(ms + eps);
                for (int d = 0; d < D; d++) y[d] = y[d] * inv * (gain ? (double)gain[d] : 1.0);
                rope(y, D, swa->rope_dims, swa->rope_theta, (double)t);
                for (int d = 0; d < D; d++) q_out[off + d] = f64_to_bf16(y[d]);
            }
        }
        free(y);
    }
    if (swa->ratio != 1) return -1;
    return csl_oracle_compress_insert(swa, bt, num_seqs, max_blocks, start_pos, cu_new, x, NULL, NULL, eps);
}

/* ------------------------------------------------------------------ */
/* Steps 2-3: DSA indexer scores + causal top-k                        */
/* ------------------------------------------------------------------ */

/* Entry i of ratio r is visible to a query at position p iff its last token
 * r(i+1)-1 is before p, i.e. r(i+1) <= p (R1; [Notes] 数学附录精要: 因果性条件
 * states that the query sees [0, p-1], and ⚠️ 注意：C128A 的因果性约束 that no
 * entry holding position >= p may be seen). */
static int64_t visible_entries(int ratio, int64_t p)
{
    return p <= 0 ? 0 : p / ratio;
}

typedef struct { double s; int64_t i; } scored;

static int by_score_then_index(const void* a, const void* b)
{
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int by_index(const void* a, const void* b)
{
    int64_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* sigma(n, i) = sum_h w[n,h] * max(0, <q_idx[n,h], K_idx[i]>) over visible
 * entries (R14), then the k highest (ties: lower index first; R15), emitted in
 * ascending index order and padded with -1.  ([Summary] DeepSeek V4 注意力架構:
 * DSA attends only to the top-k compressed tokens; [Notes] 压缩参数细节: k = 512
 * for C4A.)  kth_score[n] = sigma of the last selected entry (-inf if none);
 * all_scores[n][i] (optional) = sigma for every visible i < max_cand. */
int csl_oracle_index_topk(const csl_oracle_pool* IP, const int32_t* bt, int max_blocks, int num_q,
                          const int32_t* q_seq, const int64_t* q_pos, const uint16_t* q_idx,
                          const float* w, int n_heads, int k, int32_t* topk, double* kth_score,
                          double* all_scores, int64_t max_cand)
{
    int faults = 0;
    int D = IP->dim;
#pragma omp parallel for schedule(dynamic) reduction(+ : faults)
    for (int n = 0; n < num_q; n++) {
        int64_t nc = visible_entries(IP->ratio, q_pos[n]);
        scored* c = (scored*)malloc(sizeof(scored) * (nc > 0 ? nc : 1));
        double* key = (double*)malloc(sizeof(double) * D);
        int64_t m = 0;
        for (int64_t i = 0; i < nc; i++) {
            const uint8_t* row = entry_row(IP, bt, max_blocks, q_seq[n], i);
            double sigma = 0.0;
            if (!row) { faults++; continue; }
            load_row(row, key, D, IP->dtype);
            for (int h = 0; h < n_heads; h++) {
                const uint16_t* qh = q_idx + ((size_t)n * n_heads + h) * D;
                double dot = 0.0;
                for (int d = 0; d < D; d++) dot += bf16_to_f64(qh[d]) * key[d];
                sigma += (double)w[(size_t)n * n_heads + h] * (dot > 0.0 ? dot : 0.0);
            }
            c[m].s = sigma;
            c[m].i = i;
            m++;
            if (all_scores && i < max_cand) all_scores[(size_t)n * max_cand + i] = sigma;
        }
        if (all_scores)
            for (int64_t i = nc; i < max_cand; i++) all_scores[(size_t)n * max_cand + i] = -INFINITY;
        qsort(c, (size_t)m, sizeof(scored), by_score_then_index);
        int take = m < k ? (int)m : k;
        int32_t* out = topk + (size_t)n * k;
        for (int j = 0; j < take; j++) out[j] = (int32_t)c[j].i;
        qsort(out, (size_t)take, sizeof(int32_t), by_index);
        for (int j = take; j < k; j++) out[j] = -1;
        if (kth_score) kth_score[n] = take > 0 ? c[take - 1].s : -INFINITY;
        free(c);
        free(key);
    }
    return faults;
}

/* ------------------------------------------------------------------ */
/* Steps 4-6: hybrid attention, inverse RoPE, output store             */
/* ------------------------------------------------------------------ */

/* Query n (sequence q_seq[n], position p = q_pos[n]) attends with one softmax
 * (R13) over
 *   - the compressed entries listed in topk[n] (c4a), or, when topk is NULL,
 *     every visible compressed entry (c128a: [Notes] 压缩参数细节 "8192（全注意力）"),
 *   - the raw tokens max(0, p - swa_window) .. p - 1 ([Notes] ⚠️ 注意：C128A 的
 *     因果性约束: the window covers [p-128, p-1]; R2),
 * with K = V = the stored row ([Summary] DeepSeek V4 注意力架構: shared keys and
 * values; R9), logits = softmax_scale * <q, K> (R12).  The output of every
 * head is rotated back by RoPE^-1 at p ([Notes] Inverse RoPE 的数学原理; R8)
 * and stored as fp32, bf16, or fp8 codes with one fp32 scale per 64 elements
 * ([Notes] 融合 2：Inverse RoPE + FP8 Quant; R17).  An empty key set gives 0.
 * comp may be NULL (no compressed keys).  Topk ids of -1 are skipped; ids that
 * are not visible, and unmapped pages, are skipped and counted as faults.
 * out_f64 (optional) receives the output before the store. */
int csl_oracle_hybrid_attn(const csl_oracle_pool* comp, const csl_oracle_pool* swa, const int32_t* bt,
                           int max_blocks, int num_q, const int32_t* q_seq, const int64_t* q_pos,
                           const uint16_t* q, int n_heads, const int32_t* topk, int k, int swa_window,
                           double softmax_scale, int out_dtype, void* out, float* out_scales,
                           double* out_f64)
{
    int faults = 0;
    int D = swa->dim;
#pragma omp parallel for schedule(dynamic) reduction(+ : faults)
    for (int n = 0; n < num_q; n++) {
        int s = q_seq[n];
        int64_t p = q_pos[n];
        int64_t nc = comp ? visible_entries(comp->ratio, p) : 0;
        int64_t lo = p - swa_window < 0 ? 0 : p - swa_window;
        int64_t ncomp = comp ? (topk ? k : nc) : 0;
        int64_t cap = ncomp + (p - lo);
        double* keys = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        double* z = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        double* o = (double*)malloc(sizeof(double) * D);
        int64_t L = 0;
        /* gather the key set */
        for (int64_t j = 0; j < ncomp; j++) {
            int64_t i = topk ? topk[(size_t)n * k + j] : j;
            if (i < 0) continue;
            if (i >= nc) { faults++; continue; }
            const uint8_t* row = entry_row(comp, bt, max_blocks, s, i);
            if (!row) { faults++; continue; }
            load_row(row, keys + (size_t)L * D, D, comp->dtype);
            L++;
        }
        for (int64_t t = lo; t < p; t++) {
            const uint8_t* row = entry_row(swa, bt, max_blocks, s, t);
            if (!row) { faults++; continue; }
            load_row(row, keys + (size_t)L * D, D, swa->dtype);
            L++;
        }
        for (int h = 0; h < n_heads; h++) {
            const uint16_t* qh = q + ((size_t)n * n_heads + h) * D;
            double mx = -INFINITY, den = 0.0;
            for (int64_t j = 0; j < L; j++) {
                double dot = 0.0;
                for (int d = 0; d < D; d++) dot += bf16_to_f64(qh[d]) * keys[(size_t)j * D + d];
                z[j] = softmax_scale * dot;
                if (z[j] > mx) mx = z[j];
            }
            for (int64_t j = 0; j < L; j++) den += exp(z[j] - mx);
            for (int d = 0; d < D; d++) o[d] = 0.0;
            for (int64_t j = 0; j < L; j++) {
                double a = exp(z[j] - mx) / den;
                for (int d = 0; d < D; d++) o[d] += a * keys[(size_t)j * D + d];
            }
            rope(o, D, swa->rope_dims, swa->rope_theta, -(double)p);
            size_t base = ((size_t)n * n_heads + h) * D;
            if (out_f64) memcpy(out_f64 + base, o, sizeof(double) * D);
            if (out_dtype == O_F32) {
                for (int d = 0; d < D; d++) ((float*)out)[base + d] = (float)o[d];
            } else if (out_dtype == O_BF16) {
                for (int d = 0; d < D; d++) ((uint16_t*)out)[base + d] = f64_to_bf16(o[d]);
            } else {
                for (int g = 0; g < D / 64; g++)
                    out_scales[((size_t)n * n_heads + h) * (D / 64) + g] =
                        fp8_group(o + 64 * g, (uint8_t*)out + base + 64 * g);
            }
        }
        free(keys);
        free(z);
        free(o);
    }
    return faults;
}

int csl_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (timing only; results do not
 * depend on it). */
void csl_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
