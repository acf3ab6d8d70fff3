// Device-side building blocks shared by the gfx950 kernels: storage-format
// conversions, wavefront reductions, RoPE angles and paged addressing.
#pragma once

#include <hip/hip_runtime.h>
#include <cfloat>
#include <stdint.h>

namespace csl {

constexpr int kBlockPositions = 256;  // native positions per page
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum : uint32_t { kErrPage = 1u, kErrTopk = 2u, kErrPos = 4u, kErrSeq = 8u };

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP4 = 3 };

struct RopeFreqs {
    // theta^(-2j/R) for the R/2 rotated pairs, fp64, built on the host.
    double inv_freq[64];
};

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even fp32 -> bf16 on the conversion unit (v_cvt_pk_bf16_f32,
// two values per instruction); `lo` lands in bits 0..15.
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cvt{lo, hi}, bf16x2_cvt));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// OCP e4m3fn code -> fp32 (S.1111.111 is NaN; no infinities).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t mag = c & 0x7fu;
    float normal = __uint_as_float((mag << 20) + (120u << 23));
    float sub = (float)(c & 7u) * 0.001953125f;  // m * 2^-9
    float v = (mag >> 3) == 0 ? sub : normal;
    v = mag == 0x7fu ? __uint_as_float(0x7fc00000u) : v;
    return (c & 0x80u) ? -v : v;
}

// fp32 -> OCP e4m3fn codes, round to nearest even, saturating at +-448, NaN
// -> 0x7f with the sign.  The packed hardware conversion v_cvt_pk_fp8_f32
// rounds the same way (checked against the bitwise definition -- sign,
// exponent and mantissa rounding with subnormals at multiples of 2^-9 -- on
// every finite input below 464 in magnitude); clamping to +-448 first gives
// the saturation, and NaN is passed through by hand.
__device__ __forceinline__ float e4m3_clamp(float x) { return x != x ? x : fminf(fmaxf(x, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t e4m3_nan_fix(float x, uint32_t code, int byte) {
    return x != x ? (code & ~(0xffu << (8 * byte))) | ((((__float_as_uint(x) >> 24) & 0x80u) | 0x7fu) << (8 * byte)) : code;
}
// codes of a, b, c, d in bytes 0..3
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    uint32_t code = (uint32_t)w;
    if (__builtin_expect((a != a) | (b != b) | (c != c) | (d != d), 0)) {
        code = e4m3_nan_fix(a, code, 0);
        code = e4m3_nan_fix(b, code, 1);
        code = e4m3_nan_fix(c, code, 2);
        code = e4m3_nan_fix(d, code, 3);
    }
    return code;
}
// e4m3_pack4 for values known to be finite: saturation only
__device__ __forceinline__ uint32_t e4m3_pack4_finite(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.0f), 448.0f), fminf(fmaxf(b, -448.0f), 448.0f), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -448.0f), 448.0f), fminf(fmaxf(d, -448.0f), 448.0f), w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) { return e4m3_pack4(x, 0.f, 0.f, 0.f) & 0xffu; }

// MXFP4 block -> bf16: 32 E2M1 codes (16 bytes, element 2i in the low nibble
// of byte i) times the E8M0 scale 2^(e8 - 127), as 16 words of bf16 pairs.
// v_cvt_scalef32_pk_bf16_fp4 converts the two codes of one byte and
// multiplies by the fp32 scale; every product is exact in bf16 (checked
// against the format's definition for all bytes, scale codes 0 to 254).
__device__ __forceinline__ void mxfp4_to_bf16(const u32x4& codes, uint32_t e8, uint32_t (&out)[16]) {
    const float sc = e8 ? __uint_as_float(e8 << 23) : __uint_as_float(0x00400000u);  // 2^-127 at code 0
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        out[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[w], sc, 0));
        out[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[w], sc, 1));
        out[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[w], sc, 2));
        out[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[w], sc, 3));
    }
}

// A 16-byte load from a 4-byte aligned address (fp4 rows are 68 bytes).
__device__ __forceinline__ u32x4 load16_a4(const uint8_t* p) {
    u32x4 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
    return v;
}

// ---------------------------------------------------------------- waves

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] with the gfx950 lane-swap VALU ops
// (no LDS crossbar): permlane16_swap(v, v) returns, in every lane, the
// lower-row and the upper-row value of the lane's row pair (rows of 16 lanes);
// permlane32_swap(v, v) the same for the two 32-lane halves.  Every lane adds
// the same two operands in the same order, so all lanes hold identical sums.
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 64 lanes, identical in every lane: quad_perm swaps (lane ^ 1,
// lane ^ 2), row_half_mirror and row_mirror (the other quad, the other half
// row), then the row-pair and half-wave swaps.  Each step adds a pair of
// values that both partner lanes see, so every lane ends with the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_allsum(float v) {
    v += dpp_f32<0xb1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4e>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    v = sum_xor16(v);
    return sum_xor32(v);
}

// Prefix scans over the 64 lanes (lane 0 first) on DPP moves, no LDS: shifts
// by 1, 2, 4, 8 lanes inside each 16-lane row, then the last lane of rows 0
// and 2 into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31).  A lane whose source lies outside its row, or whose row is
// masked off, combines with 0 (the identity of both scans here).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t x) {
    x += dpp_u32<0x111>(x);
    x += dpp_u32<0x112>(x);
    x += dpp_u32<0x114>(x);
    x += dpp_u32<0x118>(x);
    x += dpp_u32<0x142, 0xa>(x);
    x += dpp_u32<0x143, 0xc>(x);
    return x;
}
__device__ __forceinline__ uint32_t wave_scan_max(uint32_t x) {
    x = max(x, dpp_u32<0x111>(x));
    x = max(x, dpp_u32<0x112>(x));
    x = max(x, dpp_u32<0x114>(x));
    x = max(x, dpp_u32<0x118>(x));
    x = max(x, dpp_u32<0x142, 0xa>(x));
    x = max(x, dpp_u32<0x143, 0xc>(x));
    return x;
}
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) { return lane_value(wave_scan_max(x), 63); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Reduce across the 8 lanes of an aligned group (lane bits 0..2).
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    return v;
}

// ---------------------------------------------------------------- RoPE

// cos/sin of pos * inv_freq.  The angle is formed and reduced to [-pi, pi] in
// fp64 (two-constant Cody-Waite split of 2*pi: 2*pi rounded to 34 significant
// bits, so k*C1 is exact for |k| < 2^19, i.e. angles up to ~3.3e6 rad), then
// the small-argument sincos runs in fp32.  Error ~1e-7 rad at 2^20 positions.
__device__ __forceinline__ void rope_cs(int64_t pos, double inv_freq, float& c, float& s) {
    constexpr double kTwoPiHi = 6.283185307402164;        // 2*pi to 34 bits
    constexpr double kTwoPiLo = -2.2257726704749154e-10;  // 2*pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = (double)pos * inv_freq;
    const double k = rint(phi * kInvTwoPi);
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, phi));
    sincosf((float)r, &s, &c);
}

// ---------------------------------------------------------------- paging

// Page of native position `t` of sequence `seq`, or -1 (unmapped / beyond the table).
__device__ __forceinline__ int32_t page_of(const int32_t* __restrict__ bt, int max_blocks, int num_pages, int seq,
                                           int64_t t) {
    int64_t b = t >> 8;
    if (t < 0 || b >= max_blocks) return -1;
    int32_t pg = bt[(int64_t)seq * max_blocks + b];
    return (pg < 0 || pg >= num_pages) ? -1 : pg;
}

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bits) { atomicOr(err, bits); }

}  // namespace csl
