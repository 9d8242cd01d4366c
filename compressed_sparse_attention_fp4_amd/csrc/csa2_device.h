// Device helpers shared by the CSA2 kernels (gfx950 only).
//
// Formats are the OCP Microscaling (MX) v1.0 ones the pages name ("DeepSeek V4.1
// Flash modeling", section "Mixed precision": index Q/K in MXFP4 with 32-element
// groups, window KV in FP8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Entries of a request visible to the query at position p ("DeepSeek V4.1 Flash
// modeling", section "CSA2": non-overlapping groups of m tokens, complete groups only;
// entry j covers tokens [j*m, j*m+m-1] and is visible iff j*m+m-1 <= p).
__device__ __forceinline__ int64_t reach(int p, int m, int n_entries)
{
    int64_t r = ((int64_t)p + 1) / m;
    return r < n_entries ? r : (int64_t)n_entries;
}

// floor(log2(a)) of a finite a > 0, subnormals included.
__device__ __forceinline__ int floor_log2(float a)
{
    uint32_t u = __float_as_uint(a);
    int e = (int)((u >> 23) & 0xFF);
    if (e == 0) return (31 - __clz(u & 0x7FFFFF)) - 149;
    return e - 127;
}

// Shared MX exponent of a block with max magnitude amax: floor(log2 amax) - emax,
// clamped to the E8M0 range; an all-zero block gets -127.
__device__ __forceinline__ int mx_shared_exp(float amax, int emax)
{
    if (amax == 0.0f) return -127;
    int e = floor_log2(amax) - emax;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 magnitude code of y >= 0, rounded to nearest with ties to the even code and
// saturated at 6: the grid is {0, .5, 1, 1.5, 2, 3, 4, 6}; the decision points are
// the midpoints, and at a midpoint the even code wins.
__device__ __forceinline__ uint32_t e2m1_code(float y)
{
    uint32_t c = 0;
    c = (y > 0.25f) ? 1u : c;
    c = (y >= 0.75f) ? 2u : c;
    c = (y > 1.25f) ? 3u : c;
    c = (y >= 1.75f) ? 4u : c;
    c = (y > 2.5f) ? 5u : c;
    c = (y >= 3.5f) ? 6u : c;
    c = (y > 5.0f) ? 7u : c;
    return c;
}

// E4M3 ("fn") magnitude code of 0 <= y, rounded to nearest even, saturated at 448.
// Below 2^-6 the grid step is 2^-9 (subnormals; code = y / 2^-9 also lands on the
// first normal code 8); above, the code is the biased exponent and 3 mantissa bits
// of y rounded at 2^(E-3), a carry into the exponent field being the next binade.
__device__ __forceinline__ uint32_t e4m3_code(float y)
{
    y = fminf(y, 448.0f);
    if (y < 0.015625f) return (uint32_t)__builtin_rintf(y * 512.0f);
    int E = floor_log2(y);
    float mant = __builtin_ldexpf(y, -E) - 1.0f;          // [0, 1), exact
    uint32_t m = (uint32_t)__builtin_rintf(mant * 8.0f);  // 0..8
    return ((uint32_t)(E + 7) << 3) + m;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Value of a positive finite E4M3 ("fn") code c < 127: (8 + m) 2^(e-10) for a biased
// exponent e > 0, m 2^-9 below.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = c >> 3, m = c & 7u;
    return e == 0 ? (float)m * 0.001953125f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
}

// E2M1 magnitude code of a / s for a >= 0 and an E4M3 scale s > 0, without dividing:
// a is compared with the grid midpoints times s.  Those products have at most 7
// significant bits and lie in fp32's normal range, so every comparison is exact and the
// decision is the one the real quotient gives (ties to the even code, saturating at 6).
__device__ __forceinline__ uint32_t e2m1_code_scaled(float a, float s)
{
    uint32_t c = 0;
    c = (a > 0.25f * s) ? 1u : c;
    c = (a >= 0.75f * s) ? 2u : c;
    c = (a > 1.25f * s) ? 3u : c;
    c = (a >= 1.75f * s) ? 4u : c;
    c = (a > 2.5f * s) ? 5u : c;
    c = (a >= 3.5f * s) ? 6u : c;
    c = (a > 5.0f * s) ? 7u : c;
    return c;
}

// Quantize one 32-element block to MXFP4: 16 packed bytes (element 2i in the low
// nibble) returned as 4 dwords, and the E8M0 byte.  The sign bit follows x.
__device__ __forceinline__ void quant_block_e2m1(const float* x, uint32_t out[4], uint32_t* scale_byte)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
    int e = mx_shared_exp(amax, 2);
    *scale_byte = (uint32_t)(e + 127);
    // The scaled conversion divides each element by its scale operand, rounds to the
    // nearest E2M1 value with ties to the even code, saturates at 6 and keeps the sign:
    // the code e2m1_code(|x| 2^-e) with x's sign bit, bit for bit (checked on the GPU for
    // every finite bf16 x and every e with |x| 2^-e < 8, the range a block produces).  The
    // operand's exponent field is what counts, so 2^-127 is passed as the subnormal float.
    const float sc = e >= -126 ? __builtin_ldexpf(1.0f, e) : __uint_as_float(0x00400000u);
#pragma unroll
    for (int w = 0; w < 4; w++) {
        uint32_t word = 0;
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[8 * w + 0], x[8 * w + 1], sc, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[8 * w + 2], x[8 * w + 3], sc, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[8 * w + 4], x[8 * w + 5], sc, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[8 * w + 6], x[8 * w + 7], sc, 3);
        out[w] = word;
    }
}

// Quantize one 16-element block to the FP4 main KV storage format: E2M1 codes (element 2i
// in the low nibble of byte i, 8 bytes as 2 dwords) and the E4M3 scale byte s = RNE(amax / 6)
// (saturating at 448).  The quotient is a correctly rounded fp32 division, which decides
// every rounding as the real quotient does: a tie point t of the E4M3 grid has at most 5
// significant bits, so 6 t lies on amax's fp32 grid, and an amax other than 6 t puts the
// real quotient at least ulp(amax) / 6 from t, further than the division's error of at
// most ulp(amax) / 8.  Elements are rounded by e2m1_code_scaled; a zero scale stores
// zero magnitudes (sign bits kept).
__device__ __forceinline__ void quant_block_fp4s16(const float* v, uint32_t out[2], uint32_t* scale_byte)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sc = e4m3_code(__fdiv_rn(amax, 6.0f));
    const float s = e4m3_value(sc);
    out[0] = out[1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        uint32_t c = s > 0.0f ? e2m1_code_scaled(fabsf(v[i]), s) : 0u;
        c |= (__float_as_uint(v[i]) >> 28) & 8u;
        out[i >> 3] |= c << (4 * (i & 7));
    }
    *scale_byte = sc;
}

// Quantize one 32-element block to MXFP8 E4M3: 32 code bytes as 8 dwords, E8M0 byte.
__device__ __forceinline__ void quant_block_e4m3(const float* x, uint32_t out[8], uint32_t* scale_byte)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
    int e = mx_shared_exp(amax, 8);
    *scale_byte = (uint32_t)(e + 127);
#pragma unroll
    for (int w = 0; w < 8; w++) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float v = x[w * 4 + j];
            uint32_t c = e4m3_code(__builtin_ldexpf(fabsf(v), -e));
            c |= (__float_as_uint(v) >> 24) & 0x80u;
            word |= c << (8 * j);
        }
        out[w] = word;
    }
}

// Monotone map of a non-NaN float to uint32 (larger float -> larger key, -0 == +0).
// Every non-NaN value maps above 0, so 0 marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Pin values: an empty asm consumes them unconditionally, so the compiler cannot sink
// their computation into the branch of a later mask (for a load, that would serialize
// every load of a thread behind a full memory round trip).
__device__ __forceinline__ void pin(uint32_t x)
{
    asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void pin(int32_t x)
{
    asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void pin(float x)
{
    asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void pin(const float4& v)
{
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

// Workgroups are dealt to the GPU's 8 XCDs (each with its own L2) round-robin by block
// index.  A grid of nrows x nchunks workgroups keeps the chunks of row r on XCD r % 8, the
// XCD every kernel of the path gives row r, so that a row's scores, selections and rows of
// KV that one kernel writes or pulls in are in the L2 the next kernel reads from.  Block
// b of each complete group of 8 rows serves row 8 (b / 8 / nchunks) + b % 8, chunk
// (b / 8) % nchunks; the rows after the last complete group take the remaining blocks in
// row-major order.  Any b below nrows x nchunks maps to one (row, chunk), and back.
__device__ __forceinline__ void xcd_row_chunk(int b, int nrows, int nchunks, int* row, int* chunk)
{
    const int full = (nrows >> 3) * nchunks * 8;  // blocks of the complete groups
    if (b < full) {
        const int g = b >> 3;
        *row = 8 * (g / nchunks) + (b & 7);
        *chunk = g % nchunks;
    } else {
        const int rb = b - full;
        *row = (nrows & ~7) + rb / nchunks;
        *chunk = rb % nchunks;
    }
}

}  // namespace csa2
