// Index-K / main-KV producer: the step that fills the caches the path reads.
//
// Pages: "DeepSeek V4.1 Flash modeling", section "CSA2" (non-overlapping compression; the
// index key is projected from the compressed main KV) and "Mixed precision" (main KV
// quantized after RoPE); "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 1
// (pairwise compression keeps incomplete pairs across decode steps) and section 5 (BF16
// weights with FP32 accumulation; ratio-2 pooling merging each completed pair in one
// kernel; RoPE, FP4 quantization and cache write fused, intermediate rounding kept).
//
// For each token row whose position p closes a group (p + 1 divisible by m) the entry
// j = (p + 1) / m - 1 is produced from the fp32 compressor outputs of its m tokens:
//   latent = token (m = 1) or (first + second) * 0.5 (m = 2; the first half comes from the
//            previous row of the call or, at a call's start, from the request's pending row)
//   main   = RoPE(latent) on dims [448, 512) at position P = j m + m - 1, stored bf16 or in
//            the FP4 storage format
//   index  = RoPE(W . bf16(latent)) on dims [64, 128) at P, fp32 accumulation by one fma
//            per term in ascending order, then MXFP4
// RoPE rotates interleaved pairs (2i, 2i+1) with cos / sin from the caller's table
// [pos][2][32]; every product and sum is rounded to fp32 on its own (no contraction).
// A second kernel, ordered after the first on the stream, stores the lone even tokens that
// end a request's rows into the pending state, so every entry reads the state as it was
// before the call.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int kLat = 512, kIdx = 128, kRope = 64;
constexpr int kEntriesPerWg = 8;

__device__ __forceinline__ float bf16_round(float x)
{
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// Rotate the pair (a, b) of the 32-pair RoPE table row at position P, pair i.
__device__ __forceinline__ void rope_pair(float* a, float* b, const float* __restrict__ rope, int64_t P, int i)
{
    const float c = rope[P * kRope + i];
    const float s = rope[P * kRope + kRope / 2 + i];
    const float x = *a, y = *b;
    *a = __fsub_rn(__fmul_rn(x, c), __fmul_rn(y, s));
    *b = __fadd_rn(__fmul_rn(x, s), __fmul_rn(y, c));
}

// One workgroup of 128 threads per 8 consecutive rows of the call.
template <int M, bool kFp4Kv>
__global__ __launch_bounds__(128) void k_kv_entries(int n, const int32_t* __restrict__ req_of_row,
                                                    const int32_t* __restrict__ pos_of_row,
                                                    const int64_t* __restrict__ row_start,
                                                    const float* __restrict__ comp,
                                                    const float* __restrict__ pending,
                                                    const uint16_t* __restrict__ w_index,
                                                    const float* __restrict__ rope, int64_t max_pos,
                                                    void* __restrict__ kv, uint8_t* __restrict__ kv_scale,
                                                    uint8_t* __restrict__ idx_codes,
                                                    uint8_t* __restrict__ idx_scales)
{
    __shared__ __attribute__((aligned(16))) float s_lat[kEntriesPerWg][kLat];
    __shared__ __attribute__((aligned(16))) float s_y[kEntriesPerWg][kLat];
    __shared__ __attribute__((aligned(16))) float s_k[kEntriesPerWg][kIdx];
    __shared__ int64_t s_P[kEntriesPerWg], s_erow[kEntriesPerWg];
    __shared__ int s_ok[kEntriesPerWg];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kEntriesPerWg;

    if (tid < kEntriesPerWg) {
        const int t = t0 + tid;
        int ok = 0;
        if (t < n) {
            const int64_t p = pos_of_row[t];
            if ((p + 1) % M == 0) {
                const int64_t j = (p + 1) / M - 1;
                const int64_t P = j * M + M - 1;
                ok = P < max_pos;
                s_P[tid] = P;
                s_erow[tid] = row_start[req_of_row[t]] + j;
            }
        }
        s_ok[tid] = ok;
    }
    __syncthreads();

    // latents (fp32) and their bf16 roundings
    for (int u = tid; u < kEntriesPerWg * (kLat / 4); u += 128) {
        const int e = u / (kLat / 4), c4 = u % (kLat / 4);
        if (!s_ok[e]) continue;
        const int t = t0 + e;
        float4 v = reinterpret_cast<const float4*>(comp + (int64_t)t * kLat)[c4];
        if (M == 2) {
            const int r = req_of_row[t];
            const bool prev_here = t > 0 && req_of_row[t - 1] == r && pos_of_row[t - 1] == pos_of_row[t] - 1;
            const float* a = prev_here ? comp + (int64_t)(t - 1) * kLat : pending + (int64_t)r * kLat;
            const float4 f = reinterpret_cast<const float4*>(a)[c4];
            v.x = __fmul_rn(__fadd_rn(f.x, v.x), 0.5f);
            v.y = __fmul_rn(__fadd_rn(f.y, v.y), 0.5f);
            v.z = __fmul_rn(__fadd_rn(f.z, v.z), 0.5f);
            v.w = __fmul_rn(__fadd_rn(f.w, v.w), 0.5f);
        }
        reinterpret_cast<float4*>(s_lat[e])[c4] = v;
        reinterpret_cast<float4*>(s_y[e])[c4] =
            make_float4(bf16_round(v.x), bf16_round(v.y), bf16_round(v.z), bf16_round(v.w));
    }
    __syncthreads();

    // index key: thread o accumulates output o of every entry, terms in ascending order
    {
        const int o = tid;
        float acc[kEntriesPerWg];
#pragma unroll
        for (int e = 0; e < kEntriesPerWg; e++) acc[e] = 0.0f;
        const uint4* wrow = reinterpret_cast<const uint4*>(w_index + (int64_t)o * kLat);
        for (int i8 = 0; i8 < kLat / 8; i8++) {
            const uint4 w4 = wrow[i8];
            const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int h = 0; h < 8; h++) {
                const float wf = __uint_as_float(h & 1 ? (ww[h >> 1] & 0xFFFF0000u) : (ww[h >> 1] << 16));
#pragma unroll
                for (int e = 0; e < kEntriesPerWg; e++) acc[e] = __builtin_fmaf(wf, s_y[e][8 * i8 + h], acc[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < kEntriesPerWg; e++) s_k[e][o] = acc[e];
    }
    // RoPE of the main latent (dims [448, 512)); the projection above read s_y only
    for (int u = tid; u < kEntriesPerWg * (kRope / 2); u += 128) {
        const int e = u / (kRope / 2), i = u % (kRope / 2);
        if (!s_ok[e]) continue;
        float* x = &s_lat[e][kLat - kRope + 2 * i];
        rope_pair(x, x + 1, rope, s_P[e], i);
    }
    __syncthreads();
    // RoPE of the index key (dims [64, 128))
    for (int u = tid; u < kEntriesPerWg * (kRope / 2); u += 128) {
        const int e = u / (kRope / 2), i = u % (kRope / 2);
        if (!s_ok[e]) continue;
        float* x = &s_k[e][kIdx - kRope + 2 * i];
        rope_pair(x, x + 1, rope, s_P[e], i);
    }
    // main KV
    if (kFp4Kv) {
        for (int u = tid; u < kEntriesPerWg * (kLat / 16); u += 128) {
            const int e = u / (kLat / 16), b = u % (kLat / 16);
            if (!s_ok[e]) continue;
            uint32_t w[2], sc;
            quant_block_fp4s16(&s_lat[e][16 * b], w, &sc);
            const int64_t er = s_erow[e];
            reinterpret_cast<uint2*>(static_cast<uint8_t*>(kv) + er * (kLat / 2))[b] = make_uint2(w[0], w[1]);
            kv_scale[er * (kLat / 16) + b] = (uint8_t)sc;
        }
    } else {
        for (int u = tid; u < kEntriesPerWg * (kLat / 8); u += 128) {
            const int e = u / (kLat / 8), c8 = u % (kLat / 8);
            if (!s_ok[e]) continue;
            const float* x = &s_lat[e][8 * c8];
            uint32_t pk[4];
#pragma unroll
            for (int h = 0; h < 4; h++)
                pk[h] = (__float_as_uint(bf16_round(x[2 * h])) >> 16) | (__float_as_uint(bf16_round(x[2 * h + 1])) & 0xFFFF0000u);
            reinterpret_cast<uint4*>(static_cast<uint16_t*>(kv) + s_erow[e] * kLat)[c8] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    }
    __syncthreads();
    // index key to MXFP4: 4 blocks of 32 per entry
    if (tid < kEntriesPerWg * (kIdx / 32)) {
        const int e = tid / (kIdx / 32), b = tid % (kIdx / 32);
        if (s_ok[e]) {
            uint32_t w[4], sc;
            quant_block_e2m1(&s_k[e][32 * b], w, &sc);
            const int64_t er = s_erow[e];
            reinterpret_cast<uint4*>(idx_codes + er * (kIdx / 2))[b] = make_uint4(w[0], w[1], w[2], w[3]);
            idx_scales[er * (kIdx / 32) + b] = (uint8_t)sc;
        }
    }
}

// Lone even tokens that end a request's rows in this call wait for their partner.
__global__ __launch_bounds__(128) void k_kv_pending(int n, const int32_t* __restrict__ req_of_row,
                                                    const int32_t* __restrict__ pos_of_row,
                                                    const float* __restrict__ comp, float* __restrict__ pending)
{
    const int t = blockIdx.x;
    const int r = req_of_row[t];
    const int p = pos_of_row[t];
    const bool next_here = t + 1 < n && req_of_row[t + 1] == r && pos_of_row[t + 1] == p + 1;
    if ((p & 1) || next_here) return;
    const float4 v = reinterpret_cast<const float4*>(comp + (int64_t)t * kLat)[threadIdx.x];
    reinterpret_cast<float4*>(pending + (int64_t)r * kLat)[threadIdx.x] = v;
}

hipError_t launch_kv_produce(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m,
                             const int64_t* row_start, const float* comp, float* pending, const uint16_t* w_index,
                             const float* rope, int64_t max_pos, bool fp4_kv, void* kv, uint8_t* kv_scale,
                             uint8_t* idx_codes, uint8_t* idx_scales, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + kEntriesPerWg - 1) / kEntriesPerWg));
#define CSA2_KV_ENTRIES(MM, F)                                                                                    \
    hipLaunchKernelGGL((k_kv_entries<MM, F>), grid, dim3(128), 0, stream, n, req_of_row, pos_of_row, row_start, \
                       comp, pending, w_index, rope, max_pos, kv, kv_scale, idx_codes, idx_scales)
    if (m == 1 && fp4_kv) CSA2_KV_ENTRIES(1, true);
    else if (m == 1) CSA2_KV_ENTRIES(1, false);
    else if (fp4_kv) CSA2_KV_ENTRIES(2, true);
    else CSA2_KV_ENTRIES(2, false);
#undef CSA2_KV_ENTRIES
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || m != 2) return e;
    static_assert(kLat / 4 == 128, "one float4 per thread");
    hipLaunchKernelGGL(k_kv_pending, dim3((unsigned)n), dim3(128), 0, stream, n, req_of_row, pos_of_row, comp, pending);
    return hipGetLastError();
}

}  // namespace csa2
