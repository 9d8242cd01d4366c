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

// The rounding of every fp32 step below is part of the result (the quantized codes it
// decides must be reproducible): no multiply-add is fused unless written as one.
#pragma clang fp contract(off)

namespace csa2 {

constexpr int kLat = 512, kIdx = 128, kRope = 64;

__device__ __forceinline__ float bf16_round(float x)
{
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// Rotate the pair (a, b) of the 32-pair RoPE table row at position P, pair i: four
// rounded products, then a rounded difference and sum.
__device__ __forceinline__ void rope_pair(float* a, float* b, const float* __restrict__ rope, int64_t P, int i)
{
    const float c = rope[P * kRope + i];
    const float s = rope[P * kRope + kRope / 2 + i];
    const float x = *a, y = *b;
    const float xc = x * c, ys = y * s, xs = x * s, yc = y * c;
    *a = xc - ys;
    *b = xs + yc;
}

// One workgroup of 128 threads per run of consecutive rows of the call: wide calls give a
// workgroup 8 m rows and process the entries they close in rounds of 8 (the projection's
// weight rows are shared by the 8 entries of a round); short calls (decode) give it one
// row and stage the 128 KiB weight matrix in LDS with coalesced loads, so that every
// entry's 512-term chains run from LDS.
template <int M, bool kFp4Kv, bool kWide>
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
    constexpr int E = kWide ? 8 : 1;          // entries per round
    constexpr int R = kWide ? 8 * M : 1;      // rows per workgroup
    __shared__ __attribute__((aligned(16))) float s_lat[E][kLat];
    __shared__ __attribute__((aligned(16))) float s_y[E][kLat];
    __shared__ __attribute__((aligned(16))) float s_k[E][kIdx];
    __shared__ int64_t s_P[R], s_erow[R];
    __shared__ int s_row[R];
    __shared__ int s_nvalid;
    // short calls: the whole weight matrix in LDS, rows 16 bytes apart from a bank multiple
    // so that 16 lanes reading 16 bytes of 16 different rows hit 64 different banks
    constexpr int kWPitch = kLat * 2 + 16;
    __shared__ __attribute__((aligned(16))) char s_w[kWide ? 16 : kIdx * kWPitch];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * R;

    // the rows of this workgroup that close a group, in order
    if (tid == 0) {
        int nv = 0;
        for (int u = 0; u < R; u++) {
            const int t = t0 + u;
            if (t >= n) break;
            const int64_t p = pos_of_row[t];
            if ((p + 1) % M != 0) continue;
            const int64_t j = (p + 1) / M - 1;
            const int64_t P = j * M + M - 1;
            if (P >= max_pos) continue;
            s_row[nv] = t;
            s_P[nv] = P;
            s_erow[nv] = row_start[req_of_row[t]] + j;
            nv++;
        }
        s_nvalid = nv;
    }
    if (!kWide) {
        // coalesced: 64 consecutive 16-byte pieces of a weight row per wave instruction
        const uint4* wg = reinterpret_cast<const uint4*>(w_index);
#pragma unroll 8
        for (int u = tid; u < kIdx * (kLat / 8); u += 128) {
            const int o = u / (kLat / 8), c = u % (kLat / 8);
            *reinterpret_cast<uint4*>(s_w + o * kWPitch + 16 * c) = wg[u];
        }
    }
    __syncthreads();
    const int nvalid = s_nvalid;

    for (int base = 0; base < nvalid; base += E) {
        const int ne = nvalid - base < E ? nvalid - base : E;
        // latents (fp32) and their bf16 roundings
        for (int u = tid; u < ne * (kLat / 4); u += 128) {
            const int e = u / (kLat / 4), c4 = u % (kLat / 4);
            const int t = s_row[base + e];
            float4 v = reinterpret_cast<const float4*>(comp + (int64_t)t * kLat)[c4];
            if (M == 2) {
                const int r = req_of_row[t];
                const bool prev_here = t > 0 && req_of_row[t - 1] == r && pos_of_row[t - 1] == pos_of_row[t] - 1;
                const float* a = prev_here ? comp + (int64_t)(t - 1) * kLat : pending + (int64_t)r * kLat;
                const float4 f = reinterpret_cast<const float4*>(a)[c4];
                v.x = (f.x + v.x) * 0.5f;
                v.y = (f.y + v.y) * 0.5f;
                v.z = (f.z + v.z) * 0.5f;
                v.w = (f.w + v.w) * 0.5f;
            }
            reinterpret_cast<float4*>(s_lat[e])[c4] = v;
            reinterpret_cast<float4*>(s_y[e])[c4] =
                make_float4(bf16_round(v.x), bf16_round(v.y), bf16_round(v.z), bf16_round(v.w));
        }
        __syncthreads();

        // index key: thread o accumulates output o of every entry of the round, one fma per
        // term in ascending order (slots past ne hold stale latents; their sums are never
        // stored).  The weight row comes from LDS (short calls) or streams from memory
        // through registers 128 bytes ahead (long calls, where 8 entries share it).
        {
            const int o = tid;
            float acc[E];
#pragma unroll
            for (int e = 0; e < E; e++) acc[e] = 0.0f;
            if (!kWide) {
                const char* wl = s_w + o * kWPitch;
                for (int u = 0; u < kLat / 8; u++) {
                    const uint4 w4 = *reinterpret_cast<const uint4*>(wl + 16 * u);
                    const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
                    const float4 lo = reinterpret_cast<const float4*>(&s_y[0][8 * u])[0];
                    const float4 hi = reinterpret_cast<const float4*>(&s_y[0][8 * u])[1];
                    const float y[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int h = 0; h < 8; h++)
                        acc[0] = __builtin_fmaf(__uint_as_float(h & 1 ? (ww[h >> 1] & 0xFFFF0000u) : (ww[h >> 1] << 16)),
                                                y[h], acc[0]);
                }
            } else {
                const uint4* wrow = reinterpret_cast<const uint4*>(w_index + (int64_t)o * kLat);
                uint4 wcur[8], wnxt[8];
#pragma unroll
                for (int u = 0; u < 8; u++) wcur[u] = wrow[u];
                for (int c = 0; c < kLat / 64; c++) {
                    if (c + 1 < kLat / 64) {
#pragma unroll
                        for (int u = 0; u < 8; u++) wnxt[u] = wrow[8 * (c + 1) + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const int i0 = 64 * c + 8 * u;
                        const uint32_t ww[4] = {wcur[u].x, wcur[u].y, wcur[u].z, wcur[u].w};
                        float y[E][8];
#pragma unroll
                        for (int e = 0; e < E; e++) {
                            const float4 lo = reinterpret_cast<const float4*>(&s_y[e][i0])[0];
                            const float4 hi = reinterpret_cast<const float4*>(&s_y[e][i0])[1];
                            y[e][0] = lo.x; y[e][1] = lo.y; y[e][2] = lo.z; y[e][3] = lo.w;
                            y[e][4] = hi.x; y[e][5] = hi.y; y[e][6] = hi.z; y[e][7] = hi.w;
                        }
#pragma unroll
                        for (int h = 0; h < 8; h++) {
                            const float wf = __uint_as_float(h & 1 ? (ww[h >> 1] & 0xFFFF0000u) : (ww[h >> 1] << 16));
#pragma unroll
                            for (int e = 0; e < E; e++) acc[e] = __builtin_fmaf(wf, y[e][h], acc[e]);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 8; u++) wcur[u] = wnxt[u];
                }
            }
#pragma unroll
            for (int e = 0; e < E; e++) s_k[e][o] = acc[e];
        }
        // RoPE of the main latent (dims [448, 512)); the projection above read s_y only
        for (int u = tid; u < ne * (kRope / 2); u += 128) {
            const int e = u / (kRope / 2), i = u % (kRope / 2);
            float* x = &s_lat[e][kLat - kRope + 2 * i];
            rope_pair(x, x + 1, rope, s_P[base + e], i);
        }
        __syncthreads();
        // RoPE of the index key (dims [64, 128))
        for (int u = tid; u < ne * (kRope / 2); u += 128) {
            const int e = u / (kRope / 2), i = u % (kRope / 2);
            float* x = &s_k[e][kIdx - kRope + 2 * i];
            rope_pair(x, x + 1, rope, s_P[base + e], i);
        }
        // main KV
        if (kFp4Kv) {
            for (int u = tid; u < ne * (kLat / 16); u += 128) {
                const int e = u / (kLat / 16), b = u % (kLat / 16);
                uint32_t w[2], sc;
                quant_block_fp4s16(&s_lat[e][16 * b], w, &sc);
                const int64_t er = s_erow[base + e];
                reinterpret_cast<uint2*>(static_cast<uint8_t*>(kv) + er * (kLat / 2))[b] = make_uint2(w[0], w[1]);
                kv_scale[er * (kLat / 16) + b] = (uint8_t)sc;
            }
        } else {
            for (int u = tid; u < ne * (kLat / 8); u += 128) {
                const int e = u / (kLat / 8), c8 = u % (kLat / 8);
                const float* x = &s_lat[e][8 * c8];
                uint32_t pk[4];
#pragma unroll
                for (int h = 0; h < 4; h++)
                    pk[h] = (__float_as_uint(bf16_round(x[2 * h])) >> 16) |
                            (__float_as_uint(bf16_round(x[2 * h + 1])) & 0xFFFF0000u);
                reinterpret_cast<uint4*>(static_cast<uint16_t*>(kv) + s_erow[base + e] * kLat)[c8] =
                    make_uint4(pk[0], pk[1], pk[2], pk[3]);
            }
        }
        __syncthreads();
        // index key to MXFP4: 4 blocks of 32 per entry
        if (tid < ne * (kIdx / 32)) {
            const int e = tid / (kIdx / 32), b = tid % (kIdx / 32);
            uint32_t w[4], sc;
            quant_block_e2m1(&s_k[e][32 * b], w, &sc);
            const int64_t er = s_erow[base + e];
            reinterpret_cast<uint4*>(idx_codes + er * (kIdx / 2))[b] = make_uint4(w[0], w[1], w[2], w[3]);
            idx_scales[er * (kIdx / 32) + b] = (uint8_t)sc;
        }
        __syncthreads();  // the next round overwrites the LDS rows
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
    const bool wide = n > 4096;
    const unsigned rows_per_wg = wide ? 8u * (unsigned)m : 1u;
    const dim3 grid((unsigned)((n + rows_per_wg - 1) / rows_per_wg));
#define CSA2_KV_ENTRIES(MM, F, W)                                                                                    \
    hipLaunchKernelGGL((k_kv_entries<MM, F, W>), grid, dim3(128), 0, stream, n, req_of_row, pos_of_row, row_start, \
                       comp, pending, w_index, rope, max_pos, kv, kv_scale, idx_codes, idx_scales)
#define CSA2_KV_ENTRIES_W(MM, F) \
    if (wide) CSA2_KV_ENTRIES(MM, F, true); else CSA2_KV_ENTRIES(MM, F, false)
    if (m == 1 && fp4_kv) { CSA2_KV_ENTRIES_W(1, true); }
    else if (m == 1) { CSA2_KV_ENTRIES_W(1, false); }
    else if (fp4_kv) { CSA2_KV_ENTRIES_W(2, true); }
    else { CSA2_KV_ENTRIES_W(2, false); }
#undef CSA2_KV_ENTRIES_W
#undef CSA2_KV_ENTRIES
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || m != 2) return e;
    static_assert(kLat / 4 == 128, "one float4 per thread");
    hipLaunchKernelGGL(k_kv_pending, dim3((unsigned)n), dim3(128), 0, stream, n, req_of_row, pos_of_row, comp, pending);
    return hipGetLastError();
}

}  // namespace csa2
