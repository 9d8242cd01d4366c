// Decoder bounded-replay tail layout and the block quantization kernels (OCP MX, and the
// FP4 main KV storage format).
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

// Row layouts of the bounded replays.  Both describe every request by a run of rows
// with consecutive absolute positions and one window lower bound; rows are packed request
// after request.
//
// Decoder tail ("SGLang: how DeepSeek V4.1 Flash late layers only process tail tokens",
// sections 2.1-2.3 and the rule block after the window table): T = min(budget, E); rows
// [S-T, S) keep their absolute positions; window lower bound S-T; tail row u maps to row
// ext_start + E - T + u of the original extend.  A decode request of a mixed batch
// ("DeepSeek V4.1 Flash modeling", section "Decoder Bounded Replay") keeps all its rows
// with lower bound 0; the borrow flag (a reading of the short-extend proposal, section
// 2.6 of the tail page) sets the bound of prefill requests to max(0, S - budget).
//
// Encoder replay ("SGLang and Miles Day-0 support for DeepSeek-V4.1", sections 4.1 and
// 4.3): the last min(P, budget) cached prefix positions, then the E extend positions,
// all bounded below by R0 = max(0, P - budget); replayed rows have no extend row (-1).
//
// One workgroup of 256 threads walks the requests in chunks of 256: block scans give
// each request's first row and first extend row, then the chunk's rows are written by
// all threads, each finding its request by binary search in the chunk's prefix.
struct LayoutReq {
    int count;  // rows of the request
    int pos0;   // absolute position of its first row
    int lo;     // window lower bound of its rows
    int nrep;   // leading rows without an extend row
    int off;    // extend row of row nrep, relative to the request's first extend row
};

template <bool kEncoder>
__device__ __forceinline__ LayoutReq layout_req(int E, int S_or_P, int decode, int budget, int flags)
{
    LayoutReq q;
    if (kEncoder) {
        const int P = S_or_P;
        const int rep = P < budget ? P : budget;
        q.count = rep + E;
        q.pos0 = P - rep;
        q.lo = q.pos0;
        q.nrep = rep;
        q.off = 0;
    } else {
        const int S = S_or_P;
        const int T = E < budget ? E : budget;
        q.count = T;
        q.pos0 = S - T;
        q.lo = decode ? 0 : ((flags & 1) ? (S - budget > 0 ? S - budget : 0) : S - T);
        q.nrep = 0;
        q.off = E - T;
    }
    return q;
}

template <bool kEncoder>
__global__ __launch_bounds__(256) void k_replay_layout(int nreq, const int32_t* __restrict__ ext_len,
                                                       const int32_t* __restrict__ len2,
                                                       const int32_t* __restrict__ is_decode, int budget, int flags,
                                                       int32_t* __restrict__ tail_len,
                                                       int32_t* __restrict__ row_start,
                                                       int32_t* __restrict__ src_row,
                                                       int32_t* __restrict__ abs_pos,
                                                       int32_t* __restrict__ win_lo,
                                                       int32_t* __restrict__ req_of_row)
{
    __shared__ int s_rstart[257];  // exclusive prefix of the row counts within the chunk (+ total)
    __shared__ int s_estart[256];  // exclusive prefix of E within the chunk
    __shared__ int s_pos0[256], s_lo[256], s_nrep[256], s_off[256];
    __shared__ int s_scan[256];
    const int tid = threadIdx.x;
    int carry_t = 0, carry_e = 0;

    for (int base = 0; base < nreq; base += 256) {
        const int r = base + tid;
        int E = 0;
        LayoutReq q{0, 0, 0, 0, 0};
        if (r < nreq) {
            E = ext_len[r];
            E = E < 0 ? 0 : E;
            q = layout_req<kEncoder>(E, len2[r], is_decode ? is_decode[r] : 0, budget, flags);
        }
        // inclusive scan of the row counts (Hillis-Steele), then of E
        s_scan[tid] = q.count;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int v = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        const int incl_t = s_scan[tid];
        const int chunk_t = s_scan[255];
        __syncthreads();
        s_scan[tid] = E;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int v = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        const int incl_e = s_scan[tid];
        const int chunk_e = s_scan[255];

        s_rstart[tid] = incl_t - q.count;
        s_estart[tid] = incl_e - E;
        s_pos0[tid] = q.pos0;
        s_lo[tid] = q.lo;
        s_nrep[tid] = q.nrep;
        s_off[tid] = q.off;
        if (tid == 0) s_rstart[256] = chunk_t;
        if (r < nreq) {
            if (!kEncoder) tail_len[r] = q.count;
            row_start[r] = carry_t + incl_t - q.count;
        }
        __syncthreads();

        for (int i = tid; i < chunk_t; i += 256) {
            // largest request slot with s_rstart <= i (slots without rows are skipped
            // because the next slot shares their start)
            int lo = 0, hi = 255;
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (s_rstart[mid] <= i) lo = mid; else hi = mid - 1;
            }
            const int u = i - s_rstart[lo];
            const int row = carry_t + i;
            src_row[row] = u < s_nrep[lo] ? -1 : carry_e + s_estart[lo] + s_off[lo] + (u - s_nrep[lo]);
            abs_pos[row] = s_pos0[lo] + u;
            win_lo[row] = s_lo[lo];
            req_of_row[row] = base + lo;
        }
        carry_t += chunk_t;
        carry_e += chunk_e;
        __syncthreads();
    }
    if (tid == 0) row_start[nreq] = carry_t;
}

// MX quantization, one thread per 32-element block.
template <bool kBf16In, bool kFp4>
__global__ __launch_bounds__(256) void k_quant_mx(const void* __restrict__ x, int64_t nblocks,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    if (kBf16In) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 32);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint4 w = p[i];
            uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[i * 8 + 2 * j] = __uint_as_float(ws[j] << 16);
                v[i * 8 + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 32);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float4 w = p[i];
            v[4 * i] = w.x;
            v[4 * i + 1] = w.y;
            v[4 * i + 2] = w.z;
            v[4 * i + 3] = w.w;
        }
    }
    uint32_t sb;
    if (kFp4) {
        uint32_t o[4];
        quant_block_e2m1(v, o, &sb);
        reinterpret_cast<uint4*>(codes)[b] = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
        uint32_t o[8];
        quant_block_e4m3(v, o, &sb);
        uint4* dst = reinterpret_cast<uint4*>(codes) + 2 * b;
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    scales[b] = (uint8_t)sb;
}

// Main KV storage format ("DeepSeek V4.1 Flash modeling", section "Mixed precision": E2M1
// data with one E4M3 scale per 16 channels and no tensor-wide scale), one thread per
// 16-element block (quant_block_fp4s16).
template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quant_fp4s16(const void* __restrict__ x, int64_t nblocks,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    float v[16];
    if (kBf16In) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 16);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint4 w = p[i];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[i * 8 + 2 * j] = __uint_as_float(ws[j] << 16);
                v[i * 8 + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 16);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float4 w = p[i];
            v[4 * i] = w.x;
            v[4 * i + 1] = w.y;
            v[4 * i + 2] = w.z;
            v[4 * i + 3] = w.w;
        }
    }
    uint32_t w[2], sc;
    quant_block_fp4s16(v, w, &sc);
    reinterpret_cast<uint2*>(codes)[b] = make_uint2(w[0], w[1]);
    scales[b] = (uint8_t)sc;
}

hipError_t launch_replay_tail_layout(int nreq, const int32_t* ext_len, const int32_t* seq_len,
                                     const int32_t* is_decode, int budget, int flags, int32_t* tail_len,
                                     int32_t* tail_row_start, int32_t* src_row, int32_t* abs_pos, int32_t* win_lo,
                                     int32_t* req_of_row, hipStream_t stream)
{
    hipLaunchKernelGGL(k_replay_layout<false>, dim3(1), dim3(256), 0, stream, nreq, ext_len, seq_len, is_decode,
                       budget, flags, tail_len, tail_row_start, src_row, abs_pos, win_lo, req_of_row);
    return hipGetLastError();
}

hipError_t launch_encoder_replay_layout(int nreq, const int32_t* prefix_len, const int32_t* ext_len, int budget,
                                        int32_t* row_start, int32_t* src_row, int32_t* abs_pos, int32_t* win_lo,
                                        int32_t* req_of_row, hipStream_t stream)
{
    hipLaunchKernelGGL(k_replay_layout<true>, dim3(1), dim3(256), 0, stream, nreq, ext_len, prefix_len,
                       (const int32_t*)nullptr, budget, 0, (int32_t*)nullptr, row_start, src_row, abs_pos, win_lo,
                       req_of_row);
    return hipGetLastError();
}

hipError_t launch_quant_mx(bool fp4, bool bf16_in, const void* x, int64_t nblocks, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream)
{
    if (nblocks == 0) return hipSuccess;
    dim3 grid((unsigned)((nblocks + 255) / 256));
    if (fp4 && bf16_in)
        hipLaunchKernelGGL((k_quant_mx<true, true>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    else if (fp4)
        hipLaunchKernelGGL((k_quant_mx<false, true>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    else if (bf16_in)
        hipLaunchKernelGGL((k_quant_mx<true, false>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    else
        hipLaunchKernelGGL((k_quant_mx<false, false>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_fp4s16(bool bf16_in, const void* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream)
{
    if (nblocks == 0) return hipSuccess;
    dim3 grid((unsigned)((nblocks + 255) / 256));
    if (bf16_in)
        hipLaunchKernelGGL((k_quant_fp4s16<true>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    else
        hipLaunchKernelGGL((k_quant_fp4s16<false>), grid, dim3(256), 0, stream, x, nblocks, codes, scales);
    return hipGetLastError();
}

}  // namespace csa2
