// Sparse + sliding-window attention: each query row attends, per head, to its selected
// compressed entries together with its own window, in one softmax.
//
// Pages: "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 1 (every query
// attends to its 128-position local window and to at most 512 compressed positions
// chosen by the indexer); "DeepSeek V4.1 Flash modeling", sections "CSA2" (Full,
// Reindex and Reuse layers all run their own attention over the selected KV) and
// "Mixed precision" (the 512-d main entry is one shared latent: key = value; the window
// cache is FP8); "SGLang: how DeepSeek V4.1 Flash late layers only process tail
// tokens", section 2.3 (a replayed tail row's window starts no lower than S - T).
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct RowKeys {
    int r, p;
    int64_t kv0;   // first main-KV row of the request
    int64_t t0;    // first window position
    int nwin;      // window rows
    const int32_t* sel;
};

__device__ __forceinline__ RowKeys row_keys(const RowsArg& rows, const CacheArg& cache, const SwaArg& swa,
                                            const int32_t* sel, int64_t sel_stride, const int32_t* sel_row_map,
                                            int row)
{
    RowKeys rk;
    rk.r = rows.req[row];
    rk.p = rows.pos[row];
    rk.kv0 = cache.row_start[rk.r];
    int64_t t0 = (int64_t)rk.p - swa.window + 1;
    const int64_t lo = rows.win_lo ? rows.win_lo[row] : 0;
    const int64_t ps = swa.pos_start[rk.r];
    t0 = t0 > lo ? t0 : lo;
    t0 = t0 > ps ? t0 : ps;
    rk.t0 = t0;
    rk.nwin = (int)((int64_t)rk.p - t0 + 1 > 0 ? (int64_t)rk.p - t0 + 1 : 0);
    rk.sel = sel ? sel + (int64_t)(sel_row_map ? sel_row_map[row] : row) * sel_stride : nullptr;
    return rk;
}

// ---------------------------------------------------------------------------- fp32
// One workgroup per (row, head): logits of every key slot into LDS (an invalid slot -1
// gets -inf), block max and sum, then each thread accumulates output dimensions.
__global__ __launch_bounds__(256) void k_attn_f32(RowsArg rows, CacheArg cache, const float* __restrict__ q, int H,
                                                  int D, const float* __restrict__ kv, const int32_t* __restrict__ sel,
                                                  int k, int64_t sel_stride, const int32_t* __restrict__ sel_row_map,
                                                  SwaArg swa, float sm_scale, const float* __restrict__ sink,
                                                  float* __restrict__ out, float* __restrict__ lse)
{
    extern __shared__ float s_logit[];
    __shared__ float s_red[4];
    const int row = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const RowKeys rk = row_keys(rows, cache, swa, sel, sel_stride, sel_row_map, row);
    const float* swa_data = static_cast<const float*>(swa.data);
    const int64_t swa_base = swa.row_start[rk.r] - swa.pos_start[rk.r];
    const int nk = k + rk.nwin;
    const float* qh = q + ((int64_t)row * H + h) * D;

    auto key_ptr = [&](int i) -> const float* {
        if (i < k) {
            const int32_t j = rk.sel[i];
            return j < 0 ? nullptr : kv + (rk.kv0 + j) * D;
        }
        return swa_data + (swa_base + rk.t0 + (i - k)) * D;
    };

    float lmax = -INFINITY;
    for (int i = tid; i < nk; i += 256) {
        const float* x = key_ptr(i);
        float l = -INFINITY;
        if (x) {
            float acc = 0.0f;
            for (int d = 0; d < D; d++) acc = __builtin_fmaf(qh[d], x[d], acc);
            l = acc * sm_scale;
        }
        s_logit[i] = l;
        lmax = fmaxf(lmax, l);
    }
    for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = lmax;
    __syncthreads();
    const float m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    float lsum = 0.0f;
    for (int i = tid; i < nk; i += 256) {
        const float pexp = (m == -INFINITY) ? 0.0f : expf(s_logit[i] - m);
        s_logit[i] = pexp;
        lsum += pexp;
    }
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
    if ((tid & 63) == 0) s_red[tid >> 6] = lsum;
    __syncthreads();
    float den = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    const bool empty = (m == -INFINITY);
    if (sink && !empty) den += expf(sink[h] - m);
    float* oh = out + ((int64_t)row * H + h) * D;
    for (int d = tid; d < D; d += 256) {
        float acc = 0.0f;
        for (int i = 0; i < nk; i++) {
            const float pexp = s_logit[i];
            if (pexp != 0.0f) acc = __builtin_fmaf(pexp, key_ptr(i)[d], acc);
        }
        oh[d] = empty ? 0.0f : acc / den;
    }
    if (lse && tid == 0) lse[(int64_t)row * H + h] = empty ? -INFINITY : m + logf(den);
}

// ----------------------------------------------------------------------------- bf16
// MQA with one shared 512-d latent (key = value) on bf16 MFMA.
//
// Workgroup = 4 waves on one query row and 16 heads (h0 .. h0+15).  The row's key list
// (selected entries with -1 removed, then window positions) is cut into tiles of 16 keys;
// wave w takes tiles w, w+4, ... and keeps its own online-softmax state and output.
//   * K tile = A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, 16 steps over 512
//     dims): lane (g, c) holds key c, dims [32s+8g, 32s+8g+8).  Window rows in FP8 are
//     dequantized to bf16 on load (exact: E4M3 times a power of two).
//   * S^T output: lane (g, c) holds keys 4g..4g+3 of head c, which is the A operand of
//     P V with v_mfma_f32_16x16x16_bf16 (keys are the contraction index).
//   * V = K transposed: v_mfma_f32_16x16x16_bf16 of a 16-key x 16-dim K slice with the
//     identity gives, in lane (g, c), keys 4g..4g+3 of one dim: the B operand of P V.
//     Output tile 2s+u column c is dim 32s + 8(c/4) + 4u + c%4.
//   * Output O: 32 tiles of 16 heads x 16 dims; lane (g, c) holds heads 4g..4g+3.
// The four waves' partial results are merged in fixed order through LDS.
// Blocks are mapped so that the head groups of one row share an XCD (and its L2): block
// b serves row 8*(b / (8*NHG)) + b%8 and head group (b/8) % NHG.
constexpr int kAttnD = 512;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 load_fp8x8_as_bf16(const uint8_t* p, float scale)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    bf16x8 r;
#define CSA2_CVT(word, b, idx) r[idx] = (__bf16)(__builtin_amdgcn_cvt_f32_fp8((int)(word), b) * scale)
    CSA2_CVT(u.x, 0, 0);
    CSA2_CVT(u.x, 1, 1);
    CSA2_CVT(u.x, 2, 2);
    CSA2_CVT(u.x, 3, 3);
    CSA2_CVT(u.y, 0, 4);
    CSA2_CVT(u.y, 1, 5);
    CSA2_CVT(u.y, 2, 6);
    CSA2_CVT(u.y, 3, 7);
#undef CSA2_CVT
    return r;
}

__global__ __launch_bounds__(256) void k_attn_bf16(RowsArg rows, CacheArg cache, const uint16_t* __restrict__ q,
                                                   int H, int nhg, const uint16_t* __restrict__ kv,
                                                   const int32_t* __restrict__ sel, int k, int64_t sel_stride,
                                                   const int32_t* __restrict__ sel_row_map, SwaArg swa,
                                                   float sm_scale, const float* __restrict__ sink,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse)
{
    __shared__ int32_t s_sel[2048];
    __shared__ int s_tmp[8];
    __shared__ float s_m[4][16], s_l[4][16];
    __shared__ float s_o[4][16][256 + 4];  // one half of the dims at a time

    const int b = blockIdx.x;
    const int row = 8 * (b / (8 * nhg)) + (b & 7);
    const int hg = (b >> 3) % nhg;
    if (row >= rows.n) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int h0 = 16 * hg;
    const RowKeys rk = row_keys(rows, cache, swa, sel, sel_stride, sel_row_map, row);

    // ---- compact the selected entries (drop -1), keeping their order
    int nsel = 0;
    for (int base = 0; base < k; base += 256) {
        const int i = base + tid;
        const int32_t j = (i < k) ? rk.sel[i] : -1;
        const int valid = j >= 0;
        const unsigned long long bal = __ballot(valid);
        const int before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) s_tmp[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, tot = 0;
        for (int w = 0; w < 4; w++) {
            before += (w < wave) ? s_tmp[w] : 0;
            tot += s_tmp[w];
        }
        if (valid) s_sel[nsel + before + before_in_wave] = j;
        nsel += tot;
        __syncthreads();
    }
    const int nk = nsel + rk.nwin;
    const int ntiles = (nk + 15) >> 4;

    // ---- Q^T as the B operand: lane (g, c) holds head h0+c, dims [32s+8g, +8)
    bf16x8 qb[16];
    {
        const uint16_t* qrow = q + ((int64_t)row * H + h0 + c) * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; s++) qb[s] = load_bf16x8(qrow + 32 * s);
    }
    // identity B operand of the transposing MFMA: lane (g, c), k-slots 4g..4g+3, column c
    s16x4 ident;
#pragma unroll
    for (int i = 0; i < 4; i++) ident[i] = (4 * g + i == c) ? (short)0x3F80 : (short)0;

    f32x4 o[32];
#pragma unroll
    for (int t = 0; t < 32; t++) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;  // state of head c (replicated over g)
    const float qk_scale = sm_scale * kLog2e;
    const uint16_t* kv_r = kv + rk.kv0 * kAttnD;
    const int64_t swa_base = swa.row_start[rk.r] - swa.pos_start[rk.r] + rk.t0;

    for (int tile = wave; tile < ntiles; tile += 4) {
        const int ki = tile * 16 + c;
        bf16x8 ka[16];
        if (ki < nsel) {
            const uint16_t* kr = kv_r + (int64_t)s_sel[ki] * kAttnD + 8 * g;
#pragma unroll
            for (int s = 0; s < 16; s++) ka[s] = load_bf16x8(kr + 32 * s);
        } else if (ki < nk) {
            const int64_t srow = swa_base + (ki - nsel);
            if (swa.dtype == 3) {
                const uint8_t* sr = static_cast<const uint8_t*>(swa.data) + srow * kAttnD + 8 * g;
                const uint8_t* sc = swa.scale + srow * (kAttnD / 32);
#pragma unroll
                for (int s = 0; s < 16; s++) ka[s] = load_fp8x8_as_bf16(sr + 32 * s, __builtin_ldexpf(1.0f, (int)sc[s] - 127));
            } else {
                const uint16_t* sr = static_cast<const uint16_t*>(swa.data) + srow * kAttnD + 8 * g;
#pragma unroll
                for (int s = 0; s < 16; s++) ka[s] = load_bf16x8(sr + 32 * s);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; s++) ka[s] = bf16x8{};
        }

        // S^T tile: lane (g, c) -> keys 4g..4g+3, head c
        f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 16; s++) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[s], st, 0, 0, 0);

        float lg[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int key = tile * 16 + 4 * g + i;
            lg[i] = (key < nk) ? st[i] * qk_scale : -INFINITY;
            tmax = fmaxf(tmax, lg[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float psum = 0.0f;
        s16x4 pa;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float pv = __builtin_amdgcn_exp2f(lg[i] - m_use);
            psum += pv;
            pa[i] = __builtin_bit_cast(short, (__bf16)pv);
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // rescale O rows (heads 4g+i) by their alpha, held by lane 4g+i
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; i++) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
        for (int t = 0; t < 32; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) o[t][i] *= al[i];

        // O += P V, V taken from the K tile through the identity MFMA
#pragma unroll
        for (int s = 0; s < 16; s++) {
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const s16x4 kh = __builtin_bit_cast(s16x4, bf16x4{ka[s][4 * u], ka[s][4 * u + 1], ka[s][4 * u + 2],
                                                                 ka[s][4 * u + 3]});
                const f32x4 tt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kh, ident, f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                          0, 0, 0);
                s16x4 vb;
#pragma unroll
                for (int i = 0; i < 4; i++) vb[i] = __builtin_bit_cast(short, (__bf16)tt[i]);
                o[2 * s + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[2 * s + u], 0, 0, 0);
            }
        }
    }

    // ---- merge the four waves: out = sum_w O_w 2^(m_w - M) / L
    if (g == 0) {
        s_m[wave][c] = m_run;
        s_l[wave][c] = l_run;
    }
    __syncthreads();
    float fac[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int hh = 4 * g + i;
        float M = -INFINITY;
        for (int w = 0; w < 4; w++) M = fmaxf(M, s_m[w][hh]);
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float L = 0.0f;
        for (int w = 0; w < 4; w++) L += s_l[w][hh] * __builtin_amdgcn_exp2f(s_m[w][hh] - Mu);
        if (sink && M != -INFINITY) L += __builtin_amdgcn_exp2f(sink[h0 + hh] * kLog2e - Mu);
        fac[i] = (L > 0.0f) ? __builtin_amdgcn_exp2f(s_m[wave][hh] - Mu) / L : 0.0f;
        if (lse && wave == 0 && c == 0)
            lse[(int64_t)row * H + h0 + hh] = (M == -INFINITY) ? -INFINITY : (M + __log2f(L)) * 0.69314718055994531f;
    }
#pragma unroll
    for (int half = 0; half < 2; half++) {
#pragma unroll
        for (int tt = 0; tt < 16; tt++) {
            const int t = 16 * half + tt;
            const int s = t >> 1, u = t & 1;
            const int d = 32 * s + 8 * (c >> 2) + 4 * u + (c & 3) - 256 * half;
#pragma unroll
            for (int i = 0; i < 4; i++) s_o[wave][4 * g + i][d] = o[t][i] * fac[i];
        }
        __syncthreads();
        for (int e = tid; e < 16 * 256; e += 256) {
            const int hh = e >> 8, d = e & 255;
            const float v = ((s_o[0][hh][d] + s_o[1][hh][d]) + s_o[2][hh][d]) + s_o[3][hh][d];
            out[((int64_t)row * H + h0 + hh) * kAttnD + 256 * half + d] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
        __syncthreads();
    }
}

hipError_t launch_attn_f32(const RowsArg& rows, const CacheArg& cache, const float* q, int heads, int dim,
                           const float* kv, const int32_t* sel, int k, int64_t sel_stride, const int32_t* sel_row_map,
                           const SwaArg& swa, float sm_scale, const float* sink, float* out, float* lse,
                           hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const size_t shmem = sizeof(float) * (size_t)(k + swa.window);
    hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)((int64_t)rows.n * heads)), dim3(256), shmem, stream, rows, cache,
                       q, heads, dim, kv, sel, k, sel_stride, sel_row_map, swa, sm_scale, sink, out, lse);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const RowsArg& rows, const CacheArg& cache, const uint16_t* q, int heads,
                            const uint16_t* kv, const int32_t* sel, int k, int64_t sel_stride,
                            const int32_t* sel_row_map, const SwaArg& swa, float sm_scale, const float* sink,
                            uint16_t* out, float* lse, hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const int nhg = heads / 16;
    const int64_t nblocks = (int64_t)((rows.n + 7) / 8) * 8 * nhg;
    hipLaunchKernelGGL(k_attn_bf16, dim3((unsigned)nblocks), dim3(256), 0, stream, rows, cache, q, heads, nhg, kv, sel,
                       k, sel_stride, sel_row_map, swa, sm_scale, sink, out, lse);
    return hipGetLastError();
}

}  // namespace csa2
