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
    __shared__ uint4 s_q[16][64];          // Q^T operand: step s, lane (g, c)

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
    // Key slots: [0, nsel) selected entries, [nsel, sel_pad) padding (masked), then the
    // window; sel_pad = nsel rounded up to a tile, so every tile is of one kind.
    const int sel_pad = (nsel + 15) & ~15;
    const int nslots = sel_pad + rk.nwin;
    const int ntiles = (nslots + 15) >> 4;
    const int sel_tiles = sel_pad >> 4;

    // ---- Q^T as the B operand, staged in LDS: lane (g, c) of step s holds head h0+c,
    //      dims [32s+8g, +8)
    for (int idx = tid; idx < 16 * 64; idx += 256) {
        const int s = idx >> 6, l = idx & 63;
        s_q[s][l] = *reinterpret_cast<const uint4*>(q + ((int64_t)row * H + h0 + (l & 15)) * kAttnD + 32 * s +
                                                   8 * (l >> 4));
    }
    __syncthreads();
    // identity B operand of the transposing MFMA: lane (g, c), k-slots 4g..4g+3, column c
    s16x4 ident;
#pragma unroll
    for (int i = 0; i < 4; i++) ident[i] = (4 * g + i == c) ? (short)0x3F80 : (short)0;

    // State of head c (replicated over g).  Exponents are taken against a reference
    // m_ref that is fixed for the whole pass: the wave's first tile maximum plus 64
    // (log2 units).  Any reference at or above the maximum gives the same softmax (the
    // numerator and the denominator share the factor) and 64 leaves the fp32 / bf16
    // exponent range ample room.  The accumulator is therefore touched only by MFMAs
    // inside the loop.  If a later logit exceeds the reference, the wave redoes its
    // tiles once with the exact maximum it has seen.
    const float qk_scale = sm_scale * kLog2e;
    const uint16_t* kv_r = kv + rk.kv0 * kAttnD;
    const int64_t swa_base = swa.row_start[rk.r] - swa.pos_start[rk.r] + rk.t0;
    f32x4 o[32];
    float m_ref = -INFINITY, l_run = 0.0f, m_true = -INFINITY;
    for (int attempt = 0; attempt < 2; attempt++) {
#pragma unroll
        for (int t = 0; t < 32; t++) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        l_run = 0.0f;
        m_ref = (attempt == 0) ? -INFINITY : m_true;
        bool over = false;
        for (int tile = wave; tile < ntiles; tile += 4) {
            // keep the Q operand in LDS: re-read it per tile instead of pinning 64 registers
            asm volatile("" ::: "memory");
            bf16x8 ka[16];
            if (tile < sel_tiles) {  // uniform: a tile of selected entries (and padding)
                const int ki = tile * 16 + c;
                const uint16_t* kr = kv_r + (int64_t)s_sel[ki < nsel ? ki : 0] * kAttnD + 8 * g;
#pragma unroll
                for (int s = 0; s < 16; s++) ka[s] = load_bf16x8(kr + 32 * s);
            } else {
                const int wi = tile * 16 + c - sel_pad;
                const int64_t srow = swa_base + (wi < rk.nwin ? wi : 0);
                if (swa.dtype == 3) {
                    const uint8_t* sr = static_cast<const uint8_t*>(swa.data) + srow * kAttnD + 8 * g;
                    const uint8_t* sc = swa.scale + srow * (kAttnD / 32);
#pragma unroll
                    for (int s = 0; s < 16; s++)
                        ka[s] = load_fp8x8_as_bf16(sr + 32 * s, __builtin_ldexpf(1.0f, (int)sc[s] - 127));
                } else {
                    const uint16_t* sr = static_cast<const uint16_t*>(swa.data) + srow * kAttnD + 8 * g;
#pragma unroll
                    for (int s = 0; s < 16; s++) ka[s] = load_bf16x8(sr + 32 * s);
                }
            }

            // S^T tile: lane (g, c) -> key slots 4g..4g+3, head c
            f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 16; s++)
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], __builtin_bit_cast(bf16x8, s_q[s][lane]), st, 0,
                                                             0, 0);
            float lg[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int slot = tile * 16 + 4 * g + i;
                const bool valid = (slot < nsel) || (slot >= sel_pad && slot < nslots);
                lg[i] = valid ? st[i] * qk_scale : -INFINITY;
                tmax = fmaxf(tmax, lg[i]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            m_true = fmaxf(m_true, tmax);
            if (m_ref == -INFINITY && tmax != -INFINITY) m_ref = tmax + 64.0f;  // the accumulator is still zero
            over |= tmax > m_ref;
            const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
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
            l_run += psum;

            // O += P V, V taken from the K tile through the identity MFMA
#pragma unroll
            for (int s = 0; s < 16; s++) {
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    const s16x4 kh = __builtin_bit_cast(
                        s16x4, bf16x4{ka[s][4 * u], ka[s][4 * u + 1], ka[s][4 * u + 2], ka[s][4 * u + 3]});
                    const f32x4 tt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kh, ident,
                                                                              f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
                    const bf16x2_t lo = __builtin_convertvector(__builtin_shufflevector(tt, tt, 0, 1), bf16x2_t);
                    const bf16x2_t hi = __builtin_convertvector(__builtin_shufflevector(tt, tt, 2, 3), bf16x2_t);
                    const s16x4 vb = __builtin_bit_cast(s16x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
                    o[2 * s + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[2 * s + u], 0, 0, 0);
                }
            }
        }
        if (!__ballot(over)) break;
    }

    // ---- merge the four waves: out = sum_w O_w 2^(m_w - M) / L
    if (g == 0) {
        s_m[wave][c] = m_ref;
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
