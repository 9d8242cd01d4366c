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
// MQA with one shared 512-d latent (key = value) on bf16 MFMA, for dim 512.
//
// Workgroup = 4 waves on one query row and 16 heads (h0 .. h0+15).  The row's key list
// (selected entries with -1 removed and padded to a multiple of 16, then the window
// positions) is cut into tiles of 16 keys; wave w takes tiles w, w+4, ... with its own
// online-softmax state and output.  Each wave double-buffers its tiles in LDS: while it
// computes on one tile, the next one is already on its way (selected rows by direct
// global-to-LDS copies, one 1 KiB row per instruction; FP8 window rows are dequantized
// to bf16 through registers: E4M3 times a power of two is exact in bf16).
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, 16 steps over the 512 dims: A = K rows
//     from LDS (lane (g, c) holds key c, dims [32s+8g, +8)), B = Q^T in registers.
//   * S^T output: lane (g, c) holds keys 4g..4g+3 of head c, which is the A operand of
//     P V with v_mfma_f32_16x16x16_bf16 (keys are the contraction index).
//   * The V operand (lane (g, c): keys 4g..4g+3 of dim c) comes straight from the row-
//     major tile with the LDS transpose read ds_read_b64_tr_b16: within a 16-lane group,
//     element j of lane i comes from the 8-byte chunk that lane 4j + i/4 addresses, so
//     lane (g, 4j+q) points at V[4g+j][16t+4q].
//   * Output O: 32 tiles of 16 heads x 16 dims (lane (g, c): heads 4g..4g+3, dim 16t+c).
// The four waves' partial results are merged in fixed order through LDS.
// Blocks are mapped so that the head groups of one row share an XCD (and its L2): block
// b serves row 8*(b / (8*NHG)) + b%8 and head group (b/8) % NHG.
constexpr int kAttnD = 512;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowBytes = kAttnD * 2 + 32;           // LDS row pitch of a tile (32 B pad)
constexpr int kTileBytes = 16 * kRowBytes;            // one tile of 16 keys
constexpr int kWaveBytes = 2 * kTileBytes;            // double buffer per wave
constexpr int kMergeBytes = 4 * 16 * (256 + 4) * 4;   // merge scratch (aliases the tiles)
static_assert(kMergeBytes <= 4 * kWaveBytes, "merge scratch must fit in the tile buffers");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}

// Copy one 1 KiB row from global memory into LDS at byte address `lds` (wave-uniform):
// lane l moves bytes [16 l, 16 l + 16).  The copy is asynchronous; it is complete once
// the wave's vector-memory counter has dropped past it (s_waitcnt vmcnt).  Issued as
// inline assembly so the compiler does not add a wait for it before unrelated LDS reads.
__device__ __forceinline__ void dma_row(const void* gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gptr)
                 : "memory", "m0");
}

// Reductions over the four 16-lane rows (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float max_over_g(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_g(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 u, float scale)
{
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
    return __builtin_bit_cast(uint4, r);
}

__global__ __launch_bounds__(256) void k_attn_bf16(RowsArg rows, CacheArg cache, const uint16_t* __restrict__ q,
                                                   int H, int nhg, const uint16_t* __restrict__ kv,
                                                   const int32_t* __restrict__ sel, int k, int64_t sel_stride,
                                                   const int32_t* __restrict__ sel_row_map, SwaArg swa,
                                                   float sm_scale, const float* __restrict__ sink,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse)
{
    __shared__ __attribute__((aligned(16))) char s_tiles[4 * kWaveBytes];
    __shared__ __attribute__((aligned(16))) int32_t s_sel[2048];
    __shared__ int s_tmp[8];
    __shared__ float s_m[4][16], s_l[4][16];

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
    if (tid < sel_pad - nsel) s_sel[nsel + tid] = s_sel[0];  // padding slots point at a real entry
    __syncthreads();
    const int nslots = sel_pad + rk.nwin;
    const int ntiles = (nslots + 15) >> 4;
    const int sel_tiles = sel_pad >> 4;

    // ---- Q^T as the B operand: lane (g, c) holds head h0+c, dims [32s+8g, +8)
    bf16x8 qb[16];
    {
        const uint16_t* qrow = q + ((int64_t)row * H + h0 + c) * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; s++) qb[s] = load_bf16x8(qrow + 32 * s);
        // Make the compiler wait for these loads here, not inside the tile loop where a
        // wait would also hold back the next tile's copies.
#pragma unroll
        for (int s = 0; s < 16; s++) asm volatile("" : "+v"(qb[s]));
    }

    const uint16_t* kv_r = kv + rk.kv0 * kAttnD;
    const int64_t swa_base = swa.row_start[rk.r] - swa.pos_start[rk.r] + rk.t0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    char* my_tiles = s_tiles + wave_u * kWaveBytes;
    const uint32_t my_tiles_lds = lds_addr(my_tiles);
    // a tile that arrives by direct copies (selected rows, or a bf16 window)
    const int dma_tiles = (swa.dtype == 3) ? sel_tiles : ntiles;

    // Start the copy of tile `tile` into buffer `buf`.  Rows that arrive by direct copy
    // are only issued here; FP8 window rows are loaded, dequantized and stored to LDS.
    auto fetch = [&](int tile, int buf) {
        const uint32_t dst = my_tiles_lds + buf * kTileBytes;
        if (tile < sel_tiles) {
            int4 jv[4];
#pragma unroll
            for (int u = 0; u < 4; u++) jv[u] = reinterpret_cast<const int4*>(s_sel + tile * 16)[u];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int32_t j = jv[r >> 2][r & 3];
                dma_row(kv_r + (int64_t)j * kAttnD + 8 * lane, dst + r * kRowBytes);
            }
        } else if (swa.dtype != 3) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int wi = tile * 16 + r - sel_pad;
                wi = wi < rk.nwin ? wi : rk.nwin - 1;
                dma_row(static_cast<const uint16_t*>(swa.data) + (swa_base + wi) * kAttnD + 8 * lane,
                        dst + r * kRowBytes);
            }
        } else {
            int wi = tile * 16 + c - sel_pad;
            wi = wi < rk.nwin ? wi : rk.nwin - 1;
            const int64_t srow = swa_base + wi;
            const uint8_t* sr = static_cast<const uint8_t*>(swa.data) + srow * kAttnD + 8 * g;
            const uint8_t* sc = swa.scale + srow * (kAttnD / 32);
            char* dp = my_tiles + buf * kTileBytes + c * kRowBytes + 16 * g;
            uint2 raw[16];
#pragma unroll
            for (int s = 0; s < 16; s++) raw[s] = *reinterpret_cast<const uint2*>(sr + 32 * s);
#pragma unroll
            for (int s = 0; s < 16; s++)
                *reinterpret_cast<uint4*>(dp + 64 * s) = fp8x8_to_bf16x8(raw[s], __builtin_ldexpf(1.0f, (int)sc[s] - 127));
        }
    };

    // State of head c (replicated over g).  Exponents are taken against a reference
    // m_ref that is fixed for the whole pass: the wave's first tile maximum plus 64
    // (log2 units).  Any reference at or above the maximum gives the same softmax (the
    // numerator and the denominator share the factor) and 64 leaves the fp32 / bf16
    // exponent range ample room.  The accumulator is therefore touched only by MFMAs
    // inside the loop.  If a later logit exceeds the reference, the wave redoes its
    // tiles once with the exact maximum it has seen.
    const float qk_scale = sm_scale * kLog2e;
    const int k_off = c * kRowBytes + 16 * g;                            // K operand, step s at +64 s
    const int v_off = (4 * g + (c >> 2)) * kRowBytes + (c & 3) * 8;     // V operand, dim tile t at +32 t
    f32x4 o[32];
    float m_ref = -INFINITY, l_run = 0.0f, m_true = -INFINITY;
    for (int attempt = 0; attempt < 2; attempt++) {
#pragma unroll
        for (int t = 0; t < 32; t++) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        l_run = 0.0f;
        m_ref = (attempt == 0) ? -INFINITY : m_true;
        bool over = false;
        int buf = 0;
        if (wave_u < ntiles) fetch(wave_u, 0);
        for (int tile = wave_u; tile < ntiles; tile += 4, buf ^= 1) {
            const bool more = tile + 4 < ntiles;
            if (more) fetch(tile + 4, buf ^ 1);
            // Wait for this tile's copies, issued one iteration ago.  When the next
            // tile's 16 copies were just issued they may stay in flight.
            if (more && tile + 4 < dma_tiles)
                asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const char* tb = my_tiles + buf * kTileBytes;

            // S^T tile: lane (g, c) -> key slots 4g..4g+3, head c.  All operand reads are
            // issued before the first product so their latencies overlap.
            bf16x8 ka[16];
#pragma unroll
            for (int s = 0; s < 16; s++)
                ka[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + k_off + 64 * s));
            __builtin_amdgcn_sched_barrier(0);
            f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 16; s++) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[s], st, 0, 0, 0);
            // V operand, read transposed from the row-major tile (in flight during the
            // softmax arithmetic below)
            s16x4 vb[32];
#pragma unroll
            for (int t = 0; t < 32; t++)
                vb[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(tb + v_off + 32 * t));
            __builtin_amdgcn_sched_barrier(0);

            float lg[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int slot = tile * 16 + 4 * g + i;
                const bool valid = (slot < nsel) || (slot >= sel_pad && slot < nslots);
                lg[i] = valid ? st[i] * qk_scale : -INFINITY;
                tmax = fmaxf(tmax, lg[i]);
            }
            tmax = max_over_g(tmax);
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
            l_run += sum_over_g(psum);
            __builtin_amdgcn_sched_barrier(0);

            // O += P V
#pragma unroll
            for (int t = 0; t < 32; t++) o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb[t], o[t], 0, 0, 0);
        }
        if (!__ballot(over)) break;
    }
    __syncthreads();  // every wave is done with its tiles: the merge reuses them

    // ---- merge the four waves: out = sum_w O_w 2^(m_w - M) / L
    float(*s_o)[16][256 + 4] = reinterpret_cast<float(*)[16][256 + 4]>(s_tiles);
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
            const int d = 16 * tt + c;
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
