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
// Workgroup = 4 waves on one query row and 16 heads (h0 .. h0+15).  The row's key slots
// are the k selected entries (tiles of 16; an entry -1 is masked and a tile with no valid
// entry is skipped) followed by the window positions.  Wave w takes tiles w, w+4, ...
// with its own online-softmax state and output, double-buffering them in LDS: while it
// computes on one tile, the next one is on its way (selected and bf16 window rows by
// direct global-to-LDS copies, one 1 KiB row per instruction; FP8 window rows are
// dequantized to bf16 through registers: E4M3 times a power of two is exact in bf16).
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
constexpr int kRowBytes = kAttnD * 2 + 48;           // LDS row pitch of a tile (48 B pad)
constexpr int kTileBytes = 16 * kRowBytes;            // one tile of 16 keys
constexpr int kWaveBytes = 2 * kTileBytes;            // double buffer per wave
constexpr int kMergeWave = 512 * 64 + 64 * 16;        // one wave's output in the merge: [dim][16 heads] + pad
constexpr int kLdsBytes = 4 * kMergeWave > 4 * kWaveBytes ? 4 * kMergeWave : 4 * kWaveBytes;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}

// Tiles are row-major in LDS with a pitch of 1072 B (1024 + 3 x 16): 16-byte chunk q of
// key r starts at 67 r + q chunks, so the 16 keys of a K-operand read (same chunk) fall
// on distinct banks, and so do the 4 keys x 4 chunks of a transposed V read.
//
// Copy 4 keys into LDS: key q (0..3) goes to byte address m0v + 1072 q (wave-uniform),
// lane l passing the global address of the key's byte 16 l minus 1072 q (the immediate
// offset moves both the global and the LDS address).  The copies are asynchronous: 4
// vector-memory instructions, complete once s_waitcnt vmcnt has dropped past them.
// Inline assembly, so the compiler adds no wait for them before unrelated LDS reads.
__device__ __forceinline__ void dma_rows4(uint32_t m0v, const void* a0, const void* a1, const void* a2,
                                          const void* a3)
{
    asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, off\n\t"
                 "global_load_lds_dwordx4 %1, off offset:1072\n\t"
                 "global_load_lds_dwordx4 %2, off offset:2144\n\t"
                 "global_load_lds_dwordx4 %3, off offset:3216"
                 :: "v"(a0), "v"(a1), "v"(a2), "v"(a3), "s"(m0v) : "memory", "m0");
}
static_assert(kRowBytes == 1072, "dma_rows4 encodes the row pitch");

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
    __shared__ __attribute__((aligned(16))) char s_tiles[kLdsBytes];
    __shared__ __attribute__((aligned(16))) int32_t s_sel[2048];
    __shared__ uint32_t s_vmask[128];
    __shared__ float s_m[4][16], s_l[4][16];

    const int b = blockIdx.x;
    const int row = 8 * (b / (8 * nhg)) + (b & 7);
    const int hg = (b >> 3) % nhg;
    if (row >= rows.n) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int h0 = 16 * hg;

    // ---- Q^T as the B operand (lane (g, c): head h0+c, dims [32s+8g, +8)), issued first
    bf16x8 qb[16];
    {
        const uint16_t* qrow = q + ((int64_t)row * H + h0 + c) * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; s++) qb[s] = load_bf16x8(qrow + 32 * s);
    }
    const RowKeys rk = row_keys(rows, cache, swa, sel, sel_stride, sel_row_map, row);

    // ---- selected slots: indices into LDS (-1 replaced by the request's entry 0, which
    // exists whenever the tile holds a valid entry) and a 16-bit validity mask per tile
    const int sel_tiles = (k + 15) >> 4;
    for (int base = 0; base < sel_tiles * 16; base += 256) {
        const int i = base + tid;
        const int32_t j = (i < k) ? rk.sel[i] : -1;
        const unsigned long long bal = __ballot(j >= 0);
        if (i < sel_tiles * 16) s_sel[i] = j >= 0 ? j : 0;
        const int t0 = (base + 64 * wave) / 16 + lane;
        if (lane < 4 && t0 < sel_tiles) s_vmask[t0] = (uint32_t)(bal >> (16 * lane)) & 0xffffu;
    }
    __syncthreads();
    const int ntiles = sel_tiles + ((rk.nwin + 15) >> 4);
    // Make the compiler wait for the Q loads here, not inside the tile loop where the
    // wait would also hold back the next tile's copies.
#pragma unroll
    for (int s = 0; s < 16; s++) asm volatile("" : "+v"(qb[s]));

    const uint16_t* kv_r = kv + rk.kv0 * kAttnD;
    const int64_t swa_base = swa.row_start[rk.r] - swa.pos_start[rk.r] + rk.t0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    char* my_tiles = s_tiles + wave_u * kWaveBytes;
    const uint32_t my_tiles_lds = lds_addr(my_tiles);
    // Per-lane copy sources: byte 16 lane of a key, less q row pitches for key q of a group
    // of 4 (the copy's immediate offset adds them back).  Window rows are addressed
    // relative to the window cache (row swa_row0 + wi for window slot wi).
    const int64_t swa_row0 = swa_base;
    const uint64_t sel_lane0 = reinterpret_cast<uint64_t>(kv_r) + 16 * lane;
    const uint64_t win_lane0 = reinterpret_cast<uint64_t>(swa.data) + 16 * lane;
    uint32_t row_bytes;  // 1024, opaque to the compiler so the address is one v_mad_u64_u32
    asm("s_mov_b32 %0, 1024" : "=s"(row_bytes));
    // tiles that arrive by direct copies: selected rows, and a bf16 window
    const int dma_tiles = (swa.dtype == 3) ? sel_tiles : ntiles;
    // the wave's next tile at or after t that holds a valid slot
    auto next_tile = [&](int t) {
        while (t < sel_tiles && s_vmask[t] == 0) t += 4;
        return __builtin_amdgcn_readfirstlane(t);
    };

    // Start the copy of tile `tile` into buffer `buf`.  Rows that arrive by direct copy
    // are only issued here; FP8 window rows are loaded, dequantized and stored to LDS.
    auto fetch = [&](int tile, int buf) {
        const uint32_t dst = my_tiles_lds + buf * kTileBytes;
        if (tile < sel_tiles || swa.dtype != 3) {
            uint32_t jr[16];  // the tile's rows, relative to the base of its source
            const bool from_sel = tile < sel_tiles;
            if (from_sel) {
                int4 jv[4];
#pragma unroll
                for (int u = 0; u < 4; u++) jv[u] = reinterpret_cast<const int4*>(s_sel + tile * 16)[u];
#pragma unroll
                for (int r = 0; r < 16; r++) jr[r] = (uint32_t)jv[r >> 2][r & 3];
            } else {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    int wi = (tile - sel_tiles) * 16 + r;
                    wi = wi < rk.nwin ? wi : rk.nwin - 1;
                    jr[r] = (uint32_t)(swa_row0 + wi);
                }
            }
            const uint64_t l0 = from_sel ? sel_lane0 : win_lane0;
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                // one multiply-add per key: row * 1024 + lane base
                const uint64_t a0 = (uint64_t)jr[4 * r4] * row_bytes + l0;
                const uint64_t a1 = (uint64_t)jr[4 * r4 + 1] * row_bytes + (l0 - kRowBytes);
                const uint64_t a2 = (uint64_t)jr[4 * r4 + 2] * row_bytes + (l0 - 2 * kRowBytes);
                const uint64_t a3 = (uint64_t)jr[4 * r4 + 3] * row_bytes + (l0 - 3 * kRowBytes);
                dma_rows4(dst + 4 * kRowBytes * r4, reinterpret_cast<const void*>(a0), reinterpret_cast<const void*>(a1),
                          reinterpret_cast<const void*>(a2), reinterpret_cast<const void*>(a3));
            }
        } else {
            int wi = (tile - sel_tiles) * 16 + c;
            wi = wi < rk.nwin ? wi : rk.nwin - 1;
            const int64_t srow = swa_base + wi;
            const uint8_t* sr = static_cast<const uint8_t*>(swa.data) + srow * kAttnD + 8 * g;
            const uint8_t* sc = swa.scale + srow * (kAttnD / 32);
            char* dp = my_tiles + buf * kTileBytes + kRowBytes * c + 16 * g;
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
    const int k_off = kRowBytes * c + 16 * g;                    // K operand, step s at +64 s
    const int v_off = kRowBytes * (4 * g + (c >> 2)) + 8 * (c & 3);  // V operand, dim tile t at +32 t
    f32x4 o[32];
    float m_ref = -INFINITY, l_run = 0.0f, m_true = -INFINITY;
    for (int attempt = 0; attempt < 2; attempt++) {
#pragma unroll
        for (int t = 0; t < 32; t++) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        l_run = 0.0f;
        m_ref = (attempt == 0) ? -INFINITY : m_true;
        bool over = false;
        int buf = 0;
        int tile = next_tile(wave_u);
        if (tile < ntiles) fetch(tile, 0);
        for (; tile < ntiles; buf ^= 1) {
            const int nxt = next_tile(tile + 4);
            const bool more = nxt < ntiles;
            if (more) fetch(nxt, buf ^ 1);
            // Wait for this tile's copies, issued one iteration ago.  When the next
            // tile's 16 copies were just issued they may stay in flight.
            if (more && nxt < dma_tiles)
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

            const uint32_t vmask = (tile < sel_tiles) ? __builtin_amdgcn_readfirstlane(s_vmask[tile]) : 0u;
            float lg[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bool valid = (tile < sel_tiles) ? ((vmask >> (4 * g + i)) & 1u) != 0
                                                      : (tile - sel_tiles) * 16 + 4 * g + i < rk.nwin;
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
            tile = nxt;
        }
        if (!__ballot(over)) break;
    }
    __syncthreads();  // every wave is done with its tiles: the merge reuses them

    // ---- merge the four waves: out = sum_w O_w 2^(m_w - M) / L.  Each wave stores its
    // scaled output as [dim][16 heads] (16 B per lane store; 16 B of padding every 8
    // dims spreads the reads over the banks), then every thread sums 4 heads x 8 dims.
    if (g == 0) {
        s_m[wave][c] = m_ref;
        s_l[wave][c] = l_run;
    }
    __syncthreads();  // also: every wave is done with its tiles, which the merge reuses
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
    auto o_off = [](int w, int d, int quad) { return w * kMergeWave + d * 64 + (d >> 3) * 16 + quad * 16; };
#pragma unroll
    for (int t = 0; t < 32; t++)
        *reinterpret_cast<f32x4*>(s_tiles + o_off(wave, 16 * t + c, g)) =
            f32x4{o[t][0] * fac[0], o[t][1] * fac[1], o[t][2] * fac[2], o[t][3] * fac[3]};
    __syncthreads();
    {
        const int quad = tid & 3, db = tid >> 2;  // heads 4 quad .. +3, dims 8 db .. +7
        f32x4 acc[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int d = 8 * db + e;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(s_tiles + o_off(0, d, quad));
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(s_tiles + o_off(1, d, quad));
            const f32x4 v2 = *reinterpret_cast<const f32x4*>(s_tiles + o_off(2, d, quad));
            const f32x4 v3 = *reinterpret_cast<const f32x4*>(s_tiles + o_off(3, d, quad));
            acc[e] = ((v0 + v1) + v2) + v3;
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            bf16x8 r;
#pragma unroll
            for (int e = 0; e < 8; e++) r[e] = (__bf16)acc[e][i];
            *reinterpret_cast<bf16x8*>(out + ((int64_t)row * H + h0 + 4 * quad + i) * kAttnD + 8 * db) = r;
        }
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
