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
    int64_t wbase;  // window row of position 0 (row_keys_spec only)
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

// row_keys for the bf16 kernel, with the request's metadata loaded speculatively: in a
// decode batch row q usually serves request q, so the per-request values of request
// `row` (when such a request exists) are loaded together with the row's own request
// number and used when it matches; only a row of another request waits for a second
// round of loads.  The result is row_keys' in every case.
__device__ __forceinline__ RowKeys row_keys_spec(const RowsArg& rows, const CacheArg& cache, const SwaArg& swa,
                                                 const int32_t* sel, int64_t sel_stride,
                                                 const int32_t* sel_row_map, int row)
{
    const int g = row < cache.nreq ? row : 0;
    const int64_t kv0_g = cache.row_start[g];
    const int64_t ps_g = swa.pos_start[g];
    const int64_t ws_g = swa.row_start[g];
    RowKeys rk;
    rk.r = rows.req[row];
    rk.p = rows.pos[row];
    const bool hit = rk.r == g;
    rk.kv0 = hit ? kv0_g : cache.row_start[rk.r];
    const int64_t ps = hit ? ps_g : swa.pos_start[rk.r];
    rk.wbase = (hit ? ws_g : swa.row_start[rk.r]) - ps;
    int64_t t0 = (int64_t)rk.p - swa.window + 1;
    const int64_t lo = rows.win_lo ? rows.win_lo[row] : 0;
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
// direct global-to-LDS copies with scalar row addresses, one 1 KiB row per instruction;
// FP8 window rows are loaded into registers a tile ahead and dequantized to bf16 by the
// scaled conversion: E4M3 times a power of two is exact in bf16).  Main KV in the FP4
// storage format ("DeepSeek V4.1 Flash modeling", section "Mixed precision": dequantized
// before attention) takes the register route too: E2M1 times its E4M3 block scale has
// at most 6 significant bits, so the decoded bf16 tile is exact and the MFMAs see the
// same operands as for a bf16 cache holding the decoded values.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, 16 steps over the 512 dims: A = K rows
//     from LDS (lane (g, c) holds key c, dims [32s+8g, +8)), B = Q^T in registers.  The
//     next tile's K operand is read while this tile's P V products run.
//   * S^T output: lane (g, c) holds keys 4g..4g+3 of head c, which is the B operand of
//     O^T = V^T P^T with v_mfma_f32_16x16x16_bf16 (keys are the contraction index).
//   * The V^T operand (lane (g, c): keys 4g..4g+3 of dim c) comes straight from the row-
//     major tile with the LDS transpose read ds_read_b64_tr_b16: within a 16-lane group,
//     element j of lane i comes from the 8-byte chunk that lane 4j + i/4 addresses, so
//     lane (g, 4j+q) points at V[4g+j][16t+4q].
//   * Output O^T: 32 tiles of 16 dims x 16 heads (lane (g, c): dims 16t+4g..+3, head c).
// The four waves' partial results are merged in fixed order through LDS.
// Blocks are mapped so that the head groups of one row share an XCD (and its L2): block
// b serves row 8*(b / (8*NHG)) + b%8 and head group (b/8) % NHG.
constexpr int kAttnD = 512;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowBytes = kAttnD * 2 + 48;           // LDS row pitch of a tile (48 B pad)
constexpr int kTileBytes = 16 * kRowBytes;            // one tile of 16 keys
constexpr int kWaveBytes = 2 * kTileBytes;            // double buffer per wave

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}

// Tiles are row-major in LDS with a pitch of 1072 B (1024 + 3 x 16): 16-byte chunk q of
// key r starts at 67 r + q chunks, so the 8 keys of each 8-lane group of a K-operand read
// (same chunk) fall on distinct bank quads, and a transposed V read conflicts at most
// 2-way.
static_assert(kRowBytes == 1072, "dma_rows4_s encodes the row pitch");

// Sum over the four 16-lane rows (lanes c, c+16, c+32, c+48).
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

// Copy 4 keys into LDS: key u (0..3) goes to byte address m0v + 1072 u, its global row
// address being au + 1072 u (au already holds the -1072 u that the immediate offset adds
// back); every lane passes the same offset 16 lane.  The copies are asynchronous: 4
// vector-memory instructions, complete once s_waitcnt vmcnt has dropped past them.
// Inline assembly, so the compiler adds no wait for them before unrelated LDS reads.
__device__ __forceinline__ void dma_rows4_s(uint32_t m0v, uint32_t voff, uint64_t a0, uint64_t a1, uint64_t a2,
                                            uint64_t a3)
{
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %2 offset:1072\n\t"
                 "global_load_lds_dwordx4 %0, %3 offset:2144\n\t"
                 "global_load_lds_dwordx4 %0, %4 offset:3216"
                 :: "v"(voff), "s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(m0v) : "memory", "m0");
}

// Float max without the NaN quieting that fmaxf adds around lane-swapped values (the
// operands here are logits or -inf, never NaN).
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 8 FP8 E4M3 codes times 2^(e - 127) to bf16 (exact: 3 mantissa bits fit in bf16's 7).
// The scaled conversion takes the E8M0 exponent as the exponent field of an fp32 scale.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8_e(uint2 u, uint32_t e)
{
    const float sc = __builtin_bit_cast(float, e << 23);
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, sc, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, sc, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, sc, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, sc, true);
    return uint4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                 __builtin_bit_cast(uint32_t, d)};
}

// 8 E2M1 codes (one dword; element 2i in the low nibble of byte i) times the block scale s
// to bf16.  The fp32 products are exact, and so is their bf16 rounding.
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t w, float s)
{
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    auto pack = [s](f32x2 f) {
        return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(f[0] * s), (__bf16)(f[1] * s)});
    };
    return uint4{pack(f0), pack(f1), pack(f2), pack(f3)};
}

template <bool kKvFp4>
__global__ __launch_bounds__(256) void k_attn_bf16(RowsArg rows, CacheArg cache, const uint16_t* __restrict__ q,
                                                   int H, int nhg, const void* __restrict__ kv,
                                                   const uint8_t* __restrict__ kv_scale,
                                                   const int32_t* __restrict__ sel, int k, int64_t sel_stride,
                                                   const int32_t* __restrict__ sel_row_map, SwaArg swa,
                                                   float sm_scale, const float* __restrict__ sink,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse)
{
    __shared__ __attribute__((aligned(16))) char s_tiles[4 * kWaveBytes];
    __shared__ __attribute__((aligned(16))) int32_t s_sel[2048];
    __shared__ uint32_t s_vmask[128];
    __shared__ float s_m[4][16], s_l[4][16];

    const int b = blockIdx.x;
    const int row = 8 * (b / (8 * nhg)) + (b & 7);
    const int hg = (b >> 3) % nhg;
    if (row >= rows.n) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int h0 = 16 * hg;

    // Wave w takes tiles w, w+4, ...: first its selected tiles (empty ones skipped),
    // then its window tiles.  Each wave stages the slots of its own selected tiles, so no
    // workgroup barrier precedes the tile loop.
    const int sel_tiles = (k + 15) >> 4;
    const int ntw = sel_tiles > wave ? (sel_tiles - wave + 3) >> 2 : 0;  // the wave's selected tiles (<= 32)
    const int32_t* selrow = sel ? sel + (int64_t)(sel_row_map ? sel_row_map[row] : row) * sel_stride : nullptr;
    // pass r, lane (g, c): slot c of the wave's tile 4r + g
    int32_t jl[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        jl[r] = -1;
        if (4 * r < ntw) {
            const int i = 4 * r + g;
            const int e = 16 * (wave + 4 * i) + c;
            if (i < ntw && e < k) jl[r] = selrow[e];
        }
    }

    // ---- Q^T as the B operand (lane (g, c): head h0+c, dims [32s+8g, +8))
    bf16x8 qb[16];
    {
        const uint16_t* qrow = q + ((int64_t)row * H + h0 + c) * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; s++) qb[s] = load_bf16x8(qrow + 32 * s);
    }
    const RowKeys rk = row_keys_spec(rows, cache, swa, sel, sel_stride, sel_row_map, row);
    const int ntiles = sel_tiles + ((rk.nwin + 15) >> 4);
    const int64_t swa_base = rk.wbase + rk.t0;
    const int win_first = wave + 4 * ntw;  // the wave's first window tile

    // FP8 window tiles go through registers: the raw rows of the wave's next window tile
    // are loaded one tile ahead (the first one here), so converting them into the LDS
    // buffer does not wait on memory.
    const bool win_fp8 = swa.dtype == 3;
    uint2 wr[16];
    uint32_t wsc[4];
    auto load_win = [&](int tile) {
        int wi = (tile - sel_tiles) * 16 + c;
        wi = wi < rk.nwin ? wi : rk.nwin - 1;
        const int64_t srow = swa_base + wi;
        const uint8_t* sr = static_cast<const uint8_t*>(swa.data) + srow * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; s++) wr[s] = *reinterpret_cast<const uint2*>(sr + 32 * s);
        const uint4 sc4 = *reinterpret_cast<const uint4*>(swa.scale + srow * (kAttnD / 32));
        wsc[0] = sc4.x;
        wsc[1] = sc4.y;
        wsc[2] = sc4.z;
        wsc[3] = sc4.w;
    };
    auto prefetch_win = [&](int tile) {
        if (win_fp8 && tile >= sel_tiles && tile < ntiles) load_win(tile);
    };
    prefetch_win(win_first);

    // ---- the wave's selected slots into LDS (-1 replaced by the request's entry 0, which
    // exists whenever the tile holds a valid entry), a 16-bit validity mask per tile, and
    // one bit per wave tile that holds any valid slot
    uint32_t nonempty = 0;
#pragma unroll
    for (int r = 0; r < 8; r++) {
        if (4 * r < ntw) {
            const int i = 4 * r + g;
            const int t = wave + 4 * i;
            const int32_t j = jl[r];
            const uint64_t bal = __ballot(j >= 0);
            if (i < ntw) {
                s_sel[16 * t + c] = j >= 0 ? j : 0;
                if (c == 0) s_vmask[t] = (uint32_t)(bal >> (16 * g)) & 0xffffu;
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
                if ((bal >> (16 * u)) & 0xffffull) nonempty |= 1u << (4 * r + u);
        }
    }

    char* my_tiles = s_tiles + wave * kWaveBytes;
    const uint32_t my_tiles_lds = lds_addr(my_tiles);
    const uint32_t voff = 16 * lane;
    // Scalar row addresses: row j of the request's main KV (selected) or window row wi
    // (bf16 window), less 1072 q for the q-th key of a group of 4.
    const uint64_t kv_r = reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(kv) + rk.kv0 * kAttnD);
    const uint64_t win_r = reinterpret_cast<uint64_t>(swa.data) + (uint64_t)swa_base * (kAttnD * 2);
    // the wave's next tile at or after t (t = wave + 4 i) that holds a valid slot
    auto next_tile = [&](int t) -> int {
        if (t < sel_tiles) {
            const int i = (t - wave) >> 2;
            const uint32_t m = nonempty >> i;
            return m ? t + 4 * (int)__builtin_ctz(m) : win_first;
        }
        return t;
    };

    // FP4 main KV: the raw rows of the wave's next selected tile are loaded one tile ahead,
    // like FP8 window rows.  Lane (g, c) holds code bytes [64 g, 64 g + 64) of slot c, i.e.
    // dims [128 g, 128 g + 128), and the 8 E4M3 scales of those dims.
    uint4 kr[4];
    uint2 ksc;
    auto prefetch_sel = [&](int tile) {
        if (!kKvFp4 || tile >= sel_tiles) return;
        const int64_t j = rk.kv0 + s_sel[16 * tile + c];
        const uint4* cp = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(kv) + j * (kAttnD / 2) + 64 * g);
#pragma unroll
        for (int i = 0; i < 4; i++) kr[i] = cp[i];
        ksc = *reinterpret_cast<const uint2*>(kv_scale + j * (kAttnD / 16) + 8 * g);
    };
    // whether tile t arrives by direct copies (else through registers)
    auto by_dma = [&](int t) -> bool { return t < sel_tiles ? !kKvFp4 : !win_fp8; };
    // after tile t has been fetched: load the registers of the wave's next tile of its kind
    auto prefetch_after = [&](int t) {
        if (t < sel_tiles)
            prefetch_sel(next_tile(t + 4));
        else
            prefetch_win(t + 4);
    };

    // Start the copy of tile `tile` into buffer `buf`; returns the tile's 16-bit mask of
    // valid slots.  Rows that arrive by direct copy are only issued here; FP8 window rows
    // and FP4 main rows are converted from registers and stored to LDS.
    auto fetch = [&](int tile, int buf) -> uint32_t {
        const uint32_t dst = my_tiles_lds + buf * kTileBytes;
        if (kKvFp4 && tile < sel_tiles) {
            // lane (g, c): slot c, dims [128 g + 8 i, +8) share scale i / 2 of the lane's 8
            char* dp = my_tiles + buf * kTileBytes + kRowBytes * c + 256 * g;
            float sv[8];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t sw = h ? ksc.y : ksc.x;
                const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
                const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, true);
                sv[4 * h] = lo[0];
                sv[4 * h + 1] = lo[1];
                sv[4 * h + 2] = hi[0];
                sv[4 * h + 3] = hi[1];
            }
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const uint32_t w = kr[i >> 2][i & 3];
                *reinterpret_cast<uint4*>(dp + 16 * i) = fp4x8_to_bf16x8(w, sv[i >> 1]);
            }
            return __builtin_amdgcn_readfirstlane(s_vmask[tile]);
        }
        if (tile < sel_tiles) {
            int4 jv[4];
#pragma unroll
            for (int u = 0; u < 4; u++) jv[u] = reinterpret_cast<const int4*>(s_sel + tile * 16)[u];
            const uint32_t vm = __builtin_amdgcn_readfirstlane(s_vmask[tile]);
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                uint64_t a[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint32_t j = __builtin_amdgcn_readfirstlane(jv[r4][u]);
                    a[u] = kv_r + ((uint64_t)j << 10) - (uint64_t)(kRowBytes * u);
                }
                dma_rows4_s(dst + 4 * kRowBytes * r4, voff, a[0], a[1], a[2], a[3]);
            }
            return vm;
        }
        const int w0 = (tile - sel_tiles) * 16;
        const int nv = rk.nwin - w0;
        const uint32_t vm = nv >= 16 ? 0xffffu : (1u << nv) - 1u;
        if (!win_fp8) {
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                uint64_t a[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int wi = w0 + 4 * r4 + u < rk.nwin ? w0 + 4 * r4 + u : rk.nwin - 1;
                    a[u] = win_r + ((uint64_t)(uint32_t)wi << 10) - (uint64_t)(kRowBytes * u);
                }
                dma_rows4_s(dst + 4 * kRowBytes * r4, voff, a[0], a[1], a[2], a[3]);
            }
        } else {
            char* dp = my_tiles + buf * kTileBytes + kRowBytes * c + 16 * g;
#pragma unroll
            for (int s = 0; s < 16; s++) {
                const uint32_t e = (wsc[s >> 2] >> (8 * (s & 3))) & 0xffu;
                *reinterpret_cast<uint4*>(dp + 64 * s) = fp8x8_to_bf16x8_e(wr[s], e);
            }
        }
        return vm;
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
        // Two tiles in flight: the current one (operands being read) and the next one
        // (arriving); the next tile's K operand is read while this tile's P V runs.
        if (attempt == 1) prefetch_win(win_first);
        int buf = 0;
        int tile = next_tile(wave);
        prefetch_sel(tile);
        uint32_t vm_cur = 0, vm_nxt = 0;
        int nxt = ntiles;
        bf16x8 ka[16];
        if (tile < ntiles) {
            vm_cur = fetch(tile, 0);
            prefetch_after(tile);
            nxt = next_tile(tile + 4);
            if (nxt < ntiles) vm_nxt = fetch(nxt, 1);
            if (nxt < ntiles && by_dma(nxt))
                asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (nxt < ntiles) prefetch_after(nxt);
#pragma unroll
            for (int s = 0; s < 16; s++)
                ka[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(my_tiles + k_off + 64 * s));
        }
        // The first copies are on their way: make the compiler wait for the Q loads here
        // (the wait above has already covered them), not inside the tile loop where its
        // wait would also hold back copies.
#pragma unroll
        for (int s = 0; s < 16; s++) asm volatile("" : "+v"(qb[s]));
        for (; tile < ntiles; buf ^= 1) {
            const char* tb = my_tiles + buf * kTileBytes;
            // S^T tile: lane (g, c) -> key slots 4g..4g+3, head c; two accumulators halve
            // the dependent chain
            f32x4 st0 = {0.0f, 0.0f, 0.0f, 0.0f}, st1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 16; s += 2) {
                st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[s], st0, 0, 0, 0);
                st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s + 1], qb[s + 1], st1, 0, 0, 0);
            }
            // V operand, read transposed from the row-major tile (in flight during the
            // softmax arithmetic below)
            s16x4 vb[32];
#pragma unroll
            for (int t = 0; t < 32; t++)
                vb[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(tb + v_off + 32 * t));
            __builtin_amdgcn_sched_barrier(0);

            float lg[4];
#pragma unroll
            for (int i = 0; i < 4; i++) lg[i] = (st0[i] + st1[i]) * qk_scale;
            if (vm_cur != 0xffffu) {
                const uint32_t bits = vm_cur >> (4 * g);
#pragma unroll
                for (int i = 0; i < 4; i++) lg[i] = (bits >> i) & 1u ? lg[i] : -INFINITY;
            }
            float tmax = vmax(vmax(lg[0], lg[1]), vmax(lg[2], lg[3]));
            {
                const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
                const auto bb = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = vmax(__uint_as_float(bb[0]), __uint_as_float(bb[1]));
            }
            m_true = vmax(m_true, tmax);
            if (m_ref == -INFINITY && tmax != -INFINITY) m_ref = tmax + 64.0f;  // the accumulator is still zero
            over |= tmax > m_ref;
            const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) pv[i] = __builtin_amdgcn_exp2f(lg[i] - m_use);
            const float psum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
            const bf16x2_t p01 = bf16x2_t{(__bf16)pv[0], (__bf16)pv[1]};
            const bf16x2_t p23 = bf16x2_t{(__bf16)pv[2], (__bf16)pv[3]};
            const s16x4 pa = __builtin_bit_cast(s16x4, uint2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)});
            l_run += sum_over_g(psum);
            __builtin_amdgcn_sched_barrier(0);

            // O^T += V^T P^T
#pragma unroll
            for (int t = 0; t < 32; t++) o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb[t], pa, o[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);

            // This buffer is free (its V operand is in registers): it takes the tile after
            // next.  Then wait for the next tile and read its K operand while P V runs.
            int n2 = ntiles;
            uint32_t vm_n2 = 0;
            if (nxt < ntiles) {
                n2 = next_tile(nxt + 4);
                if (n2 < ntiles) vm_n2 = fetch(n2, buf);
                if (n2 < ntiles && by_dma(n2))
                    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (n2 < ntiles) prefetch_after(n2);
                const char* tn = my_tiles + (buf ^ 1) * kTileBytes;
#pragma unroll
                for (int s = 0; s < 16; s++)
                    ka[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tn + k_off + 64 * s));
            }
            tile = nxt;
            nxt = n2;
            vm_cur = vm_nxt;
            vm_nxt = vm_n2;
        }
        if (!__ballot(over)) break;
    }

    // ---- merge the four waves: out = sum_w O_w 2^(m_w - M) / L.  Each wave stores its
    // unscaled O^T into its own tile area as [16 heads][512 dims] with a head pitch of
    // 2064 B (516 dwords: the 8 lanes of each 8-lane group of a 16-byte store fall on
    // distinct bank quads) as soon as its loop ends; after one barrier wave w combines
    // dims [128 w, 128 w + 128) of the 16 heads, reading the four waves' values with the
    // same lane pattern.
    constexpr int kHeadPitch = 2064;
    static_assert(16 * kHeadPitch <= kWaveBytes, "a wave's output fits its tile area");
    {
        char* ob = my_tiles + kHeadPitch * c + 16 * g;
#pragma unroll
        for (int t = 0; t < 32; t++) *reinterpret_cast<f32x4*>(ob + 64 * t) = o[t];
    }
    if (g == 0) {
        s_m[wave][c] = m_ref;
        s_l[wave][c] = l_run;
    }
    __syncthreads();
    float fac[4];
    {
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            mw[w] = s_m[w][c];
            M = fmaxf(M, mw[w]);
        }
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            fac[w] = __builtin_amdgcn_exp2f(mw[w] - Mu);
            L += s_l[w][c] * fac[w];
        }
        if (sink && M != -INFINITY) L += __builtin_amdgcn_exp2f(sink[h0 + c] * kLog2e - Mu);
        const float rL = (L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) fac[w] *= rL;
        if (lse && wave == 0 && g == 0)
            lse[(int64_t)row * H + h0 + c] = (M == -INFINITY) ? -INFINITY : (M + __log2f(L)) * 0.69314718055994531f;
    }
    {
        const char* ib = s_tiles + kHeadPitch * c + 16 * g + 512 * wave;
        uint16_t* orow = out + ((int64_t)row * H + h0 + c) * kAttnD + 128 * wave + 4 * g;
#pragma unroll
        for (int u = 0; u < 8; u++) {
            f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < 4; w++) a += *reinterpret_cast<const f32x4*>(ib + w * kWaveBytes + 64 * u) * fac[w];
            const bf16x2_t r01 = bf16x2_t{(__bf16)a[0], (__bf16)a[1]};
            const bf16x2_t r23 = bf16x2_t{(__bf16)a[2], (__bf16)a[3]};
            *reinterpret_cast<uint2*>(orow + 16 * u) =
                uint2{__builtin_bit_cast(uint32_t, r01), __builtin_bit_cast(uint32_t, r23)};
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
                            const void* kv, const uint8_t* kv_scale, const int32_t* sel, int k, int64_t sel_stride,
                            const int32_t* sel_row_map, const SwaArg& swa, float sm_scale, const float* sink,
                            uint16_t* out, float* lse, hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const int nhg = heads / 16;
    const int64_t nblocks = (int64_t)((rows.n + 7) / 8) * 8 * nhg;
    if (kv_scale)
        hipLaunchKernelGGL((k_attn_bf16<true>), dim3((unsigned)nblocks), dim3(256), 0, stream, rows, cache, q, heads,
                           nhg, kv, kv_scale, sel, k, sel_stride, sel_row_map, swa, sm_scale, sink, out, lse);
    else
        hipLaunchKernelGGL((k_attn_bf16<false>), dim3((unsigned)nblocks), dim3(256), 0, stream, rows, cache, q, heads,
                           nhg, kv, kv_scale, sel, k, sel_stride, sel_row_map, swa, sm_scale, sink, out, lse);
    return hipGetLastError();
}

}  // namespace csa2
