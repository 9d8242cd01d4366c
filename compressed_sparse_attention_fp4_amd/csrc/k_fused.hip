// Fused pool scoring + top-k: the restricted scoring and the selection of a Reindex
// layer in one kernel, with no score written to memory.
//
// Pages: "DeepSeek V4.1 Flash modeling", section "Hierarchical Sparse Indexer" (later index
// layers rescore only the shared candidate pool and take their own top-k inside it; the
// section's measurement notes ask for the fused module of restricted scoring and
// selection and its data movement); "SGLang and Miles Day-0 support for DeepSeek-V4.1",
// section 5 (the indexer scores the FP4 cache directly, MQA form).
//
// One workgroup per query row and segment of pool columns: launches over many rows take
// a whole pool of up to 16,384 columns (2,048 blocks of 8) per 1024-thread workgroup;
// few rows (a decode batch) split the pool into segments of 4,096 columns on 512
// threads, so that the scoring spreads over every CU.  Its waves score the segment exactly as
// csa2_index_score does for a pool (the same MXFP4 MFMA tiles, head permutation and fixed
// head-sum order, so every score is bit for bit the same), turn each score into its order
// key in LDS (a column past the pool, or a pool position past the row's reach, is no
// candidate), and run the radix selection of csa2_topk over those keys: thread t takes
// keys [KPT t, KPT t + KPT), whole pool blocks, so positions follow from the block ids in
// LDS.  A one-segment pool writes the index set directly, with no second launch; longer
// pools write each segment's top-k as (key, position) lists, which csa2_topk's exact list
// merge reduces to the index set.  The result is what csa2_index_score + csa2_topk give,
// without the 64 KiB score row per query going to memory and back.
#include "csa2_device.h"
#include "csa2_launch.h"
#include "csa2_score.h"
#include "csa2_select.h"

#pragma clang fp contract(off)

namespace csa2 {

// Segment shapes: a whole pool of up to 16,384 columns in one workgroup (no merge), or
// segments of 4,096 columns merged afterwards.
constexpr int kWholeNT = 1024, kWholeKPT = 16, kWholeCap = kWholeNT * kWholeKPT;
constexpr int kSegNT = 512, kSegKPT = 8, kSegCap = kSegNT * kSegKPT;
// Key groups in flight per wave: 1024-thread workgroups have 128 VGPRs per lane, 512-thread
// ones 256 (a group takes 20).
constexpr int kWholeDepth = 2, kSegDepth = 2;

template <int NHT, int kFusedNT, int kFusedKPT, int DEPTH>
__global__ __launch_bounds__(kFusedNT) void k_score_topk_pool(RowsArg rows, CacheArg cache, const void* __restrict__ q,
                                                         const uint8_t* __restrict__ q_scale,
                                                         const float* __restrict__ w, int64_t w_stride,
                                                         const uint8_t* __restrict__ kdata,
                                                         const uint8_t* __restrict__ kscale, PoolArg pool, int k,
                                                         int nseg, int32_t* __restrict__ out_idx,
                                                         uint2* __restrict__ out_list)
{
    constexpr int H = NHT * 16;
    constexpr int G = H / 4;
    constexpr int NW = kFusedNT / 64;
    constexpr int kFusedCap = kFusedNT * kFusedKPT;
    // the selection takes each thread's pool block ids from its own slots of s_bid
    static_assert(kFusedKPT % 8 == 0, "each thread holds whole pool blocks of 8 candidates");
    __shared__ uint4 s_qa[NHT][64];
    __shared__ uint32_t s_qs[NHT][64];
    __shared__ int32_t s_bid[kFusedCap / 8];
    __shared__ __attribute__((aligned(16))) uint32_t s_key[kFusedCap];

    int row, seg;
    xcd_row_chunk(blockIdx.x, rows.n, nseg, &row, &seg);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The pool row's block count and block ids are read beside the row's request lookups,
    // not after them (a row without reach ignores them; its pool row is valid all the same).
    const int prow = pool.row_map ? pool.row_map[row] : row;
    const int nb_pool = pool.nblocks[prow];
    const int r = rows.req[row];
    const int64_t R = reach(rows.pos[row], cache.ratio_m, cache.n_entries[r]);
    const int nb_row = R > 0 ? nb_pool : 0;  // <= max_blocks <= 2048 (host-checked)
    const int ncol_row = nb_row * 8;
    const int c_begin = seg * kFusedCap;            // the segment's first pool column
    const int nb0 = c_begin / 8;                    // and block
    int nbs = nb_row - nb0;                         // blocks of the segment
    nbs = nbs < 0 ? 0 : (nbs > kFusedCap / 8 ? kFusedCap / 8 : nbs);
    const int ncol = __builtin_amdgcn_readfirstlane(nbs * 8);  // columns of the segment
    const int R32 = __builtin_amdgcn_readfirstlane((int)R);  // positions < n_entries fit 32 bits

    // ---- the row's index q quantized into A operands (one 32-element block per thread;
    // with q_scale, its MXFP4 codes and scale as given), the pool's block ids and the lane
    // group's head weights
    if (tid < NHT * 64 && q_scale) {
        const int t = tid >> 6, l = tid & 63;
        const int m = l & 15, blk = l >> 4;
        const int64_t rh = (int64_t)row * H + G * (m >> 2) + 4 * t + (m & 3);
        const u32x4_t c = gload_x4<0>(static_cast<const uint8_t*>(q) + rh * 64 + blk * 16);
        s_qa[t][l] = make_uint4(c[0], c[1], c[2], c[3]);
        s_qs[t][l] = (uint32_t)gload_u8<0>(q_scale + rh * 4 + blk);
    } else if (tid < NHT * 64) {
        const int t = tid >> 6, l = tid & 63;
        const int m = l & 15, blk = l >> 4;
        const int head = G * (m >> 2) + 4 * t + (m & 3);
        const uint16_t* src = static_cast<const uint16_t*>(q) + ((int64_t)row * H + head) * 128 + blk * 32;
        u32x4_t x[4] = {gload_x4<0>(src), gload_x4<16>(src), gload_x4<32>(src), gload_x4<48>(src)};
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                v[i * 8 + 2 * jj] = __uint_as_float(x[i][jj] << 16);
                v[i * 8 + 2 * jj + 1] = __uint_as_float(x[i][jj] & 0xFFFF0000u);
            }
        uint32_t o[4], sb;
        quant_block_e2m1(v, o, &sb);
        s_qa[t][l] = make_uint4(o[0], o[1], o[2], o[3]);
        s_qs[t][l] = sb;
    }
    {
        const int32_t* bid_row = pool.blocks + (int64_t)prow * pool.max_blocks + nb0;
        const int nslot = pool.max_blocks - nb0;  // slots of the pool row from the segment on (> 0)
        for (int i = tid; i < kFusedCap / 8; i += kFusedNT) {
            const int32_t b = bid_row[i < nslot ? i : 0];
            s_bid[i] = i < nbs ? b : 0;
        }
    }
    const int g = lane >> 4;
    float wr[NHT * 4];
    {
        const float* wrow = w + (int64_t)row * w_stride + G * g;
#pragma unroll
        for (int t = 0; t < NHT; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) wr[4 * t + i] = wrow[4 * t + i];
    }
    __syncthreads();
    i32x8 a[NHT];
    int sa[NHT];
#pragma unroll
    for (int t = 0; t < NHT; t++) {
        const uint4 u = s_qa[t][lane];
        a[t] = i32x8{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        sa[t] = (int)s_qs[t][lane];
    }

    // ---- scores of 64 columns per wave and group; wave w takes groups w, w + NW, ...,
    // loading the next group's key tiles while it scores the current one
    const int64_t krow0 = cache.row_start[r];
    const uint8_t* kd_base = kdata + krow0 * 64 + 16 * (lane >> 4);
    // Each lane loads all four block scales of its key (one dword) and takes its own byte
    // where the MFMA reads it: a byte load would leave 8-bit loop-carried registers that
    // the compiler widens at the loop's back edge, waiting there for the tiles just issued.
    const uint8_t* ks_base = kscale + krow0 * 4;
    const int sshift = 8 * (lane >> 4);
    // Lane (g, c) of tile u takes column off0 + 16 u + c.  The four block-id lookups are
    // issued together (no lane skips one: a column past the segment looks column 0 up),
    // and the lane keeps the position of column off0 + lane (tile g, its own column of the
    // group's scores) for the candidate test after scoring: -1 when that column is no
    // candidate.
    auto load = [&](int off0, u32x4_t (&kd)[4], int (&sk)[4], int& mypos) {
        int oc[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int off = off0 + 16 * u + (lane & 15);
            oc[u] = off < ncol ? off : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) bv[u] = s_bid[oc[u] >> 3];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int off = off0 + 16 * u + (lane & 15);
            const int pos = (bv[u] << 3) | (oc[u] & 7);
            const bool cand = (off < ncol) & (pos < R32);
            const int j = cand ? pos : 0;
            mypos = (u == g) ? (cand ? pos : -1) : mypos;
            kd[u] = gload_x4<0>(kd_base + ((uint64_t)(uint32_t)j << 6));
            sk[u] = gload_i32<0>(ks_base + ((uint64_t)(uint32_t)j << 2));
        }
    };
    auto score_group = [&](int off0, const u32x4_t (&kd)[4], const int (&sk)[4], int mypos) {
        float P[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            f32x4 d[NHT];
            const i32x8 b = i32x8{(int)kd[u][0], (int)kd[u][1], (int)kd[u][2], (int)kd[u][3], 0, 0, 0, 0};
            const int sb = (int)(((uint32_t)sk[u] >> sshift) & 0xffu);
#pragma unroll
            for (int t = 0; t < NHT; t++) {
                const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                d[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[t], b, zero, 4, 4, 0, sa[t], 0, sb);
            }
            float pp = 0.0f;
#pragma unroll
            for (int t = 0; t < NHT; t++)
#pragma unroll
                for (int i = 0; i < 4; i++) pp = __builtin_fmaf(wr[4 * t + i], relu_bits(d[t][i]), pp);
            P[u] = pp;
        }
        // lane group g holds P_g of tiles 0..3; after the swaps lane (g, c) holds the score
        // of tile g, position c, i.e. column off0 + lane
        auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(P[0]), __float_as_uint(P[1]), false, false);
        auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(P[2]), __float_as_uint(P[3]), false, false);
        const float h01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
        const float h23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(h01), __float_as_uint(h23), false, false);
        const float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        s_key[off0 + lane] = mypos >= 0 ? order_key(score) : 0u;
    };
    const int ngrp = (ncol + 63) >> 6;
    const int mine = wave < ngrp ? (ngrp - wave + NW - 1) / NW : 0;  // groups of this wave
    if (mine > 0) {
        // A ring of DEPTH key groups: group i is scored while groups i + 1 .. i + DEPTH - 1
        // are in flight.  Every pass issues the same loads (a group past the wave's last
        // reads column 0 again, never scored), so the compiler's wait before each group's
        // products is the same on every path and leaves the later groups in flight.
        u32x4_t kr[DEPTH][4];
        int sr[DEPTH][4], pr[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; d++) load(64 * (wave + NW * d), kr[d], sr[d], pr[d]);
        for (int i = 0; i < mine; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; d++) {
                if (i + d < mine) score_group(64 * (wave + NW * (i + d)), kr[d], sr[d], pr[d]);
                load(64 * (wave + NW * (i + d + DEPTH)), kr[d], sr[d], pr[d]);
            }
        }
    }
    // groups past the pool hold no candidate
    for (int c = 64 * ngrp + tid; c < kFusedCap; c += kFusedNT) s_key[c] = 0u;
    __syncthreads();

    // ---- selection over the LDS keys
    uint32_t key[kFusedKPT];
    {
        const uint4* kp = reinterpret_cast<const uint4*>(s_key + kFusedKPT * tid);
#pragma unroll
        for (int v4 = 0; v4 < kFusedKPT / 4; v4++) {
            const uint4 u = kp[v4];
            key[4 * v4] = u.x;
            key[4 * v4 + 1] = u.y;
            key[4 * v4 + 2] = u.z;
            key[4 * v4 + 3] = u.w;
        }
    }
    int32_t bid[bid_slots(kFusedKPT)];
#pragma unroll
    for (int b8 = 0; b8 < bid_slots(kFusedKPT); b8++) bid[b8] = s_bid[bid_slots(kFusedKPT) * tid + b8];
    SelArgs sel{};
    sel.src.rows = rows;
    sel.src.cache = cache;
    sel.src.pool = pool;
    sel.src.stride = (int64_t)pool.block * pool.max_blocks;
    sel.block = 8;
    sel.block_shift = 3;
    sel.k = k;
    sel.nseg = nseg;
    sel.seg_len = kFusedCap;
    sel.out_idx = out_idx;
    sel.out_list = out_list;
    sel.out_stride = k;
    sel.out_mode = nseg > 1 ? OUT_LIST : OUT_IDX;
    select_core<kFusedKPT, SRC_POOL, kFusedNT>(sel, row, seg, R, (int64_t)ncol_row, prow, c_begin,
                                               (int64_t)kFusedKPT * tid, key, bid, true);
}

// The exact merge of a decode batch's segment lists (each segment's top-k as (key, position)
// pairs, at most 2,048 candidates per row): the selection of csa2_topk's list merge, built in
// this file so that it shares its scheduling.  One 1024-thread workgroup per row, 2
// candidates per thread (slightly ahead of 512 threads of 4; 256 of 8 was behind), the
// row's workgroup on the XCD of its segments.
constexpr int kMergeNT = 1024, kMergeKPT = 2;

__global__ __launch_bounds__(kMergeNT) void k_merge_segment_lists(SelArgs a)
{
    int row, seg;
    xcd_row_chunk(blockIdx.x, a.src.rows.n, 1, &row, &seg);
    // list entries carry their positions and index outputs need neither the reach nor the
    // pool row, so no row metadata is loaded before the lists
    const int64_t R = 0, ncol = 0;
    const int prow = row;
    const int64_t e0 = (int64_t)threadIdx.x * kMergeKPT;
    const int64_t lim = (int64_t)a.nlists_prev * a.k;
    const uint2* in = a.in + (int64_t)row * lim;
    uint32_t v[kMergeKPT], key[kMergeKPT];
#pragma unroll
    for (int i = 0; i < kMergeKPT; i++) v[i] = in[e0 + i < lim ? e0 + i : 0].x;
#pragma unroll
    for (int i = 0; i < kMergeKPT; i++) pin(v[i]);
#pragma unroll
    for (int i = 0; i < kMergeKPT; i++) key[i] = e0 + i < lim ? v[i] : 0u;
    int32_t bid[bid_slots(kMergeKPT)] = {0};
    select_core<kMergeKPT, SRC_LIST, kMergeNT>(a, row, 0, R, ncol, prow, 0, e0, key, bid, false);
}

// Rows from which a launch takes whole pools.  One workgroup then scores a row's whole
// pool on one CU, so with fewer rows most CUs would idle; from half the CU count on, the
// saved list merge (a second launch) outweighs that (measured: 128 rows of 8,192 pool
// columns 27.6 against 31.7 us, 256 rows 28.3 against 51.1 us; 64 rows of 16,384 columns
// 44.0 against 28.8 us).
constexpr int kWholeRows = 128;

// Columns per segment: the whole pool when it fits one workgroup and the launch has rows
// enough.
static int64_t fused_cap(int n, int64_t cols)
{
    return (n >= kWholeRows && cols <= kWholeCap) ? kWholeCap : kSegCap;
}

size_t score_topk_pool_workspace(int n, int64_t cols, int k)
{
    const int64_t cap = fused_cap(n, cols);
    const int64_t nseg = (cols + cap - 1) / cap;
    return nseg > 1 ? (size_t)n * nseg * k * sizeof(uint2) : 0;
}

hipError_t launch_score_topk_pool(const RowsArg& rows, const CacheArg& cache, const IndexQ& qin, int heads,
                                  const float* w, int64_t w_stride, const uint8_t* kdata, const uint8_t* kscale,
                                  const PoolArg& pool, int k, int32_t* out_idx, void* ws, hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const int64_t cols = (int64_t)pool.block * pool.max_blocks;
    const bool whole = fused_cap(rows.n, cols) == kWholeCap;
    const int nseg = whole ? 1 : (int)((cols + kSegCap - 1) / kSegCap);
    uint2* lists = nseg > 1 ? static_cast<uint2*>(ws) : nullptr;
    const dim3 grid((unsigned)((int64_t)rows.n * nseg));
#define CSA2_FUSED_LAUNCH(T, NT, KPT, DEPTH)                                                                 \
    hipLaunchKernelGGL((k_score_topk_pool<T, NT, KPT, DEPTH>), grid, dim3(NT), 0, stream, rows, cache, qin.q, \
                       qin.q_scale, w, w_stride, kdata, kscale, pool, k, nseg, out_idx, lists)
#define CSA2_FUSED_CASE(T)                                           \
    case T:                                                          \
        if (whole)                                                   \
            CSA2_FUSED_LAUNCH(T, kWholeNT, kWholeKPT, kWholeDepth);  \
        else                                                         \
            CSA2_FUSED_LAUNCH(T, kSegNT, kSegKPT, kSegDepth);        \
        break;
    switch (heads / 16) {
        CSA2_FUSED_CASE(1)
        CSA2_FUSED_CASE(2)
        CSA2_FUSED_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef CSA2_FUSED_CASE
#undef CSA2_FUSED_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nseg == 1) return e;
    SelSource src{nullptr, cols, rows, cache, pool};
    if ((int64_t)nseg * k > (int64_t)kMergeNT * kMergeKPT) return launch_list_merge(src, k, nseg, lists, out_idx, stream);
    SelArgs a{};
    a.src = src;
    a.k = k;
    a.nseg = 1;
    a.seg_len = nseg;
    a.nlists_prev = nseg;
    a.in = lists;
    a.out_idx = out_idx;
    a.out_stride = k;
    a.out_mode = OUT_IDX;
    hipLaunchKernelGGL(k_merge_segment_lists, dim3((unsigned)rows.n), dim3(kMergeNT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
