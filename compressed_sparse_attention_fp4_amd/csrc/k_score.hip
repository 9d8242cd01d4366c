// Index scoring: s_j = sum_h w_h * ReLU(q_h . k_j) over every reachable compressed
// position of a query row, or over the row's candidate pool.
//
// Pages: "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 5 (the indexer
// scores the FP4 cache directly; MQA form: one key per position shared by all index
// heads, heads replicated); "DeepSeek V4.1 Flash modeling", sections "Mixed precision"
// (index Q/K are MXFP4 with 32-element groups) and "Hierarchical Sparse Indexer"
// (Reindex layers rescore only the candidate pool).
//
// Head order.  The head sum is taken in fp32 in one fixed order: 4 contiguous head
// groups, P_g = fma(w_h, max(d_h, 0), P_g) over the group's heads in ascending order
// from +0, s = (P_0 + P_1) + (P_2 + P_3).  In the MFMA kernel the A-operand rows are
// permuted so that the 16x16 output tile of a lane group holds consecutive heads of
// one group: A row m of head tile t is head (H/4)*(m/4) + 4t + m%4, and the output
// rows 4g..4g+3 that lane group g holds are therefore heads (H/4)*g + 4t + 0..3.  Each
// lane runs its group's fma chain in registers; two lane swaps finish the sum.
#include "csa2_device.h"
#include "csa2_launch.h"
#include "csa2_score.h"

#pragma clang fp contract(off)

namespace csa2 {

constexpr int kScoreMaxBlocks = 1024;  // pool blocks per workgroup chunk (block ids staged in LDS)

__device__ __forceinline__ int64_t row_columns(const RowsArg& rows, const CacheArg& cache, const PoolArg& pool,
                                               int row, int64_t stride, int64_t* R_out, int* prow_out)
{
    const int r = rows.req[row];
    const int64_t R = reach(rows.pos[row], cache.ratio_m, cache.n_entries[r]);
    int64_t ncol = R;
    int prow = row;
    if (pool.blocks) {
        prow = pool.row_map ? pool.row_map[row] : row;
        ncol = R > 0 ? (int64_t)pool.nblocks[prow] * pool.block : 0;
    }
    *R_out = R;
    *prow_out = prow;
    return ncol < stride ? ncol : stride;
}

// Columns a row's output covers: every position below score_stride (full range), or
// the max_blocks * block columns of a pool row (score_stride is then its pitch).
__device__ __forceinline__ int64_t output_columns(const PoolArg& pool, int64_t stride)
{
    return pool.blocks ? (int64_t)pool.block * pool.max_blocks : stride;
}

// -inf into columns [from, to) of a score row, by all threads of the workgroup.
__device__ __forceinline__ void fill_neg_inf(float* rowp, int64_t from, int64_t to)
{
    for (int64_t c = from + threadIdx.x; c < to; c += blockDim.x) rowp[c] = -INFINITY;
}

__device__ __forceinline__ int64_t column_position(const PoolArg& pool, int prow, int64_t c)
{
    if (!pool.blocks) return c;
    const int64_t i = c / pool.block;
    return (int64_t)pool.blocks[(int64_t)prow * pool.max_blocks + i] * pool.block + (c - i * pool.block);
}

// ----------------------------------------------------------------------------- fp32
// One thread per (row, column): the dot product is an fma chain over the dimension in
// ascending order from +0, then the canonical head reduction.
__global__ __launch_bounds__(256) void k_score_f32(RowsArg rows, CacheArg cache, const float* __restrict__ q,
                                                   int H, int D, const float* __restrict__ w, int64_t w_stride,
                                                   const float* __restrict__ keys, PoolArg pool,
                                                   float* __restrict__ scores, int64_t stride, int nchunks)
{
    int row, chk;
    xcd_row_chunk(blockIdx.x, rows.n, nchunks, &row, &chk);
    int64_t R;
    int prow;
    const int64_t ncol = row_columns(rows, cache, pool, row, stride, &R, &prow);
    const int64_t c = (int64_t)chk * blockDim.x + threadIdx.x;
    float* dst = scores + (int64_t)row * stride + c;
    if (c >= ncol) {
        // columns past the row's reach (or past its pool) hold -inf
        if (c < output_columns(pool, stride)) *dst = -INFINITY;
        return;
    }
    const int64_t j = column_position(pool, prow, c);
    if (j >= R) {
        *dst = -INFINITY;
        return;
    }
    const float* kr = keys + (cache.row_start[rows.req[row]] + j) * D;
    const float* wr = w + (int64_t)row * w_stride;
    const int G = H / 4;
    float P[4];
    for (int g = 0; g < 4; g++) {
        float acc = 0.0f;
        for (int h = g * G; h < (g + 1) * G; h++) {
            const float* qr = q + ((int64_t)row * H + h) * D;
            float d = 0.0f;
            for (int i = 0; i < D; i++) d = __builtin_fmaf(qr[i], kr[i], d);
            acc = __builtin_fmaf(wr[h], fmaxf(d, 0.0f), acc);
        }
        P[g] = acc;
    }
    *dst = (P[0] + P[1]) + (P[2] + P[3]);
}

// ---------------------------------------------------------------------------- MXFP4
// Workgroup = 4 waves on NR query rows and a chunk of columns.  Each row's bf16 index q
// is quantized once per workgroup into LDS (one 32-element block per lane, which is
// exactly the lane's slice of the MFMA A operand).  Each wave then takes 64 columns
// at a time: 4 key tiles of 16 positions, each scored against NHT head tiles with
// v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1, E8M0 block scales): key tile lane
// (g, c) loads position c's 16-byte code block g (one 32-element block) and its scale.
// With NR = 2 the two rows belong to one request and share every key tile (prefill rows
// reach nearly the same positions): each row still has its own products, its own head
// sum in the canonical order and its own stores, so its scores are those of NR = 1.
template <int NHT, bool POOL, int NR>
__device__ __forceinline__ void score_rows(const RowsArg& rows, const CacheArg& cache, const void* __restrict__ q,
                                           const uint8_t* __restrict__ q_scale, const float* __restrict__ w,
                                           int64_t w_stride,
                                           const uint8_t* __restrict__ kdata, const uint8_t* __restrict__ kscale,
                                           const PoolArg& pool, float* __restrict__ scores, int64_t stride,
                                           int chunk, int chk, const int (&rowv)[NR])
{
    static_assert(NR == 1 || !POOL, "rows share key tiles only over the full range");
    constexpr int H = NHT * 16;
    constexpr int G = H / 4;
    __shared__ uint4 s_qa[NR][NHT][64];
    __shared__ uint32_t s_qs[NR][NHT][64];
    __shared__ int32_t s_bid[POOL ? kScoreMaxBlocks : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
    const int64_t c_begin = (int64_t)chk * chunk;
    // the chunk's columns past a row's reach (or its pool) hold -inf
    const int64_t cover = output_columns(pool, stride) < c_begin + chunk ? output_columns(pool, stride)
                                                                           : c_begin + chunk;
    // (the rows' sizes are read through vector loads; readfirstlane makes the branches on
    // them scalar, so that no wave runs both sides of one)
    int nccr[NR];  // columns of this chunk each row covers (<= 8192)
    int ncc = 0;   // columns whose keys are loaded: the most any row covers
    int R32 = 0;   // positions are below n_entries, so 32 bits hold them
    int prow = rowv[0];
#pragma unroll
    for (int r = 0; r < NR; r++) {
        int64_t R;
        const int64_t ncol = row_columns(rows, cache, pool, rowv[r], stride, &R, &prow);
        const int64_t c_end = (c_begin + chunk < ncol) ? c_begin + chunk : ncol;
        nccr[r] = __builtin_amdgcn_readfirstlane((int)(c_end > c_begin ? c_end - c_begin : 0));
        ncc = nccr[r] > ncc ? nccr[r] : ncc;
        const int r32 = __builtin_amdgcn_readfirstlane((int)R);
        R32 = r32 > R32 ? r32 : R32;
    }
    if (ncc == 0) {
#pragma unroll
        for (int r = 0; r < NR; r++) fill_neg_inf(scores + (int64_t)rowv[r] * stride, c_begin, cover);
        return;
    }

    const int64_t krow0 = cache.row_start[rows.req[rowv[0]]];
    // Pool rows: the chunk's block ids go to LDS (a chunk starts on a block boundary and
    // spans at most kScoreMaxBlocks blocks; the block size is a power of two).
    const int bshift = POOL ? __builtin_ctz((unsigned)pool.block) : 0;

    // Position of chunk column `off` (0 <= off < ncc); R or beyond when the column lies
    // past the row's reach.
    auto pos_of = [&](int off) -> int {
        if (!POOL) return (int)c_begin + off;
        return (s_bid[off >> bshift] << bshift) | (off & (pool.block - 1));
    };
    const int32_t* bid_row = POOL ? pool.blocks + (int64_t)prow * pool.max_blocks + (c_begin >> bshift) : nullptr;
    const uint8_t* kd_base = kdata + krow0 * 64 + 16 * (lane >> 4);
    const uint8_t* ks_base = kscale + krow0 * 4 + (lane >> 4);

    // Key tile loader: lane (g, c) of tile u takes position c's 32-element block g (an
    // unreachable column reads position 0 and is masked when stored); it issues exactly
    // eight loads (four 16-byte code blocks, four scale bytes), after looking the row
    // addresses up (gather_b).  It has no branch (a column past the chunk looks up column
    // 0), so the compiler sees one sequence of loads on every path and waits for each key
    // tile just before its products.
    auto lookup_b = [&](int off0, int (&jj)[4]) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int off = off0 + 16 * u + (lane & 15);
            jj[u] = pos_of(off < ncc ? off : 0);
        }
    };
    auto address_b = [&](int off0, const int (&jj)[4], const uint8_t* (&kp)[4], const uint8_t* (&sp)[4]) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int off = off0 + 16 * u + (lane & 15);
            const int j = (off < ncc && jj[u] < R32) ? jj[u] : 0;
            kp[u] = kd_base + ((uint64_t)(uint32_t)j << 6);
            sp[u] = ks_base + ((uint64_t)(uint32_t)j << 2);
        }
    };
    auto gather_b = [&](int off0, const uint8_t* (&kp)[4], const uint8_t* (&sp)[4]) {
        int jj[4];
        lookup_b(off0, jj);
        address_b(off0, jj, kp, sp);
    };
    auto issue_b = [&](const uint8_t* const (&kp)[4], const uint8_t* const (&sp)[4], u32x4_t (&kd)[4], int (&sk)[4]) {
#pragma unroll
        for (int u = 0; u < 4; u++) kd[u] = gload_x4<0>(kp[u]);
#pragma unroll
        for (int u = 0; u < 4; u++) sk[u] = gload_u8<0>(sp[u]);
    };
    auto load = [&](int off0, u32x4_t (&kd)[4], int (&sk)[4]) {
        if (!POOL && off0 + 64 <= ncc) {
            // a whole group inside a full-range chunk: positions c_begin + off0 + 16 u + c,
            // all reachable, one address per lane and the tiles at immediate offsets (the
            // same eight loads in the same order as below)
            const uint32_t j = (uint32_t)c_begin + (uint32_t)off0 + (uint32_t)(lane & 15);
            const uint8_t* kp = kd_base + ((uint64_t)j << 6);
            const uint8_t* sp = ks_base + ((uint64_t)j << 2);
            kd[0] = gload_x4<0>(kp);
            kd[1] = gload_x4<1024>(kp);
            kd[2] = gload_x4<2048>(kp);
            kd[3] = gload_x4<3072>(kp);
            sk[0] = gload_u8<0>(sp);
            sk[1] = gload_u8<64>(sp);
            sk[2] = gload_u8<128>(sp);
            sk[3] = gload_u8<192>(sp);
            return;
        }
        const uint8_t* kp[4];
        const uint8_t* sp[4];
        gather_b(off0, kp, sp);
        issue_b(kp, sp, kd, sk);
    };
    // ---- loads, all issued before their first use: the rows' index q (one 32-element
    // block per thread and pass: bf16 values, or with q_scale its MXFP4 codes and scale),
    // the head weights and the pool block ids, then (full rows) the wave's first two groups
    // of key tiles, so that HBM is busy from the start.
    constexpr int QP = (NHT * 64 + 255) / 256;
    const bool q4 = q_scale != nullptr;  // the same for every thread
    u32x4_t qraw[NR][QP][4];
    u32x4_t qcode[NR][QP];
    int qsc[NR][QP];
#pragma unroll
    for (int r = 0; r < NR; r++) {
#pragma unroll
        for (int pp = 0; pp < QP; pp++) {
            const int idx = threadIdx.x + 256 * pp;
            if (idx < NHT * 64) {
                const int t = idx >> 6, l = idx & 63;
                const int m = l & 15, blk = l >> 4;
                const int head = G * (m >> 2) + 4 * t + (m & 3);
                const int64_t rh = (int64_t)rowv[r] * H + head;
                if (q4) {
                    qcode[r][pp] = gload_x4<0>(static_cast<const uint8_t*>(q) + rh * 64 + blk * 16);
                    qsc[r][pp] = gload_u8<0>(q_scale + rh * 4 + blk);
                } else {
                    const uint16_t* src = static_cast<const uint16_t*>(q) + rh * 128 + blk * 32;
                    qraw[r][pp][0] = gload_x4<0>(src);
                    qraw[r][pp][1] = gload_x4<16>(src);
                    qraw[r][pp][2] = gload_x4<32>(src);
                    qraw[r][pp][3] = gload_x4<48>(src);
                }
            }
        }
    }
    const int g = lane >> 4;
    float wr[NR][NHT * 4];
#pragma unroll
    for (int r = 0; r < NR; r++) {
        const float* wrow = w + (int64_t)rowv[r] * w_stride + G * g;
#pragma unroll
        for (int t = 0; t < NHT; t++) {
            wr[r][4 * t + 0] = gload_f32<0>(wrow + 4 * t);
            wr[r][4 * t + 1] = gload_f32<4>(wrow + 4 * t);
            wr[r][4 * t + 2] = gload_f32<8>(wrow + 4 * t);
            wr[r][4 * t + 3] = gload_f32<12>(wrow + 4 * t);
        }
    }
    constexpr int BPT = POOL ? kScoreMaxBlocks / 256 : 1;  // pool block ids staged per thread
    const int nb = POOL ? (ncc + pool.block - 1) >> bshift : 0;
    int32_t bidv[BPT];
    if (POOL) {
#pragma unroll
        for (int i = 0; i < BPT; i++) {  // branch-free within a pass: past the chunk, block 0 again
            const int idx = threadIdx.x + 256 * i;
            bidv[i] = 256 * i < nb ? gload_i32<0>(bid_row + (idx < nb ? idx : 0)) : 0;
        }
    }
    // The wave scores groups 64 wave + 256 i, i < n, from two key buffers that alternate.
    // Both first loads are issued even when the wave has fewer than two groups (load
    // then reads position 0 for their columns), so the same loads are in flight on every
    // path and the compiler's waits need not depend on the group count.
    const int off0 = 64 * wave;
    const int n = off0 < ncc ? (ncc - off0 + 255) >> 8 : 0;
    u32x4_t ka[4], kb[4];
    int sa4[4], sb4[4];
    if (!POOL) {
        // pool rows look their positions up in the staged block ids: their first key
        // tiles follow the barrier below
        load(off0, ka, sa4);
        load(off0 + 256, kb, sb4);
    }

    // ---- pool block ids to LDS; the rows' index q quantized into A operands
    if (POOL) {
#pragma unroll
        for (int i = 0; i < BPT; i++) {
            const int idx = threadIdx.x + 256 * i;
            if (256 * i < nb && idx < nb) s_bid[idx] = bidv[i];
        }
    }
#pragma unroll
    for (int r = 0; r < NR; r++) {
#pragma unroll
        for (int pp = 0; pp < QP; pp++) {
            const int idx = threadIdx.x + 256 * pp;
            if (idx < NHT * 64 && q4) {
                const int t = idx >> 6, l = idx & 63;
                s_qa[r][t][l] = make_uint4(qcode[r][pp][0], qcode[r][pp][1], qcode[r][pp][2], qcode[r][pp][3]);
                s_qs[r][t][l] = (uint32_t)qsc[r][pp];
            } else if (idx < NHT * 64) {
                const int t = idx >> 6, l = idx & 63;
                float v[32];
#pragma unroll
                for (int i = 0; i < 4; i++) {
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) {
                        v[i * 8 + 2 * jj] = __uint_as_float(qraw[r][pp][i][jj] << 16);
                        v[i * 8 + 2 * jj + 1] = __uint_as_float(qraw[r][pp][i][jj] & 0xFFFF0000u);
                    }
                }
                uint32_t o[4], sb;
                quant_block_e2m1(v, o, &sb);
                s_qa[r][t][l] = make_uint4(o[0], o[1], o[2], o[3]);
                s_qs[r][t][l] = sb;
            }
        }
    }
    __syncthreads();

    i32x8 a[NR][NHT];
    int sa[NR][NHT];
#pragma unroll
    for (int r = 0; r < NR; r++) {
#pragma unroll
        for (int t = 0; t < NHT; t++) {
            const uint4 u = s_qa[r][t][lane];
            a[r][t] = i32x8{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
            sa[r][t] = (int)s_qs[r][t][lane];
        }
    }
    if (POOL) {
        load(off0, ka, sa4);
        load(off0 + 256, kb, sb4);
    }

    // score the 64 columns off0 .. off0 + 63 from their key tiles
    auto score_group = [&](int off0, const u32x4_t (&kd)[4], const int (&sk)[4]) {
        // tiles one at a time: NHT products per row into separate registers, then the
        // rows' head sums
        float P[NR][4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const i32x8 b = i32x8{(int)kd[u][0], (int)kd[u][1], (int)kd[u][2], (int)kd[u][3], 0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < NR; r++) {
                f32x4 d[NHT];
#pragma unroll
                for (int t = 0; t < NHT; t++) {
                    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    d[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[r][t], b, zero, 4, 4, 0, sa[r][t], 0,
                                                                           sk[u]);
                }
                float pp = 0.0f;
#pragma unroll
                for (int t = 0; t < NHT; t++)
#pragma unroll
                    for (int i = 0; i < 4; i++) pp = __builtin_fmaf(wr[r][4 * t + i], relu_bits(d[t][i]), pp);
                P[r][u] = pp;
            }
        }
        const int off = off0 + lane;
        float score[NR];
#pragma unroll
        for (int r = 0; r < NR; r++) {
            // Lane group g holds P_g for tiles 0..3.  Pair groups (0,1) and (2,3) per
            // tile, then (01, 23): lane (g, c) ends with the score of tile g, position c.
            auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(P[r][0]), __float_as_uint(P[r][1]), false,
                                                        false);
            auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(P[r][2]), __float_as_uint(P[r][3]), false,
                                                        false);
            const float h01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
            const float h23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(h01), __float_as_uint(h23), false, false);
            score[r] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        // Every row's scores are computed before the first (lane-masked) store: otherwise
        // the compiler sinks a row's products past the previous row's store branch, and
        // the block boundary keeps them from overlapping that row's head sums.
#pragma unroll
        for (int r = 0; r < NR; r++) pin(score[r]);
#pragma unroll
        for (int r = 0; r < NR; r++) {
            if (off < nccr[r]) {
                if (POOL && pos_of(off) >= R32) score[r] = -INFINITY;
                scores[(int64_t)rowv[r] * stride + c_begin + off] = score[r];
            }
        }
    };

    // Groups i and i + 1 are in flight while group i is scored.  The loop runs while both
    // reloads are real groups; the last two or three groups follow, so that each wait
    // (and the load count it assumes) is fixed along every path.
    {
        int i = 0;
        for (; i + 3 < n; i += 2) {
            score_group(off0 + 256 * i, ka, sa4);
            load(off0 + 256 * (i + 2), ka, sa4);
            score_group(off0 + 256 * (i + 1), kb, sb4);
            load(off0 + 256 * (i + 3), kb, sb4);
        }
        const int rest = n - i;  // 0 .. 3
        if (rest == 3) {
            score_group(off0 + 256 * i, ka, sa4);
            load(off0 + 256 * (i + 2), ka, sa4);
            score_group(off0 + 256 * (i + 1), kb, sb4);
            score_group(off0 + 256 * (i + 2), ka, sa4);
        } else if (rest == 2) {
            score_group(off0 + 256 * i, ka, sa4);
            score_group(off0 + 256 * (i + 1), kb, sb4);
        } else {
            if (rest == 1) score_group(off0 + 256 * i, ka, sa4);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; r++)
        if (c_begin + nccr[r] < cover) fill_neg_inf(scores + (int64_t)rowv[r] * stride, c_begin + nccr[r], cover);
}

// One query row per workgroup.
template <int NHT, bool POOL>
__global__ __launch_bounds__(256) void k_score_mxfp4(RowsArg rows, CacheArg cache, const void* __restrict__ q,
                                                     const uint8_t* __restrict__ q_scale,
                                                     const float* __restrict__ w, int64_t w_stride,
                                                     const uint8_t* __restrict__ kdata,
                                                     const uint8_t* __restrict__ kscale, PoolArg pool,
                                                     float* __restrict__ scores, int64_t stride, int chunk,
                                                     int nchunks)
{
    int row, chk;
    xcd_row_chunk(blockIdx.x, rows.n, nchunks, &row, &chk);
    const int rv[1] = {row};
    score_rows<NHT, POOL, 1>(rows, cache, q, q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk, chk,
                             rv);
}

// Rows 2 i and 2 i + 1 per workgroup (full range, launches over many rows): one pass
// over shared key tiles when both belong to one request, else one row after the other.
template <int NHT>
__global__ __launch_bounds__(256, 3) void k_score_mxfp4_pair(RowsArg rows, CacheArg cache,
                                                          const void* __restrict__ q,
                                                          const uint8_t* __restrict__ q_scale,
                                                          const float* __restrict__ w, int64_t w_stride,
                                                          const uint8_t* __restrict__ kdata,
                                                          const uint8_t* __restrict__ kscale, PoolArg pool,
                                                          float* __restrict__ scores, int64_t stride, int chunk,
                                                          int nchunks)
{
    int pair, chk;
    xcd_row_chunk(blockIdx.x, (rows.n + 1) >> 1, nchunks, &pair, &chk);
    const int r0 = 2 * pair, r1 = r0 + 1;
    const bool shared =
        __builtin_amdgcn_readfirstlane((int)(r1 < rows.n && rows.req[r0] == rows.req[r1])) != 0;
    if (shared) {
        const int rv[2] = {r0, r1};
        score_rows<NHT, false, 2>(rows, cache, q, q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk,
                                  chk, rv);
        return;
    }
    const int a0[1] = {r0};
    score_rows<NHT, false, 1>(rows, cache, q, q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk, chk,
                              a0);
    if (r1 < rows.n) {
        __syncthreads();  // the second row reuses the first one's LDS
        const int a1[1] = {r1};
        score_rows<NHT, false, 1>(rows, cache, q, q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk,
                                  chk, a1);
    }
}

static int pick_chunk(int n, int64_t cols, int block)
{
    // Each workgroup quantizes its row's index q once, so columns per workgroup should be
    // many (1024..8192); shrink only while there are fewer than 2048 workgroups (about two
    // rounds of the 256 CUs at 4 workgroups each, which evens out the finish; 512
    // workgroups of 8192 columns were no faster for a decode batch of 64 rows over 65,536
    // positions, and 32 rows over 262,144 do not depend on it).  A pool chunk spans at most
    // kScoreMaxBlocks blocks (1024 columns suffice for block 1).
    int64_t chunk = 8192;
    while (chunk > 1024 && (int64_t)n * ((cols + chunk - 1) / chunk) < 2048) chunk >>= 1;
    while (block > 0 && chunk / block > kScoreMaxBlocks) chunk >>= 1;
    return (int)chunk;
}

// Full-range launches over at least this many rows (prefill) score rows in pairs.
constexpr int kPairRows = 1024;

hipError_t launch_index_score_mxfp4(const RowsArg& rows, const CacheArg& cache, const IndexQ& qin, int heads,
                                    const float* w, int64_t w_stride, const uint8_t* kdata, const uint8_t* kscale,
                                    const PoolArg& pool, float* scores, int64_t stride, hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const int64_t cols = pool.blocks ? (int64_t)pool.block * pool.max_blocks : stride;
    const bool pairs = !pool.blocks && rows.n >= kPairRows;
    const int units = pairs ? (rows.n + 1) / 2 : rows.n;  // workgroup rows
    const int chunk = pick_chunk(units, cols, pool.blocks ? pool.block : 0);
    const int nchunks = (int)((cols + chunk - 1) / chunk);
    dim3 grid((unsigned)((int64_t)nchunks * units));
#define CSA2_SCORE_CASE(T)                                                                               \
    case T:                                                                                              \
        if (pool.blocks)                                                                                 \
            hipLaunchKernelGGL((k_score_mxfp4<T, true>), grid, dim3(256), 0, stream, rows, cache, qin.q,   \
                               qin.q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk,       \
                               nchunks);                                                                 \
        else if (pairs)                                                                                  \
            hipLaunchKernelGGL((k_score_mxfp4_pair<T>), grid, dim3(256), 0, stream, rows, cache, qin.q,    \
                               qin.q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk,       \
                               nchunks);                                                                 \
        else                                                                                             \
            hipLaunchKernelGGL((k_score_mxfp4<T, false>), grid, dim3(256), 0, stream, rows, cache, qin.q,  \
                               qin.q_scale, w, w_stride, kdata, kscale, pool, scores, stride, chunk,       \
                               nchunks);                                                                 \
        break;
    switch (heads / 16) {
        CSA2_SCORE_CASE(1)
        CSA2_SCORE_CASE(2)
        CSA2_SCORE_CASE(3)
        CSA2_SCORE_CASE(4)
        CSA2_SCORE_CASE(5)
        CSA2_SCORE_CASE(6)
        CSA2_SCORE_CASE(7)
        CSA2_SCORE_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef CSA2_SCORE_CASE
    return hipGetLastError();
}

hipError_t launch_index_score_f32(const RowsArg& rows, const CacheArg& cache, const float* q, int heads, int dim,
                                  const float* w, int64_t w_stride, const float* keys, const PoolArg& pool,
                                  float* scores, int64_t stride, hipStream_t stream)
{
    if (rows.n == 0) return hipSuccess;
    const int64_t cols = pool.blocks ? (int64_t)pool.block * pool.max_blocks : stride;
    const int nchunks = (int)((cols + 255) / 256);
    dim3 grid((unsigned)((int64_t)nchunks * rows.n));
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), 0, stream, rows, cache, q, heads, dim, w, w_stride, keys, pool,
                       scores, stride, nchunks);
    return hipGetLastError();
}

}  // namespace csa2
