// Top-k selection: flat (over every reachable position), over a candidate pool, and
// the hierarchical block pass.
//
// Pages: "DeepSeek V4.1 Flash modeling", section "Hierarchical Sparse Indexer" (top-512
// per query; blocks of 8 positions scored by their maximum, at most 2,048 blocks; later
// index layers select inside that pool); "SGLang and Miles Day-0 support for
// DeepSeek-V4.1", section 2 (the block holding the newest position is always kept; the
// same pass takes its own top-512 over all reachable positions).  Ties go to the lower
// position (the workload definition; the pages are silent).
//
// Method.  Candidates are mapped to order-preserving 32-bit keys (0 = no candidate).  One
// workgroup (1024 threads; 256 for launches over many rows) holds up to threads*KPT
// candidates in registers, blocked: thread t owns candidates [t*KPT, (t+1)*KPT), so thread
// order is candidate order.  An MSB-first radix select finds the threshold key T: the
// first digit (11 bits) starts at the highest bit where the largest and smallest keys
// differ, later digits take 8 bits of the keys still in the threshold bin; a pass whose
// threshold bin is taken whole ends the search, and a threshold bin of at most 64 keys is
// ranked directly by one wave.  Histograms are LDS atomics; the threshold bin is found by
// a cooperative scan from the top.  The selection is every key above T plus the
// lowest-indexed keys equal to T; one block scan of per-thread counts gives each selected
// candidate its output slot in ascending candidate order.  Rows longer than one
// workgroup are cut into segments whose top-k lists are merged by another pass (the
// order is total, so the merge is exact).
#include "csa2_device.h"
#include "csa2_launch.h"
#include "csa2_select.h"

namespace csa2 {

template <int KPT, int SRC>
__device__ __forceinline__ void load_keys(const SelArgs& a, int row, int64_t R, int64_t ncol, int prow, int64_t base,
                                          int64_t e0, uint32_t (&key)[KPT], int32_t (&bid)[bid_slots(KPT)],
                                          bool& bid_ok)
{
    // Every path issues all of the thread's loads first, with addresses clamped by bounds
    // known without the row's geometry, then pins them (one wait) and masks afterwards.
    bid_ok = false;
    const SelSource& s = a.src;
    if (SRC == SRC_LIST) {
        const int64_t lim_e = (int64_t)a.seg_len * a.k;
        const int64_t lim_l = (int64_t)a.nlists_prev * a.k;
        const uint2* in = a.in + (int64_t)row * lim_l;
        uint32_t v[KPT];
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int64_t li = base + e0 + i;
            v[i] = in[li < lim_l ? li : 0].x;
        }
#pragma unroll
        for (int i = 0; i < KPT; i++) pin(v[i]);
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int64_t e = e0 + i;
            key[i] = (e < lim_e && base + e < lim_l) ? v[i] : 0u;
        }
        return;
    }
    if (SRC == SRC_BMAX) {
        // every block but the newest (its key is 0 in the array, and it is past lim)
        const uint32_t* kp = a.bmax + (int64_t)row * a.bstride;
        uint32_t v[KPT];
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int64_t c = base + e0 + i;
            v[i] = kp[c < a.bstride ? c : 0];
        }
#pragma unroll
        for (int i = 0; i < KPT; i++) pin(v[i]);
        const int64_t lim = ((ncol + 7) >> 3) - 1;
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int64_t c = base + e0 + i;
            key[i] = ((e0 + i < a.seg_len) && (c < lim)) ? v[i] : 0u;
        }
        return;
    }
    if constexpr (SRC == SRC_PGATHER) {
        // candidate c is pool position blocks[c / 8] * 8 + c % 8 of the full score row;
        // a thread's KPT candidates are KPT / 8 whole blocks
        static_assert(KPT % 8 == 0, "whole blocks per thread");
        const float* rowp = s.scores + (int64_t)row * s.stride;
        const bool vec = ((reinterpret_cast<uintptr_t>(rowp) & 15) == 0) && (s.stride % 8 == 0);
        int32_t bl[KPT / 8];
#pragma unroll
        for (int b8 = 0; b8 < KPT / 8; b8++) {
            const int64_t cb = ((base + e0) >> 3) + b8;
            bl[b8] = s.pool.blocks[(int64_t)prow * s.pool.max_blocks + (cb < s.pool.max_blocks ? cb : 0)];
        }
#pragma unroll
        for (int b8 = 0; b8 < KPT / 8; b8++) pin(bl[b8]);
        float f[KPT];
#pragma unroll
        for (int b8 = 0; b8 < KPT / 8; b8++) {
            const int64_t p0 = (int64_t)bl[b8] * 8;
            if (vec) {
                const int64_t pc = (p0 >= 0 && p0 + 8 <= s.stride) ? p0 : 0;
                const float4 u = reinterpret_cast<const float4*>(rowp + pc)[0];
                const float4 v = reinterpret_cast<const float4*>(rowp + pc)[1];
                f[8 * b8] = u.x; f[8 * b8 + 1] = u.y; f[8 * b8 + 2] = u.z; f[8 * b8 + 3] = u.w;
                f[8 * b8 + 4] = v.x; f[8 * b8 + 5] = v.y; f[8 * b8 + 6] = v.z; f[8 * b8 + 7] = v.w;
            } else {
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    const int64_t pq = p0 + q;
                    f[8 * b8 + q] = rowp[(pq >= 0 && pq < s.stride) ? pq : 0];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KPT; i++) pin(f[i]);
        const int64_t lim = (a.seg_len < ncol - base) ? base + a.seg_len : ncol;
        // positions the block pass saw: reachable ones that lie inside the score row
        const int64_t rlim = R < s.stride ? R : s.stride;
#pragma unroll
        for (int b8 = 0; b8 < KPT / 8; b8++) {
            const int64_t c = base + e0 + 8 * b8;
            const bool okb = c < lim;
            const int64_t blk = okb ? bl[b8] : 0;
            bid[b8] = (int32_t)blk;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const bool ok = okb && (c + q < lim) && (blk * 8 + q < rlim);
                key[8 * b8 + q] = ok ? order_key(f[8 * b8 + q]) : 0u;
            }
        }
        bid_ok = ((base + e0) & 7) == 0;
        return;
    }
    if (SRC == SRC_BLOCK) {
        // every block but the newest; all their members are reachable (block == 8)
        const float* rowp = s.scores + (int64_t)row * s.stride;
        const bool vec = ((reinterpret_cast<uintptr_t>(rowp) & 15) == 0);
        const int64_t nfull = s.stride >> 3;  // whole blocks inside the row
        const int64_t nblk = (ncol + 7) >> 3;
        constexpr int NB = KPT < 4 ? KPT : 4;  // blocks loaded together (registers)
#pragma unroll
        for (int i0 = 0; i0 < KPT; i0 += NB) {
            float f[NB][8];
#pragma unroll
            for (int j = 0; j < NB; j++) {
                const int64_t c = base + e0 + i0 + j;
                const float* sp = rowp + ((c < nfull ? c : 0) << 3);
                if (vec) {
                    const float4 u = reinterpret_cast<const float4*>(sp)[0];
                    const float4 v = reinterpret_cast<const float4*>(sp)[1];
                    f[j][0] = u.x; f[j][1] = u.y; f[j][2] = u.z; f[j][3] = u.w;
                    f[j][4] = v.x; f[j][5] = v.y; f[j][6] = v.z; f[j][7] = v.w;
                } else {
#pragma unroll
                    for (int q = 0; q < 8; q++) f[j][q] = sp[q];
                }
            }
#pragma unroll
            for (int j = 0; j < NB; j++)
#pragma unroll
                for (int q = 0; q < 8; q++) pin(f[j][q]);
#pragma unroll
            for (int j = 0; j < NB; j++) {
                const int64_t c = base + e0 + i0 + j;
                const bool ok = (e0 + i0 + j < a.seg_len) && (c < nblk - 1);
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < 8; q++) m = max(m, order_key(f[j][q]));
                key[i0 + j] = ok ? m : 0u;
            }
        }
        return;
    }
    const float* rowp = s.scores + (int64_t)row * s.stride;
    const int64_t c0 = base + e0;
    float v[KPT];
    if (KPT % 4 == 0 && c0 + KPT <= s.stride && ((reinterpret_cast<uintptr_t>(rowp + c0) & 15) == 0)) {
#pragma unroll
        for (int i = 0; i < KPT; i += 4) {
            const float4 u = *reinterpret_cast<const float4*>(rowp + c0 + i);
            v[i] = u.x; v[i + 1] = u.y; v[i + 2] = u.z; v[i + 3] = u.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int64_t c = c0 + i;
            v[i] = rowp[c < s.stride ? c : 0];
        }
    }
    const bool pool_bids = SRC == SRC_POOL && KPT % 8 == 0 && a.block_shift == 3 && (c0 & 7) == 0;
    if (pool_bids) {
#pragma unroll
        for (int b8 = 0; b8 < bid_slots(KPT); b8++) {
            const int64_t cb = (c0 >> 3) + b8;
            bid[b8] = s.pool.blocks[(int64_t)prow * s.pool.max_blocks + (cb < s.pool.max_blocks ? cb : 0)];
        }
#pragma unroll
        for (int b8 = 0; b8 < bid_slots(KPT); b8++) pin(bid[b8]);
    }
#pragma unroll
    for (int i = 0; i < KPT; i++) pin(v[i]);
    const int64_t lim = (a.seg_len < ncol - base) ? base + a.seg_len : ncol;  // columns of this slice
#pragma unroll
    for (int i = 0; i < KPT; i++) key[i] = (c0 + i < lim) ? order_key(v[i]) : 0u;
    if (SRC == SRC_POOL) {
        // a pool position past the reachable range (only in the newest block) is no candidate
        if (pool_bids) {
#pragma unroll
            for (int i = 0; i < KPT; i++) {
                const int64_t pp = ((int64_t)bid[i >> 3] << 3) + (i & 7);
                key[i] = (pp >= R) ? 0u : key[i];
            }
            bid_ok = true;
        } else {
#pragma unroll
            for (int i = 0; i < KPT; i++) {
                const int64_t c = c0 + i;
                const int64_t pp = pool_position(s, a.block_shift, prow, c < lim ? c : 0);
                key[i] = (pp >= R) ? 0u : key[i];
            }
        }
    }
}

template <int KPT, int SRC, int NT = kNT>
__global__ __launch_bounds__(NT) void k_select(SelArgs a)
{
    const int nseg = a.nseg;
    int row, seg;
    xcd_row_chunk(blockIdx.x, a.src.rows.n, nseg, &row, &seg);
    const int tid = threadIdx.x;
    const SelSource& s = a.src;

    int64_t R = 0, ncol = 0;
    int prow = row;
    // a merge level's entries carry their positions: only a level that writes a pool
    // (whose newest block follows from the row's columns) needs the row metadata, and no
    // other waits for it before its loads
    if (SRC != SRC_LIST || a.out_mode == OUT_BLOCKS) row_info(s, row, &R, &ncol, &prow);
    const int64_t base = (int64_t)seg * (SRC == SRC_LIST ? a.seg_len * a.k : a.seg_len);
    const int64_t e0 = (int64_t)tid * KPT;  // blocked: thread t owns [t*KPT, (t+1)*KPT)

    uint32_t key[KPT];
    int32_t bid[bid_slots(KPT)];
    bool bid_ok;
    load_keys<KPT, SRC>(a, row, R, ncol, prow, base, e0, key, bid, bid_ok);
    select_core<KPT, SRC, NT>(a, row, seg, R, ncol, prow, base, e0, key, bid, bid_ok);
}

// ------------------------------------------------------------------------ host plans
struct Plan {
    bool ok;     // every level fits the workgroups that run it, and the last one leaves one list
    int levels;
    int64_t seg_len[8];  // candidates (level 0) or lists (merge) per workgroup
    int nseg[8];         // lists per row produced by each level
    int64_t cap[8];      // candidates one workgroup holds at this level
};

// Largest first-level segment per source: 32768 candidates from plain score rows, 16384
// when each candidate needs a pool lookup or a block maximum (more live registers).
static int64_t first_cap(int mode) { return (mode == SRC_FULL) ? kMaxCap : 16384; }

static Plan make_plan(int64_t cols, int k, int mode)
{
    Plan p{};
    p.ok = true;
    p.levels = 1;
    if (cols < 1) cols = 1;
    const int64_t cap0 = first_cap(mode);
    if (k == 0 || cols <= cap0) {
        p.seg_len[0] = cols;
        p.nseg[0] = 1;
        p.cap[0] = cols;
        return p;
    }
    // first level: segments of up to kMaxCap columns, at least 2k each so that selecting
    // actually reduces the data
    int64_t nseg = (cols + cap0 - 1) / cap0;
    p.seg_len[0] = (cols + nseg - 1) / nseg;
    p.nseg[0] = (int)nseg;
    p.cap[0] = p.seg_len[0];
    int64_t cur = nseg;
    // lists merged per workgroup: a merge level selects with at most 16 candidates per
    // thread (launch_level), so a group holds at most kListCap candidates
    const int64_t group = kListCap / k;
    while (cur > 1 && p.levels < 8) {
        const int64_t g = cur < group ? cur : group;
        const int64_t nxt = (cur + g - 1) / g;
        p.seg_len[p.levels] = g;
        p.nseg[p.levels] = (int)nxt;
        p.cap[p.levels] = g * k;
        p.levels++;
        cur = nxt;
    }
    p.ok = cur == 1;
    return p;
}

static size_t level_bytes(const Plan& p, int l, int n, int k)
{
    return (size_t)n * p.nseg[l] * (size_t)(k > 0 ? k : 1) * sizeof(uint2);
}

static size_t plan_workspace(const Plan& p, int n, int k)
{
    if (p.levels <= 1) return 0;
    size_t a = 0, b = 0;
    for (int l = 0; l + 1 < p.levels; l++) {
        const size_t sz = level_bytes(p, l, n, k);
        if (l % 2 == 0) a = sz > a ? sz : a; else b = sz > b ? sz : b;
    }
    return ((a + 255) & ~(size_t)255) + b;
}

// Launches over many rows (a prefill, a replay over thousands of extend rows) select
// with small workgroups: a workgroup's passes are a chain of barriers whose cost grows
// with its wave count, and more of them fit on a CU, so rows per second rise.  Slices
// of up to 4096 candidates take 256 threads; 8192 take 512 threads of 16 (32 per thread
// on 256 threads needs 170 VGPRs, two workgroups per CU: 27,328 rows of 8192 took 686
// against 518 us).  Few rows (a decode batch) keep 1024 threads, which finish one row
// sooner.  The selection is exact either way.
constexpr int kManyRows = 1024;

// Launch one level; every variant holds threads x KPT candidates, and a level whose
// workgroups would hold more (a plan the variants cannot take) is refused rather than
// losing candidates.
template <int SRC>
static hipError_t launch_level(dim3 grid, int64_t cap, int nrows, const SelArgs& a, hipStream_t stream)
{
    if (nrows >= kManyRows && cap <= 8192) {
        if (cap <= 2048)
            hipLaunchKernelGGL((k_select<8, SRC, 256>), grid, dim3(256), 0, stream, a);
        else if (cap <= 4096)
            hipLaunchKernelGGL((k_select<16, SRC, 256>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((k_select<16, SRC, 512>), grid, dim3(512), 0, stream, a);
        return hipSuccess;
    }
    if (cap <= 4096)  // (pool gathers take whole blocks: at least 8 per thread)
        hipLaunchKernelGGL((k_select<SRC == SRC_PGATHER ? 16 : 4, SRC>), grid, dim3(kNT), 0, stream, a);
    else if (cap <= 8192)  // e.g. the 8,192 block maxima of a 65,536-entry row: every slot used
        hipLaunchKernelGGL((k_select<8, SRC>), grid, dim3(kNT), 0, stream, a);
    else if (cap <= kListCap)
        hipLaunchKernelGGL((k_select<16, SRC>), grid, dim3(kNT), 0, stream, a);
    else if (SRC == SRC_FULL && cap <= kMaxCap)
        hipLaunchKernelGGL((k_select<SRC == SRC_FULL ? kMaxKPT : 16, SRC>), grid, dim3(kNT), 0,
                           stream, a);
    else
        return hipErrorInvalidValue;
    return hipSuccess;
}

static int ilog2(int x)
{
    int s = 0;
    while ((1 << s) < x) s++;
    return s;
}

static hipError_t run_plan(const SelSource& src, int mode, int block, int k, int64_t cols, int out_mode,
                           int32_t* out_idx, int out_stride, int32_t* out_nblocks, void* ws, hipStream_t stream,
                           const uint32_t* bmax = nullptr, int64_t bstride = 0)
{
    const int n = src.rows.n;
    if (n == 0) return hipSuccess;
    const Plan p = make_plan(cols, k, mode);
    if (!p.ok) return hipErrorInvalidValue;
    size_t sza = 0;
    for (int l = 0; l + 1 < p.levels; l += 2) {
        const size_t sz = level_bytes(p, l, n, k);
        sza = sz > sza ? sz : sza;
    }
    sza = (sza + 255) & ~(size_t)255;
    uint2* bufA = static_cast<uint2*>(ws);
    uint2* bufB = reinterpret_cast<uint2*>(static_cast<char*>(ws) + sza);
    const uint2* prev = nullptr;
    for (int l = 0; l < p.levels; l++) {
        SelArgs a{};
        a.src = src;
        a.block = block > 0 ? block : (src.pool.blocks ? src.pool.block : 1);
        a.block_shift = ilog2(a.block);
        a.k = k;
        a.nseg = p.nseg[l];
        a.seg_len = p.seg_len[l];
        a.nlists_prev = (l == 0) ? 0 : p.nseg[l - 1];
        a.in = prev;
        const bool last = (l + 1 == p.levels);
        a.out_mode = last ? out_mode : OUT_LIST;
        a.out_list = (l % 2 == 0) ? bufA : bufB;
        a.out_idx = out_idx;
        a.out_nblocks = out_nblocks;
        a.out_stride = out_stride;
        a.bmax = bmax;
        a.bstride = bstride;
        const dim3 grid((unsigned)((int64_t)n * p.nseg[l]));
        hipError_t e;
        if (l > 0)
            e = launch_level<SRC_LIST>(grid, p.cap[l], n, a, stream);
        else if (mode == SRC_FULL)
            e = launch_level<SRC_FULL>(grid, p.cap[l], n, a, stream);
        else if (mode == SRC_POOL)
            e = launch_level<SRC_POOL>(grid, p.cap[l], n, a, stream);
        else if (mode == SRC_BMAX)
            e = launch_level<SRC_BMAX>(grid, p.cap[l], n, a, stream);
        else if (mode == SRC_PGATHER)
            e = launch_level<SRC_PGATHER>(grid, p.cap[l], n, a, stream);
        else
            e = launch_level<SRC_BLOCK>(grid, p.cap[l], n, a, stream);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return e;
        prev = a.out_list;
    }
    return hipSuccess;
}

static int64_t select_cols(const SelSource& src)
{
    return src.pool.blocks ? (int64_t)src.pool.block * src.pool.max_blocks : src.stride;
}

size_t topk_workspace(int n, int64_t stride, int k, bool pool)
{
    return plan_workspace(make_plan(stride, k, pool ? SRC_POOL : SRC_FULL), n, k);
}

hipError_t launch_list_merge(const SelSource& src, int k, int nlists, const uint2* lists, int32_t* out,
                             hipStream_t stream)
{
    SelArgs a{};
    a.src = src;
    a.k = k;
    a.nseg = 1;
    a.seg_len = nlists;
    a.nlists_prev = nlists;
    a.in = lists;
    a.out_idx = out;
    a.out_stride = k;
    a.out_mode = OUT_IDX;
    if ((int64_t)nlists * k <= 2048 && src.rows.n < kManyRows) {
        // a decode batch's few short lists: 512 threads pass the barriers sooner than 1024
        hipLaunchKernelGGL((k_select<4, SRC_LIST, 512>), dim3((unsigned)src.rows.n), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    hipError_t e = launch_level<SRC_LIST>(dim3((unsigned)src.rows.n), (int64_t)nlists * k, src.rows.n, a, stream);
    return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_topk(const SelSource& src, int k, int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    (void)ws_bytes;
    return run_plan(src, src.pool.blocks ? SRC_POOL : SRC_FULL, 0, k, select_cols(src), OUT_IDX, out, k, nullptr,
                    ws, stream);
}

// Block maxima of the full score row as order-preserving keys: key of block b is the
// maximum over its 8 members for every block but the newest (whose members may be partly
// unreachable; it is always kept), 0 (no candidate) for the newest block and beyond.
__global__ __launch_bounds__(256) void k_block_max(SelSource s, uint32_t* __restrict__ bmax, int64_t bstride,
                                                   int chunks)
{
    int row, chk;
    xcd_row_chunk(blockIdx.x, s.rows.n, chunks, &row, &chk);
    const int64_t c = (int64_t)chk * 256 + threadIdx.x;
    if (c >= bstride) return;
    int64_t R, ncol;
    int prow;
    row_info(s, row, &R, &ncol, &prow);
    const int64_t nblk = (ncol + 7) >> 3;
    uint32_t m = 0;
    if (c < nblk - 1) {
        const float* sp = s.scores + (int64_t)row * s.stride + c * 8;
        if ((reinterpret_cast<uintptr_t>(sp) & 15) == 0) {
            const float4 u = reinterpret_cast<const float4*>(sp)[0];
            const float4 v = reinterpret_cast<const float4*>(sp)[1];
            m = max(max(max(order_key(u.x), order_key(u.y)), max(order_key(u.z), order_key(u.w))),
                    max(max(order_key(v.x), order_key(v.y)), max(order_key(v.z), order_key(v.w))));
        } else {
#pragma unroll
            for (int q = 0; q < 8; q++) m = max(m, order_key(sp[q]));
        }
    }
    bmax[(int64_t)row * bstride + c] = m;
}

// Pools of rows whose every block fits: blocks 0 .. ceil(ncol / block) - 1 ascending, -1
// padded (the hierarchy keeps every block of such a row, the newest included).
__global__ __launch_bounds__(256) void k_pool_all(SelSource s, int block_shift, int32_t* __restrict__ out_blocks,
                                                  int max_blocks, int32_t* __restrict__ out_nblocks)
{
    const int row = blockIdx.x;
    int64_t R, ncol;
    int prow;
    row_info(s, row, &R, &ncol, &prow);
    const int nblk = (int)((ncol + (1 << block_shift) - 1) >> block_shift);  // <= max_blocks (host-checked)
    int32_t* o = out_blocks + (int64_t)row * max_blocks;
    for (int i = threadIdx.x; i < max_blocks; i += blockDim.x) o[i] = i < nblk ? i : -1;
    if (threadIdx.x == 0) out_nblocks[row] = nblk;
}

// The two-stage hierarchy (blocks of 8, k <= max_blocks - 1): block maxima, the pool's
// blocks selected from them, then the flat top-k taken over the pool's positions only.
// The last step is exact: an entry outside the pool lies in a non-newest block with at
// least max_blocks - 1 >= k other blocks ranked above it, and each of their maxima ranks
// above the entry in (score desc, position asc) order, so the entry is not in the top-k.
static bool two_stage(int k, int block, int max_blocks) { return block == 8 && k >= 1 && k <= max_blocks - 1; }

static size_t bmax_bytes(int n, int64_t stride)
{
    return (((size_t)n * (size_t)((stride + 7) / 8) * sizeof(uint32_t)) + 255) & ~(size_t)255;
}

size_t topk_hier_workspace(int n, int64_t stride, int k, int block, int max_blocks)
{
    if ((stride + block - 1) / block <= max_blocks) return plan_workspace(make_plan(stride, k, SRC_FULL), n, k);
    if (two_stage(k, block, max_blocks)) {
        const int64_t bstride = (stride + 7) / 8;
        const size_t blk = plan_workspace(make_plan(bstride, max_blocks - 1, SRC_BMAX), n, max_blocks - 1);
        const size_t flat = plan_workspace(make_plan((int64_t)max_blocks * 8, k, SRC_PGATHER), n, k);
        return bmax_bytes(n, stride) + (blk > flat ? blk : flat);
    }
    const size_t flat = plan_workspace(make_plan(stride, k, SRC_FULL), n, k);
    const int64_t nblk = (stride + block - 1) / block;
    const size_t blk = plan_workspace(make_plan(nblk, max_blocks - 1, SRC_BLOCK), n, max_blocks - 1);
    return flat > blk ? flat : blk;
}

hipError_t launch_topk_hier(const SelSource& src, int k, int block, int max_blocks, int32_t* out_idx,
                            int32_t* out_blocks, int32_t* out_nblocks, void* ws, size_t ws_bytes, hipStream_t stream)
{
    (void)ws_bytes;
    const int n = src.rows.n;
    if (n == 0) return hipSuccess;
    if ((src.stride + block - 1) / block <= max_blocks) {
        // Every row keeps all its blocks (a score row has at most ceil(stride / block)), so
        // the pool needs no selection and the flat top-k runs over the score rows directly
        // (e.g. a replay's source layer: 8192 positions, pools of 2048 blocks).
        hipError_t e = run_plan(src, SRC_FULL, 0, k, src.stride, OUT_IDX, out_idx, k, nullptr, ws, stream);
        if (e != hipSuccess) return e;
        SelSource sb = src;
        sb.pool = PoolArg{nullptr, nullptr, nullptr, block, max_blocks};
        hipLaunchKernelGGL(k_pool_all, dim3((unsigned)n), dim3(256), 0, stream, sb, ilog2(block), out_blocks,
                           max_blocks, out_nblocks);
        return hipGetLastError();
    }
    if (two_stage(k, block, max_blocks)) {
        const int64_t bstride = (src.stride + 7) / 8;
        uint32_t* bmax = static_cast<uint32_t*>(ws);
        void* ws2 = static_cast<char*>(ws) + bmax_bytes(n, src.stride);
        const int chunks = (int)((bstride + 255) / 256);
        SelSource sb = src;
        sb.pool = PoolArg{nullptr, nullptr, nullptr, 8, max_blocks};
        hipLaunchKernelGGL(k_block_max, dim3((unsigned)((int64_t)n * chunks)), dim3(256), 0, stream, sb, bmax, bstride,
                           chunks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = run_plan(sb, SRC_BMAX, 8, max_blocks - 1, bstride, OUT_BLOCKS, out_blocks, max_blocks, out_nblocks, ws2,
                     stream, bmax, bstride);
        if (e != hipSuccess) return e;
        SelSource sp = src;
        sp.pool = PoolArg{out_blocks, out_nblocks, nullptr, 8, max_blocks};
        return run_plan(sp, SRC_PGATHER, 8, k, (int64_t)max_blocks * 8, OUT_IDX, out_idx, k, nullptr, ws2, stream);
    }
    hipError_t e = run_plan(src, SRC_FULL, 0, k, src.stride, OUT_IDX, out_idx, k, nullptr, ws, stream);
    if (e != hipSuccess) return e;
    const int64_t nblk = (src.stride + block - 1) / block;
    return run_plan(src, SRC_BLOCK, block, max_blocks - 1, nblk, OUT_BLOCKS, out_blocks, max_blocks, out_nblocks,
                    ws, stream);
}

}  // namespace csa2
