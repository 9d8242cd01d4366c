// Top-k selection: flat (over every reachable position), over a candidate pool, and
// the hierarchical block pass.
//
// Pages: "DeepSeek V4.1 Flash modeling", section "Hierarchical Sparse Indexer" (top-512
// per query; blocks of 8 positions scored by their maximum, at most 2,048 blocks; later
// index layers select inside that pool); "SGLang and Miles Day-0 support for
// DeepSeek-V4.1", section 2 (the block holding the newest position is always kept; the
// same pass takes its own top-512 over all reachable positions).  Ties go to the lower
// position (problem statement).
//
// Method.  Candidates are mapped to order-preserving 32-bit keys (0 = no candidate).
// One workgroup selects the k best of up to NT*KPT candidates held in registers
// (blocked: thread t owns candidates [t*KPT, (t+1)*KPT), so thread order is candidate
// order): an MSB-first radix select over LDS histograms finds the threshold key T (the
// first pass starts at the highest bit where the largest and smallest keys differ, so
// concentrated score ranges still spread over the bins); the selection is every key
// above T plus the lowest-indexed keys equal to T; two block scans give each thread its
// output offset, so the output is in ascending candidate order.  Rows longer than one
// workgroup's capacity are cut into segments whose local top-k lists are merged by
// further passes (a total order makes the merge exact).
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

enum SrcMode { SRC_FULL = 0, SRC_POOL = 1, SRC_BLOCK = 2, SRC_LIST = 3 };
enum OutMode { OUT_IDX = 0, OUT_LIST = 1, OUT_BLOCKS = 2 };

constexpr int kNT = 512;       // threads per selection workgroup
constexpr int kSegCols = 8192; // candidates per first-level segment (KPT 16)
constexpr int kMergeCap = 16384;  // candidates per merge workgroup (KPT 32)

struct SelArgs {
    SelSource src;
    int mode;           // SrcMode of the first level
    int block;          // SRC_BLOCK: positions per block
    int k;              // entries kept per row
    int nseg;           // segments (lists) per row at this level
    int seg_len;        // candidates per segment (first level) or lists per group (merge)
    int nlists_prev;    // merge level: lists per row in the input
    const uint2* in;    // merge level input lists [n][nlists_prev][k] (key, pos)
    uint2* out_list;    // OUT_LIST target [n][nseg][k]
    int32_t* out_idx;   // OUT_IDX target [n][k] / OUT_BLOCKS target [n][max_blocks]
    int32_t* out_nblocks;
    int out_stride;     // row stride of out_idx (k, or max_blocks)
    int out_mode;
};

__device__ __forceinline__ void row_info(const SelSource& s, int row, int64_t* R, int64_t* ncol, int* prow)
{
    const int r = s.rows.req[row];
    *R = reach(s.rows.pos[row], s.cache.ratio_m, s.cache.n_entries[r]);
    int64_t nc = *R;
    *prow = row;
    if (s.pool.blocks) {
        *prow = s.pool.row_map ? s.pool.row_map[row] : row;
        nc = *R > 0 ? (int64_t)s.pool.nblocks[*prow] * s.pool.block : 0;
    }
    *ncol = nc < s.stride ? nc : s.stride;
}

__device__ __forceinline__ int64_t pool_position(const SelSource& s, int prow, int64_t c)
{
    const int64_t i = c / s.pool.block;
    return (int64_t)s.pool.blocks[(int64_t)prow * s.pool.max_blocks + i] * s.pool.block + (c - i * s.pool.block);
}

template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* s_tmp, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) {
        const int t = s_tmp[w];
        before += (w < wave) ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* s_tmp)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) r = max(r, s_tmp[w]);
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* s_tmp)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, 64));
    if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) r = min(r, s_tmp[w]);
    __syncthreads();
    return r;
}

// Candidate e of a first-level segment: its key (0 = none).
__device__ __forceinline__ uint32_t first_level_key(const SelArgs& a, int row, int64_t R, int64_t ncol, int prow,
                                                    int64_t c)
{
    const SelSource& s = a.src;
    if (a.mode == SRC_BLOCK) {
        // blocks other than the newest: [0, nblk - 1); all their members are reachable
        const int64_t nblk = (ncol + a.block - 1) / a.block;
        if (c >= nblk - 1) return 0u;
        const float* sp = s.scores + (int64_t)row * s.stride + c * a.block;
        uint32_t m = 0;
        for (int u = 0; u < a.block; u++) m = max(m, order_key(sp[u]));
        return m;
    }
    if (c >= ncol) return 0u;
    if (a.mode == SRC_POOL && pool_position(s, prow, c) >= R) return 0u;
    return order_key(s.scores[(int64_t)row * s.stride + c]);
}

template <int KPT>
__global__ __launch_bounds__(kNT) void k_select(SelArgs a, int first_level)
{
    constexpr int NT = kNT;
    constexpr int CAP = NT * KPT;
    __shared__ uint32_t s_keys[CAP + CAP / 32];
    __shared__ int s_hist[256];
    __shared__ int s_tmp[NT / 64];
    __shared__ uint32_t s_res[3];

    const int nseg = a.nseg;
    const int row = blockIdx.x / nseg;
    const int seg = blockIdx.x % nseg;
    const int tid = threadIdx.x;
    const SelSource& s = a.src;

    int64_t R, ncol;
    int prow;
    row_info(s, row, &R, &ncol, &prow);

    // ---- gather keys: striped into LDS (coalesced), then blocked into registers
    const int64_t base = (int64_t)seg * (first_level ? a.seg_len : (int64_t)a.seg_len * a.k);
    for (int i = 0; i < KPT; i++) {
        const int e = i * NT + tid;
        uint32_t key = 0;
        if (first_level) {
            if (e < a.seg_len) key = first_level_key(a, row, R, ncol, prow, base + e);
        } else {
            const int64_t li = base + e;  // index into this row's concatenated lists
            if (e < a.seg_len * a.k && li < (int64_t)a.nlists_prev * a.k)
                key = a.in[(int64_t)row * a.nlists_prev * a.k + li].x;
        }
        s_keys[e + (e >> 5)] = key;
    }
    __syncthreads();
    uint32_t key[KPT];
    int nvalid = 0;
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
        const int e = tid * KPT + i;
        key[i] = s_keys[e + (e >> 5)];
        nvalid += key[i] != 0;
        kmax = max(kmax, key[i]);
        if (key[i] != 0) kmin = min(kmin, key[i]);
    }
    int nv;
    (void)block_exclusive_sum<NT>(nvalid, s_tmp, &nv);
    const int k = a.k;

    // ---- threshold: select key > T, plus the first need_eq keys equal to T
    bool ge_mode = false;  // true: select key >= T (and key != 0)
    uint32_t T = 0;
    int need_eq = 0;
    if (k == 0) {
        ge_mode = true;   // nothing: no non-NaN key reaches 0xFFFFFFFF
        T = 0xFFFFFFFFu;
    } else if (nv <= k) {
        ge_mode = true;
        T = 1;
    } else {
        kmax = block_max_u32<NT>(kmax, reinterpret_cast<uint32_t*>(s_tmp));
        kmin = block_min_u32<NT>(kmin, reinterpret_cast<uint32_t*>(s_tmp));
        const uint32_t diff = kmax ^ kmin;
        if (diff == 0) {
            T = kmax;
            need_eq = k;
        } else {
            int sb = 31 - __clz(diff);
            uint32_t prefix = (sb >= 31) ? 0u : (kmax & (~0u << (sb + 1)));
            int need = k;
            while (true) {
                const int nbits = sb + 1 < 8 ? sb + 1 : 8;
                const int shift = sb + 1 - nbits;
                const uint32_t hm = (sb >= 31) ? 0u : (~0u << (sb + 1));
                const uint32_t dmask = (1u << nbits) - 1u;
                if (tid < 256) s_hist[tid] = 0;
                __syncthreads();
#pragma unroll
                for (int i = 0; i < KPT; i++)
                    if (key[i] != 0 && (key[i] & hm) == (prefix & hm))
                        atomicAdd(&s_hist[(key[i] >> shift) & dmask], 1);
                __syncthreads();
                if (tid < 64) {
                    int c[4], sum = 0;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        c[j] = s_hist[255 - 4 * tid - j];
                        sum += c[j];
                    }
                    int incl = sum;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const int y = __shfl_up(incl, off, 64);
                        if (tid >= off) incl += y;
                    }
                    const int excl = incl - sum;
                    if (excl < need && need <= incl) {
                        int acc = excl;
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            if (acc + c[j] >= need) {
                                s_res[0] = (uint32_t)(255 - 4 * tid - j);
                                s_res[1] = (uint32_t)acc;
                                s_res[2] = (uint32_t)c[j];
                                break;
                            }
                            acc += c[j];
                        }
                    }
                }
                __syncthreads();
                const uint32_t b = s_res[0];
                const int above = (int)s_res[1];
                const int cnt = (int)s_res[2];
                __syncthreads();
                prefix |= b << shift;
                need -= above;
                if (cnt == need) {
                    ge_mode = true;
                    T = prefix;
                    break;
                }
                if (shift == 0) {
                    T = prefix;
                    need_eq = need;
                    break;
                }
                sb = shift - 1;
            }
        }
    }

    // ---- ordered compaction
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
        const bool is_gt = ge_mode ? (key[i] != 0 && key[i] >= T) : (key[i] > T);
        const bool is_eq = !ge_mode && key[i] == T;
        gt += is_gt;
        eq += is_eq;
    }
    int eq_total;
    const int eq_before = block_exclusive_sum<NT>(eq, s_tmp, &eq_total);
    int take = need_eq - eq_before;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    int nsel;
    int off = block_exclusive_sum<NT>(gt + take, s_tmp, &nsel);

    int taken = 0;
    const int64_t row_out = (int64_t)row * nseg + seg;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
        const bool is_gt = ge_mode ? (key[i] != 0 && key[i] >= T) : (key[i] > T);
        bool sel = is_gt;
        if (!ge_mode && key[i] == T) {
            sel = taken < take;
            taken++;
        }
        if (sel) {
            const int e = tid * KPT + i;
            int32_t pos;
            if (first_level) {
                const int64_t c = base + e;
                pos = (int32_t)((a.mode == SRC_POOL) ? pool_position(s, prow, c) : c);
            } else {
                pos = (int32_t)a.in[(int64_t)row * a.nlists_prev * k + base + e].y;
            }
            if (a.out_mode == OUT_LIST)
                a.out_list[row_out * k + off] = make_uint2(key[i], (uint32_t)pos);
            else
                a.out_idx[(int64_t)row * a.out_stride + off] = pos;
            off++;
        }
    }
    // ---- padding (and the newest block of the hierarchical pool)
    if (a.out_mode == OUT_LIST) {
        for (int i = nsel + tid; i < k; i += NT) a.out_list[row_out * k + i] = make_uint2(0u, 0xFFFFFFFFu);
    } else if (a.out_mode == OUT_IDX) {
        for (int i = nsel + tid; i < a.out_stride; i += NT) a.out_idx[(int64_t)row * a.out_stride + i] = -1;
    } else {
        const int64_t nblk = (ncol + a.block - 1) / a.block;
        int tot = nsel;
        if (nblk > 0) {
            if (tid == 0) a.out_idx[(int64_t)row * a.out_stride + nsel] = (int32_t)(nblk - 1);
            tot = nsel + 1;
        }
        for (int i = tot + tid; i < a.out_stride; i += NT) a.out_idx[(int64_t)row * a.out_stride + i] = -1;
        if (tid == 0) a.out_nblocks[row] = tot;
    }
}

// ------------------------------------------------------------------------ host plans
struct Plan {
    int levels;
    int nseg[8];  // lists per row produced by each level (last level: 1)
};

static Plan make_plan(int64_t cols, int k)
{
    Plan p{};
    int64_t n0 = (cols + kSegCols - 1) / kSegCols;
    if (n0 < 1 || k == 0) n0 = 1;
    p.levels = 1;
    p.nseg[0] = (int)n0;
    int64_t cur = n0;
    const int group = k > 0 ? kMergeCap / k : kMergeCap;
    while (cur > 1 && p.levels < 8) {
        cur = (cur + group - 1) / group;
        p.nseg[p.levels++] = (int)cur;
    }
    return p;
}

static size_t plan_workspace(const Plan& p, int n, int k)
{
    if (p.levels <= 1) return 0;
    // level 0 output in buffer A, level 1 in B, level 2 in A, ...
    size_t a = 0, b = 0;
    for (int l = 0; l + 1 < p.levels; l++) {
        size_t sz = (size_t)n * p.nseg[l] * (size_t)(k > 0 ? k : 1) * sizeof(uint2);
        if (l % 2 == 0) a = sz > a ? sz : a; else b = sz > b ? sz : b;
    }
    return ((a + 255) & ~(size_t)255) + b;
}

static hipError_t run_plan(const SelSource& src, int mode, int block, int k, int64_t cols, int out_mode,
                           int32_t* out_idx, int out_stride, int32_t* out_nblocks, void* ws, hipStream_t stream)
{
    const int n = src.rows.n;
    if (n == 0) return hipSuccess;
    const Plan p = make_plan(cols, k);
    const size_t sza = [&] {
        size_t a = 0;
        for (int l = 0; l + 1 < p.levels; l += 2) {
            size_t sz = (size_t)n * p.nseg[l] * (size_t)(k > 0 ? k : 1) * sizeof(uint2);
            a = sz > a ? sz : a;
        }
        return (a + 255) & ~(size_t)255;
    }();
    uint2* bufA = static_cast<uint2*>(ws);
    uint2* bufB = reinterpret_cast<uint2*>(static_cast<char*>(ws) + sza);
    const uint2* prev = nullptr;
    for (int l = 0; l < p.levels; l++) {
        SelArgs a{};
        a.src = src;
        a.mode = mode;
        a.block = block;
        a.k = k;
        a.nseg = p.nseg[l];
        a.seg_len = (l == 0) ? kSegCols : kMergeCap / (k > 0 ? k : 1);
        a.nlists_prev = (l == 0) ? 0 : p.nseg[l - 1];
        a.in = prev;
        const bool last = (l + 1 == p.levels);
        a.out_mode = last ? out_mode : OUT_LIST;
        a.out_list = (l % 2 == 0) ? bufA : bufB;
        a.out_idx = out_idx;
        a.out_nblocks = out_nblocks;
        a.out_stride = out_stride;
        dim3 grid((unsigned)((int64_t)n * p.nseg[l]));
        if (l == 0)
            hipLaunchKernelGGL((k_select<kSegCols / kNT>), grid, dim3(kNT), 0, stream, a, 1);
        else
            hipLaunchKernelGGL((k_select<kMergeCap / kNT>), grid, dim3(kNT), 0, stream, a, 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        prev = a.out_list;
    }
    return hipSuccess;
}

static int64_t select_cols(const SelSource& src)
{
    return src.pool.blocks ? (int64_t)src.pool.block * src.pool.max_blocks : src.stride;
}

size_t topk_workspace(int n, int64_t stride, int k) { return plan_workspace(make_plan(stride, k), n, k); }

hipError_t launch_topk(const SelSource& src, int k, int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    (void)ws_bytes;
    return run_plan(src, src.pool.blocks ? SRC_POOL : SRC_FULL, 0, k, select_cols(src), OUT_IDX, out, k, nullptr,
                    ws, stream);
}

size_t topk_hier_workspace(int n, int64_t stride, int k, int block, int max_blocks)
{
    const size_t flat = plan_workspace(make_plan(stride, k), n, k);
    const int64_t nblk = (stride + block - 1) / block;
    const size_t blk = plan_workspace(make_plan(nblk, max_blocks - 1), n, max_blocks - 1);
    return flat > blk ? flat : blk;
}

hipError_t launch_topk_hier(const SelSource& src, int k, int block, int max_blocks, int32_t* out_idx,
                            int32_t* out_blocks, int32_t* out_nblocks, void* ws, size_t ws_bytes, hipStream_t stream)
{
    (void)ws_bytes;
    hipError_t e = run_plan(src, SRC_FULL, 0, k, src.stride, OUT_IDX, out_idx, k, nullptr, ws, stream);
    if (e != hipSuccess) return e;
    const int64_t nblk = (src.stride + block - 1) / block;
    return run_plan(src, SRC_BLOCK, block, max_blocks - 1, nblk, OUT_BLOCKS, out_blocks, max_blocks, out_nblocks,
                    ws, stream);
}

}  // namespace csa2
