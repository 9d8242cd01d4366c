// Device-side check of the device-array preconditions the entry points state: query
// rows (request, position, window floor), the cache geometry, candidate pools and
// selected index sets.  Nothing is computed from the checked values; each violation
// sets its bit in a caller-owned error word.  Every read stays inside the arrays as
// their host-checked sizes give them: a row's request, pool row or index row is used
// as an index only after it has been found in range.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

// Bit values (the same as the CSA2_BAD_* constants of the header).
enum : uint32_t {
    kBadReq = 1u, kBadPos = 2u, kBadWinLo = 4u, kBadCache = 8u,
    kBadPoolMap = 16u, kBadPool = 32u, kBadSelMap = 64u, kBadSel = 128u,
};

// OR of a value over the wave.
__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    for (int off = 32; off >= 1; off >>= 1) v |= (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

__global__ __launch_bounds__(64) void k_clear_word(uint32_t* __restrict__ word) { if (threadIdx.x == 0) *word = 0u; }

// One workgroup per query row (grid-strided); the first workgroup also checks the
// cache geometry of every request.
__global__ __launch_bounds__(256) void k_check_inputs(RowsArg rows, int nreq, CacheArg cache, PoolArg pool,
                                                      int pool_rows, const int32_t* __restrict__ sel, int k,
                                                      int64_t sel_stride, const int32_t* __restrict__ sel_row_map,
                                                      int sel_rows, uint32_t* __restrict__ word)
{
    const int tid = threadIdx.x;
    uint32_t bad = 0;
    if (blockIdx.x == 0) {
        for (int r = tid; r < nreq; r += blockDim.x)
            if (cache.n_entries[r] < 0 || cache.row_start[r] < 0) bad |= kBadCache;
    }
    // block ids must keep b * block + block - 1 inside an int32 position
    const int64_t max_bid = pool.blocks ? (int64_t)INT32_MAX / pool.block - 1 : 0;
    for (int row = blockIdx.x; row < rows.n; row += gridDim.x) {
        const int r = rows.req[row];
        const int p = rows.pos[row];
        const bool req_ok = r >= 0 && r < nreq;
        if (!req_ok) bad |= kBadReq;
        if (p < 0) bad |= kBadPos;
        if (rows.win_lo) {
            const int lo = rows.win_lo[row];
            if (lo < 0 || lo > p) bad |= kBadWinLo;
        }
        if (!req_ok || p < 0) continue;  // no reach to check against
        const int ne = cache.n_entries[r];
        const int64_t R = ne < 0 ? 0 : reach(p, cache.ratio_m, ne);
        if (sel) {
            const int srow = sel_row_map ? sel_row_map[row] : row;
            if (srow < 0 || srow >= sel_rows) {
                bad |= kBadSelMap;
            } else {
                const int32_t* s = sel + (int64_t)srow * sel_stride;
                for (int i = tid; i < k; i += blockDim.x) {
                    const int32_t j = s[i];
                    if (j != -1 && (j < 0 || (int64_t)j >= R)) bad |= kBadSel;
                }
            }
        }
        if (pool.blocks) {
            const int prow = pool.row_map ? pool.row_map[row] : row;
            if (prow < 0 || prow >= pool_rows) {
                bad |= kBadPoolMap;
            } else {
                const int nb = pool.nblocks[prow];
                if (nb < 0 || nb > pool.max_blocks) {
                    bad |= kBadPool;
                } else {
                    const int32_t* b = pool.blocks + (int64_t)prow * pool.max_blocks;
                    for (int i = tid; i < nb; i += blockDim.x) {
                        const int32_t v = b[i];
                        if (v < 0 || (int64_t)v > max_bid || (i > 0 && b[i - 1] >= v)) bad |= kBadPool;
                    }
                }
            }
        }
    }
    bad = wave_or(bad);
    if ((tid & 63) == 0 && bad) atomicOr(word, bad);
}

hipError_t launch_check_inputs(const RowsArg& rows, int nreq, const CacheArg& cache, const PoolArg& pool,
                               int pool_rows, const int32_t* sel, int k, int64_t sel_stride,
                               const int32_t* sel_row_map, int sel_rows, uint32_t* word, hipStream_t stream)
{
    hipLaunchKernelGGL(k_clear_word, dim3(1), dim3(64), 0, stream, word);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = rows.n < 1 ? 1 : (rows.n < 4096 ? rows.n : 4096);
    hipLaunchKernelGGL(k_check_inputs, dim3(grid), dim3(256), 0, stream, rows, nreq, cache, pool, pool_rows, sel, k,
                       sel_stride, sel_row_map, sel_rows, word);
    return hipGetLastError();
}

}  // namespace csa2
