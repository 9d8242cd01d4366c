// C ABI of the CSA2 hot path: argument validation, workspace sizing and dispatch to
// the gfx950 kernels.  Every check on scalar or host-visible arguments happens before
// any HIP call, so argument errors are reported identically with or without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/csa2.h"
#include "csa2_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return CSA2_OK;
}

int launch_result(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(CSA2_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The kernels use gfx950 instructions (scaled FP4 MFMA, lane swaps): refuse others.
int check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA2_E_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    static std::mutex mu;
    static int known[64] = {0};  // 0 unknown, 1 gfx950, 2 other
    if (dev < 0 || dev >= 64) return fail(CSA2_E_UNSUPPORTED, "device index %d out of range", dev);
    {
        std::lock_guard<std::mutex> lock(mu);
        if (known[dev] == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess) return fail(CSA2_E_LAUNCH, "hipGetDeviceProperties: %s", hipGetErrorString(e));
            known[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        }
        if (known[dev] != 1) return fail(CSA2_E_UNSUPPORTED, "device %d is not gfx950", dev);
    }
    return CSA2_OK;
}

// The kernels move element data in 8- and 16-byte vectors.
bool misaligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) != 0; }

int check_rows(const csa2_rows* rows)
{
    if (!rows) return fail(CSA2_E_ARG, "rows is NULL");
    if (rows->n < 0) return fail(CSA2_E_ARG, "rows->n = %d < 0", rows->n);
    if (rows->n > 0 && (!rows->req_of_row || !rows->pos_of_row))
        return fail(CSA2_E_ARG, "rows->req_of_row / pos_of_row is NULL");
    return CSA2_OK;
}

int check_cache(const csa2_cache* cache)
{
    if (!cache) return fail(CSA2_E_ARG, "cache is NULL");
    if (cache->nreq < 1) return fail(CSA2_E_ARG, "cache->nreq = %d < 1", cache->nreq);
    if (cache->ratio_m != 1 && cache->ratio_m != 2)
        return fail(CSA2_E_UNSUPPORTED, "cache->ratio_m = %d (1 or 2)", cache->ratio_m);
    if (!cache->n_entries || !cache->row_start) return fail(CSA2_E_ARG, "cache->n_entries / row_start is NULL");
    return CSA2_OK;
}

int check_pool(const csa2_pool* pool, int64_t score_stride)
{
    if (!pool) return CSA2_OK;
    if (!pool->blocks || !pool->nblocks) return fail(CSA2_E_ARG, "pool->blocks / nblocks is NULL");
    if (pool->block < 1 || pool->block > 64 || (pool->block & (pool->block - 1)))
        return fail(CSA2_E_ARG, "pool->block = %d (a power of two, 1..64)", pool->block);
    if (pool->max_blocks < 1 || pool->max_blocks > 65536)
        return fail(CSA2_E_ARG, "pool->max_blocks = %d (1..65536)", pool->max_blocks);
    if ((int64_t)pool->block * pool->max_blocks > score_stride)
        return fail(CSA2_E_ARG, "pool columns %lld exceed score_stride %lld",
                    (long long)pool->block * pool->max_blocks, (long long)score_stride);
    return CSA2_OK;
}

csa2::RowsArg rows_arg(const csa2_rows* r) { return csa2::RowsArg{r->n, r->req_of_row, r->pos_of_row, r->win_lo}; }
csa2::CacheArg cache_arg(const csa2_cache* c)
{
    return csa2::CacheArg{c->ratio_m, c->n_entries, c->row_start, c->nreq};
}
csa2::PoolArg pool_arg(const csa2_pool* p)
{
    if (!p) return csa2::PoolArg{nullptr, nullptr, nullptr, 0, 0};
    return csa2::PoolArg{p->blocks, p->nblocks, p->row_map, p->block, p->max_blocks};
}

// Scratch of csa2_topk_hier_noalloc: one array per device, held until the process ends.
// Its name is a host-side stand-in for the device copy, so host code never passes it to
// a kernel: the device address comes from hipGetSymbolAddress, taken once per device
// with that device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

int scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA2_E_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(CSA2_E_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CSA2_E_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA2_OK;
}

}  // namespace

extern "C" {

const char* csa2_last_error(void) { return g_err.c_str(); }

int csa2_version(void) { return CSA2_VERSION; }

size_t csa2_workspace_size(int op, int32_t n, int64_t cols, int32_t k, int32_t max_blocks)
{
    if (n <= 0 || cols <= 0) return 0;
    switch (op) {
        case CSA2_OP_TOPK:
            // cols = score columns (full range) or block*max_blocks (pool): the plan for
            // the pool source is never smaller, so size for it
            return csa2::topk_workspace(n, cols, k, true);
        case CSA2_OP_TOPK_HIER:
            return csa2::topk_hier_workspace(n, cols, k, 8, max_blocks > 0 ? max_blocks : 1);
        case CSA2_OP_ATTN:
            return 0;
        case CSA2_OP_TOPK_POOL_FUSED:
            // cols = block * max_blocks of the pool
            return csa2::score_topk_pool_workspace(n, cols, k);
        default:
            return 0;
    }
}

// Index q of the MXFP4 kernels: BF16, or MXFP4 codes with their E8M0 scale plane.
static int check_index_q(const void* q_idx, csa2_dtype q_dtype, const uint8_t* q_scale, const char* who)
{
    if (q_dtype != CSA2_BF16 && q_dtype != CSA2_MXFP4)
        return fail(CSA2_E_UNSUPPORTED, "%s: index q dtype %d (BF16 or MXFP4)", who, (int)q_dtype);
    if ((q_dtype == CSA2_MXFP4) != (q_scale != nullptr))
        return fail(CSA2_E_ARG, q_dtype == CSA2_MXFP4 ? "%s: MXFP4 index q without q_scale"
                                                      : "%s: q_scale given for a BF16 index q", who);
    if (misaligned(q_idx, 16)) return fail(CSA2_E_ARG, "%s: q_idx must start on a 16-byte boundary", who);
    return CSA2_OK;
}

int csa2_index_score(const csa2_rows* rows, const csa2_cache* cache, const void* q_idx, csa2_dtype q_dtype,
                     const uint8_t* q_scale, int32_t heads, const float* w, int64_t w_row_stride,
                     const csa2_index_keys* keys, const csa2_pool* pool, float* scores, int64_t score_stride,
                     void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!keys) return fail(CSA2_E_ARG, "keys is NULL");
    if (!q_idx || !w || !scores || !keys->data) return fail(CSA2_E_ARG, "q_idx / w / scores / keys->data is NULL");
    if (score_stride < 1) return fail(CSA2_E_ARG, "score_stride = %lld < 1", (long long)score_stride);
    if (w_row_stride < 0) return fail(CSA2_E_ARG, "w_row_stride < 0");
    if ((rc = check_pool(pool, score_stride))) return rc;
    if (keys->dtype == CSA2_MXFP4) {
        if ((rc = check_index_q(q_idx, q_dtype, q_scale, "MXFP4 keys"))) return rc;
        if (keys->dim != 128) return fail(CSA2_E_UNSUPPORTED, "MXFP4 keys: dim %d (128 supported)", keys->dim);
        if (!keys->scale) return fail(CSA2_E_ARG, "MXFP4 keys without a scale plane");
        if (misaligned(keys->data, 16)) return fail(CSA2_E_ARG, "keys->data must start on a 16-byte boundary");
        if (heads < 16 || heads > 128 || heads % 16)
            return fail(CSA2_E_UNSUPPORTED, "MXFP4 scoring: heads %d (multiple of 16, at most 128)", heads);
        if (w_row_stride != 0 && w_row_stride < heads) return fail(CSA2_E_ARG, "w_row_stride < heads");
    } else if (keys->dtype == CSA2_F32) {
        if (q_dtype != CSA2_F32) return fail(CSA2_E_UNSUPPORTED, "F32 keys need an F32 index q");
        if (q_scale) return fail(CSA2_E_ARG, "q_scale given for an F32 index q");
        if (keys->dim < 1 || keys->dim > 1024) return fail(CSA2_E_UNSUPPORTED, "F32 keys: dim %d", keys->dim);
        if (heads < 4 || heads > 128 || heads % 4)
            return fail(CSA2_E_UNSUPPORTED, "F32 scoring: heads %d (multiple of 4, at most 128)", heads);
        if (w_row_stride != 0 && w_row_stride < heads) return fail(CSA2_E_ARG, "w_row_stride < heads");
    } else {
        return fail(CSA2_E_UNSUPPORTED, "index key dtype %d", (int)keys->dtype);
    }
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (keys->dtype == CSA2_MXFP4)
        return launch_result(csa2::launch_index_score_mxfp4(rows_arg(rows), cache_arg(cache),
                                                            csa2::IndexQ{q_idx, q_scale}, heads, w,
                                                            w_row_stride, static_cast<const uint8_t*>(keys->data),
                                                            keys->scale, pool_arg(pool), scores, score_stride, s),
                             "csa2_index_score");
    return launch_result(csa2::launch_index_score_f32(rows_arg(rows), cache_arg(cache), static_cast<const float*>(q_idx),
                                                      heads, keys->dim, w, w_row_stride,
                                                      static_cast<const float*>(keys->data), pool_arg(pool), scores,
                                                      score_stride, s),
                         "csa2_index_score");
}

int csa2_index_topk_pool(const csa2_rows* rows, const csa2_cache* cache, const void* q_idx, csa2_dtype q_dtype,
                         const uint8_t* q_scale, int32_t heads, const float* w, int64_t w_row_stride,
                         const csa2_index_keys* keys, const csa2_pool* pool, int32_t k, int32_t* out_idx,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!keys || !pool) return fail(CSA2_E_ARG, "keys / pool is NULL");
    if (!q_idx || !w || !out_idx || !keys->data) return fail(CSA2_E_ARG, "q_idx / w / out_idx / keys->data is NULL");
    if (w_row_stride < 0) return fail(CSA2_E_ARG, "w_row_stride < 0");
    if (k < 1 || k > 2048) return fail(CSA2_E_ARG, "k = %d (1..2048)", k);
    if (pool->block != 8) return fail(CSA2_E_UNSUPPORTED, "pool block %d (8 supported)", pool->block);
    if (pool->max_blocks < 1 || pool->max_blocks > 2048)
        return fail(CSA2_E_UNSUPPORTED, "pool max_blocks %d (1..2048: the pool fits one workgroup)", pool->max_blocks);
    if ((rc = check_pool(pool, (int64_t)pool->block * pool->max_blocks))) return rc;
    if (keys->dtype != CSA2_MXFP4 || keys->dim != 128 || !keys->scale)
        return fail(CSA2_E_UNSUPPORTED, "fused pool top-k: MXFP4 keys of dim 128 with a scale plane");
    if ((rc = check_index_q(q_idx, q_dtype, q_scale, "fused pool top-k"))) return rc;
    if (heads != 16 && heads != 32 && heads != 64)
        return fail(CSA2_E_UNSUPPORTED, "fused pool top-k: heads %d (16, 32 or 64)", heads);
    if (w_row_stride != 0 && w_row_stride < heads) return fail(CSA2_E_ARG, "w_row_stride < heads");
    if (misaligned(keys->data, 16)) return fail(CSA2_E_ARG, "keys->data must start on a 16-byte boundary");
    if (misaligned(keys->scale, 4)) return fail(CSA2_E_ARG, "keys->scale must start on a 4-byte boundary");
    if (rows->n == 0) return ok();
    const size_t need = csa2::score_topk_pool_workspace(rows->n, (int64_t)pool->block * pool->max_blocks, k);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(CSA2_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if ((rc = check_device())) return rc;
    return launch_result(csa2::launch_score_topk_pool(rows_arg(rows), cache_arg(cache),
                                                      csa2::IndexQ{q_idx, q_scale}, heads, w, w_row_stride,
                                                      static_cast<const uint8_t*>(keys->data), keys->scale,
                                                      pool_arg(pool), k, out_idx, workspace,
                                                      static_cast<hipStream_t>(stream)),
                         "csa2_index_topk_pool");
}

int csa2_topk(const csa2_rows* rows, const csa2_cache* cache, const float* scores, int64_t score_stride,
              const csa2_pool* pool, int32_t k, int32_t* out_idx, void* workspace, size_t workspace_bytes,
              void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!scores || !out_idx) return fail(CSA2_E_ARG, "scores / out_idx is NULL");
    if (k < 1 || k > 2048) return fail(CSA2_E_ARG, "k = %d (1..2048)", k);
    if (score_stride < 1) return fail(CSA2_E_ARG, "score_stride = %lld < 1", (long long)score_stride);
    if ((rc = check_pool(pool, score_stride))) return rc;
    const int64_t cols = pool ? (int64_t)pool->block * pool->max_blocks : score_stride;
    const size_t need = csa2::topk_workspace(rows->n, cols, k, pool != nullptr);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(CSA2_E_WORKSPACE, "csa2_topk needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    csa2::SelSource src{scores, score_stride, rows_arg(rows), cache_arg(cache), pool_arg(pool)};
    return launch_result(csa2::launch_topk(src, k, out_idx, workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                         "csa2_topk");
}

int csa2_topk_hier(const csa2_rows* rows, const csa2_cache* cache, const float* scores, int64_t score_stride,
                   int32_t k, int32_t block, int32_t max_blocks, int32_t* out_idx, int32_t* out_pool_blocks,
                   int32_t* out_pool_nblocks, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!scores || !out_idx || !out_pool_blocks || !out_pool_nblocks)
        return fail(CSA2_E_ARG, "scores / out_idx / out_pool_blocks / out_pool_nblocks is NULL");
    if (k < 1 || k > 2048) return fail(CSA2_E_ARG, "k = %d (1..2048)", k);
    if (block != 8) return fail(CSA2_E_UNSUPPORTED, "block = %d (8 supported)", block);
    if (max_blocks < 1 || max_blocks > 4096) return fail(CSA2_E_ARG, "max_blocks = %d (1..4096)", max_blocks);
    if (score_stride < 1) return fail(CSA2_E_ARG, "score_stride = %lld < 1", (long long)score_stride);
    const size_t need = csa2::topk_hier_workspace(rows->n, score_stride, k, block, max_blocks);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(CSA2_E_WORKSPACE, "csa2_topk_hier needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    csa2::SelSource src{scores, score_stride, rows_arg(rows), cache_arg(cache), pool_arg(nullptr)};
    return launch_result(csa2::launch_topk_hier(src, k, block, max_blocks, out_idx, out_pool_blocks, out_pool_nblocks,
                                                workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                         "csa2_topk_hier");
}

int csa2_topk_hier_noalloc(const csa2_rows* rows, const csa2_cache* cache, const float* scores,
                           int64_t score_stride, int32_t k, int32_t block, int32_t max_blocks, int32_t* out_idx,
                           int32_t* out_pool_blocks, int32_t* out_pool_nblocks, void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!scores || !out_idx || !out_pool_blocks || !out_pool_nblocks)
        return fail(CSA2_E_ARG, "scores / out_idx / out_pool_blocks / out_pool_nblocks is NULL");
    if (k < 1 || k > 2048) return fail(CSA2_E_ARG, "k = %d (1..2048)", k);
    if (block != 8) return fail(CSA2_E_UNSUPPORTED, "block = %d (8 supported)", block);
    if (max_blocks < 1 || max_blocks > 4096) return fail(CSA2_E_ARG, "max_blocks = %d (1..4096)", max_blocks);
    if (score_stride < 1) return fail(CSA2_E_ARG, "score_stride = %lld < 1", (long long)score_stride);
    const size_t need = csa2::topk_hier_workspace(rows->n, score_stride, k, block, max_blocks);
    if (need > kScratchBytes)
        return fail(CSA2_E_WORKSPACE,
                    "csa2_topk_hier_noalloc: %d rows x %lld columns need %zu scratch bytes, more than its %zu; "
                    "use csa2_topk_hier with a workspace",
                    rows->n, (long long)score_stride, need, kScratchBytes);
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    void* ws = nullptr;
    if (need > 0 && (rc = scratch_address(&ws))) return rc;
    csa2::SelSource src{scores, score_stride, rows_arg(rows), cache_arg(cache), pool_arg(nullptr)};
    return launch_result(csa2::launch_topk_hier(src, k, block, max_blocks, out_idx, out_pool_blocks, out_pool_nblocks,
                                                ws, need, static_cast<hipStream_t>(stream)),
                         "csa2_topk_hier_noalloc");
}

int csa2_sparse_swa_attn(const csa2_rows* rows, const csa2_cache* cache, const void* q, csa2_dtype q_dtype,
                         int32_t heads, int32_t dim, const void* kv, csa2_dtype kv_dtype, const uint8_t* kv_scale,
                         const int32_t* sel_idx, int32_t k, int64_t sel_stride, const int32_t* sel_row_map,
                         const csa2_swa* swa, float sm_scale, const float* sink, void* out, csa2_dtype out_dtype,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    (void)workspace;
    (void)workspace_bytes;
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!q || !kv || !out || !swa) return fail(CSA2_E_ARG, "q / kv / out / swa is NULL");
    if (k < 0 || k > 2048) return fail(CSA2_E_ARG, "k = %d (0..2048)", k);
    if (k > 0 && !sel_idx) return fail(CSA2_E_ARG, "sel_idx is NULL with k = %d", k);
    if (k > sel_stride) return fail(CSA2_E_ARG, "k = %d exceeds sel_stride %lld", k, (long long)sel_stride);
    if (!swa->data || !swa->row_start || !swa->pos_start) return fail(CSA2_E_ARG, "swa data / row_start / pos_start is NULL");
    if (swa->window < 1 || swa->window > 4096) return fail(CSA2_E_ARG, "swa->window = %d (1..4096)", swa->window);
    if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(CSA2_E_ARG, "sm_scale must be positive and finite");
    if (heads < 1 || dim < 1) return fail(CSA2_E_ARG, "heads / dim < 1");
    const bool f32 = q_dtype == CSA2_F32 && kv_dtype == CSA2_F32 && swa->dtype == CSA2_F32 && out_dtype == CSA2_F32;
    const bool kv_fp4 = kv_dtype == CSA2_FP4_S16;
    const bool bf = q_dtype == CSA2_BF16 && (kv_dtype == CSA2_BF16 || kv_fp4) &&
                    (swa->dtype == CSA2_MXFP8_E4M3 || swa->dtype == CSA2_BF16) && out_dtype == CSA2_BF16;
    if (kv_fp4 != (kv_scale != nullptr))
        return fail(CSA2_E_ARG, kv_fp4 ? "FP4_S16 kv without kv_scale" : "kv_scale given for a kv dtype without scales");
    if (f32) {
        if (dim > 256) return fail(CSA2_E_UNSUPPORTED, "F32 attention: dim %d > 256", dim);
        if (heads > 1024) return fail(CSA2_E_UNSUPPORTED, "F32 attention: heads %d > 1024", heads);
    } else if (bf) {
        if (dim != 512) return fail(CSA2_E_UNSUPPORTED, "BF16 attention: dim %d (512 supported)", dim);
        if (heads % 16 || heads > 1024) return fail(CSA2_E_UNSUPPORTED, "BF16 attention: heads %d (multiple of 16)", heads);
        if (swa->dtype == CSA2_MXFP8_E4M3 && !swa->scale) return fail(CSA2_E_ARG, "MXFP8 window without scales");
        if (misaligned(q, 16) || misaligned(kv, 16) || misaligned(out, 16) || misaligned(swa->data, 16) ||
            (swa->scale && misaligned(swa->scale, 16)) || (kv_scale && misaligned(kv_scale, 16)))
            return fail(CSA2_E_ARG,
                        "q / kv / kv_scale / out / swa->data / swa->scale must start on a 16-byte boundary");
    } else {
        return fail(CSA2_E_UNSUPPORTED, "attention dtypes (q %d, kv %d, window %d, out %d)", (int)q_dtype,
                    (int)kv_dtype, (int)swa->dtype, (int)out_dtype);
    }
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    csa2::SwaArg sa{(int)swa->dtype, swa->data, swa->scale, swa->row_start, swa->pos_start, swa->window};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (f32)
        return launch_result(csa2::launch_attn_f32(rows_arg(rows), cache_arg(cache), static_cast<const float*>(q), heads,
                                                   dim, static_cast<const float*>(kv), sel_idx, k, sel_stride,
                                                   sel_row_map, sa, sm_scale, sink, static_cast<float*>(out), lse, s),
                             "csa2_sparse_swa_attn");
    return launch_result(csa2::launch_attn_bf16(rows_arg(rows), cache_arg(cache), static_cast<const uint16_t*>(q), heads,
                                                kv, kv_scale, sel_idx, k, sel_stride, sel_row_map, sa, sm_scale, sink,
                                                static_cast<uint16_t*>(out), lse, s),
                         "csa2_sparse_swa_attn");
}

int csa2_replay_tail_layout(int32_t nreq, const int32_t* ext_len, const int32_t* seq_len, const int32_t* is_decode,
                            int32_t budget, int32_t flags, int32_t* tail_len, int32_t* tail_row_start,
                            int32_t* src_row, int32_t* abs_pos, int32_t* win_lo, int32_t* req_of_row,
                            int32_t capacity, void* stream)
{
    if (nreq < 0) return fail(CSA2_E_ARG, "nreq = %d < 0", nreq);
    if (budget < 1) return fail(CSA2_E_ARG, "budget = %d < 1", budget);
    if (flags & ~CSA2_TAIL_BORROW_PREFIX_WINDOW) return fail(CSA2_E_ARG, "unknown flags 0x%x", flags);
    if (!tail_row_start) return fail(CSA2_E_ARG, "tail_row_start is NULL");
    if (nreq > 0 && (!ext_len || !seq_len || !tail_len || !src_row || !abs_pos || !win_lo || !req_of_row))
        return fail(CSA2_E_ARG, "a tail-layout array is NULL");
    if ((int64_t)capacity < (int64_t)budget * nreq)
        return fail(CSA2_E_ARG, "capacity %d < budget %d x nreq %d", capacity, budget, nreq);
    if ((int64_t)budget * nreq > 0x7FFFFFFF) return fail(CSA2_E_ARG, "budget x nreq overflows int32");
    int rc;
    if ((rc = check_device())) return rc;
    return launch_result(csa2::launch_replay_tail_layout(nreq, ext_len, seq_len, is_decode, budget, flags, tail_len,
                                                         tail_row_start, src_row, abs_pos, win_lo, req_of_row,
                                                         static_cast<hipStream_t>(stream)),
                         "csa2_replay_tail_layout");
}

int csa2_encoder_replay_layout(int32_t nreq, const int32_t* prefix_len, const int32_t* ext_len, int64_t n_ext,
                               int32_t budget, int32_t* row_start, int32_t* src_row, int32_t* abs_pos,
                               int32_t* win_lo, int32_t* req_of_row, int32_t capacity, void* stream)
{
    if (nreq < 0) return fail(CSA2_E_ARG, "nreq = %d < 0", nreq);
    if (budget < 1) return fail(CSA2_E_ARG, "budget = %d < 1", budget);
    if (n_ext < 0) return fail(CSA2_E_ARG, "n_ext = %lld < 0", (long long)n_ext);
    if (!row_start) return fail(CSA2_E_ARG, "row_start is NULL");
    if (nreq > 0 && (!prefix_len || !ext_len || !src_row || !abs_pos || !win_lo || !req_of_row))
        return fail(CSA2_E_ARG, "an encoder-replay layout array is NULL");
    const int64_t bound = (int64_t)budget * nreq + n_ext;
    if (bound > 0x7FFFFFFF) return fail(CSA2_E_ARG, "budget x nreq + n_ext overflows int32");
    if ((int64_t)capacity < bound)
        return fail(CSA2_E_ARG, "capacity %d < budget %d x nreq %d + n_ext %lld", capacity, budget, nreq,
                    (long long)n_ext);
    int rc;
    if ((rc = check_device())) return rc;
    return launch_result(csa2::launch_encoder_replay_layout(nreq, prefix_len, ext_len, budget, row_start, src_row,
                                                            abs_pos, win_lo, req_of_row,
                                                            static_cast<hipStream_t>(stream)),
                         "csa2_encoder_replay_layout");
}

int csa2_kv_produce(const csa2_rows* rows, const csa2_cache* cache, const float* comp, float* pending,
                    const uint16_t* w_index, const float* rope, int64_t max_pos, csa2_dtype kv_dtype, void* kv,
                    uint8_t* kv_scale, uint8_t* index_codes, uint8_t* index_scales, void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!comp || !w_index || !rope || !kv || !index_codes || !index_scales)
        return fail(CSA2_E_ARG, "comp / w_index / rope / kv / index_codes / index_scales is NULL");
    if (cache->ratio_m == 2 && !pending) return fail(CSA2_E_ARG, "pending is NULL with ratio_m = 2");
    if (max_pos < 1) return fail(CSA2_E_ARG, "max_pos = %lld < 1", (long long)max_pos);
    if (kv_dtype != CSA2_FP4_S16 && kv_dtype != CSA2_BF16)
        return fail(CSA2_E_UNSUPPORTED, "kv_dtype %d (FP4_S16 or BF16)", (int)kv_dtype);
    if ((kv_dtype == CSA2_FP4_S16) != (kv_scale != nullptr))
        return fail(CSA2_E_ARG, "kv_scale goes with FP4_S16 main KV only");
    if (misaligned(comp, 16) || misaligned(pending, 16) || misaligned(w_index, 16) || misaligned(kv, 16) ||
        misaligned(index_codes, 16))
        return fail(CSA2_E_ARG, "comp / pending / w_index / kv / index_codes must start on a 16-byte boundary");
    if (rows->n == 0) return ok();
    if ((rc = check_device())) return rc;
    return launch_result(csa2::launch_kv_produce(rows->n, rows->req_of_row, rows->pos_of_row, cache->ratio_m,
                                                 cache->row_start, comp, pending, w_index, rope, max_pos,
                                                 kv_dtype == CSA2_FP4_S16, kv, kv_scale, index_codes, index_scales,
                                                 static_cast<hipStream_t>(stream)),
                         "csa2_kv_produce");
}

int csa2_quant_mx(csa2_dtype fmt, const void* x, csa2_dtype x_dtype, int64_t nblocks, uint8_t* codes,
                  uint8_t* scales, void* stream)
{
    if (fmt != CSA2_MXFP4 && fmt != CSA2_MXFP8_E4M3 && fmt != CSA2_FP4_S16)
        return fail(CSA2_E_UNSUPPORTED, "fmt %d", (int)fmt);
    if (x_dtype != CSA2_F32 && x_dtype != CSA2_BF16) return fail(CSA2_E_UNSUPPORTED, "x_dtype %d", (int)x_dtype);
    if (nblocks < 0) return fail(CSA2_E_ARG, "nblocks < 0");
    if (nblocks > 0 && (!x || !codes || !scales)) return fail(CSA2_E_ARG, "x / codes / scales is NULL");
    if (misaligned(x, 16) || misaligned(codes, 16)) return fail(CSA2_E_ARG, "x / codes must start on a 16-byte boundary");
    if (nblocks == 0) return ok();
    int rc;
    if ((rc = check_device())) return rc;
    const bool bf16_in = x_dtype == CSA2_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == CSA2_FP4_S16)
        return launch_result(csa2::launch_quant_fp4s16(bf16_in, x, nblocks, codes, scales, s), "csa2_quant_mx");
    return launch_result(csa2::launch_quant_mx(fmt == CSA2_MXFP4, bf16_in, x, nblocks, codes, scales, s),
                         "csa2_quant_mx");
}


int csa2_check_inputs(const csa2_rows* rows, const csa2_cache* cache, const csa2_pool* pool, int32_t pool_rows,
                      const int32_t* sel, int32_t k, int64_t sel_stride, const int32_t* sel_row_map,
                      int32_t sel_rows, uint32_t* error_word, void* stream)
{
    int rc;
    if ((rc = check_rows(rows)) || (rc = check_cache(cache))) return rc;
    if (!error_word) return fail(CSA2_E_ARG, "error_word is NULL");
    if (misaligned(error_word, 4)) return fail(CSA2_E_ARG, "error_word must start on a 4-byte boundary");
    if (pool) {
        if ((rc = check_pool(pool, (int64_t)pool->block * pool->max_blocks))) return rc;
        if (pool_rows < 1) return fail(CSA2_E_ARG, "pool_rows = %d < 1", pool_rows);
    }
    if (sel) {
        if (k < 0) return fail(CSA2_E_ARG, "k = %d < 0", k);
        if (sel_stride < k) return fail(CSA2_E_ARG, "sel_stride %lld < k %d", (long long)sel_stride, k);
        if (sel_row_map && sel_rows < 1) return fail(CSA2_E_ARG, "sel_rows = %d < 1", sel_rows);
    } else if (sel_row_map) {
        return fail(CSA2_E_ARG, "sel_row_map without sel");
    }
    if ((rc = check_device())) return rc;
    return launch_result(csa2::launch_check_inputs(rows_arg(rows), cache->nreq, cache_arg(cache), pool_arg(pool),
                                                   pool ? pool_rows : 0, sel, sel ? k : 0, sel_stride, sel_row_map,
                                                   sel_row_map ? sel_rows : rows->n, error_word,
                                                   static_cast<hipStream_t>(stream)),
                         "csa2_check_inputs");
}

}  // extern "C"
