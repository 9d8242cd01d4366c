// Internal launchers of the CSA2 kernels (host side).  The C ABI in csa2_api.cpp
// validates arguments and calls these; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Row / cache / pool descriptors flattened for kernel arguments.
struct RowsArg {
    int n;
    const int32_t* req;
    const int32_t* pos;
    const int32_t* win_lo;  // may be null
};

struct CacheArg {
    int ratio_m;
    const int32_t* n_entries;
    const int64_t* row_start;
    int nreq;  // entries of n_entries / row_start
};

struct PoolArg {
    const int32_t* blocks;   // null: full range
    const int32_t* nblocks;
    const int32_t* row_map;  // may be null
    int block;
    int max_blocks;
};

hipError_t launch_replay_tail_layout(int nreq, const int32_t* ext_len, const int32_t* seq_len,
                                     const int32_t* is_decode, int budget, int flags, int32_t* tail_len,
                                     int32_t* tail_row_start, int32_t* src_row, int32_t* abs_pos, int32_t* win_lo,
                                     int32_t* req_of_row, hipStream_t stream);
hipError_t launch_encoder_replay_layout(int nreq, const int32_t* prefix_len, const int32_t* ext_len, int budget,
                                        int32_t* row_start, int32_t* src_row, int32_t* abs_pos, int32_t* win_lo,
                                        int32_t* req_of_row, hipStream_t stream);

hipError_t launch_quant_mx(bool fp4, bool bf16_in, const void* x, int64_t nblocks, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);
// Main KV storage format: 16-element blocks, E2M1 codes + one E4M3 scale per block.
hipError_t launch_quant_fp4s16(bool bf16_in, const void* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream);

// Index q of the MXFP4 scoring kernels: bf16 [n][heads][128] (quantized in-kernel), or with
// q_scale non-null its MXFP4 codes [n][heads][64 B] and E8M0 scales [n][heads][4].
struct IndexQ {
    const void* q;
    const uint8_t* q_scale;
};

// Index scores.  MXFP4 path: q as above; F32 path: q, keys fp32.
hipError_t launch_index_score_mxfp4(const RowsArg& rows, const CacheArg& cache, const IndexQ& q, int heads,
                                    const float* w, int64_t w_stride, const uint8_t* kdata, const uint8_t* kscale,
                                    const PoolArg& pool, float* scores, int64_t stride, hipStream_t stream);
hipError_t launch_index_score_f32(const RowsArg& rows, const CacheArg& cache, const float* q, int heads, int dim,
                                  const float* w, int64_t w_stride, const float* keys, const PoolArg& pool,
                                  float* scores, int64_t stride, hipStream_t stream);

// Selection.  Source of the candidate rows of a top-k.
struct SelSource {
    const float* scores;
    int64_t stride;
    RowsArg rows;
    CacheArg cache;
    PoolArg pool;  // pool.blocks non-null: candidates are the row's pool columns
};

size_t topk_workspace(int n, int64_t stride, int k, bool pool);

// Exact merge of nlists (key, position) lists of k per row into the row's top-k indices.
hipError_t launch_list_merge(const SelSource& src, int k, int nlists, const uint2* lists, int32_t* out,
                             hipStream_t stream);

// Fused pool scoring + top-k (block 8, at most 2048 blocks; heads 16, 32 or 64); pools
// of more than 4096 columns need the segment lists' workspace.
size_t score_topk_pool_workspace(int n, int64_t cols, int k);
hipError_t launch_score_topk_pool(const RowsArg& rows, const CacheArg& cache, const IndexQ& q, int heads,
                                  const float* w, int64_t w_stride, const uint8_t* kdata, const uint8_t* kscale,
                                  const PoolArg& pool, int k, int32_t* out_idx, void* ws, hipStream_t stream);
hipError_t launch_topk(const SelSource& src, int k, int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

size_t topk_hier_workspace(int n, int64_t stride, int k, int block, int max_blocks);
hipError_t launch_topk_hier(const SelSource& src, int k, int block, int max_blocks, int32_t* out_idx,
                            int32_t* out_blocks, int32_t* out_nblocks, void* ws, size_t ws_bytes,
                            hipStream_t stream);

// Attention.
struct SwaArg {
    int dtype;  // 0 f32, 1 bf16, 3 mxfp8
    const void* data;
    const uint8_t* scale;
    const int64_t* row_start;
    const int32_t* pos_start;
    int window;
};

hipError_t launch_attn_f32(const RowsArg& rows, const CacheArg& cache, const float* q, int heads, int dim,
                           const float* kv, const int32_t* sel, int k, int64_t sel_stride, const int32_t* sel_row_map,
                           const SwaArg& swa, float sm_scale, const float* sink, float* out, float* lse,
                           hipStream_t stream);
// kv: bf16 [rows][512] (kv_scale null) or FP4_S16 codes [rows][256] with E4M3 scales [rows][32].
hipError_t launch_attn_bf16(const RowsArg& rows, const CacheArg& cache, const uint16_t* q, int heads,
                            const void* kv, const uint8_t* kv_scale, const int32_t* sel, int k, int64_t sel_stride,
                            const int32_t* sel_row_map, const SwaArg& swa, float sm_scale, const float* sink,
                            uint16_t* out, float* lse, hipStream_t stream);

// Index-K / main-KV producer (m = 1 or 2; main KV bf16 or FP4_S16).
hipError_t launch_kv_produce(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m,
                             const int64_t* row_start, const float* comp, float* pending, const uint16_t* w_index,
                             const float* rope, int64_t max_pos, bool fp4_kv, void* kv, uint8_t* kv_scale,
                             uint8_t* idx_codes, uint8_t* idx_scales, hipStream_t stream);

// Debug check of device-array preconditions into an error word (cleared first).
hipError_t launch_check_inputs(const RowsArg& rows, int nreq, const CacheArg& cache, const PoolArg& pool,
                               int pool_rows, const int32_t* sel, int k, int64_t sel_stride,
                               const int32_t* sel_row_map, int sel_rows, uint32_t* word, hipStream_t stream);

}  // namespace csa2
