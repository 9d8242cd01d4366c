/*
 * csa2.h -- C ABI of the CSA2 compressed-sparse-attention hot path on MI355X (gfx950).
 *
 * The path (one layer of DeepSeek V4.1 Flash's "Compressed Sparse Attention 2"):
 *   1. csa2_index_score      MQA-style index scores over FP4 (MXFP4) index keys
 *   2. csa2_topk             top-k per query (flat, or restricted to a candidate pool)
 *   3. csa2_topk_hier        flat top-k plus the hierarchical candidate pool
 *   4. csa2_sparse_swa_attn  attention over the selected compressed entries and the
 *                            query's own sliding window, one joint softmax
 *   5. csa2_replay_tail_layout  per-request tail rows of the decoder bounded replay
 *      csa2_encoder_replay_layout  rows of an extend under the encoder-side replay
 *   0. csa2_kv_produce      the step before: pooled main KV and index keys into the caches
 *
 * Pages (cited by title and section):
 *   [MOD]  "DeepSeek V4.1 Flash modeling" (pages.haorui.li): sections "CSA2",
 *          "Hierarchical Sparse Indexer", "Decoder Bounded Replay", "Mixed precision".
 *   [TAIL] "SGLang: how DeepSeek V4.1 Flash late layers only process tail tokens"
 *          (lab.ttaoai.cn): sections 2.1, 2.2, 2.3, 2.6, 3.1.
 *   [DAY0] "SGLang and Miles Day-0 support for DeepSeek-V4.1" (theainews.cc summary of
 *          the LMSYS post): sections 1, 2, 4.2, 5.
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or retains memory; scratch space comes in through `workspace`
 *     (size from csa2_workspace_size).  Structs are passed by host pointer and read
 *     during the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call validates its
 *     scalar arguments on the host, enqueues kernels on `stream` and returns without
 *     synchronizing.  Inputs must stay valid until the stream reaches the work.
 *   - Return value: CSA2_OK, or an error code; nothing is enqueued when the error is
 *     detected before launch (every CSA2_E_ARG / CSA2_E_UNSUPPORTED / CSA2_E_WORKSPACE).
 *     csa2_last_error() gives a message for the calling thread.
 *   - Device-array contents (positions, lengths, indices) are preconditions stated per
 *     call; the calls do not check them.  csa2_check_inputs checks the row, cache, pool
 *     and index-set ones on the device into an error word, for debugging callers.
 *   - Element arrays move in 16-byte vectors and must start on a 16-byte boundary (every
 *     hipMalloc / torch allocation does): q_idx and keys->data of csa2_index_score (MXFP4);
 *     q, kv, kv_scale, out, swa->data and swa->scale of csa2_sparse_swa_attn (BF16); x and
 *     codes of csa2_quant_mx; keys->scale of csa2_index_topk_pool moves in 4-byte words and
 *     must start on a 4-byte boundary.  A misaligned pointer is CSA2_E_ARG.  Row pitches follow from
 *     the shapes (64 + 4 bytes per MXFP4 key, 1 KiB per bf16 KV row, 256 + 32 bytes per
 *     FP4_S16 KV row), so aligned bases keep every row aligned.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs, and a
 *     row's outputs do not depend on the other rows of the batch.
 *   - Calls are reentrant.  The only state kept between calls is a per-device flag,
 *     filled on a device's first call, that records whether it is a gfx950 (guarded by
 *     a mutex); nothing else persists.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_VERSION 4

enum {
    CSA2_OK = 0,
    CSA2_E_ARG = 1,         /* null pointer, count/stride/size out of range */
    CSA2_E_UNSUPPORTED = 2, /* dtype / dim / head-count combination, or device is not gfx950 */
    CSA2_E_WORKSPACE = 3,   /* workspace missing or smaller than csa2_workspace_size */
    CSA2_E_LAUNCH = 4       /* a HIP launch or runtime call failed */
};

typedef enum csa2_dtype {
    CSA2_F32 = 0,        /* IEEE binary32 */
    CSA2_BF16 = 1,       /* bfloat16 */
    CSA2_MXFP4 = 2,      /* OCP MX: E2M1 codes, two per byte (element 2i in the low nibble),
                            one E8M0 scale byte per 32 elements in a separate plane */
    CSA2_MXFP8_E4M3 = 3, /* OCP MX: E4M3 ("fn") codes, one per byte, one E8M0 scale per 32 */
    CSA2_FP4_S16 = 4     /* main KV storage format ([MOD] "Mixed precision"): E2M1 codes, two per
                            byte (element 2i in the low nibble), one E4M3 ("fn") scale byte per
                            16 elements in a separate plane, no tensor-wide scale; a 512-d entry
                            is 256 + 32 = 288 bytes */
} csa2_dtype;

/* Query rows of one call.  Row q belongs to request req_of_row[q] and sits at
 * absolute token position pos_of_row[q] (0-based; the original position is kept
 * for replayed tail rows, [TAIL] section 2.2).  win_lo[q] is the lowest absolute
 * position the row's sliding window may read (the replay lower bound of [TAIL]
 * section 2.3); NULL means 0. */
typedef struct csa2_rows {
    int32_t n;
    const int32_t* req_of_row; /* [n] */
    const int32_t* pos_of_row; /* [n] */
    const int32_t* win_lo;     /* [n] or NULL */
} csa2_rows;

/* Geometry of a KV owner's compressed cache ([MOD] "CSA2": non-overlapping groups of
 * ratio_m tokens; only complete groups are entries).  Entry j of request r covers
 * tokens [j*m, j*m+m-1] and is visible to the query at position p iff j*m+m-1 <= p,
 * so R(q) = min(floor((p+1)/m), n_entries[r]) entries are reachable.  Entry j of
 * request r lives in row row_start[r] + j of every per-entry buffer of the owner
 * (index keys and main KV share the row numbering). */
typedef struct csa2_cache {
    int32_t nreq;
    int32_t ratio_m;          /* 1 or 2 */
    const int32_t* n_entries; /* [nreq] complete entries C_r */
    const int64_t* row_start; /* [nreq] */
} csa2_cache;

/* Index keys of the owner ([MOD] "Mixed precision": MXFP4 with 32-element groups, 68 B
 * per 128-d entry = 64 B codes + 4 B scales, stored as two planes). */
typedef struct csa2_index_keys {
    csa2_dtype dtype;     /* CSA2_MXFP4 (dim 128) or CSA2_F32 (dim 1..1024) */
    int32_t dim;
    const void* data;     /* MXFP4: uint8[rows][dim/2]; F32: float[rows][dim] */
    const uint8_t* scale; /* MXFP4: uint8[rows][dim/32] E8M0; F32: NULL */
} csa2_index_keys;

/* Candidate pool of the hierarchical indexer ([MOD] "Hierarchical Sparse Indexer";
 * [DAY0] section 2): per pool row, nblocks[r] ascending block ids in blocks[r][0..);
 * block b holds positions [b*block, b*block+block), block a power of two.  A query row q uses pool row
 * row_map[q] (NULL = q). */
typedef struct csa2_pool {
    int32_t block;          /* positions per block, 8 on the pages (power of two, 1..64) */
    int32_t max_blocks;     /* row stride of `blocks`, 2048 on the pages */
    const int32_t* blocks;  /* [pool_rows][max_blocks] */
    const int32_t* nblocks; /* [pool_rows], each <= max_blocks */
    const int32_t* row_map; /* [n] or NULL */
} csa2_pool;

/* Sliding-window KV of one layer ([DAY0] section 1: every layer keeps its own FP8
 * window of the last 128 positions; [MOD] "Mixed precision").  Position t of request
 * r is row row_start[r] + (t - pos_start[r]); the buffer must hold every position
 * the windows read: [max(win_lo, p - window + 1, pos_start[r]), p]. */
typedef struct csa2_swa {
    csa2_dtype dtype;         /* CSA2_MXFP8_E4M3, CSA2_BF16 or CSA2_F32 */
    const void* data;         /* [rows][dim] */
    const uint8_t* scale;     /* MXFP8: uint8[rows][dim/32] E8M0; otherwise NULL */
    const int64_t* row_start; /* [nreq] */
    const int32_t* pos_start; /* [nreq] */
    int32_t window;           /* W (128 on the pages): the window of p is [p-W+1, p] */
} csa2_swa;

/* ---------------------------------------------------------------------------------
 * csa2_index_score -- indexer scores over every reachable compressed position, or over
 * a candidate pool.
 *
 * Defines ([DAY0] section 5: the indexer scores the FP4 cache directly, heads
 * replicated; the formula is the workload definition's ReLU-weighted MQA form):
 *     s_j = sum_h w_h * ReLU(q_h . k_j)
 * With MXFP4 keys the BF16 index q is first quantized to MXFP4 (32-element blocks,
 * OCP MX rule; [MOD] "Mixed precision": index Q/K are MXFP4), so every q_h . k_j is an
 * exact product sum; the head sum is taken in fp32 in a fixed order: 4 contiguous
 * head groups, P_g = fma(w_h, max(d_h,0), P_g) over the group in ascending h from +0,
 * s = (P_0 + P_1) + (P_2 + P_3).
 *
 * q_idx   [n][heads][keys->dim]: BF16 or MXFP4 for MXFP4 keys, F32 for F32 keys (q_dtype
 *         says which).  MXFP4 q is the quantized BF16 q as csa2_quant_mx (MXFP4) writes it
 *         for the [n * heads * dim / 32] blocks: q_idx the E2M1 codes [n][heads][dim / 2]
 *         (element 2i in the low nibble), q_scale the E8M0 bytes [n][heads][dim / 32]; the
 *         scores are then exactly those of the BF16 q it came from (the same quantization
 *         happens in-kernel for BF16 q).  q_scale is NULL for the other dtypes.
 * heads   MXFP4: a multiple of 16, at most 128; F32: a multiple of 4, at most 128.
 * w       float [n][heads] with row stride w_row_stride (0: one row shared by all).
 * pool    NULL: column j of row q is compressed position j; every column j < score_stride
 *         is written, the score for j < R(q) and -inf from R(q) on.  Non-NULL: column c
 *         is position blocks[c/block]*block + c%block of the row's pool; the columns
 *         c < block*max_blocks are written, -inf where the position is not reachable and
 *         from block*nblocks on; requires block*max_blocks <= score_stride, and the
 *         columns from block*max_blocks to score_stride are row padding, not written.
 * scores  float [n][score_stride].
 * Errors: E_ARG (null pointers, n < 0, bad strides), E_UNSUPPORTED (dtype/dim/heads).
 * ------------------------------------------------------------------------------- */
int csa2_index_score(const csa2_rows* rows, const csa2_cache* cache, const void* q_idx, csa2_dtype q_dtype,
                     const uint8_t* q_scale, int32_t heads, const float* w, int64_t w_row_stride,
                     const csa2_index_keys* keys, const csa2_pool* pool, float* scores, int64_t score_stride,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_topk -- the k best candidates of every row ([MOD] "Hierarchical Sparse Indexer":
 * top-512 per query; [DAY0] section 1: at most 512 positions).
 *
 * Candidates: positions j < min(R(q), score_stride) (pool == NULL), or the reachable
 * positions of the row's pool (pool != NULL, columns as in csa2_index_score).
 * Order: larger score first (-0 equals +0), then lower position; the first k are kept.
 * Scores must not be NaN.  out_idx [n][k]: the kept absolute compressed positions in
 * ascending order, then -1 padding (fewer than k candidates keeps them all).
 * k: 1..2048.  workspace: csa2_workspace_size(CSA2_OP_TOPK, ...).
 * ------------------------------------------------------------------------------- */
int csa2_topk(const csa2_rows* rows, const csa2_cache* cache, const float* scores, int64_t score_stride,
              const csa2_pool* pool, int32_t k, int32_t* out_idx, void* workspace, size_t workspace_bytes,
              void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_index_topk_pool -- csa2_index_score over a candidate pool and csa2_topk over its
 * scores in one call, with no score written to memory ([MOD] "Hierarchical Sparse
 * Indexer": Reindex layers rescore only the shared pool and select inside it; the
 * section's measurement notes name the fused module of restricted scoring and selection).
 * out_idx [n][k] is exactly what csa2_index_score (pool) followed by csa2_topk (pool) give:
 * the k best pool positions below the row's reach, ascending, -1 padded (ties to the lower
 * position).  Supported: MXFP4 keys of dim 128, BF16 or MXFP4 index q (q_idx / q_scale as
 * for csa2_index_score), heads 16 / 32 / 64, pool
 * block 8 with max_blocks <= 2048 (the pages' 16,384-position pool), k 1..2048.
 * Calls over 128 rows or more score and select each row's whole pool in one workgroup
 * and need no workspace.  Fewer rows (a decode batch) split each pool into segments of
 * 4096 columns, spread over the CUs; pools of more than one segment then need workspace
 * (csa2_workspace_size(CSA2_OP_TOPK_POOL_FUSED, n, block * max_blocks, k, 0): each
 * segment's top-k as (key, position) lists, merged exactly by a second launch).
 * ------------------------------------------------------------------------------- */
int csa2_index_topk_pool(const csa2_rows* rows, const csa2_cache* cache, const void* q_idx, csa2_dtype q_dtype,
                         const uint8_t* q_scale, int32_t heads, const float* w, int64_t w_row_stride,
                         const csa2_index_keys* keys, const csa2_pool* pool, int32_t k, int32_t* out_idx,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_topk_hier -- the source pass of the hierarchical indexer ([MOD] "Hierarchical
 * Sparse Indexer"; [DAY0] section 2, "two-level selection"): the flat top-k over all
 * reachable positions (as csa2_topk without a pool) AND the candidate pool: blocks
 * [b*block, b*block+block) are scored by the maximum over their reachable members;
 * when ceil(R/block) <= max_blocks every block is kept, otherwise the block holding
 * the newest reachable position plus the max_blocks-1 best other blocks by (block
 * score desc, block id asc).  out_pool_blocks [n][max_blocks] ascending ids, -1 padded;
 * out_pool_nblocks [n].  block 8 (the pages' block; other sizes are CSA2_E_UNSUPPORTED),
 * max_blocks 1..4096, k 1..2048.
 * ------------------------------------------------------------------------------- */
int csa2_topk_hier(const csa2_rows* rows, const csa2_cache* cache, const float* scores, int64_t score_stride,
                   int32_t k, int32_t block, int32_t max_blocks, int32_t* out_idx, int32_t* out_pool_blocks,
                   int32_t* out_pool_nblocks, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_topk_hier_noalloc -- csa2_topk_hier for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same selection, the same outputs, with its scratch taken from a library-owned
 * 32 MiB array per device instead of a caller workspace.  Arguments as csa2_topk_hier.
 *   - Allocates nothing: no hipMalloc / hipFree; the array is static device memory that
 *     each device holds until the process ends; its address is looked up once per
 *     device (the first call on it).
 *   - Sizes whose scratch exceeds 32 MiB (csa2_workspace_size(CSA2_OP_TOPK_HIER, ...) >
 *     33554432, e.g. more than about 1,000 rows of 65,536 columns) are refused with
 *     CSA2_E_WORKSPACE before anything is enqueued.
 *   - Every call on one device shares that device's array: calls that may overlap on one
 *     device (different streams, or different host threads) race and must be ordered by
 *     the caller.  Nothing in the array needs to start at zero; each call writes what it
 *     reads.
 * ------------------------------------------------------------------------------- */
int csa2_topk_hier_noalloc(const csa2_rows* rows, const csa2_cache* cache, const float* scores,
                           int64_t score_stride, int32_t k, int32_t block, int32_t max_blocks, int32_t* out_idx,
                           int32_t* out_pool_blocks, int32_t* out_pool_nblocks, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_sparse_swa_attn -- each query row attends, per head, to its selected compressed
 * entries together with its own sliding window, in one softmax ([DAY0] section 1;
 * [MOD] "CSA2": Full, Reindex and Reuse layers all keep their own attention; Reuse
 * passes the latest top-k of its KV group as sel_idx).
 *
 * Keys = values: the main entry is one shared 512-d latent ([MOD] "Mixed precision").
 * For row q at position p of request r, head h:
 *   set  = { kv[row_start[r] + j] : j = sel_idx[s][i] >= 0 }   (s = sel_row_map ? sel_row_map[q] : q)
 *        U { window row of t : max(win_lo[q], p - W + 1, pos_start[r]) <= t <= p }
 *   out  = sum_x softmax_x(sm_scale * q_h . x) * x; the optional sink adds exp(sink_h - max)
 *          to the denominator only; lse = max + log(denominator) (natural log).
 * Selected indices must be < R(q) (or -1); k = 0 gives window-only attention.
 *
 * q [n][heads][dim] and out [n][heads][dim]; lse float [n][heads] or NULL.
 * kv: F32 / BF16 [rows][dim] (kv_scale NULL), or CSA2_FP4_S16 codes uint8 [rows][dim/2]
 * with kv_scale uint8 [rows][dim/16] E4M3 ([MOD] "Mixed precision": the main KV is stored
 * in 4 bits and dequantized before attention; each element is its E2M1 value times its
 * block's scale, exact in bf16, so the result is attention over the decoded values).
 * Scale bytes must be finite E4M3 codes (not 0x7F / 0xFF), as csa2_quant_mx writes them.
 * Supported: (q, kv, window, out) = (F32, F32, F32, F32) with dim <= 256 and any heads;
 *            (BF16, BF16 or FP4_S16, MXFP8_E4M3 or BF16, BF16) with dim = 512 and
 *            heads % 16 == 0.
 * sel_idx [*][sel_stride] int32, k <= sel_stride, k 0..2048.
 * ------------------------------------------------------------------------------- */
int csa2_sparse_swa_attn(const csa2_rows* rows, const csa2_cache* cache, const void* q, csa2_dtype q_dtype,
                         int32_t heads, int32_t dim, const void* kv, csa2_dtype kv_dtype, const uint8_t* kv_scale,
                         const int32_t* sel_idx, int32_t k, int64_t sel_stride, const int32_t* sel_row_map, const csa2_swa* swa,
                         float sm_scale, const float* sink, void* out, csa2_dtype out_dtype, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_replay_tail_layout -- per-request tail rows of the decoder bounded replay
 * ([TAIL] sections 2.1-2.3 and the rule block after the window table; [DAY0] 4.2).
 * For request r with extend length E = ext_len[r] and total length S = seq_len[r]:
 *   T = min(budget, E); the late layers process absolute positions [S - T, S);
 *   the window lower bound of those rows is S - T (also for E < budget, [TAIL] 2.6);
 *   tail row u of r is row ext_start(r) + E - T + u of the original extend, where
 *   ext_start(r) = sum of ext_len over the requests before r.
 * Mixed batches ([MOD] "Decoder Bounded Replay": the new tokens of decode requests still
 * pass through the whole trunk): is_decode[r] != 0 marks a decode request, whose E rows
 * (E <= budget) are all kept, with window lower bound 0.  is_decode NULL = all prefill.
 * flags: CSA2_TAIL_BORROW_PREFIX_WINDOW sets the lower bound of prefill requests to
 * max(0, S - budget), so a short extend sees the cached prefix's window (a reading of
 * the proposal discussed in [TAIL] 2.6; off reproduces the page's pinned behaviour).
 * Outputs: tail_len [nreq]; tail_row_start [nreq+1] (exclusive prefix sum of tail_len);
 * per tail row (at most capacity): src_row, abs_pos, win_lo, req_of_row.
 * Precondition 0 <= E <= S.  capacity >= budget*nreq (host-checked), budget >= 1.
 * ------------------------------------------------------------------------------- */
enum { CSA2_TAIL_BORROW_PREFIX_WINDOW = 1 };

int csa2_replay_tail_layout(int32_t nreq, const int32_t* ext_len, const int32_t* seq_len, const int32_t* is_decode,
                            int32_t budget, int32_t flags, int32_t* tail_len, int32_t* tail_row_start,
                            int32_t* src_row, int32_t* abs_pos, int32_t* win_lo, int32_t* req_of_row,
                            int32_t capacity, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_encoder_replay_layout -- rows of an extend batch under encoder-side bounded replay
 * ([DAY0] section 4.1: on a prefix-cache hit the last 128 tokens of the cached prefix
 * are recomputed to rebuild the window, the cached compressed KV and indexer keys stay;
 * section 4.3: local attention is cut at the rebuild boundary).
 * Request r has P = prefix_len[r] cached tokens and E = ext_len[r] new ones.  Its rows
 * are the absolute positions [R0, P + E) with R0 = max(0, P - budget): first the
 * min(P, budget) replayed prefix positions, then the extend.  Every row's window lower
 * bound is R0.  src_row is the extend input row (ext_start(r) + t - P) of an extend row
 * and -1 for a replayed prefix row.  row_start [nreq+1] is the exclusive prefix sum of
 * the per-request row counts min(P, budget) + E.
 * n_ext = sum of ext_len (a precondition); capacity >= budget*nreq + n_ext (host-checked).
 * ------------------------------------------------------------------------------- */
int csa2_encoder_replay_layout(int32_t nreq, const int32_t* prefix_len, const int32_t* ext_len, int64_t n_ext,
                               int32_t budget, int32_t* row_start, int32_t* src_row, int32_t* abs_pos,
                               int32_t* win_lo, int32_t* req_of_row, int32_t capacity, void* stream);

/* ---------------------------------------------------------------------------------
 * csa2_kv_produce -- the index-K / main-KV producer that fills the caches the path reads
 * ([MOD] "CSA2": non-overlapping compression, the index key projected from the
 * compressed main KV; [MOD] "Mixed precision": main KV quantized after RoPE; [DAY0]
 * section 1: pairwise compression keeps incomplete pairs across decode steps; section 5:
 * BF16 weights with FP32 accumulation, ratio-2 pooling of each completed pair, RoPE, FP4
 * quantization and cache write fused with the intermediate rounding kept).
 *
 * rows: the call's token rows (win_lo unused); rows of one request are consecutive and
 * at ascending consecutive positions.  comp float [n][512]: the compressor's fp32 output
 * of each token.  Row t at position p closes entry j = (p + 1) / m - 1 when (p + 1) % m
 * == 0 (m = cache->ratio_m, 1 or 2); that entry, at row cache->row_start[r] + j of every
 * cache buffer, is
 *   latent = comp[t] (m = 1), or (first + comp[t]) * 0.5 in fp32 (m = 2), where first is
 *            the previous row of the call when it holds position p - 1, else pending[r]
 *   main   = latent with dims [448, 512) rotated (RoPE) at position P = j m + m - 1, in
 *            interleaved pairs (2i, 2i+1): x' = x c - y s, y' = x s + y c, each product
 *            and sum rounded to fp32, c = rope[P][0][i], s = rope[P][1][i]; stored to kv
 *            as bf16 (nearest even) [rows][512], or as FP4_S16 codes [rows][256] with
 *            kv_scale [rows][32]
 *   index  = k_o = sum_i w_index[o][i] * bf16(latent_i) (fp32, one fma per term in
 *            ascending i), dims [64, 128) rotated the same way, then MXFP4 into
 *            index_codes [rows][64] and index_scales [rows][4] (csa2_quant_mx's rule).
 * pending float [nreq][512] (m = 2; may be NULL for m = 1): a request whose rows in the
 * call end at an even position leaves that token's comp row there; entries read pending
 * as it was before the call.  Rows that close no entry write no cache row.
 * w_index bf16 [128][512]; rope float [max_pos][2][32]; entries with P >= max_pos are
 * not written (a precondition violation).  Buffers: comp, pending, w_index, kv and
 * index_codes start on a 16-byte boundary.
 * ------------------------------------------------------------------------------- */
int csa2_kv_produce(const csa2_rows* rows, const csa2_cache* cache, const float* comp, float* pending,
                    const uint16_t* w_index, const float* rope, int64_t max_pos, csa2_dtype kv_dtype, void* kv,
                    uint8_t* kv_scale, uint8_t* index_codes, uint8_t* index_scales, void* stream);

/* ---------------------------------------------------------------------------------
 * Helpers.
 * ------------------------------------------------------------------------------- */
enum { CSA2_OP_TOPK = 1, CSA2_OP_TOPK_HIER = 2, CSA2_OP_ATTN = 3, CSA2_OP_TOPK_POOL_FUSED = 4 };

/* Workspace bytes for an op: n rows, `cols` = score_stride (TOPK / TOPK_HIER), the pool's
 * block * max_blocks (TOPK_POOL_FUSED) or the number of selected entries k (ATTN), k,
 * max_blocks (TOPK_HIER). */
size_t csa2_workspace_size(int op, int32_t n, int64_t cols, int32_t k, int32_t max_blocks);

/* ---------------------------------------------------------------------------------
 * csa2_check_inputs -- debug check of the device-array preconditions the calls above
 * state, for callers that want them verified (the calls themselves assume them): on
 * `stream`, *error_word (a device uint32, 4-byte aligned) is cleared, then every
 * violation found ORs its bit in.  Nothing else is written.  The caller reads the word
 * after the stream reaches the check; 0 means every checked precondition holds.
 *   rows, cache: required.  CSA2_BAD_REQ: req_of_row outside [0, nreq);
 *     CSA2_BAD_POS: pos_of_row < 0; CSA2_BAD_WIN_LO: win_lo < 0 or > pos_of_row;
 *     CSA2_BAD_CACHE: n_entries < 0 or row_start < 0 (every request).
 *   pool (or NULL) with pool_rows rows of blocks / nblocks: CSA2_BAD_POOL_MAP: a row's
 *     pool row (row_map, else the row itself) outside [0, pool_rows); CSA2_BAD_POOL:
 *     nblocks outside [0, max_blocks], or a pool row's block ids not strictly ascending,
 *     negative, or so large that a position of the block overflows int32.
 *   sel (or NULL) [sel_rows][sel_stride], k per row, read through sel_row_map (or NULL:
 *     row q reads sel row q): CSA2_BAD_SEL_MAP: a mapped row outside [0, sel_rows);
 *     CSA2_BAD_SEL: an index neither -1 nor in [0, R(q)).
 * Only the pool and index rows that some query row reads are checked; a row whose
 * request or position is invalid has no reach, so its pool and index rows are skipped.
 * Two launches (clear, check); the check reads each checked array once.
 * ------------------------------------------------------------------------------- */
enum {
    CSA2_BAD_REQ = 1, CSA2_BAD_POS = 2, CSA2_BAD_WIN_LO = 4, CSA2_BAD_CACHE = 8,
    CSA2_BAD_POOL_MAP = 16, CSA2_BAD_POOL = 32, CSA2_BAD_SEL_MAP = 64, CSA2_BAD_SEL = 128
};
int csa2_check_inputs(const csa2_rows* rows, const csa2_cache* cache, const csa2_pool* pool, int32_t pool_rows,
                      const int32_t* sel, int32_t k, int64_t sel_stride, const int32_t* sel_row_map,
                      int32_t sel_rows, uint32_t* error_word, void* stream);

/* Message of the calling thread's last error ("" after success). */
const char* csa2_last_error(void);

int csa2_version(void);

/* Block quantization of x (F32 or BF16, contiguous), nblocks blocks, into codes and one
 * scale byte per block.  Inputs must be finite.
 *   fmt CSA2_MXFP4 / CSA2_MXFP8_E4M3 (OCP MX): 32-element blocks, codes 16 / 32 B per
 *     block, E8M0 scale = shared exponent floor(log2(max|x|)) - emax (emax 2 for E2M1, 8
 *     for E4M3; -127 for an all-zero block), elements rounded to nearest even and
 *     saturated, the sign bit copied from x.  This is the quantizer csa2_index_score
 *     applies to the BF16 index q; it also prepares index keys and window KV.
 *   fmt CSA2_FP4_S16 (the main KV format, [MOD] "Mixed precision"; applied after RoPE):
 *     16-element blocks, codes 8 B per block, E4M3 scale s = max|x| / 6 rounded to the
 *     nearest E4M3 value (ties to even, saturating at 448); element = |x| / s rounded to
 *     the nearest E2M1 value (ties to even, saturating at 6) with x's sign bit; a block
 *     whose s rounds to 0 stores zero magnitudes.  (The pages fix the format, not its
 *     rounding; this is the NVFP4 rule without the tensor-wide scale.) */
int csa2_quant_mx(csa2_dtype fmt, const void* x, csa2_dtype x_dtype, int64_t nblocks, uint8_t* codes,
                  uint8_t* scales, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
