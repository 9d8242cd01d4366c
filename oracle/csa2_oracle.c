/*
 * csa2_oracle.c -- plain, slow CPU oracle for the CSA2 sparse-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * cpu_baseline leg may load this code.  It shares no code, header, table or
 * helper with the HIP library; it has its own codecs.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "DeepSeek V4.1 Flash modeling" (pages.haorui.li), sections "CSA2",
 *       "Hierarchical Sparse Indexer", "Decoder Bounded Replay", "Mixed precision".
 *  [P2] "SGLang: how DeepSeek V4.1 Flash late layers only process tail tokens"
 *       (lab.ttaoai.cn), sections 2.1 (tail rule), 2.3 (window), 2.6 (short extend),
 *       3.1 (token x layer counts).
 *  [P4] "SGLang and Miles Day-0 support for DeepSeek-V4.1" (theainews.cc summary of the
 *       LMSYS post), sections 1 (architecture), 2 (sharing and retrieval), 5 (kernels).
 *  The indexer score formula sum_h w_h * ReLU(q_h . k) and the lowest-index tie break
 *  are not on the pages; they come from the workload definition that accompanies them.
 *  OCP Microscaling Formats (MX) v1.0 defines E2M1, E4M3, E8M0 and block scaling.
 *
 * Precision: attention is computed in double from dequantized inputs.  The index
 * score decides an integer result (the top-k set), so it is computed in the fp32
 * canonical order that the GPU kernel also follows (see orc_canon_reduce).
 *
 * Built with -O2 -ffp-contract=off: no implicit fused multiply-add anywhere;
 * fmaf() appears only where the canonical order says fma.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

#define ORC_E2M1 0
#define ORC_E4M3 1

/* Host threads of the OpenMP loops (timing the oracle at a stated thread count). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------- */
/* Element formats (OCP MX v1.0).                                             */
/* ------------------------------------------------------------------------- */

/* E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
 * subnormal (value = mantissa * 0.5).  No inf, no NaN. */
double orc_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m * 0.5, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (the OCP "fn" variant): bias 7, exponent field 0 subnormal
 * (mantissa/8 * 2^-6), S.1111.111 is NaN, no infinities. */
double orc_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0 scale byte b encodes 2^(b-127); 0xFF is NaN (never produced here). */
double orc_e8m0_value(int b) { return b == 255 ? NAN : ldexp(1.0, b - 127); }

/* Round a non-negative finite y to the nearest value of a small binary float
 * format (mbits mantissa bits, unbiased minimum normal exponent emin), ties to
 * even, then saturate at maxval.  Textbook RNE: the quantum of y's binade (or
 * of the subnormal range) is 2^(E-mbits); rint() rounds half to even. */
static double round_to_format(double y, int mbits, int emin, double maxval)
{
    if (y == 0.0) return 0.0;
    int E;
    frexp(y, &E);
    E -= 1;                       /* y in [2^E, 2^(E+1)) */
    if (E < emin) E = emin;       /* subnormals share the min-normal quantum */
    double quantum = ldexp(1.0, E - mbits);
    double r = rint(y / quantum) * quantum;
    return r > maxval ? maxval : r;
}

/* Code of a non-negative element value on the grid (exact search). */
static int encode_magnitude(double r, int fmt)
{
    int ncodes = (fmt == ORC_E2M1) ? 8 : 127; /* positive codes, E4M3 NaN excluded */
    for (int c = 0; c < ncodes; c++) {
        double v = (fmt == ORC_E2M1) ? orc_e2m1_value(c) : orc_e4m3_value(c);
        if (v == r) return c;
    }
    return -1; /* unreachable for r produced by round_to_format */
}

/* MX quantization of one 32-element block (OCP MX v1.0 conversion):
 *   shared exponent e = floor(log2(max|x|)) - emax_elem, clamped to the E8M0 range
 *   (emax_elem = 2 for E2M1, 8 for E4M3; an all-zero block gets e = -127);
 *   element i = RNE(x_i / 2^e) on the element grid, saturating at +-6 / +-448;
 *   the sign bit is the sign of x_i (so a negative value that rounds to zero
 *   keeps its sign bit).
 * codes[i] receives one code per element (unpacked); *scale the E8M0 byte. */
void orc_mx_quant_block(const double* x, int fmt, uint8_t* codes, uint8_t* scale)
{
    const int emax_elem = (fmt == ORC_E2M1) ? 2 : 8;
    const int mbits = (fmt == ORC_E2M1) ? 1 : 3;
    const int emin = (fmt == ORC_E2M1) ? 0 : -6;
    const double maxval = (fmt == ORC_E2M1) ? 6.0 : 448.0;
    const int signbit = (fmt == ORC_E2M1) ? 8 : 128;

    double amax = 0.0;
    for (int i = 0; i < 32; i++)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int E;
        frexp(amax, &E);          /* amax in [2^(E-1), 2^E) */
        e = (E - 1) - emax_elem;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    *scale = (uint8_t)(e + 127);
    for (int i = 0; i < 32; i++) {
        double y = ldexp(fabs(x[i]), -e);
        double r = round_to_format(y, mbits, emin, maxval);
        int c = encode_magnitude(r, fmt);
        if (signbit(x[i])) c |= signbit;
        codes[i] = (uint8_t)c;
    }
}

/* Quantize nblocks consecutive 32-element blocks of x (fp32 values).
 * E2M1 output is packed two codes per byte, element 2i in the low nibble;
 * E4M3 output is one code per byte.  scales[b] is the E8M0 byte of block b. */
void orc_mx_quant(int fmt, const float* x, int64_t nblocks, uint8_t* out, uint8_t* scales)
{
    for (int64_t b = 0; b < nblocks; b++) {
        double xb[32];
        uint8_t codes[32];
        for (int i = 0; i < 32; i++) xb[i] = x[b * 32 + i];
        orc_mx_quant_block(xb, fmt, codes, &scales[b]);
        if (fmt == ORC_E2M1) {
            for (int i = 0; i < 16; i++)
                out[b * 16 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        } else {
            memcpy(out + b * 32, codes, 32);
        }
    }
}

/* Dequantize: value of element i of an MX tensor (row-major, dim per row). */
static double mx_elem(int fmt, const uint8_t* data, const uint8_t* scales, int64_t row, int dim, int i)
{
    int code;
    if (fmt == ORC_E2M1) {
        uint8_t byte = data[row * (dim / 2) + i / 2];
        code = (i & 1) ? (byte >> 4) : (byte & 15);
    } else {
        code = data[row * dim + i];
    }
    double v = (fmt == ORC_E2M1) ? orc_e2m1_value(code) : orc_e4m3_value(code);
    return v * orc_e8m0_value(scales[row * (dim / 32) + i / 32]);
}

/* ------------------------------------------------------------------------- */
/* Main KV storage format ([P1] "Mixed precision", the table of per-entry bytes): */
/* E2M1 elements with one E4M3 scale per 16 channels and no second-level global   */
/* scale (the NVFP4 block layout without its tensor-wide scale); 512 channels make */
/* 256 code bytes + 32 scale bytes = 288 B per entry.  Element 2i is the low      */
/* nibble.  The pages fix the format, not the rounding; the reading taken is the  */
/* NVFP4 rule with the global scale removed: s = E4M3 nearest-even rounding of    */
/* amax / 6 (saturating at 448); element = E2M1 nearest-even rounding of |x| / s  */
/* (saturating at 6) with the sign bit of x; a block whose s rounds to zero       */
/* stores zero magnitudes.                                                        */
/* ------------------------------------------------------------------------- */
void orc_fp4s16_quant_block(const double* x, uint8_t* codes, uint8_t* scale)
{
    double amax = 0.0;
    for (int i = 0; i < 16; i++)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    double s = round_to_format(amax / 6.0, 3, -6, 448.0);
    *scale = (uint8_t)encode_magnitude(s, ORC_E4M3);
    for (int i = 0; i < 16; i++) {
        int c = 0;
        if (s > 0.0) c = encode_magnitude(round_to_format(fabs(x[i]) / s, 1, 0, 6.0), ORC_E2M1);
        if (signbit(x[i])) c |= 8;
        codes[i] = (uint8_t)c;
    }
}

/* Quantize nblocks consecutive 16-element blocks of x: 8 packed code bytes and one
 * E4M3 scale byte per block. */
void orc_fp4s16_quant(const float* x, int64_t nblocks, uint8_t* out, uint8_t* scales)
{
    for (int64_t b = 0; b < nblocks; b++) {
        double xb[16];
        uint8_t codes[16];
        for (int i = 0; i < 16; i++) xb[i] = x[b * 16 + i];
        orc_fp4s16_quant_block(xb, codes, &scales[b]);
        for (int i = 0; i < 8; i++) out[b * 8 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
    }
}

/* Value of element i of a row in the main KV format: E2M1 code times its block's
 * E4M3 scale. */
static double fp4s16_elem(const uint8_t* data, const uint8_t* scales, int64_t row, int dim, int i)
{
    uint8_t byte = data[row * (dim / 2) + i / 2];
    int code = (i & 1) ? (byte >> 4) : (byte & 15);
    return orc_e2m1_value(code) * orc_e4m3_value(scales[row * (dim / 16) + i / 16]);
}

/* ------------------------------------------------------------------------- */
/* Reachability: [P1] "CSA2" (non-overlapping compression; only complete groups   */
/* are entries) and "Mixed precision" (incomplete groups are separate state);    */
/* causal visibility "position i sees nothing later than i" ([P1] "CED").         */
/* Entry j of a request covers tokens [j*m, j*m+m-1]; it is visible to the query */
/* at absolute position p iff its last token j*m+m-1 <= p.                        */
/* ------------------------------------------------------------------------- */
int64_t orc_reach(int64_t p, int m, int64_t n_entries)
{
    int64_t R = 0;
    for (int64_t j = 0; j < n_entries; j++)
        if (j * m + m - 1 <= p) R = j + 1;
    return R;
}

/* ------------------------------------------------------------------------- */
/* Index score.  Problem statement: s_j = sum_h w_h * ReLU(q_h . k_j), an MQA    */
/* form over one shared key per position ([P4] section 5: FP4 index scoring reads */
/* the FP4 cache directly, heads replicated).  Index q and k are MXFP4 with a     */
/* 32-element block ([P1] "Mixed precision": Indexer Q/K use MXFP4, group 32).    */
/*                                                                            */
/* Canonical fp32 head reduction (the order the GPU also uses, so the top-k set  */
/* is decided identically): split the H heads into 4 contiguous groups;          */
/* P_g = fma(w_h, max(d_h, 0), P_g) over the group's heads in ascending order,   */
/* starting at +0; s = (P_0 + P_1) + (P_2 + P_3).                                 */
/* ------------------------------------------------------------------------- */
static float orc_canon_reduce(const float* d, const float* w, int H)
{
    int G = H / 4;
    float P[4];
    for (int g = 0; g < 4; g++) {
        float acc = 0.0f;
        for (int h = g * G; h < (g + 1) * G; h++) {
            float r = d[h] > 0.0f ? d[h] : 0.0f;
            acc = fmaf(w[h], r, acc);
        }
        P[g] = acc;
    }
    return (P[0] + P[1]) + (P[2] + P[3]);
}

/* Absolute compressed position of score column c of a row, or -1 if the column
 * holds no position.  Full range: c itself.  Pool: block blocks[c / B], member
 * c % B (columns are the selected blocks' positions in ascending order). */
static int64_t column_position(int64_t c, const int32_t* blocks, const int32_t* nblocks, int64_t prow,
                               int block, int max_blocks)
{
    if (!blocks) return c;
    int64_t i = c / block;
    if (i >= nblocks[prow]) return -1;
    return (int64_t)blocks[prow * max_blocks + i] * block + c % block;
}

/* Exact MXFP4 x MXFP4 dot product over dim elements.  Each product of two E2M1
 * values is a multiple of 1/4 with |.| <= 36; a 32-block sums to an integer
 * multiple of 2^(e_q + e_k - 2) below 2^13, so the per-block sums are exact
 * integers.  The (at most 8) block terms are added in double, which is exact
 * while their exponents lie within 39 of each other; *inexact is set otherwise
 * or when the result is not an fp32 value (then no fp32 order is exact). */
static double mxfp4_dot(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, int dim,
                        int* inexact)
{
    double total = 0.0;
    int emin = 1000, emax = -1000;
    for (int b = 0; b < dim / 32; b++) {
        long isum = 0;
        for (int i = b * 32; i < b * 32 + 32; i++) {
            int cq = (i & 1) ? (qc[i / 2] >> 4) : (qc[i / 2] & 15);
            int ck = (i & 1) ? (kc[i / 2] >> 4) : (kc[i / 2] & 15);
            long a2 = (long)llround(2.0 * orc_e2m1_value(cq));
            long b2 = (long)llround(2.0 * orc_e2m1_value(ck));
            isum += a2 * b2;
        }
        int ex = (qs[b] - 127) + (ks[b] - 127) - 2;
        if (isum != 0) {
            if (ex < emin) emin = ex;
            if (ex > emax) emax = ex;
        }
        total += ldexp((double)isum, ex);
    }
    if (emax >= emin && emax - emin > 39) *inexact = 1;
    if ((double)(float)total != total) *inexact = 1;
    return total;
}

/* Score every reachable column of every row (MXFP4 keys, index q given as fp32
 * values that the method quantizes to MXFP4 first).  Returns the number of
 * (row, column, head) dot products that were not exact in fp32 (expected 0). */
long orc_index_score_mxfp4(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m,
                           const int32_t* n_entries, const int64_t* row_start, int H, int dim,
                           const float* q, const float* w, int64_t w_row_stride, const uint8_t* kdata,
                           const uint8_t* kscale, const int32_t* pool_blocks, const int32_t* pool_nblocks,
                           int block, int max_blocks, const int32_t* pool_row_map, float* scores,
                           int64_t score_stride)
{
    long bad = 0;
    int nb = dim / 32;
    uint8_t* qcodes = (uint8_t*)malloc((size_t)n * H * (dim / 2));
    uint8_t* qscales = (uint8_t*)malloc((size_t)n * H * nb);
    orc_mx_quant(ORC_E2M1, q, (int64_t)n * H * nb, qcodes, qscales);

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int row = 0; row < n; row++) {
        int r = req_of_row[row];
        int64_t R = orc_reach(pos_of_row[row], m, n_entries[r]);
        int64_t prow = pool_row_map ? pool_row_map[row] : row;
        int64_t ncol = pool_blocks ? (int64_t)pool_nblocks[prow] * block : R;
        if (ncol > score_stride) ncol = score_stride;
        float* d = (float*)malloc(sizeof(float) * H);
        const float* wr = w + (int64_t)row * w_row_stride;
        for (int64_t c = 0; c < ncol; c++) {
            int64_t j = column_position(c, pool_blocks, pool_nblocks, prow, block, max_blocks);
            if (j < 0 || j >= R) {
                scores[(int64_t)row * score_stride + c] = -INFINITY;
                continue;
            }
            int64_t krow = row_start[r] + j;
            for (int h = 0; h < H; h++) {
                int inexact = 0;
                int64_t qi = (int64_t)row * H + h;
                double dd = mxfp4_dot(qcodes + qi * (dim / 2), qscales + qi * nb, kdata + krow * (dim / 2),
                                      kscale + krow * nb, dim, &inexact);
                bad += inexact;
                d[h] = (float)dd;
            }
            scores[(int64_t)row * score_stride + c] = orc_canon_reduce(d, wr, H);
        }
        free(d);
    }
    free(qcodes);
    free(qscales);
    return bad;
}

/* fp32 variant (q and keys fp32): d_h = fma chain over the dimension in
 * ascending order from +0, then the canonical head reduction. */
void orc_index_score_f32(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m,
                         const int32_t* n_entries, const int64_t* row_start, int H, int dim, const float* q,
                         const float* w, int64_t w_row_stride, const float* keys, const int32_t* pool_blocks,
                         const int32_t* pool_nblocks, int block, int max_blocks, const int32_t* pool_row_map,
                         float* scores, int64_t score_stride)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int row = 0; row < n; row++) {
        int r = req_of_row[row];
        int64_t R = orc_reach(pos_of_row[row], m, n_entries[r]);
        int64_t prow = pool_row_map ? pool_row_map[row] : row;
        int64_t ncol = pool_blocks ? (int64_t)pool_nblocks[prow] * block : R;
        if (ncol > score_stride) ncol = score_stride;
        float* d = (float*)malloc(sizeof(float) * H);
        const float* wr = w + (int64_t)row * w_row_stride;
        for (int64_t c = 0; c < ncol; c++) {
            int64_t j = column_position(c, pool_blocks, pool_nblocks, prow, block, max_blocks);
            if (j < 0 || j >= R) {
                scores[(int64_t)row * score_stride + c] = -INFINITY;
                continue;
            }
            const float* kr = keys + (row_start[r] + j) * dim;
            for (int h = 0; h < H; h++) {
                const float* qr = q + ((int64_t)row * H + h) * dim;
                float acc = 0.0f;
                for (int i = 0; i < dim; i++) acc = fmaf(qr[i], kr[i], acc);
                d[h] = acc;
            }
            scores[(int64_t)row * score_stride + c] = orc_canon_reduce(d, wr, H);
        }
        free(d);
    }
}

/* ------------------------------------------------------------------------- */
/* Top-k ([P1] "Hierarchical Sparse Indexer": top-512 per query; [P4] section 1: */
/* at most 512 compressed positions).  Candidates are ordered by score (larger  */
/* first; -0 equals +0) and then by lower position; the first k are taken; the   */
/* output lists them in ascending position and pads with -1.                     */
/* ------------------------------------------------------------------------- */
typedef struct {
    float s;
    int64_t j;
} orc_cand;

static int cand_cmp(const void* a, const void* b)
{
    const orc_cand* x = (const orc_cand*)a;
    const orc_cand* y = (const orc_cand*)b;
    float sx = x->s + 0.0f, sy = y->s + 0.0f; /* -0 -> +0 */
    if (sx > sy) return -1;
    if (sx < sy) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int i64_cmp(const void* a, const void* b)
{
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Select from cands[0..nc) (sorted in place); write k outputs (ascending, -1 pad). */
static void take_topk(orc_cand* cands, int64_t nc, int k, int32_t* out)
{
    qsort(cands, (size_t)nc, sizeof(orc_cand), cand_cmp);
    int64_t t = nc < k ? nc : k;
    int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (t > 0 ? t : 1));
    for (int64_t i = 0; i < t; i++) sel[i] = cands[i].j;
    qsort(sel, (size_t)t, sizeof(int64_t), i64_cmp);
    for (int64_t i = 0; i < k; i++) out[i] = i < t ? (int32_t)sel[i] : -1;
    free(sel);
}

void orc_topk(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m, const int32_t* n_entries,
              const float* scores, int64_t score_stride, const int32_t* pool_blocks,
              const int32_t* pool_nblocks, int block, int max_blocks, const int32_t* pool_row_map, int k,
              int32_t* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int row = 0; row < n; row++) {
        int r = req_of_row[row];
        int64_t R = orc_reach(pos_of_row[row], m, n_entries[r]);
        int64_t prow = pool_row_map ? pool_row_map[row] : row;
        int64_t ncol = pool_blocks ? (int64_t)pool_nblocks[prow] * block : R;
        if (ncol > score_stride) ncol = score_stride;
        orc_cand* cands = (orc_cand*)malloc(sizeof(orc_cand) * (ncol > 0 ? ncol : 1));
        int64_t nc = 0;
        for (int64_t c = 0; c < ncol; c++) {
            int64_t j = column_position(c, pool_blocks, pool_nblocks, prow, block, max_blocks);
            if (j < 0 || j >= R) continue;
            cands[nc].s = scores[(int64_t)row * score_stride + c];
            cands[nc].j = j;
            nc++;
        }
        take_topk(cands, nc, k, out + (int64_t)row * k);
        free(cands);
    }
}

/* ------------------------------------------------------------------------- */
/* Hierarchical selection ([P1] "Hierarchical Sparse Indexer"; [P4] section 2,   */
/* "two-level selection"): positions are grouped 8 to a block; a block's score   */
/* is the maximum over its reachable members; at most max_blocks blocks are kept, */
/* always including the block that holds the newest reachable position; the rest */
/* are the best others by (block score desc, block id asc).  The same pass also  */
/* takes its own flat top-k over all reachable positions.                         */
/* ------------------------------------------------------------------------- */
void orc_topk_hier(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m, const int32_t* n_entries,
                   const float* scores, int64_t score_stride, int k, int block, int max_blocks,
                   int32_t* out_idx, int32_t* out_blocks, int32_t* out_nblocks)
{
    orc_topk(n, req_of_row, pos_of_row, m, n_entries, scores, score_stride, NULL, NULL, 0, 0, NULL, k, out_idx);
#pragma omp parallel for schedule(dynamic, 1)
    for (int row = 0; row < n; row++) {
        int r = req_of_row[row];
        int64_t R = orc_reach(pos_of_row[row], m, n_entries[r]);
        if (R > score_stride) R = score_stride;
        int64_t nblk = (R + block - 1) / block;
        int32_t* ob = out_blocks + (int64_t)row * max_blocks;
        for (int i = 0; i < max_blocks; i++) ob[i] = -1;
        if (nblk <= max_blocks) {
            for (int64_t b = 0; b < nblk; b++) ob[b] = (int32_t)b;
            out_nblocks[row] = (int32_t)nblk;
            continue;
        }
        int64_t newest = nblk - 1;
        orc_cand* cands = (orc_cand*)malloc(sizeof(orc_cand) * newest);
        for (int64_t b = 0; b < newest; b++) {
            float mx = -INFINITY;
            for (int64_t j = b * block; j < b * block + block && j < R; j++) {
                float s = scores[(int64_t)row * score_stride + j] + 0.0f;
                if (s > mx) mx = s;
            }
            cands[b].s = mx;
            cands[b].j = b;
        }
        int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * max_blocks);
        take_topk(cands, newest, max_blocks - 1, tmp);
        for (int i = 0; i < max_blocks - 1; i++) ob[i] = tmp[i];
        ob[max_blocks - 1] = (int32_t)newest; /* largest id: stays ascending */
        out_nblocks[row] = max_blocks;
        free(tmp);
        free(cands);
    }
}

/* ------------------------------------------------------------------------- */
/* Sparse + sliding-window attention ([P4] section 1: every query attends to its */
/* own 128-position window and to at most 512 compressed positions chosen by the */
/* indexer; [P1] "Mixed precision": the 512-d main entry is one shared latent,   */
/* used as key and value; SWA KV is FP8).  One softmax over the union of the two */
/* sets, computed in double.  The window of query p is [max(lo, p-W+1), p] where */
/* lo is the replay lower bound ([P2] section 2.3) and the first cached window   */
/* position.  A sink, when given, adds exp(sink_h - max) to the denominator.     */
/* Data types: 0 = f32, 1 = bf16 (raw 16-bit patterns), 3 = MXFP8 E4M3 (+E8M0),  */
/* 4 = the main KV storage format (E2M1 + one E4M3 scale per 16, defined above).  */
/* ------------------------------------------------------------------------- */
static double load_val(const void* base, int dt, const uint8_t* scales, int64_t row, int dim, int i)
{
    if (dt == 0) return ((const float*)base)[row * dim + i];
    if (dt == 1) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[row * dim + i] << 16;
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    if (dt == 4) return fp4s16_elem((const uint8_t*)base, scales, row, dim, i);
    return mx_elem(ORC_E4M3, (const uint8_t*)base, scales, row, dim, i);
}

static void attend_set(const double* qh, int D, const double* keys, int64_t nk, double sm_scale, const float* sink,
                       int h, double* out, double* lse)
{
    if (nk == 0) {
        for (int d = 0; d < D; d++) out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double* logit = (double*)malloc(sizeof(double) * nk);
    double mx = -INFINITY;
    for (int64_t t = 0; t < nk; t++) {
        double acc = 0.0;
        for (int d = 0; d < D; d++) acc += qh[d] * keys[t * D + d];
        logit[t] = sm_scale * acc;
        if (logit[t] > mx) mx = logit[t];
    }
    double den = 0.0;
    for (int d = 0; d < D; d++) out[d] = 0.0;
    for (int64_t t = 0; t < nk; t++) {
        double p = exp(logit[t] - mx);
        den += p;
        for (int d = 0; d < D; d++) out[d] += p * keys[t * D + d];
    }
    if (sink) den += exp((double)sink[h] - mx);
    for (int d = 0; d < D; d++) out[d] /= den;
    *lse = mx + log(den);
    free(logit);
}

/* Gathers the key/value set of one row: selected entries (if sel != NULL) or
 * all reachable entries (dense mode), then the window rows. */
static int64_t gather_row(int row, int r, int p, int64_t R, int D, const void* kv, int kv_dt,
                          const uint8_t* kv_scale, const int64_t* row_start, const int32_t* sel, int k, const void* swa, int swa_dt,
                          const uint8_t* swa_scale, const int64_t* swa_row_start, const int32_t* swa_pos_start,
                          int window, int lo, double* keys)
{
    int64_t nk = 0;
    if (sel) {
        for (int i = 0; i < k; i++) {
            int32_t j = sel[i];
            if (j < 0) continue;
            for (int d = 0; d < D; d++) keys[nk * D + d] = load_val(kv, kv_dt, kv_scale, row_start[r] + j, D, d);
            nk++;
        }
    } else {
        for (int64_t j = 0; j < R; j++) {
            for (int d = 0; d < D; d++) keys[nk * D + d] = load_val(kv, kv_dt, kv_scale, row_start[r] + j, D, d);
            nk++;
        }
    }
    int64_t t0 = (int64_t)p - window + 1;
    if (t0 < lo) t0 = lo;
    if (t0 < swa_pos_start[r]) t0 = swa_pos_start[r];
    for (int64_t t = t0; t <= p; t++) {
        int64_t srow = swa_row_start[r] + (t - swa_pos_start[r]);
        for (int d = 0; d < D; d++) keys[nk * D + d] = load_val(swa, swa_dt, swa_scale, srow, D, d);
        nk++;
    }
    (void)row;
    return nk;
}

static void attn_common(int dense, int n, const int32_t* req_of_row, const int32_t* pos_of_row,
                        const int32_t* win_lo, int m, const int32_t* n_entries, const int64_t* row_start,
                        const void* q, int q_dt, int H, int D, const void* kv, int kv_dt,
                        const uint8_t* kv_scale, const int32_t* sel_idx,
                        int k, int64_t sel_stride, const int32_t* sel_row_map, const void* swa, int swa_dt,
                        const uint8_t* swa_scale, const int64_t* swa_row_start, const int32_t* swa_pos_start,
                        int window, double sm_scale, const float* sink, double* out, double* lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int row = 0; row < n; row++) {
        int r = req_of_row[row];
        int p = pos_of_row[row];
        int lo = win_lo ? win_lo[row] : 0;
        int64_t R = orc_reach(p, m, n_entries[r]);
        int64_t cap = (dense ? R : k) + window;
        double* keys = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        const int32_t* sel = NULL;
        if (!dense) sel = sel_idx + (int64_t)(sel_row_map ? sel_row_map[row] : row) * sel_stride;
        int64_t nk = gather_row(row, r, p, R, D, kv, kv_dt, kv_scale, row_start, sel, k, swa, swa_dt, swa_scale,
                                swa_row_start, swa_pos_start, window, lo, keys);
        double* qh = (double*)malloc(sizeof(double) * D);
        for (int h = 0; h < H; h++) {
            for (int d = 0; d < D; d++) qh[d] = load_val(q, q_dt, NULL, (int64_t)row * H + h, D, d);
            double l;
            attend_set(qh, D, keys, nk, sm_scale, sink, h, out + ((int64_t)row * H + h) * D, &l);
            if (lse) lse[(int64_t)row * H + h] = l;
        }
        free(qh);
        free(keys);
    }
}

void orc_sparse_swa_attn(int n, const int32_t* req_of_row, const int32_t* pos_of_row, const int32_t* win_lo, int m,
                         const int32_t* n_entries, const int64_t* row_start, const void* q, int q_dt, int H, int D,
                         const void* kv, int kv_dt, const uint8_t* kv_scale, const int32_t* sel_idx, int k,
                         int64_t sel_stride, const int32_t* sel_row_map, const void* swa, int swa_dt, const uint8_t* swa_scale,
                         const int64_t* swa_row_start, const int32_t* swa_pos_start, int window, double sm_scale,
                         const float* sink, double* out, double* lse)
{
    attn_common(0, n, req_of_row, pos_of_row, win_lo, m, n_entries, row_start, q, q_dt, H, D, kv, kv_dt, kv_scale,
                sel_idx, k, sel_stride, sel_row_map, swa, swa_dt, swa_scale, swa_row_start, swa_pos_start, window, sm_scale,
                sink, out, lse);
}

/* Dense brute force: every reachable compressed entry plus the window, no index set. */
void orc_dense_attn(int n, const int32_t* req_of_row, const int32_t* pos_of_row, const int32_t* win_lo, int m,
                    const int32_t* n_entries, const int64_t* row_start, const void* q, int q_dt, int H, int D,
                    const void* kv, int kv_dt, const uint8_t* kv_scale, const void* swa, int swa_dt,
                    const uint8_t* swa_scale, const int64_t* swa_row_start, const int32_t* swa_pos_start, int window, double sm_scale,
                    const float* sink, double* out, double* lse)
{
    attn_common(1, n, req_of_row, pos_of_row, win_lo, m, n_entries, row_start, q, q_dt, H, D, kv, kv_dt, kv_scale,
                NULL, 0, 0, NULL, swa, swa_dt, swa_scale, swa_row_start, swa_pos_start, window, sm_scale, sink, out, lse);
}

/* ------------------------------------------------------------------------- */
/* Index-K producer, the step that fills the caches the path reads ([P1] "CSA2":   */
/* non-overlapping compression, index K projected from the compressed main KV;    */
/* [P4] section 1: pairwise compression keeps incomplete pairs across decode      */
/* steps; [P4] section 5: compressor projection with BF16 weights and FP32        */
/* accumulation and output, ratio-2 pooling merging each completed pair, RoPE and */
/* FP4 quantization/pack/cache write fused while keeping the intermediate        */
/* rounding; [P1] "Mixed precision": main KV quantized after RoPE).              */
/* Readings (the pages name the steps, not their arithmetic):                    */
/*  - input: the compressor's per-token fp32 outputs (512-d); m tokens pool into  */
/*    one entry by their mean, (a + b) * 0.5 in fp32 for m = 2, the token itself  */
/*    for m = 1; entry j covers tokens [j m, j m + m - 1] and is produced when   */
/*    its last token arrives; a lone first token waits in `pending` [nreq][512]. */
/*  - RoPE: the last 64 dims of the 512-d latent and of the 128-d index key,     */
/*    rotated in interleaved pairs (2i, 2i+1) at the entry's last token position */
/*    P = j m + m - 1, with cos / sin taken from a caller table [pos][2][32]:     */
/*    x' = x c - y s, y' = x s + y c, each product and sum rounded to fp32.      */
/*  - index K: k_o = sum_i W[o][i] * bf16(latent_i) over the pre-RoPE latent,    */
/*    accumulated in fp32 by one fma per term in ascending i (a fixed order, so  */
/*    that the MXFP4 codes it decides are reproducible), then RoPE, then MXFP4.  */
/*  - main KV: the RoPE'd latent, stored bf16 (nearest even) or in the FP4       */
/*    storage format above.                                                      */
/* Rows of one request in a call are consecutive ascending positions.  Reads of   */
/* `pending` see its state before the call.                                      */
/* ------------------------------------------------------------------------- */
#define ORC_KV_DIM 512
#define ORC_IDX_DIM 128
#define ORC_ROPE_DIM 64

static float orc_bf16_round(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

static void orc_rope(float* x, const float* rope, int64_t P)
{
    const float* c = rope + P * ORC_ROPE_DIM;
    const float* sn = c + ORC_ROPE_DIM / 2;
    for (int i = 0; i < ORC_ROPE_DIM / 2; i++) {
        float a = x[2 * i], b = x[2 * i + 1];
        float t1 = a * c[i], t2 = b * sn[i], t3 = a * sn[i], t4 = b * c[i];
        x[2 * i] = t1 - t2;
        x[2 * i + 1] = t3 + t4;
    }
}

static void orc_produce_entry(const float* latent, int64_t P, int64_t erow, const uint16_t* w_index,
                              const float* rope, int kv_dt, void* kv, uint8_t* kv_scale, uint8_t* idx_codes,
                              uint8_t* idx_scales)
{
    float x[ORC_KV_DIM], k[ORC_IDX_DIM], y[ORC_KV_DIM];
    for (int i = 0; i < ORC_KV_DIM; i++) {
        x[i] = latent[i];
        y[i] = orc_bf16_round(latent[i]);
    }
    /* index key */
    for (int o = 0; o < ORC_IDX_DIM; o++) {
        float acc = 0.0f;
        for (int i = 0; i < ORC_KV_DIM; i++) {
            uint32_t wb = (uint32_t)w_index[(int64_t)o * ORC_KV_DIM + i] << 16;
            float wf;
            memcpy(&wf, &wb, 4);
            acc = fmaf(wf, y[i], acc);
        }
        k[o] = acc;
    }
    orc_rope(k + ORC_IDX_DIM - ORC_ROPE_DIM, rope, P);
    orc_mx_quant(ORC_E2M1, k, ORC_IDX_DIM / 32, idx_codes + erow * (ORC_IDX_DIM / 2), idx_scales + erow * (ORC_IDX_DIM / 32));
    /* main KV */
    orc_rope(x + ORC_KV_DIM - ORC_ROPE_DIM, rope, P);
    if (kv_dt == 4) {
        orc_fp4s16_quant(x, ORC_KV_DIM / 16, (uint8_t*)kv + erow * (ORC_KV_DIM / 2), kv_scale + erow * (ORC_KV_DIM / 16));
    } else {
        uint16_t* o = (uint16_t*)kv + erow * ORC_KV_DIM;
        for (int i = 0; i < ORC_KV_DIM; i++) {
            float r = orc_bf16_round(x[i]);
            uint32_t u;
            memcpy(&u, &r, 4);
            o[i] = (uint16_t)(u >> 16);
        }
    }
}

/* Returns 0, or -1 for an argument the producer does not take. */
int orc_kv_produce(int n, const int32_t* req_of_row, const int32_t* pos_of_row, int m, const int64_t* row_start,
                   const float* comp, float* pending, const uint16_t* w_index, const float* rope, int64_t max_pos,
                   int kv_dt, void* kv, uint8_t* kv_scale, uint8_t* idx_codes, uint8_t* idx_scales)
{
    if (m != 1 && m != 2) return -1;
    if (kv_dt != 1 && kv_dt != 4) return -1;
    /* entries first (they read `pending` as it was before the call), then the new lone tokens */
    for (int t = 0; t < n; t++) {
        int r = req_of_row[t];
        int64_t p = pos_of_row[t];
        if ((p + 1) % m != 0) continue;
        int64_t j = (p + 1) / m - 1;
        int64_t P = j * m + m - 1;
        if (P >= max_pos) return -1;
        float latent[ORC_KV_DIM];
        const float* b = comp + (int64_t)t * ORC_KV_DIM;
        if (m == 1) {
            for (int i = 0; i < ORC_KV_DIM; i++) latent[i] = b[i];
        } else {
            int prev_here = t > 0 && req_of_row[t - 1] == r && pos_of_row[t - 1] == p - 1;
            const float* a = prev_here ? comp + (int64_t)(t - 1) * ORC_KV_DIM : pending + (int64_t)r * ORC_KV_DIM;
            for (int i = 0; i < ORC_KV_DIM; i++) latent[i] = (a[i] + b[i]) * 0.5f;
        }
        orc_produce_entry(latent, P, row_start[r] + j, w_index, rope, kv_dt, kv, kv_scale, idx_codes, idx_scales);
    }
    if (m == 2) {
        for (int t = 0; t < n; t++) {
            int r = req_of_row[t];
            int64_t p = pos_of_row[t];
            int next_here = t + 1 < n && req_of_row[t + 1] == r && pos_of_row[t + 1] == p + 1;
            if (p % 2 == 0 && !next_here)
                memcpy(pending + (int64_t)r * ORC_KV_DIM, comp + (int64_t)t * ORC_KV_DIM, sizeof(float) * ORC_KV_DIM);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Decoder bounded-replay tail layout ([P2] sections 2.1 and 2.3, restated in the */
/* rule block after the window table): per request, T = min(budget, E); the     */
/* late layers keep the absolute positions [S - T, S); the window lower bound is */
/* S - T; the tail row u of request r is row (start of r in the extend) + E - T + u */
/* of the original extend.  Computed per request, never per batch.               */
/* Mixed batches ([P1] "Decoder Bounded Replay": in a mixed batch the new tokens */
/* of decode requests still pass through the whole trunk): a request flagged as  */
/* decode keeps all of its E rows (E <= budget) and no window cut (lower bound   */
/* 0; the window cache's own first position still bounds what exists).          */
/* flags bit 0 (reading of the short-extend proposal in [P2] section 2.6, which */
/* lets the late layers see the cached prefix's window): the lower bound of a   */
/* prefill request becomes max(0, S - budget) instead of S - T; it differs only */
/* when E < budget.                                                              */
/* ------------------------------------------------------------------------- */
int orc_replay_tail_layout(int nreq, const int32_t* ext_len, const int32_t* seq_len, const int32_t* is_decode,
                           int budget, int flags, int32_t* tail_len, int32_t* tail_row_start, int32_t* src_row,
                           int32_t* abs_pos, int32_t* win_lo, int32_t* req_of_row, int capacity)
{
    int64_t ext_start = 0, out = 0;
    for (int r = 0; r < nreq; r++) {
        int E = ext_len[r], S = seq_len[r];
        int decode = is_decode && is_decode[r];
        if (E < 0 || E > S) return -1;
        if (decode && E > budget) return -3;
        int T = (decode || E < budget) ? E : budget;
        int lo;
        if (decode)
            lo = 0;
        else if (flags & 1)
            lo = S - budget > 0 ? S - budget : 0;
        else
            lo = S - T;
        tail_len[r] = T;
        tail_row_start[r] = (int32_t)out;
        for (int u = 0; u < T; u++) {
            if (out >= capacity) return -2;
            src_row[out] = (int32_t)(ext_start + E - T + u);
            abs_pos[out] = S - T + u;
            win_lo[out] = lo;
            req_of_row[out] = r;
            out++;
        }
        ext_start += E;
    }
    tail_row_start[nreq] = (int32_t)out;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Encoder-side bounded replay layout ([P4] section 4.1; [P4] section 4.3: both */
/* replay modes cut local attention at the rebuild boundary).  Request r has a  */
/* cached prefix of P tokens (its compressed KV and indexer keys are kept, its  */
/* window is not) and an extend of E new tokens.  The rows of the call are the  */
/* last min(P, budget) prefix positions, recomputed to rebuild the window, then */
/* the E extend positions: absolute positions [R0, P + E) with R0 =             */
/* max(0, P - budget), all with window lower bound R0.  src_row is the row of   */
/* the extend input for extend rows and -1 for replayed prefix rows (whose      */
/* tokens come from the cache).  row_start[r] is the first row of request r.    */
/* ------------------------------------------------------------------------- */
int orc_encoder_replay_layout(int nreq, const int32_t* prefix_len, const int32_t* ext_len, int budget,
                              int32_t* row_start, int32_t* src_row, int32_t* abs_pos, int32_t* win_lo,
                              int32_t* req_of_row, int capacity)
{
    int64_t ext_start = 0, out = 0;
    for (int r = 0; r < nreq; r++) {
        int P = prefix_len[r], E = ext_len[r];
        if (P < 0 || E < 0) return -1;
        int R0 = P - budget > 0 ? P - budget : 0;
        row_start[r] = (int32_t)out;
        for (int t = R0; t < P + E; t++) {
            if (out >= capacity) return -2;
            src_row[out] = t < P ? -1 : (int32_t)(ext_start + (t - P));
            abs_pos[out] = t;
            win_lo[out] = R0;
            req_of_row[out] = r;
            out++;
        }
        ext_start += E;
    }
    row_start[nreq] = (int32_t)out;
    return 0;
}
