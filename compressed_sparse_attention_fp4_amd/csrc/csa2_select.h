// Radix top-k selection shared by the selection kernels and the fused score + select
// kernel (device code only).  See k_topk.hip for the method.
#pragma once

#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

// Candidate sources: FULL (score row, column = position), POOL (compact pool score row,
// column c = pool position c), BLOCK (block maxima computed from the score row), LIST (a
// previous level's (key, position) lists), BMAX (precomputed block-maximum keys), PGATHER
// (the pool's positions gathered from the full score row).
enum SrcMode { SRC_FULL = 0, SRC_POOL = 1, SRC_BLOCK = 2, SRC_LIST = 3, SRC_BMAX = 4, SRC_PGATHER = 5 };
enum OutMode { OUT_IDX = 0, OUT_LIST = 1, OUT_BLOCKS = 2 };

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;
constexpr int kMaxKPT = 32;
constexpr int64_t kMaxCap = (int64_t)kNT * kMaxKPT;  // 32768 candidates per workgroup
constexpr int64_t kListCap = (int64_t)kNT * 16;      // 16384 candidates per merge workgroup

struct SelArgs {
    SelSource src;
    int block;          // SRC_BLOCK: positions per block (a power of two)
    int block_shift;    // log2(block) for pool / block addressing
    int k;              // entries kept per row
    int nseg;           // workgroups (segments / groups) per row at this level
    int64_t seg_len;    // candidates per segment (first level) or lists per group (merge)
    int nlists_prev;    // merge level: lists per row in the input
    const uint2* in;    // merge input lists [n][nlists_prev][k] (key, pos)
    uint2* out_list;    // OUT_LIST target [n][nseg][k]
    int32_t* out_idx;   // OUT_IDX target [n][out_stride] / OUT_BLOCKS target
    int32_t* out_nblocks;
    int out_stride;
    int out_mode;
    const uint32_t* bmax;  // SRC_BMAX: block-maximum keys [n][bstride]
    int64_t bstride;
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

__device__ __forceinline__ int64_t pool_position(const SelSource& s, int shift, int prow, int64_t c)
{
    const int64_t i = c >> shift;
    return ((int64_t)s.pool.blocks[(int64_t)prow * s.pool.max_blocks + i] << shift) + (c & ((1 << shift) - 1));
}

constexpr int bid_slots(int kpt) { return kpt / 8 > 0 ? kpt / 8 : 1; }

// Keys of candidates [e0, e0 + KPT) of this workgroup's slice (blocked layout), loaded
// without per-element branches: addresses are clamped and invalid slots masked after.
// Pool sources with whole blocks per thread (KPT % 8 == 0, slice start % 8 == 0) also
// return the thread's pool block ids, so the output needs no second lookup.
// Wave-wide scans and reductions on DPP (register-to-register lane moves, no LDS round
// trip): Hillis-Steele shifts inside each 16-lane row (row_shr 1, 2, 4, 8), then row
// broadcasts carry row 0's last lane into row 1, row 2's into row 3 (row_bcast:15) and
// lane 31 into rows 2 and 3 (row_bcast:31).  Lanes a move does not reach read the
// operation's identity.
enum : int { kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118, kDppBcast15 = 0x142,
             kDppBcast31 = 0x143 };

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t identity, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xf, false);
}

// inclusive prefix of op over lanes 0..lane
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl(uint32_t v, uint32_t identity, Op op)
{
    v = op(v, dpp_move<kDppShr1, 0xf>(identity, v));
    v = op(v, dpp_move<kDppShr2, 0xf>(identity, v));
    v = op(v, dpp_move<kDppShr4, 0xf>(identity, v));
    v = op(v, dpp_move<kDppShr8, 0xf>(identity, v));
    v = op(v, dpp_move<kDppBcast15, 0xa>(identity, v));
    v = op(v, dpp_move<kDppBcast31, 0xc>(identity, v));
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int x, int)
{
    return (int)wave_incl((uint32_t)x, 0u, [](uint32_t p, uint32_t q) { return p + q; });
}

// wave-uniform reductions (the inclusive result of the last lane)
__device__ __forceinline__ int wave_sum(int x)
{
    return __builtin_amdgcn_readlane((int)wave_incl((uint32_t)x, 0u, [](uint32_t p, uint32_t q) { return p + q; }),
                                     63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane(
        (int)wave_incl(x, 0u, [](uint32_t p, uint32_t q) { return p > q ? p : q; }), 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane(
        (int)wave_incl(x, 0xFFFFFFFFu, [](uint32_t p, uint32_t q) { return p < q ? p : q; }), 63);
}

// Exclusive block scan of two counters at once (one barrier); NW waves.  s_w is not
// protected afterwards: the caller must not write it again (k_select scans once).
template <int NW>
__device__ __forceinline__ void block_scan2(int a, int b, int* s_w, int lane, int wave, int* ea, int* eb, int* ta,
                                            int* tb)
{
    const int ia = wave_incl_scan(a, lane);
    const int ib = wave_incl_scan(b, lane);
    if (lane == 63) {
        s_w[2 * wave] = ia;
        s_w[2 * wave + 1] = ib;
    }
    __syncthreads();
    int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        const int va = s_w[2 * w], vb = s_w[2 * w + 1];
        pa += (w < wave) ? va : 0;
        pb += (w < wave) ? vb : 0;
        sa += va;
        sb += vb;
    }
    *ea = pa + ia - a;
    *eb = pb + ib - b;
    *ta = sa;
    *tb = sb;
}

constexpr int kBins1 = 2048;  // first digit: 11 bits
constexpr int kBins = 256;    // later digits: 8 bits

// Threshold bin of a histogram of NB bins, scanned from the top: the bin b where the
// count of keys in bins above b is < need <= that count plus hist[b].  All threads
// cooperate: thread t of NT takes NB/NT adjacent bins from the top (conflict-free reads),
// one block scan orders the partial sums, and the thread holding the crossing publishes
// (bin, count above, bin count) through LDS.
template <int NB, int NT>
__device__ __forceinline__ void find_bin(const int* hist, int need, int* s_w, int* s_res, int tid, int lane,
                                         int wave, int* bin, int* above, int* cnt)
{
    constexpr int PER = NB / NT > 0 ? NB / NT : 1;
    int c[PER], sum = 0;
    const bool act = tid * PER < NB;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        c[j] = act ? hist[NB - 1 - (tid * PER + j)] : 0;
        sum += c[j];
    }
    const int incl = wave_incl_scan(sum, lane);
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) before += (w < wave) ? s_w[w] : 0;
    int acc = before + incl - sum;
    if (act && acc < need && need <= acc + sum) {
#pragma unroll
        for (int j = 0; j < PER; j++) {
            if (acc + c[j] >= need) {
                s_res[0] = NB - 1 - (tid * PER + j);
                s_res[1] = acc;
                s_res[2] = c[j];
                break;
            }
            acc += c[j];
        }
    }
    __syncthreads();
    *bin = s_res[0];
    *above = s_res[1];
    *cnt = s_res[2];
}

// The selection itself, for keys already in registers (blocked: thread t owns candidates
// [e0, e0 + KPT) of its row's slice starting at base): finds the threshold, then writes the
// selected positions (or (key, position) lists) in candidate order, and the padding.
template <int KPT, int SRC, int NT>
__device__ __forceinline__ void select_core(const SelArgs a, int row, int seg, int64_t R, int64_t ncol, int prow,
                                            int64_t base, int64_t e0, uint32_t (&key)[KPT],
                                            int32_t (&bid)[bid_slots(KPT)], bool bid_ok)
{
    __shared__ int s_h1[kBins1];        // first pass
    __shared__ int s_h[3][kBins];       // later passes, rotating (cleared one pass ahead)
    constexpr int NW = NT / 64;
    __shared__ uint32_t s_red[3][NW];
    __shared__ int s_w[2 * NW];
    __shared__ int s_fw[2][NW];    // find_bin partial sums (alternating between passes)
    __shared__ int s_res[2][3];
    __shared__ uint32_t s_cand[64];  // the threshold bin's keys once it holds at most 64
    __shared__ int s_ncand;
    __shared__ uint32_t s_fin[2];

    const int nseg = a.nseg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const SelSource& s = a.src;
    const int k = a.k;
    (void)R;
    int nvalid = 0;
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
    uint64_t live = 0;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
        const bool v = key[i] != 0;
        nvalid += v;
        live |= (uint64_t)v << i;
        kmax = max(kmax, key[i]);
        kmin = v ? min(kmin, key[i]) : kmin;
    }
    nvalid = wave_sum(nvalid);
    kmax = wave_max(kmax);
    kmin = wave_min(kmin);
    if (lane == 0) {
        s_red[0][wave] = (uint32_t)nvalid;
        s_red[1][wave] = kmax;
        s_red[2][wave] = kmin;
    }
    for (int i = tid; i < kBins1; i += NT) s_h1[i] = 0;
    if (tid == 0) s_ncand = 0;
    if (tid < kBins) s_h[1][tid] = 0;  // pass 1's histogram
    __syncthreads();
    int nv = 0;
    kmax = 0;
    kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        nv += (int)s_red[0][w];
        kmax = max(kmax, s_red[1][w]);
        kmin = min(kmin, s_red[2][w]);
    }

    // ---- threshold: select key > T (ge_mode: key >= T), plus the first need_eq keys == T
    bool ge_mode = true;
    uint32_t T = 1;  // nv <= k: every valid key
    int need_eq = 0;
    if (k == 0) {
        T = 0xFFFFFFFFu;  // nothing (no non-NaN key reaches it)
    } else if (nv > k) {
        const uint32_t diff = kmax ^ kmin;
        if (diff == 0) {
            ge_mode = false;
            T = kmax;
            need_eq = k;
        } else {
            int sb = 31 - __clz(diff);
            uint32_t prefix = (sb >= 31) ? 0u : (kmax & (~0u << (sb + 1)));
            int need = k;
            int pass = 0;
            while (true) {
                const int width = pass == 0 ? 11 : 8;
                const int nbits = sb + 1 < width ? sb + 1 : width;
                const int shift = sb + 1 - nbits;
                const uint32_t dmask = (1u << nbits) - 1u;
                int* hist = pass == 0 ? s_h1 : s_h[pass % 3];
                // clear the next pass's buffer: its last readers were two passes back and
                // finished before the previous pass's barrier
                if (pass > 0 && tid < kBins) s_h[(pass + 1) % 3][tid] = 0;
                if (pass == 0) {
                    // every valid key shares the prefix above sb.  An empty slot adds 0 to
                    // a bin picked by its slot number: no branch, and no pile-up of
                    // same-address atomics (one shared dummy bin serialized thousands of
                    // them when a row fills only part of the slots).
#pragma unroll
                    for (int i = 0; i < KPT; i++) {
                        const int bin = key[i] ? (int)((key[i] >> shift) & dmask) : (int)((e0 + i) & dmask);
                        atomicAdd(&hist[bin], key[i] ? 1 : 0);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < KPT; i++)
                        if ((live >> i) & 1) atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
                }
                __syncthreads();
                int bsel, above, cnt;
                if (pass == 0)
                    find_bin<kBins1, NT>(hist, need, s_fw[pass & 1], s_res[pass & 1], tid, lane, wave, &bsel, &above,
                                     &cnt);
                else
                    find_bin<kBins, NT>(hist, need, s_fw[pass & 1], s_res[pass & 1], tid, lane, wave, &bsel, &above,
                                    &cnt);
                prefix |= (uint32_t)bsel << shift;
                need -= above;
                // keep only the keys of the threshold bin for the next pass
                const uint32_t hm = ~0u << shift;
                uint64_t nl = 0;
#pragma unroll
                for (int i = 0; i < KPT; i++) nl |= (uint64_t)(((live >> i) & 1) && ((key[i] & hm) == prefix)) << i;
                live = nl;
                pass++;
                if (cnt == need) {
                    T = prefix;  // the whole bin is taken: keys >= prefix
                    break;
                }
                if (shift == 0) {
                    ge_mode = false;
                    T = prefix;
                    need_eq = need;
                    break;
                }
                if (cnt <= 64) {
                    // Few keys left in the threshold bin: gather them and let one wave
                    // find the need-th largest, T, directly (no further histogram pass).
                    // Then the selection is every key above T plus the first need - (keys
                    // above T in the bin) keys equal to T, in candidate order.
                    // (one LDS atomic per thread that holds any of them)
                    const int nlive = __builtin_popcountll(live);
                    if (nlive) {
                        int at = atomicAdd(&s_ncand, nlive);
#pragma unroll
                        for (int i = 0; i < KPT; i++)
                            if ((live >> i) & 1) s_cand[at++] = key[i];
                    }
                    __syncthreads();
                    if (wave == 0) {
                        // lane j holds candidate j; each lane counts the candidates above
                        // and at or above its own through register reads of every lane
                        const uint32_t v = lane < cnt ? s_cand[lane] : 0u;
                        int gt = 0, ge = 0;
                        for (int j = 0; j < cnt; j++) {
                            const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
                            gt += c > v;
                            ge += c >= v;
                        }
                        // exactly the lanes holding T satisfy gt < need <= ge; they agree
                        if (lane < cnt && gt < need && need <= ge) {
                            s_fin[0] = v;
                            s_fin[1] = (uint32_t)(need - gt);
                        }
                    }
                    __syncthreads();
                    ge_mode = false;
                    T = s_fin[0];
                    need_eq = (int)s_fin[1];
                    break;
                }
                sb = shift - 1;
            }
        }
    }

    // ---- ordered output: thread order is candidate order (blocked layout)
    int gt = 0, eq = 0;
    uint64_t selbits = 0, eqbits = 0;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
        const bool isgt = ge_mode ? (key[i] != 0 && key[i] >= T) : (key[i] > T);
        const bool iseq = !ge_mode && key[i] == T;
        gt += isgt;
        eq += iseq;
        selbits |= (uint64_t)isgt << i;
        eqbits |= (uint64_t)iseq << i;
    }
    // One scan of both counts: selected before this thread = keys above T before it plus
    // the equal keys before it, capped at need_eq; of its own equal keys it takes the
    // first need_eq - (equal keys before it).
    int gt_before, eq_before, nsel_gt, eq_tot;
    block_scan2<NW>(gt, eq, s_w, lane, wave, &gt_before, &eq_before, &nsel_gt, &eq_tot);
    int take = 0;
    if (!ge_mode) {
        take = need_eq - eq_before;
        take = take < 0 ? 0 : (take > eq ? eq : take);
        int seen = 0;
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const bool e = (eqbits >> i) & 1;
            selbits |= (uint64_t)(e && seen < take) << i;
            seen += e;
        }
    }
    int off = gt_before + (ge_mode ? 0 : (eq_before < need_eq ? eq_before : need_eq));
    const int nsel = nsel_gt + (ge_mode ? 0 : (eq_tot < need_eq ? eq_tot : need_eq));
    const int64_t row_out = (int64_t)row * nseg + seg;
    // Index outputs whose positions follow from the slot alone (score rows, block maxima,
    // pools with their block ids in registers) loop over the thread's selected slots only:
    // a thread holds few of them, and the general loop below branches on every slot.
    const bool slots_only = a.out_mode != OUT_LIST && SRC != SRC_LIST &&
                            (!(SRC == SRC_POOL || SRC == SRC_PGATHER) || bid_ok);
    if (slots_only) {
        int32_t* orow = a.out_idx + (int64_t)row * a.out_stride;
        for (uint64_t m = selbits; m; m &= m - 1) {
            const int i = __builtin_ctzll(m);
            int32_t pos;
            if (SRC == SRC_POOL || SRC == SRC_PGATHER) {
                int32_t blk = bid[0];
#pragma unroll
                for (int b8 = 1; b8 < bid_slots(KPT); b8++) blk = ((i >> 3) == b8) ? bid[b8] : blk;
                pos = (blk << 3) + (i & 7);
            } else {
                pos = (int32_t)(base + e0 + i);
            }
            orow[off++] = pos;
        }
    }
#pragma unroll
    for (int i = 0; i < KPT && !slots_only; i++) {
        if ((selbits >> i) & 1) {
            const int64_t e = e0 + i;
            int32_t pos;
            if (SRC == SRC_LIST)
                pos = (int32_t)a.in[(int64_t)row * a.nlists_prev * k + base + e].y;
            else if (SRC == SRC_POOL || SRC == SRC_PGATHER)
                pos = bid_ok ? (bid[i >> 3] << 3) + (i & 7) : (int32_t)pool_position(s, a.block_shift, prow, base + e);
            else
                pos = (int32_t)(base + e);
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
        const int64_t nblk = (ncol + a.block - 1) >> a.block_shift;
        int tot = nsel;
        if (nblk > 0) {
            if (tid == 0) a.out_idx[(int64_t)row * a.out_stride + nsel] = (int32_t)(nblk - 1);
            tot = nsel + 1;
        }
        for (int i = tot + tid; i < a.out_stride; i += NT) a.out_idx[(int64_t)row * a.out_stride + i] = -1;
        if (tid == 0) a.out_nblocks[row] = tot;
    }
}


}  // namespace csa2
