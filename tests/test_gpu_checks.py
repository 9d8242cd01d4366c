"""csa2_check_inputs: the device-side check of the stated device-array preconditions.

Seeded random rows, cache geometry, pools and index sets, valid or with violations
planted at random, are checked on the device; the error word must equal the bits a
plain host evaluation of the same preconditions gives (include/csa2.h, csa2_check_inputs).
Valid inputs from the library's own selection calls give 0.  The check kernel only
compares the planted values; none of them reaches a compute kernel."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B

from gpu_util import DEV, dev_cache, dev_rows, i32, say

pytestmark = pytest.mark.gpu

I32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def expected_bits(rows, cache, pool, pool_rows, sel, sel_map):
    """The preconditions evaluated on the host, bit by bit."""
    req, pos, lo = rows["req_of_row"], rows["pos_of_row"], rows.get("win_lo")
    ne, rs, m = cache["n_entries"], cache["row_start"], cache["ratio_m"]
    nreq = len(ne)
    bad = 0
    if np.any(ne < 0) or np.any(rs < 0):
        bad |= B.BAD_CACHE
    for q in range(len(req)):
        r, p = int(req[q]), int(pos[q])
        ok = 0 <= r < nreq
        if not ok:
            bad |= B.BAD_REQ
        if p < 0:
            bad |= B.BAD_POS
        if lo is not None and (lo[q] < 0 or lo[q] > p):
            bad |= B.BAD_WIN_LO
        if not ok or p < 0:
            continue
        R = 0 if ne[r] < 0 else min((p + 1) // m, int(ne[r]))
        if sel is not None:
            srow = int(sel_map[q]) if sel_map is not None else q
            if not 0 <= srow < sel.shape[0]:
                bad |= B.BAD_SEL_MAP
            else:
                s = sel[srow].astype(np.int64)
                if np.any((s != -1) & ((s < 0) | (s >= R))):
                    bad |= B.BAD_SEL
        if pool is not None:
            prow = int(pool["row_map"][q]) if pool.get("row_map") is not None else q
            if not 0 <= prow < pool_rows:
                bad |= B.BAD_POOL_MAP
                continue
            nb = int(pool["nblocks"][prow])
            if nb < 0 or nb > pool["blocks"].shape[1]:
                bad |= B.BAD_POOL
                continue
            b = pool["blocks"][prow, :nb].astype(np.int64)
            if np.any(b < 0) or np.any(b > I32_MAX // pool["block"] - 1) or np.any(np.diff(b) <= 0):
                bad |= B.BAD_POOL
    return bad


def _valid_case(rng, n=300, nreq=12, m=2, k=64, nb_max=32):
    ne = rng.integers(0, 3000, nreq).astype(np.int32)
    rs = np.concatenate([[0], np.cumsum(ne)[:-1]]).astype(np.int64)
    req = rng.integers(0, nreq, n).astype(np.int32)
    pos = np.array([rng.integers(0, 2 * int(ne[r]) + 40) for r in req], np.int32)
    lo = np.array([rng.integers(0, p + 1) for p in pos], np.int32)
    prows = n + 7
    row_map = rng.permutation(prows)[:n].astype(np.int32)
    blocks = np.full((prows, nb_max), -1, np.int32)
    nblocks = np.zeros(prows, np.int32)
    for q in range(n):
        R = min((int(pos[q]) + 1) // m, int(ne[req[q]]))
        nbk = (R + 7) // 8
        take = min(nbk, int(rng.integers(0, nb_max + 1)))
        ids = np.sort(rng.choice(nbk, take, replace=False)) if take else np.zeros(0, np.int64)
        blocks[row_map[q], :take] = ids
        nblocks[row_map[q]] = take
    sel_rows = n + 5
    sel_map = rng.permutation(sel_rows)[:n].astype(np.int32)
    sel = np.full((sel_rows, k), -1, np.int32)
    for q in range(n):
        R = min((int(pos[q]) + 1) // m, int(ne[req[q]]))
        t = min(R, k)
        if t:
            sel[sel_map[q], :t] = rng.choice(R, t, replace=False)
    rows = dict(req_of_row=req, pos_of_row=pos, win_lo=lo)
    cache = dict(ratio_m=m, n_entries=ne, row_start=rs)
    pool = dict(blocks=blocks, nblocks=nblocks, block=8, row_map=row_map)
    return rows, cache, pool, prows, sel, sel_map


def _plant(rng, rows, cache, pool, prows, sel, sel_map):
    """One random precondition violation."""
    n = len(rows["req_of_row"])
    q = int(rng.integers(0, n))
    kind = int(rng.integers(0, 10))
    if kind == 0:
        rows["req_of_row"][q] = rng.choice([-1, len(cache["n_entries"]), 1 << 30])
    elif kind == 1:
        rows["pos_of_row"][q] = -int(rng.integers(1, 5))
    elif kind == 2:
        rows["win_lo"][q] = rows["pos_of_row"][q] + 1 if rng.integers(0, 2) else -1
    elif kind == 3:
        r = int(rng.integers(0, len(cache["n_entries"])))
        if rng.integers(0, 2):
            cache["n_entries"][r] = -1
        else:
            cache["row_start"][r] = -5
    elif kind == 4:
        pool["row_map"][q] = rng.choice([-1, prows, prows + 100])
    elif kind == 5:
        p = int(pool["row_map"][q])
        pool["nblocks"][p] = rng.choice([-1, pool["blocks"].shape[1] + 1])
    elif kind == 6:
        p = int(pool["row_map"][q])
        nb = int(pool["nblocks"][p])
        if nb >= 2:
            pool["blocks"][p, nb - 1] = pool["blocks"][p, nb - 2]  # not strictly ascending
        elif nb == 1:
            pool["blocks"][p, 0] = rng.choice([-3, I32_MAX // 8])
    elif kind == 7:
        sel_map[q] = rng.choice([-1, sel.shape[0]])
    elif kind == 8:
        sel[sel_map[q], int(rng.integers(0, sel.shape[1]))] = rng.choice([-2, 1 << 30])
    else:
        sel[sel_map[q], int(rng.integers(0, sel.shape[1]))] = 10 ** 6  # past any reach here


def _device_word(rows, cache, pool, prows, sel, sel_map):
    pd = B.Pool(i32(pool["blocks"]).to(DEV), i32(pool["nblocks"]).to(DEV), pool["block"],
                i32(pool["row_map"]).to(DEV))
    assert pd.blocks.shape[0] == prows
    word = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)  # cleared by the call
    B.check_inputs(dev_rows(rows), dev_cache(cache), pd, i32(sel).to(DEV), i32(sel_map).to(DEV), word=word)
    return int(word.cpu().item()) & 0xFFFFFFFF


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6])
def test_check_inputs_matches_host_evaluation(seed):
    rng = np.random.default_rng(700 + seed)
    case = _valid_case(rng)
    say("case: check_inputs seed %d, valid inputs" % seed)
    assert expected_bits(*case[:4], case[4], case[5]) == 0
    assert _device_word(*case) == 0
    for trial in range(6):
        case = _valid_case(rng)
        for _ in range(int(rng.integers(1, 4))):
            _plant(rng, *case)
        want = expected_bits(*case[:4], case[4], case[5])
        say("  trial %d: expected bits 0x%x" % (trial, want))
        assert _device_word(*case) == want


def test_check_inputs_on_selection_outputs():
    """Pools and index sets from csa2_topk_hier over valid rows pass the check."""
    say("case: check_inputs on csa2_topk_hier outputs")
    rng = np.random.default_rng(77)
    nreq, m = 6, 2
    ne = rng.integers(100, 9000, nreq).astype(np.int32)
    rs = np.concatenate([[0], np.cumsum(ne)[:-1]]).astype(np.int64)
    req = np.repeat(np.arange(nreq), 4).astype(np.int32)
    pos = np.array([rng.integers(0, 2 * int(ne[r])) for r in req], np.int32)
    rows = dict(req_of_row=req, pos_of_row=pos)
    cache = dict(ratio_m=m, n_entries=ne, row_start=rs)
    C = int(ne.max())
    sc = torch.randn((len(req), C), generator=torch.Generator().manual_seed(5)).to(DEV)
    rd, cd = dev_rows(rows), dev_cache(cache)
    idx, pb, pn = B.topk_hier(rd, cd, sc, 512, 8, 256)
    word = B.check_inputs(rd, cd, B.Pool(pb, pn, 8), idx)
    assert int(word.cpu().item()) == 0
