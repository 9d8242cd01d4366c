"""Pins of the oracle's top-k and hierarchical selection (CPU only).

Pages: "DeepSeek V4.1 Flash modeling", section "Hierarchical Sparse Indexer" (top-512;
blocks of 8 positions scored by their maximum; at most 2,048 blocks, i.e. at most
16,384 candidates); "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 2
(the block holding the newest position is always kept; the pass also takes its own
top-512 from all reachable positions; nothing is excluded when every reachable
position fits the 16,384 budget).  Ties go to the lowest index (the workload definition; the pages are silent).

Pins: brute force with Python's sort on tiny inputs (tie-heavy too), and the
invariants the pages state.
"""
import numpy as np
import pytest


def _rows(R_list, m=1):
    # one request per row, query at the last position so that R = n_entries
    n = len(R_list)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([r * m + m - 1 if r > 0 else 0 for r in R_list]))
    cache = dict(ratio_m=m, n_entries=np.array(R_list), row_start=np.cumsum([0] + R_list[:-1]))
    return rows, cache


def _brute_topk(s, k):
    order = sorted(range(len(s)), key=lambda j: (-(s[j] + 0.0), j))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("tie_levels", [None, 3, 1])
def test_topk_brute_force(orc, tie_levels):
    rng = np.random.default_rng(21 if tie_levels is None else tie_levels)
    R_list = [0, 1, 7, 33, 64, 65, 100, 200]
    rows, cache = _rows(R_list)
    stride = 256
    scores = np.full((len(R_list), stride), np.nan, np.float32)
    for i, R in enumerate(R_list):
        v = rng.standard_normal(R).astype(np.float32)
        if tie_levels is not None:
            v = np.floor(v * tie_levels).astype(np.float32)
        v[v == 0] = rng.choice([0.0, -0.0], size=int(np.sum(v == 0)))  # mix +0 and -0
        scores[i, :R] = v
    for k in (1, 5, 64, 128):
        out = orc.topk(rows, cache, scores, k)
        for i, R in enumerate(R_list):
            assert list(out[i]) == _brute_topk(list(scores[i, :R]), k), (i, k)


def test_topk_invariants(orc):
    rng = np.random.default_rng(22)
    R_list = [300, 511, 512, 513, 1000]
    rows, cache = _rows(R_list)
    scores = np.full((len(R_list), 1024), np.nan, np.float32)
    for i, R in enumerate(R_list):
        scores[i, :R] = rng.standard_normal(R)
    k = 512
    out = orc.topk(rows, cache, scores, k)
    for i, R in enumerate(R_list):
        sel = out[i][out[i] >= 0]
        assert len(sel) == min(k, R)
        assert np.all(np.diff(sel) > 0)
        if R > k:
            chosen = set(sel.tolist())
            worst_sel = min((scores[i, j], -j) for j in chosen)
            best_rest = max((scores[i, j], -j) for j in range(R) if j not in chosen)
            assert best_rest < worst_sel


def _brute_hier(s, B, NB):
    R = len(s)
    nblk = (R + B - 1) // B
    if nblk <= NB:
        return list(range(nblk))
    newest = nblk - 1
    bmax = [max(s[b * B:min(R, b * B + B)]) + 0.0 for b in range(newest)]
    order = sorted(range(newest), key=lambda b: (-bmax[b], b))
    return sorted(order[:NB - 1]) + [newest]


@pytest.mark.parametrize("ties", [False, True])
def test_hier_brute_force(orc, ties):
    rng = np.random.default_rng(31 + ties)
    B, NB, k = 8, 4, 5
    R_list = [0, 3, 8, 9, 31, 32, 33, 40, 57, 100]
    rows, cache = _rows(R_list)
    scores = np.full((len(R_list), 128), np.nan, np.float32)
    for i, R in enumerate(R_list):
        v = rng.standard_normal(R).astype(np.float32)
        if ties:
            v = np.floor(v).astype(np.float32)
        scores[i, :R] = v
    idx, blocks, nblocks = orc.topk_hier(rows, cache, scores, k, block=B, max_blocks=NB)
    for i, R in enumerate(R_list):
        want = _brute_hier(list(scores[i, :R]), B, NB)
        assert nblocks[i] == len(want)
        assert list(blocks[i, :nblocks[i]]) == want
        assert np.all(blocks[i, nblocks[i]:] == -1)
        assert list(idx[i]) == _brute_topk(list(scores[i, :R]), k)


def test_hier_invariants(orc):
    """Pool <= NB*B; newest block kept; everything kept when it fits; and (derived)
    the flat top-k lies inside the pool whenever NB-1 >= k."""
    rng = np.random.default_rng(33)
    B, NB, k = 8, 16, 12
    R_list = [1, 127, 128, 129, 300, 1000]
    rows, cache = _rows(R_list)
    scores = np.full((len(R_list), 1024), np.nan, np.float32)
    for i, R in enumerate(R_list):
        scores[i, :R] = rng.standard_normal(R)
    idx, blocks, nblocks = orc.topk_hier(rows, cache, scores, k, block=B, max_blocks=NB)
    for i, R in enumerate(R_list):
        nb = nblocks[i]
        bl = blocks[i, :nb]
        assert nb <= NB
        assert bl[-1] == (R + B - 1) // B - 1
        if R <= NB * B:
            assert list(bl) == list(range((R + B - 1) // B))
        pool_pos = {b * B + u for b in bl for u in range(B) if b * B + u < R}
        assert set(idx[i][idx[i] >= 0].tolist()) <= pool_pos


def test_pool_topk_matches_restricted_brute_force(orc):
    rng = np.random.default_rng(34)
    B, NB, k = 8, 6, 10
    R_list = [50, 90, 200]
    rows, cache = _rows(R_list)
    scores = np.full((len(R_list), NB * B), np.nan, np.float32)
    blocks = np.full((len(R_list), NB), -1, np.int32)
    nblocks = np.zeros(len(R_list), np.int32)
    full = []
    for i, R in enumerate(R_list):
        s = rng.standard_normal(R).astype(np.float32)
        full.append(s)
        nb = (R + B - 1) // B
        pick = sorted(set(rng.choice(nb - 1, size=NB - 1, replace=False).tolist()) | {nb - 1})
        blocks[i, :len(pick)] = pick
        nblocks[i] = len(pick)
        for c in range(len(pick) * B):
            j = pick[c // B] * B + c % B
            scores[i, c] = s[j] if j < R else -np.inf
    pool = dict(blocks=blocks, nblocks=nblocks, block=B, max_blocks=NB)
    out = orc.topk(rows, cache, scores, k, pool=pool)
    for i, R in enumerate(R_list):
        cand = [blocks[i, c // B] * B + c % B for c in range(nblocks[i] * B)]
        cand = [j for j in cand if j < R]
        order = sorted(cand, key=lambda j: (-float(full[i][j]), j))
        want = sorted(order[:k]) + [-1] * max(0, k - len(cand))
        assert list(out[i]) == want
