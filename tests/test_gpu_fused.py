"""GPU parity of the fused pool scoring + top-k (csa2_index_topk_pool).

Its result is defined as csa2_index_score over the pool followed by csa2_topk over those
scores, so the index sets must equal that two-launch path and the oracle's index sets bit
for bit: pools of every size up to 2048 blocks (partial pools, the newest block cut by the
reach, empty rows), a row map, heads 16 / 32 / 64, k from 1 to 2048, and rows whose scores
tie; decode-sized calls (pool segments and a list merge) and calls over 128 rows or more
(whole pools per workgroup)."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B
from compressed_sparse_attention_fp4_amd import synth

from gpu_util import DEV, POISON_I32, dev_cache, dev_rows, i32, poison, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _case(seed, R_list, H, nb_max=2048, map_rows=False):
    """Rows at positions R - 1 (m = 1) with pools drawn over their reachable blocks (all of
    them when they fit, else a random set plus the newest block)."""
    rng = np.random.default_rng(seed)
    n = len(R_list)
    C = max(R_list + [1])
    geom = synth.Geometry([max(R, 1) for R in R_list], 1)
    rows = dict(req_of_row=np.arange(n, dtype=np.int32), pos_of_row=np.array([max(R, 1) - 1 for R in R_list], np.int32))
    n_ent = np.array([R for R in R_list], np.int32)
    cache = dict(ratio_m=1, n_entries=n_ent, row_start=np.array(geom.row_start))
    prows = 2 * n if map_rows else n
    blocks = np.full((prows, nb_max), -1, np.int32)
    nblocks = np.zeros(prows, np.int32)
    row_map = rng.permutation(prows)[:n].astype(np.int32) if map_rows else np.arange(n, dtype=np.int32)
    for i, R in enumerate(R_list):
        nb = (R + 7) // 8
        pick = list(range(nb)) if nb <= nb_max else \
            sorted(set(rng.choice(nb - 1, nb_max - 1, replace=False).tolist()) | {nb - 1})
        blocks[row_map[i], :len(pick)] = pick
        nblocks[row_map[i]] = len(pick)
    keys = synth.normal((geom.total_entries, 128), seed, "index_keys")
    qi = synth.normal_bf16((n, H, 128), seed, "index_q")
    w = synth.uniform((n, H), seed, "index_w")
    pool = dict(blocks=blocks, nblocks=nblocks, block=8, max_blocks=nb_max, row_map=row_map if map_rows else None)
    return rows, cache, keys, qi, w, pool, C


def _both(rows, cache, keys, qi, w, pool, k):
    """Fused and two-launch results on the device (outputs poisoned)."""
    kd, ksd = B.quant_mx(B.MXFP4, keys.to(DEV))
    K = B.IndexKeys(kd, ksd, 128)
    rd, cd = dev_rows(rows), dev_cache(cache)
    pd = B.Pool(i32(pool["blocks"]).to(DEV), i32(pool["nblocks"]).to(DEV), 8,
                None if pool["row_map"] is None else i32(pool["row_map"]).to(DEV))
    n = len(rows["req_of_row"])
    fused = B.index_topk_pool(rd, cd, qi.to(DEV), w.to(DEV), K, pd, k, out=poison((n, k), torch.int32))
    sc = B.index_score(rd, cd, qi.to(DEV), w.to(DEV), K, pool=pd, score_stride=8 * pool["max_blocks"])
    two = B.topk(rd, cd, sc, k, pool=pd, out=poison((n, k), torch.int32))
    return fused.cpu().numpy(), two.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("H", [64, 32, 16])
@pytest.mark.parametrize("k", [512, 1, 2048])
def test_fused_equals_two_launches_and_oracle(orc, H, k):
    say("case: fused pool top-k H=%d k=%d" % (H, k))
    R_list = [65536, 16384, 16390, 9000, 2049, 100, 8, 1, 0, 30000] * 2
    rows, cache, keys, qi, w, pool, C = _case(300 + H + k, R_list, H)
    fused, two, sc = _both(rows, cache, keys, qi, w, pool, k)
    assert not np.any(fused == POISON_I32)
    assert np.array_equal(fused, two)
    ko, kso = orc.mx_quant(orc.E2M1, keys.numpy())
    sample = [0, 2, 4, 6, 7, 8, 9]
    rs = {key: v[sample] for key, v in rows.items()}
    pool_o = dict(pool, blocks=pool["blocks"][sample], nblocks=pool["nblocks"][sample])
    s_o, bad = orc.index_score(rs, cache, qi[sample].float().numpy(), w[sample].numpy(), ko, key_scales=kso, heads=H,
                               dim=128, score_stride=8 * pool["max_blocks"], pool=pool_o)
    assert bad == 0
    i_o = orc.topk(rs, cache, s_o, k, pool=pool_o)
    assert np.array_equal(fused[sample], i_o)


@pytest.mark.parametrize("H,k,map_rows,nb_max", [(64, 512, False, 2048), (16, 2048, True, 2048), (32, 1, False, 2048),
                                                  (64, 128, True, 64), (64, 512, False, 1000)])
def test_fused_whole_pools(orc, H, k, map_rows, nb_max):
    """Launches over 128 rows or more score and select each row's whole pool in one
    workgroup (no list merge): the same index sets as the two launches and the oracle,
    for full and small pools."""
    say("case: fused pool top-k over 160 rows (whole pools) H=%d k=%d map=%s max_blocks=%d" % (H, k, map_rows, nb_max))
    R_list = [16390, 3000, 2049, 100, 8, 1, 0, 5000] * 20
    rows, cache, keys, qi, w, pool, C = _case(330 + H + k + nb_max, R_list, H, nb_max=nb_max, map_rows=map_rows)
    fused, two, sc = _both(rows, cache, keys, qi, w, pool, k)
    assert not np.any(fused == POISON_I32)
    assert np.array_equal(fused, two)
    ko, kso = orc.mx_quant(orc.E2M1, keys.numpy())
    sample = [0, 1, 2, 6, 7, 159]
    rs = {key: v[sample] for key, v in rows.items()}
    pr = pool["row_map"][sample] if map_rows else np.array(sample)
    pool_o = dict(pool, blocks=pool["blocks"][pr], nblocks=pool["nblocks"][pr], row_map=None)
    s_o, bad = orc.index_score(rs, cache, qi[sample].float().numpy(), w[sample].numpy(), ko, key_scales=kso, heads=H,
                               dim=128, score_stride=8 * pool["max_blocks"], pool=pool_o)
    assert bad == 0
    i_o = orc.topk(rs, cache, s_o, k, pool=pool_o)
    assert np.array_equal(fused[sample], i_o)


def test_fused_row_map_and_small_pools(orc):
    say("case: fused pool top-k through a row map, max_blocks 64 and 1000")
    for nb_max in (64, 1000):
        rows, cache, keys, qi, w, pool, C = _case(311 + nb_max, [65536, 700, 20000, 513, 0, 9999], 64, nb_max=nb_max,
                                                  map_rows=True)
        fused, two, _ = _both(rows, cache, keys, qi, w, pool, 128)
        assert np.array_equal(fused, two)


def test_fused_ties(orc):
    """Index q of zeros: every reachable pool score is +0, so the top-k are the lowest pool
    positions (ties to the lower position), the same on both paths."""
    say("case: fused pool top-k with all scores equal")
    rows, cache, keys, qi, w, pool, C = _case(321, [65536, 5000, 16384], 64)
    qi = torch.zeros_like(qi)
    fused, two, sc = _both(rows, cache, keys, qi, w, pool, 512)
    assert np.array_equal(fused, two)
    for i in range(3):
        nb = pool["nblocks"][i]
        pos = (pool["blocks"][i, :nb, None] * 8 + np.arange(8)[None, :]).ravel()
        pos = np.sort(pos[pos < [65536, 5000, 16384][i]])
        assert fused[i].tolist() == pos[:512].tolist()
