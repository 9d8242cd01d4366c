"""Seeded random sweeps of the scoring, selection and attention calls against the oracle.

Each case draws its own shapes: row counts on both sides of the many-row and whole-pool
launch shapes, score strides from a few entries to multi-level rows, reaches that cut the
newest block anywhere (or reach past the score row), k from 1 to 2048, pool capacities
below and above k, and scores with or without ties.  Index sets, pools, counts and index
scores must match bit for bit, attention within the bf16 tolerance of the other attention
tests; outputs start poisoned.  The case parameters are printed before each launch."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B

from gpu_util import DEV, POISON_I32, dev_cache, dev_rows, poison, quant_both, say
from test_gpu_fused import _both, _case
from test_gpu_parity import _attn_bf16_case, _check_bf16_attn, _run_attn_bf16, _score_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _rows_scores(rng, n, stride, ties):
    """Rows at positions R - 1 (m = 1); scores past a row's reach are NaN (never read)."""
    edge = [0, 1, 7, 8, 9, stride - 1, stride, stride + 5]
    R_list = [int(rng.choice(edge)) if rng.random() < 0.3 else int(rng.integers(0, stride + 1)) for _ in range(n)]
    R_list = [max(R, 0) for R in R_list]
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([max(R - 1, 0) for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(n, np.int64))
    scores = np.full((n, stride), np.nan, np.float32)
    for i, R in enumerate(R_list):
        v = (rng.standard_normal(min(R, stride)) * 30 + 150).astype(np.float32)
        if ties is not None:
            v = np.floor(v / ties).astype(np.float32) * ties
        scores[i, :min(R, stride)] = v
    return rows, cache, scores, R_list


@pytest.mark.parametrize("seed", range(12))
def test_random_topk_hier(orc, seed):
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.choice([1, 3, 17, 40]))
    stride = int(rng.choice([int(rng.integers(1, 4000)), int(rng.integers(4000, 70000)), int(rng.integers(70000, 140000))]))
    k = int(rng.choice([1, 3, 64, 511, 512, 1500, 2048]))
    max_blocks = int(rng.choice([1, 2, 8, 64, 600, 2048, 4096]))
    ties = [None, 2.0, 1000.0][int(rng.integers(0, 3))]
    rows, cache, scores, R_list = _rows_scores(rng, n, stride, ties)
    say("case: random topk_hier seed=%d n=%d stride=%d k=%d max_blocks=%d ties=%s R=%s" %
        (seed, n, stride, k, max_blocks, ties, R_list[:6]))
    out = (poison((n, k), torch.int32), poison((n, max_blocks), torch.int32), poison((n,), torch.int32))
    idx, blocks, nblocks = B.topk_hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k, 8,
                                       max_blocks, out=out)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, k, 8, max_blocks)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)


@pytest.mark.parametrize("seed", range(10))
def test_random_topk_flat(orc, seed):
    rng = np.random.default_rng(4100 + seed)
    n = int(rng.choice([1, 5, 33]))
    stride = int(rng.choice([int(rng.integers(1, 3000)), int(rng.integers(3000, 40000)),
                             int(rng.integers(40000, 300000))]))
    k = int(rng.choice([1, 2, 100, 512, 2047, 2048]))
    ties = [None, 4.0, 1000.0][int(rng.integers(0, 3))]
    rows, cache, scores, R_list = _rows_scores(rng, n, stride, ties)
    say("case: random topk seed=%d n=%d stride=%d k=%d ties=%s R=%s" % (seed, n, stride, k, ties, R_list[:6]))
    got = B.topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k,
                 out=poison((n, k), torch.int32)).cpu().numpy()
    assert np.array_equal(got, orc.topk(rows, cache, scores, k))


@pytest.mark.parametrize("seed", range(8))
def test_random_fused_pool_topk(orc, seed):
    """csa2_index_topk_pool equals csa2_index_score over the pool + csa2_topk on every row
    and the oracle on sampled rows, for decode-sized calls (segments and a list merge) and
    calls of 128 rows or more (whole pools)."""
    rng = np.random.default_rng(4200 + seed)
    many = bool(rng.random() < 0.4)
    n = int(rng.integers(128, 150)) if many else int(rng.integers(1, 24))
    H = int(rng.choice([16, 32, 64]))
    k = int(rng.choice([1, 100, 512, 2048]))
    nb_max = int(rng.choice([8, 64, 1000, 2048]))
    map_rows = bool(rng.random() < 0.5)
    R_hi = 3000 if many else 30000  # host key arrays stay a few hundred MB
    R_list = [int(rng.choice([0, 1, 8, 9, 2048, 2049])) if rng.random() < 0.25 else int(rng.integers(0, R_hi))
              for _ in range(n)]
    say("case: random fused pool top-k seed=%d n=%d H=%d k=%d max_blocks=%d map=%s R=%s" %
        (seed, n, H, k, nb_max, map_rows, R_list[:6]))
    rows, cache, keys, qi, w, pool, C = _case(4300 + seed, R_list, H, nb_max=nb_max, map_rows=map_rows)
    fused, two, sc = _both(rows, cache, keys, qi, w, pool, k)
    assert not np.any(fused == POISON_I32)
    assert np.array_equal(fused, two)
    ko, kso = orc.mx_quant(orc.E2M1, keys.numpy())
    sample = sorted(set([0, n - 1] + rng.choice(n, size=min(n, 2), replace=False).tolist()))
    rs = {key: v[sample] for key, v in rows.items()}
    pr = pool["row_map"][sample] if map_rows else np.array(sample)
    pool_o = dict(pool, blocks=pool["blocks"][pr], nblocks=pool["nblocks"][pr], row_map=None)
    s_o, bad = orc.index_score(rs, cache, qi[sample].float().numpy(), w[sample].numpy(), ko, key_scales=kso, heads=H,
                               dim=128, score_stride=8 * nb_max, pool=pool_o)
    assert bad == 0
    assert np.array_equal(fused[sample], orc.topk(rs, cache, s_o, k, pool=pool_o))


@pytest.mark.parametrize("seed", range(8))
def test_random_index_score(orc, seed):
    """Full-range MXFP4 index scores bit for bit on sampled rows; columns past the reach are
    -inf.  Row counts reach the paired-row launch (1,024 rows or more) in some cases."""
    rng = np.random.default_rng(4400 + seed)
    nreq = int(rng.integers(1, 4))
    S = tuple(int(rng.integers(1, 5000)) for _ in range(nreq))
    m = int(rng.choice([1, 2]))
    H = int(rng.choice([16, 32, 64]))
    per = int(rng.choice([3, 40, 600]))
    rows, cache, keys, q, w = _score_case(4500 + seed, S, m, H, 128, min(per, min(S)))
    n = len(rows["req_of_row"])
    stride = int(rng.choice([max(cache["n_entries"]), int(rng.integers(1, 3000))]))
    stride = max(stride, 1)
    say("case: random index_score seed=%d S=%s m=%d H=%d rows=%d stride=%d" % (seed, S, m, H, n, stride))
    (kd, ksd), (ko, kso) = quant_both(orc, B.MXFP4, orc.E2M1, keys)
    s_d = B.index_score(dev_rows(rows), dev_cache(cache), q.to(DEV), w.to(DEV), B.IndexKeys(kd, ksd, 128),
                        scores=poison((n, stride), torch.float32))
    got = s_d.cpu().numpy()
    sample = sorted(set([0, n - 1] + rng.choice(n, size=min(n, 10), replace=False).tolist()))
    rs = {key: v[sample] for key, v in rows.items()}
    s_o, bad = orc.index_score(rs, cache, q[sample].float().numpy(), w[sample].numpy(), ko, key_scales=kso, heads=H,
                               dim=128, score_stride=stride)
    assert bad == 0
    for j, i in enumerate(sample):
        r, p = rows["req_of_row"][i], rows["pos_of_row"][i]
        R = min((p + 1) // m, cache["n_entries"][r])
        assert np.all(got[i, R:] == -np.inf), "row %d: columns past R=%d not -inf" % (i, R)
        assert np.array_equal(got[i, :R], s_o[j, :R]), "row %d (p=%d R=%d) differs" % (i, p, R)


@pytest.mark.parametrize("seed", range(8))
def test_random_attn_bf16(orc, seed):
    """Sparse + window attention against the oracle's float64 attention: random request
    lengths, ratio, heads, k (with -1 holes), FP8 or bf16 window, window floors, sinks and
    the FP4 main KV format."""
    rng = np.random.default_rng(4600 + seed)
    nreq = int(rng.integers(1, 3))
    S = tuple(int(rng.integers(1, 3000)) for _ in range(nreq))
    m = int(rng.choice([1, 2]))
    H = int(rng.choice([16, 32, 64, 80, 128]))
    k = int(rng.choice([0, 1, 17, 64, 512, 1000, 2048]))
    swa_fp8 = bool(rng.random() < 0.6)
    tail = bool(rng.random() < 0.4)
    kv_fp4 = bool(rng.random() < 0.3)
    sink = (rng.standard_normal(H) * 2).astype(np.float32) if rng.random() < 0.3 else None
    sm_scale = float(rng.choice([1 / math.sqrt(512), 0.02, 0.3]))
    say("case: random attention seed=%d S=%s m=%d H=%d k=%d fp8=%s tail=%s fp4kv=%s sink=%s scale=%g" %
        (seed, S, m, H, k, swa_fp8, tail, kv_fp4, sink is not None, sm_scale))
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(4700 + seed, S, m, H, k, min(5, min(S)),
                                                            win_lo_tail=tail)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, H, sm_scale,
                                            swa_fp8=swa_fp8, sink=sink, kv_fp4=kv_fp4)
    _check_bf16_attn(got, ref, lse_g, lse_r)
