"""GPU parity of every entry point against the oracle, on seeded inputs sized so that the
oracle finishes in seconds while the kernels still cross several tiles and a ragged
tail.  Index sets and scores must match bit for bit; attention outputs within
|g - r| <= atol + rtol |r| (bf16: 2e-2 + 1e-2 |r|, plus a per-row relative L2 error
<= 1e-2; fp32: 1e-4 + 1e-4 |r|)."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B
from compressed_sparse_attention_fp4_amd import synth

from gpu_util import (DEV, POISON_I32, allclose_report, dev_cache, dev_rows, fp4_decode_torch, i32, i64, poison,
                      quant_both, quant_fp4_both, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _topk(rows_d, cache_d, scores_d, k, pool=None):
    """csa2_topk into a poisoned output (every slot must be written: positions or -1)."""
    out = poison((rows_d.n, k), torch.int32)
    return B.topk(rows_d, cache_d, scores_d, k, pool=pool, out=out)


def _hier(rows_d, cache_d, scores_d, k, block, max_blocks):
    """csa2_topk_hier into poisoned outputs."""
    n = rows_d.n
    out = (poison((n, k), torch.int32), poison((n, max_blocks), torch.int32), poison((n,), torch.int32))
    return B.topk_hier(rows_d, cache_d, scores_d, k, block, max_blocks, out=out)


# ------------------------------------------------------------------ quantizer
def test_quant_mx_all_bf16_patterns(orc):
    say("case: quant_mx over every bf16 bit pattern (finite), MXFP4 and MXFP8")
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals)]
    vals = vals[: (vals.numel() // 32) * 32]
    # shuffle so blocks mix magnitudes (several shared exponents per pattern)
    g = torch.Generator().manual_seed(0)
    for rep in range(3):
        x = vals[torch.randperm(vals.numel(), generator=g)].reshape(-1, 32).contiguous()
        quant_both(orc, B.MXFP4, orc.E2M1, x)
        quant_both(orc, B.MXFP8_E4M3, orc.E4M3, x)
    # also from bf16 input directly
    x = vals[torch.randperm(vals.numel(), generator=g)].reshape(-1, 32).contiguous()
    cd, sd = B.quant_mx(B.MXFP4, x.to(torch.bfloat16).to(DEV))
    co, so = orc.mx_quant(orc.E2M1, x.numpy())
    assert np.array_equal(cd.cpu().numpy(), co) and np.array_equal(sd.cpu().numpy(), so)


def _every_value_under_every_scale():
    """Blocks of 32 bf16 values: the first pins the block's shared exponent e (its maximum
    magnitude lies in [2^(e+2), 2^(e+3)), or below 2^-125 for the clamped e = -127), the
    other 31 run through every finite bf16 value whose magnitude does not exceed it, so
    every (value, e) pair a block can produce is quantized once."""
    b = np.arange(65536, dtype=np.uint32)
    expo = (b >> 7) & 0xFF
    finite = expo < 255
    blocks = []
    for e in range(-127, 126):
        if e == -127:
            amax_bits, lim = 0x00FF, 0x00FF                      # just below 2^-125
        else:
            amax_bits = ((e + 2 + 127) << 7) | 0x7F              # 1.9921875 * 2^(e + 2)
            lim = amax_bits
        mag = b & 0x7FFF
        xs = b[finite & (mag <= lim)].astype(np.uint16)
        pad = (-len(xs)) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        head = np.full((xs.shape[0], 1), amax_bits, np.uint16)
        blocks.append(np.concatenate([head, xs], axis=1))
    allb = np.concatenate(blocks).astype(np.uint16)
    return torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16)


def test_quant_mxfp4_every_value_under_every_scale(orc):
    """The E2M1 rounding of csa2_quant_mx (and of every kernel that quantizes index q or
    keys in-kernel, which share its block routine) equals the oracle's for every finite
    bf16 value under every shared exponent a block can give it."""
    say("case: quant_mx MXFP4, every finite bf16 value under every shared exponent")
    x = _every_value_under_every_scale()
    cd, sd = B.quant_mx(B.MXFP4, x.to(DEV))
    co, so = orc.mx_quant(orc.E2M1, x.float().numpy())
    assert np.array_equal(sd.cpu().numpy(), so), "scales"
    assert np.array_equal(cd.cpu().numpy(), co), "codes"


def test_quant_mx_ties_and_ranges(orc):
    say("case: quant_mx ties, saturation, zero blocks, tiny and huge magnitudes")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4096, 32)).astype(np.float32)
    x *= (2.0 ** rng.integers(-120, 120, size=(4096, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :8] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x[2, :4] = [448.0, 460.0, 470.0, 511.0]
    x[3] = -0.0
    quant_both(orc, B.MXFP4, orc.E2M1, torch.from_numpy(x))
    quant_both(orc, B.MXFP8_E4M3, orc.E4M3, torch.from_numpy(x))


# ---------------------------------------------------------------- tail layout
def test_replay_tail_layout(orc):
    say("case: replay tail layout, page examples and a random batch")
    cases = [([8192], [8192]), ([64], [8256]), ([8192] * 4, [8192, 16384, 24576, 32768]),
             (synth.C2_EXTENDS, [8192] * 8), ([0, 1, 127, 128, 129, 5, 0], [10, 50, 127, 1000, 129, 5, 7])]
    rng = np.random.default_rng(4)
    e = rng.integers(0, 400, size=700)
    cases.append((e.tolist(), (e + rng.integers(0, 1000, size=700)).tolist()))
    for ext, seq in cases:
        nreq = len(ext)
        cap = 128 * nreq
        t = dict(tail_len=poison((nreq,), torch.int32), tail_row_start=poison((nreq + 1,), torch.int32))
        for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
            t[name] = poison((cap,), torch.int32)
        B.replay_tail_layout(i32(ext).to(DEV), i32(seq).to(DEV), 128, out=t)
        o = orc.replay_tail_layout(ext, seq, 128)
        tot = int(o["tail_row_start"][-1])
        assert t["tail_len"].cpu().numpy().tolist() == o["tail_len"].tolist()
        assert t["tail_row_start"].cpu().numpy().tolist() == o["tail_row_start"].tolist()
        for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
            assert np.array_equal(t[name][:tot].cpu().numpy(), o[name]), name


# --------------------------------------------------------------------- scores
def _score_case(seed, S, m, H, D, nrows_per_req, fp4=True):
    rng = np.random.default_rng(seed)
    geom = synth.Geometry(list(S), m)
    req, pos = [], []
    for r, s in enumerate(S):
        special = [0, 1, 2, m * 16 - 1, m * 16, s - 1, s - 2, min(s - 1, 8191), min(s - 1, 8192)]
        pick = set(p for p in special if 0 <= p < s) | set(rng.choice(s, size=nrows_per_req, replace=False).tolist())
        for p in sorted(pick):
            req.append(r)
            pos.append(p)
    rows = dict(req_of_row=np.array(req), pos_of_row=np.array(pos))
    cache = dict(ratio_m=m, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    keys = synth.normal((geom.total_entries, D), seed, "index_keys")
    n = len(req)
    if fp4:
        q = synth.normal_bf16((n, H, D), seed, "index_q")
    else:
        q = synth.normal((n, H, D), seed, "index_q")
    w = synth.uniform((n, H), seed, "index_w")
    return rows, cache, keys, q, w


@pytest.mark.parametrize("H", [64, 32, 16])
def test_index_score_mxfp4_full_range(orc, H):
    say("case: index_score MXFP4 full range, heads=%d" % H)
    rows, cache, keys, q, w = _score_case(10 + H, (3000, 1234, 77), 2, H, 128, 12)
    stride = 1536
    (kd, ksd), (ko, kso) = quant_both(orc, B.MXFP4, orc.E2M1, keys)
    n = len(rows["req_of_row"])
    s_d = B.index_score(dev_rows(rows), dev_cache(cache), q.to(DEV), w.to(DEV), B.IndexKeys(kd, ksd, 128),
                        scores=poison((n, stride), torch.float32))
    s_o, bad = orc.index_score(rows, cache, q.float().numpy(), w.numpy(), ko, key_scales=kso, heads=H, dim=128,
                               score_stride=stride)
    assert bad == 0
    got = s_d.cpu().numpy()
    for i in range(len(rows["req_of_row"])):
        r, p = rows["req_of_row"][i], rows["pos_of_row"][i]
        R = min((p + 1) // 2, cache["n_entries"][r])
        assert np.all(got[i, R:] == -np.inf), "row %d: columns past R=%d not -inf" % (i, R)
        if not np.array_equal(got[i, :R], s_o[i, :R]):
            bad_cols = np.nonzero(got[i, :R] != s_o[i, :R])[0]
            raise AssertionError("row %d (p=%d R=%d): %d columns differ, first %s: gpu %r oracle %r" % (
                i, p, R, len(bad_cols), bad_cols[:8], got[i, bad_cols[:4]], s_o[i, bad_cols[:4]]))


@pytest.mark.parametrize("H", [64, 16])
def test_index_score_mxfp4_row_pairs(orc, H):
    """Full-range calls over 1024 rows or more score rows in pairs that share key tiles
    when both rows belong to one request.  Requests of odd lengths put pairs across
    request boundaries (scored one row after the other) and the row count is odd: every
    row must equal the same row scored in calls of fewer rows (one row per workgroup),
    bit for bit, and sampled rows the oracle."""
    say("case: index_score MXFP4 in row pairs, heads=%d" % H)
    rng = np.random.default_rng(40 + H)
    lens = [301, 4, 1, 516, 233, 77, 1]           # prefill rows per request (sum 1133, odd)
    S = [600, 5, 2, 1100, 240, 77, 3000]
    m = 2
    geom = synth.Geometry(S, m)
    req = np.concatenate([np.full(L, r) for r, L in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.sort(rng.choice(s, size=L, replace=False)) for s, L in zip(S, lens)]).astype(np.int32)
    rows = dict(req_of_row=req, pos_of_row=pos)
    cache = dict(ratio_m=m, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    n = len(req)
    assert n >= 1024 and n % 2 == 1
    keys = synth.normal((geom.total_entries, 128), 40 + H, "index_keys")
    q = synth.normal_bf16((n, H, 128), 40 + H, "index_q")
    w = synth.uniform((n, H), 40 + H, "index_w")
    stride = 1600
    (kd, ksd), (ko, kso) = quant_both(orc, B.MXFP4, orc.E2M1, keys)
    K = B.IndexKeys(kd, ksd, 128)
    qd, wd = q.to(DEV), w.to(DEV)
    whole = B.index_score(dev_rows(rows), dev_cache(cache), qd, wd, K, scores=poison((n, stride), torch.float32))
    parts = poison((n, stride), torch.float32)
    for a in range(0, n, 400):
        b = min(n, a + 400)
        sub = {k: v[a:b] for k, v in rows.items()}
        B.index_score(dev_rows(sub), dev_cache(cache), qd[a:b], wd[a:b], K, scores=parts[a:b])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int32), parts.view(torch.int32))
    sample = sorted(set([0, 1, 2, 300, 301, 302, 304, 305, 306, 821, 822, n - 2, n - 1]) |
                    set(rng.choice(n, 12, replace=False).tolist()))
    rs = {k: v[sample] for k, v in rows.items()}
    s_o, bad = orc.index_score(rs, cache, q[sample].float().numpy(), w[sample].numpy(), ko, key_scales=kso, heads=H,
                               dim=128, score_stride=stride)
    assert bad == 0
    got = whole.cpu().numpy()[sample]
    for i in range(len(sample)):
        R = min((int(rs["pos_of_row"][i]) + 1) // m, int(cache["n_entries"][rs["req_of_row"][i]]))
        assert np.array_equal(got[i, :R], s_o[i, :R]), "row %d" % sample[i]
        assert np.all(got[i, R:] == -np.inf)


def test_index_score_mxfp4_q_input(orc):
    """MXFP4 index q (codes and E8M0 scales from csa2_quant_mx of the bf16 q) gives the
    scores of that bf16 q bit for bit: one row per workgroup, row pairs (1024 rows or
    more) and pool columns, and through the fused pool top-k."""
    say("case: index_score with MXFP4 index q")
    rng = np.random.default_rng(50)
    lens, S, m = [700, 450, 1], [1400, 900, 5000], 2
    geom = synth.Geometry(S, m)
    req = np.concatenate([np.full(L, r) for r, L in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.sort(rng.choice(s_, size=L, replace=False)) for s_, L in zip(S, lens)]).astype(np.int32)
    rows = dict(req_of_row=req, pos_of_row=pos)
    cache = dict(ratio_m=m, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    n = len(req)
    keys = synth.normal((geom.total_entries, 128), 50, "index_keys")
    q = synth.normal_bf16((n, 64, 128), 50, "index_q").to(DEV)
    w = synth.uniform((n, 64), 50, "index_w").to(DEV)
    kd, ksd = B.quant_mx(B.MXFP4, keys.to(DEV))
    K = B.IndexKeys(kd, ksd, 128)
    qc, qs = B.quant_mx(B.MXFP4, q)
    assert qc.shape == (n, 64, 64) and qs.shape == (n, 64, 4)
    rd, cd = dev_rows(rows), dev_cache(cache)
    stride = 2600
    for part in (slice(0, n), slice(0, 300)):          # pairs (n >= 1024), then one row per workgroup
        sub = {k_: v[part] for k_, v in rows.items()}
        a = B.index_score(dev_rows(sub), cd, q[part], w[part], K, scores=poison((len(sub["req_of_row"]), stride),
                                                                              torch.float32))
        b = B.index_score(dev_rows(sub), cd, qc[part], w[part], K, q_scale=qs[part],
                          scores=poison((len(sub["req_of_row"]), stride), torch.float32))
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # pool columns and the fused pool top-k
    NB = 96
    blocks = np.full((n, NB), -1, np.int32)
    nblocks = np.zeros(n, np.int32)
    for i in range(n):
        R = min((int(pos[i]) + 1) // m, geom.n_entries[req[i]])
        nb = (R + 7) // 8
        pick = list(range(nb)) if nb <= NB else sorted(set(rng.choice(nb - 1, NB - 1, replace=False).tolist()) | {nb - 1})
        blocks[i, :len(pick)] = pick
        nblocks[i] = len(pick)
    pd = B.Pool(i32(blocks).to(DEV), i32(nblocks).to(DEV), 8)
    a = B.index_score(rd, cd, q, w, K, pool=pd, scores=poison((n, NB * 8), torch.float32))
    b = B.index_score(rd, cd, qc, w, K, pool=pd, scores=poison((n, NB * 8), torch.float32), q_scale=qs)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    fa = B.index_topk_pool(rd, cd, q, w, K, pd, 128, out=poison((n, 128), torch.int32))
    fb = B.index_topk_pool(rd, cd, qc, w, K, pd, 128, out=poison((n, 128), torch.int32), q_scale=qs)
    assert torch.equal(fa, fb)
    # the decode-sized shape (fewer than 128 rows: pool segments) gives the same sets
    few = {k_: v[:100] for k_, v in rows.items()}
    pf = B.Pool(pd.blocks[:100].contiguous(), pd.nblocks[:100].contiguous(), 8)
    fc = B.index_topk_pool(dev_rows(few), cd, qc[:100], w[:100], K, pf, 128, out=poison((100, 128), torch.int32),
                           q_scale=qs[:100])
    assert torch.equal(fc, fa[:100])
    # and the bf16 scores are the oracle's (sampled rows)
    sample = [0, 1, 699, 700, 1149, 1150]
    rs = {k_: v[sample] for k_, v in rows.items()}
    ko, kso = orc.mx_quant(orc.E2M1, keys.numpy())
    s_o, bad = orc.index_score(rs, cache, q[sample].float().cpu().numpy(), w[sample].cpu().numpy(), ko, key_scales=kso,
                               heads=64, dim=128, score_stride=stride)
    assert bad == 0
    full = B.index_score(rd, cd, qc, w, K, q_scale=qs, scores=poison((n, stride), torch.float32)).cpu().numpy()
    for i, r in enumerate(sample):
        R = min((int(pos[r]) + 1) // m, geom.n_entries[req[r]])
        assert np.array_equal(full[r, :R], s_o[i, :R])


def test_index_score_mxfp4_pool(orc):
    say("case: index_score MXFP4 over a candidate pool (ragged newest block, row map)")
    rows, cache, keys, q, w = _score_case(21, (4000, 999), 1, 64, 128, 10)
    rng = np.random.default_rng(22)
    n = len(rows["req_of_row"])
    B_, NB = 8, 64
    blocks = np.full((n, NB), -1, np.int32)
    nblocks = np.zeros(n, np.int32)
    for i in range(n):
        r, p = rows["req_of_row"][i], rows["pos_of_row"][i]
        R = min(p + 1, cache["n_entries"][r])
        nb = (R + B_ - 1) // B_
        others = rng.choice(max(nb - 1, 1), size=min(NB - 1, max(nb - 1, 0)), replace=False) if nb > 1 else []
        pick = sorted(set(np.asarray(others).tolist()) | {nb - 1}) if nb > 0 else []
        blocks[i, :len(pick)] = pick
        nblocks[i] = len(pick)
    # the row map sends every row to its own pool row in reverse storage order
    perm = np.arange(n)[::-1].copy()
    pool_blocks = np.empty_like(blocks)
    pool_n = np.empty_like(nblocks)
    pool_blocks[perm] = blocks
    pool_n[perm] = nblocks
    pool_o = dict(blocks=pool_blocks, nblocks=pool_n, block=B_, max_blocks=NB, row_map=perm)
    pool_d = B.Pool(i32(pool_blocks).to(DEV), i32(pool_n).to(DEV), B_, i32(perm).to(DEV))
    stride = NB * B_
    (kd, ksd), (ko, kso) = quant_both(orc, B.MXFP4, orc.E2M1, keys)
    # score_stride is the pool width plus padding that the call must leave alone
    pad = poison((n, stride + 24), torch.float32)
    s_d = B.index_score(dev_rows(rows), dev_cache(cache), q.to(DEV), w.to(DEV), B.IndexKeys(kd, ksd, 128),
                        pool=pool_d, scores=pad)
    s_o, bad = orc.index_score(rows, cache, q.float().numpy(), w.numpy(), ko, key_scales=kso, heads=64, dim=128,
                               score_stride=stride, pool=pool_o)
    assert bad == 0
    got = s_d.cpu().numpy()
    for i in range(n):
        ncol = nblocks[i] * B_
        assert np.array_equal(got[i, :ncol], s_o[i, :ncol]), i
        assert np.all(got[i, ncol:stride] == -np.inf), i
        assert np.all(np.isnan(got[i, stride:])), i


def test_index_score_f32_c0(orc):
    say("case: index_score fp32 (C0 shapes)")
    cfg = synth.config(0)
    rows_t = synth.prefill_rows(cfg.geom)
    rows = {k: v.numpy() for k, v in rows_t.items()}
    g = cfg.geom
    cache = dict(ratio_m=g.ratio_m, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    n = len(rows["req_of_row"])
    keys = synth.normal((g.total_entries, cfg.index_dim), 0, "index_keys")
    q = synth.normal((n, cfg.index_heads, cfg.index_dim), 0, "index_q")
    w = synth.uniform((n, cfg.index_heads), 0, "index_w")
    stride = 512
    s_d = B.index_score(dev_rows(rows), dev_cache(cache), q.to(DEV), w.to(DEV), B.IndexKeys(keys.to(DEV), None, 64),
                        scores=poison((n, stride), torch.float32))
    s_o, _ = orc.index_score(rows, cache, q.numpy(), w.numpy(), keys.numpy(), heads=8, dim=64, score_stride=stride)
    got = s_d.cpu().numpy()
    for i in range(n):
        R = min((rows["pos_of_row"][i] + 1) // 2, 512)
        assert np.array_equal(got[i, :R], s_o[i, :R]), i
        assert np.all(got[i, R:] == -np.inf), i


# ---------------------------------------------------------------------- top-k
def _topk_inputs(seed, R_list, stride, ties=None):
    rng = np.random.default_rng(seed)
    n = len(R_list)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([max(R - 1, 0) for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(n, np.int64))
    scores = np.full((n, stride), np.nan, np.float32)
    for i, R in enumerate(R_list):
        v = (rng.standard_normal(R) * 30 + 150).astype(np.float32)
        if ties is not None:
            v = np.floor(v / ties).astype(np.float32) * ties
        scores[i, :min(R, stride)] = v[:stride]
    return rows, cache, scores


@pytest.mark.parametrize("ties", [None, 4.0, 1000.0])
@pytest.mark.parametrize("k", [64, 512, 2048])
def test_topk_flat(orc, k, ties):
    say("case: topk flat k=%d ties=%s" % (k, ties))
    R_list = [0, 1, 511, 512, 513, 2047, 2048, 2049, 5000, 8191, 8192, 8193, 16385, 40000]
    stride = 40960
    rows, cache, scores = _topk_inputs(100 + k, R_list, stride, ties)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k).cpu().numpy()
    ref = orc.topk(rows, cache, scores, k)
    for i in range(len(R_list)):
        assert np.array_equal(got[i], ref[i]), (i, R_list[i])


@pytest.mark.parametrize("stride", [2048, 4096, 8192])
@pytest.mark.parametrize("ties", [None, 4.0])
def test_topk_many_rows(orc, stride, ties):
    """At least 1024 rows select with small workgroups (256 threads of 8 or 16 candidates,
    512 threads of 16, by the row length): ragged reaches around k and the slice sizes, with and
    without ties, checked row by row against the oracle; the same rows in a batch of
    16 (1024-thread workgroups) give the same index sets."""
    say("case: topk many rows stride=%d ties=%s" % (stride, ties))
    base = [0, 1, 100, 511, 512, 513, 1000, 2047, 2048, 2049, 4095, 4096, 4097, 6000, 8191, 8192]
    R_list = [min(base[i % len(base)], stride) for i in range(1024)]
    rows, cache, scores = _topk_inputs(700 + stride, R_list, stride, ties)
    sd = torch.from_numpy(scores).to(DEV)
    got = _topk(dev_rows(rows), dev_cache(cache), sd, 512).cpu().numpy()
    ref = orc.topk(rows, cache, scores, 512)
    for i in range(len(R_list)):
        assert np.array_equal(got[i], ref[i]), (i, R_list[i])
    few = {k: v[:16] for k, v in rows.items()}
    fc = dict(ratio_m=1, n_entries=cache["n_entries"][:16], row_start=cache["row_start"][:16])
    got16 = _topk(dev_rows(few), dev_cache(fc), sd[:16].contiguous(), 512).cpu().numpy()
    assert np.array_equal(got16, got[:16])


@pytest.mark.parametrize("stride", [8192, 16384])
def test_topk_small_threshold_bin(orc, stride):
    """Rows whose threshold falls among a few repeated values: after the first pass the
    threshold bin holds at most 64 keys (the direct ranking path) or just more (another
    histogram pass), with ties broken by the lowest index."""
    say("case: topk small threshold bin, stride=%d" % stride)
    rng = np.random.default_rng(31 + stride)
    k = 512
    R = stride
    rows_scores = []
    for above, groups in [(500, [(50.0, 30)]),             # 12 of 30 copies of the threshold value
                          (505, [(50.0, 20), (50.5, 20)]),  # 7 of the 20 copies of 50.5
                          (448, [(50.0, 64)]),              # exactly 64 keys in the bin
                          (440, [(50.0, 65)]),              # one more than the direct path takes
                          (511, [(50.0, 1), (49.0, 40)])]:  # the threshold is a single key
        v = rng.uniform(0.0, 1.0, R).astype(np.float32)
        pos = rng.permutation(R)
        v[pos[:above]] = (100.0 + rng.permutation(above)).astype(np.float32)
        at = above
        for val, cnt in groups:
            v[pos[at:at + cnt]] = np.float32(val)
            at += cnt
        rows_scores.append(v)
    n = len(rows_scores)
    scores = np.stack(rows_scores)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.full(n, R - 1))
    cache = dict(ratio_m=1, n_entries=np.full(n, R), row_start=np.arange(n, dtype=np.int64) * R)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k).cpu().numpy()
    ref = orc.topk(rows, cache, scores, k)
    for i in range(n):
        assert np.array_equal(got[i], ref[i]), i


def test_topk_pool(orc):
    say("case: topk over a pool")
    rng = np.random.default_rng(7)
    R_list = [100, 8000, 20000, 65536]
    B_, NB = 8, 2048
    rows = dict(req_of_row=np.arange(4), pos_of_row=np.array([R - 1 for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(4, np.int64))
    blocks = np.full((4, NB), -1, np.int32)
    nb_ = np.zeros(4, np.int32)
    for i, R in enumerate(R_list):
        nb = (R + B_ - 1) // B_
        if nb <= NB:
            pick = list(range(nb))
        else:
            pick = sorted(set(rng.choice(nb - 1, NB - 1, replace=False).tolist()) | {nb - 1})
        blocks[i, :len(pick)] = pick
        nb_[i] = len(pick)
    scores = np.full((4, NB * B_), np.nan, np.float32)
    for i, R in enumerate(R_list):
        for c in range(nb_[i] * B_):
            j = blocks[i, c // B_] * B_ + c % B_
            scores[i, c] = -np.inf if j >= R else np.float32(rng.standard_normal() * 20 + 100)
    pool_o = dict(blocks=blocks, nblocks=nb_, block=B_, max_blocks=NB)
    pool_d = B.Pool(i32(blocks).to(DEV), i32(nb_).to(DEV), B_)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, pool=pool_d).cpu().numpy()
    ref = orc.topk(rows, cache, scores, 512, pool=pool_o)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("ties", [None, 2.0])
def test_topk_hier(orc, ties):
    say("case: topk_hier ties=%s" % ties)
    R_list = [1, 9, 100, 16383, 16384, 16385, 16392, 16393, 30000, 65536]
    stride = 65536
    rows, cache, scores = _topk_inputs(55, R_list, stride, ties)
    idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8, 2048)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, 2048)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)


@pytest.mark.parametrize("ties,max_blocks,k", [(None, 1025, 512), (2.0, 2048, 512), (None, 1100, 2048)])
def test_topk_hier_all_blocks_fit(orc, ties, max_blocks, k):
    """Score rows of at most max_blocks blocks (a replay's source layer: 8192 positions, pools
    of 2048 blocks): every row keeps all its blocks and the flat top-k runs on the score
    rows directly; ragged reaches, a stride that is not a multiple of the block, ties."""
    say("case: topk_hier with every block in the pool ties=%s max_blocks=%d k=%d" % (ties, max_blocks, k))
    R_list = [0, 1, 7, 9, 100, 513, 4096, 8191, 8199, 8200, 8200, 3000]
    stride = 8200
    rows, cache, scores = _topk_inputs(57, R_list, stride, ties)
    idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k, 8,
                                 max_blocks)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, k, 8, max_blocks)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)


# ------------------------------------------------------------------ attention
def test_attn_f32_c0(orc):
    say("case: sparse+window attention fp32 (C0), k=64 and k=512 (dense equivalence)")
    cfg = synth.config(0)
    g = cfg.geom
    rows_t = synth.prefill_rows(g)
    rows = {k: v.numpy() for k, v in rows_t.items()}
    n = len(rows["req_of_row"])
    cache = dict(ratio_m=2, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    q = synth.normal((n, 8, 64), 0, "q")
    kv = synth.normal((g.total_entries, 64), 0, "kv")
    win = synth.window_cache_geometry(g, 128, rows_held=g.seq_len)
    swa_data = synth.normal((win["rows"], 64), 0, "swa")
    rng = np.random.default_rng(0)
    sel = np.full((n, 64), -1, np.int32)
    for i in range(n):
        R = min((rows["pos_of_row"][i] + 1) // 2, 512)
        take = min(R, 64)
        sel[i, :take] = np.sort(rng.choice(R, size=take, replace=False)) if take else []
    scale = 1.0 / 8.0
    wd = B.Window(swa_data.to(DEV), None, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    wo = dict(data=swa_data.numpy(), dtype=0, scale=None, row_start=win["row_start"].numpy(),
              pos_start=win["pos_start"].numpy(), window=128)
    out_d, lse_d = B.sparse_swa_attn(dev_rows(rows), dev_cache(cache), q.to(DEV), kv.to(DEV), i32(sel).to(DEV), wd,
                                     scale, out=poison((n, 8, 64), torch.float32), lse=poison((n, 8), torch.float32))
    out_o, lse_o = orc.sparse_swa_attn(rows, cache, q.numpy(), 0, kv.numpy(), 0, sel, wo, heads=8, dim=64,
                                       sm_scale=scale)
    nb, emax, _ = allclose_report(out_d.cpu().numpy(), out_o, 1e-4, 1e-4)
    assert nb == 0, (nb, emax)
    assert allclose_report(lse_d.cpu().numpy(), lse_o, 1e-4, 1e-4)[0] == 0
    # k = 512 >= R: equal to dense brute force over every reachable entry
    sel_all = np.full((n, 512), -1, np.int32)
    for i in range(n):
        R = min((rows["pos_of_row"][i] + 1) // 2, 512)
        sel_all[i, :R] = np.arange(R)
    out_d2 = B.sparse_swa_attn(dev_rows(rows), dev_cache(cache), q.to(DEV), kv.to(DEV), i32(sel_all).to(DEV), wd, scale,
                               out=poison((n, 8, 64), torch.float32))
    dense, _ = orc.sparse_swa_attn(rows, cache, q.numpy(), 0, kv.numpy(), 0, None, wo, heads=8, dim=64, sm_scale=scale,
                                   dense=True)
    nb, emax, _ = allclose_report(out_d2.cpu().numpy(), dense, 1e-4, 1e-4)
    assert nb == 0, (nb, emax)


def _attn_bf16_case(seed, S, m, H, k, nrows_per_req, win_lo_tail=False, swa_fp8=True):
    rng = np.random.default_rng(seed)
    geom = synth.Geometry(list(S), m)
    req, pos = [], []
    for r, s in enumerate(S):
        special = [0, 1, 126, 127, 128, 129, s - 1]
        pick = set(p for p in special if 0 <= p < s) | set(rng.choice(s, size=nrows_per_req, replace=False).tolist())
        for p in sorted(pick):
            req.append(r)
            pos.append(p)
    n = len(req)
    rows = dict(req_of_row=np.array(req), pos_of_row=np.array(pos))
    if win_lo_tail:
        rows["win_lo"] = np.array([max(0, p - int(rng.integers(0, 130))) for p in pos])
    cache = dict(ratio_m=m, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    D = 512
    q = synth.normal_bf16((n, H, D), seed, "q")
    kv = synth.normal_bf16((geom.total_entries, D), seed, "kv")
    win = synth.window_cache_geometry(geom, 128, rows_held=geom.seq_len)
    swa_raw = synth.normal((win["rows"], D), seed, "swa")
    sel = np.full((n, k), -1, np.int32)
    for i in range(n):
        R = min((pos[i] + 1) // m, geom.n_entries[req[i]])
        take = min(R, k)
        if take:
            chosen = rng.choice(R, size=take, replace=False)
            slots = rng.choice(k, size=take, replace=False)   # -1 holes anywhere
            sel[i, np.sort(slots)] = np.sort(chosen)
    return rows, cache, q, kv, win, swa_raw, sel


def _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, H, sm_scale, swa_fp8=True, sel_row_map=None,
                   sink=None, kv_fp4=False):
    """kv_fp4: the main KV goes in the FP4 storage format, quantized on each side from
    the same bf16 rows (identical bytes asserted)."""
    n = len(rows["req_of_row"])
    if swa_fp8:
        (cd, sd), (co, so) = quant_both(orc, B.MXFP8_E4M3, orc.E4M3, swa_raw)
        wd = B.Window(cd, sd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
        wo = dict(data=co, dtype=3, scale=so, row_start=win["row_start"].numpy(), pos_start=win["pos_start"].numpy(),
                  window=128)
    else:
        sb = swa_raw.to(torch.bfloat16)
        wd = B.Window(sb.to(DEV), None, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
        wo = dict(data=sb.view(torch.int16).numpy().view(np.uint16), dtype=1, scale=None,
                  row_start=win["row_start"].numpy(), pos_start=win["pos_start"].numpy(), window=128)
    if kv_fp4:
        (kv_d, kvs_d), (kv_o, kvs_o) = quant_fp4_both(orc, kv)
        kv_dt_o = orc.DT_FP4S16
    else:
        kv_d, kvs_d = kv.to(DEV), None
        kv_o, kvs_o, kv_dt_o = kv.view(torch.int16).numpy().view(np.uint16), None, 1
    out_d, lse_d = B.sparse_swa_attn(dev_rows(rows), dev_cache(cache), q.to(DEV), kv_d, i32(sel).to(DEV), wd,
                                     sm_scale, sel_row_map=None if sel_row_map is None else i32(sel_row_map).to(DEV),
                                     sink=None if sink is None else torch.from_numpy(sink).to(DEV),
                                     out=poison(tuple(q.shape), torch.bfloat16), lse=poison((n, H), torch.float32),
                                     kv_scale=kvs_d)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    out_o, lse_o = orc.sparse_swa_attn(rows, cache, qb, 1, kv_o, kv_dt_o, sel, wo, heads=H, dim=512,
                                       sm_scale=sm_scale, sel_row_map=sel_row_map, sink=sink, kv_scale=kvs_o)
    return out_d.float().cpu().numpy(), lse_d.cpu().numpy(), out_o, lse_o


def _check_bf16_attn(got, ref, lse_g, lse_r):
    nb, emax, _ = allclose_report(got, ref, 2e-2, 1e-2)
    assert nb == 0, ("elements out of tolerance", nb, emax)
    n, H, D = ref.shape
    rel = np.linalg.norm((got - ref).reshape(n * H, D), axis=1) / (np.linalg.norm(ref.reshape(n * H, D), axis=1) + 1e-30)
    assert rel.max() <= 1e-2, ("row relative L2", rel.max())
    nb, emax, _ = allclose_report(lse_g, lse_r, 1e-3, 1e-3)
    assert nb == 0, ("lse", nb, emax)


@pytest.mark.parametrize("H,k,swa_fp8,tail", [(64, 512, True, False), (16, 64, True, True), (32, 512, False, False),
                                              (64, 0, True, False), (16, 2048, True, False), (128, 512, True, True),
                                              (80, 96, False, True)])
def test_attn_bf16(orc, H, k, swa_fp8, tail):
    say("case: sparse+window attention bf16 H=%d k=%d fp8=%s tail=%s" % (H, k, swa_fp8, tail))
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(30 + H + k, (2600, 700), 2 if k != 2048 else 1, H, k, 6,
                                                            win_lo_tail=tail)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, H, 1 / math.sqrt(512),
                                            swa_fp8=swa_fp8)
    _check_bf16_attn(got, ref, lse_g, lse_r)


@pytest.mark.parametrize("sm_scale", [1.0, 3.0])
def test_attn_bf16_wide_logits(orc, sm_scale):
    # Logits spread over far more than 64 (log2 units) between a wave's first tile and the
    # row maximum, so the exponent reference taken from the first tile is exceeded and the
    # wave redoes its tiles with the exact maximum.
    say("case: bf16 attention with logits spread wider than the first-tile reference, scale %g" % sm_scale)
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(61, (2600, 700), 2, 16, 512, 6)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 16, sm_scale)
    _check_bf16_attn(got, ref, lse_g, lse_r)


def test_attn_bf16_dense_equivalence(orc):
    say("case: bf16 attention with every reachable entry selected equals dense brute force")
    rows, cache, q, kv, win, swa_raw, _ = _attn_bf16_case(77, (900,), 2, 16, 512, 8)
    n = len(rows["req_of_row"])
    sel = np.full((n, 512), -1, np.int32)
    for i in range(n):
        R = min((rows["pos_of_row"][i] + 1) // 2, 450)
        sel[i, :R] = np.arange(R)
    got, lse_g, _, _ = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 16, 1 / math.sqrt(512))
    (cd, sd), (co, so) = quant_both(orc, B.MXFP8_E4M3, orc.E4M3, swa_raw)
    wo = dict(data=co, dtype=3, scale=so, row_start=win["row_start"].numpy(), pos_start=win["pos_start"].numpy(),
              window=128)
    dense, lse_dense = orc.sparse_swa_attn(rows, cache, q.view(torch.int16).numpy().view(np.uint16), 1,
                                           kv.view(torch.int16).numpy().view(np.uint16), 1, None, wo, heads=16, dim=512,
                                           sm_scale=1 / math.sqrt(512), dense=True)
    _check_bf16_attn(got, dense, lse_g, lse_dense)


def test_attn_bf16_reuse_row_map(orc):
    say("case: Reuse layer reads another layer's index rows through sel_row_map")
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(88, (1500,), 2, 16, 512, 10)
    n = len(rows["req_of_row"])
    rng = np.random.default_rng(1)
    # producer rows live in a larger table; each consumer row maps to its producer row
    table = np.full((3 * n, 512), -1, np.int32)
    row_map = rng.permutation(3 * n)[:n].astype(np.int32)
    table[row_map] = sel
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, table, 16, 0.05,
                                            sel_row_map=row_map)
    _check_bf16_attn(got, ref, lse_g, lse_r)
    got2, _, _, _ = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 16, 0.05)
    assert np.array_equal(got, got2)  # same indices through the map: bitwise identical


def test_determinism_and_batch_invariance(orc):
    say("case: run twice bitwise equal; a row alone equals the row inside a batch")
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(99, (1200, 800), 2, 32, 512, 6)
    a, la, ref, lref = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 32, 0.04)
    _check_bf16_attn(a, ref, la, lref)
    b, _, _, _ = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 32, 0.04)
    assert np.array_equal(a, b)
    i = 3
    rows1 = {k: v[i:i + 1] for k, v in rows.items()}
    c, _, _, _ = _run_attn_bf16(orc, rows1, cache, q[i:i + 1].contiguous(), kv, win, swa_raw, sel[i:i + 1], 32, 0.04)
    assert np.array_equal(a[i:i + 1], c)


@pytest.mark.parametrize("k", [512, 2048])
def test_topk_multilevel(orc, k):
    say("case: topk over rows longer than one workgroup (segments + merge), k=%d" % k)
    R_list = [70000, 131072, 262144, 200001, 65536, 65537]
    rows, cache, scores = _topk_inputs(300 + k, R_list, 262144, ties=None)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k).cpu().numpy()
    ref = orc.topk(rows, cache, scores, k)
    assert np.array_equal(got, ref)
    # and with heavy ties, where the merge must keep the lowest positions
    rows, cache, scores = _topk_inputs(301 + k, R_list, 262144, ties=50.0)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), k).cpu().numpy()
    ref = orc.topk(rows, cache, scores, k)
    assert np.array_equal(got, ref)


def test_topk_hier_long(orc):
    say("case: topk_hier on 262144-entry rows (C4 shape)")
    R_list = [262144, 100000]
    rows, cache, scores = _topk_inputs(400, R_list, 262144)
    idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8, 2048)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, 2048)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)


# ------------------------------------------------ hierarchy: single-stage path, ties
@pytest.mark.parametrize("max_blocks", [64, 512])
def test_topk_hier_single_stage(orc, max_blocks):
    """k >= max_blocks takes the single-stage path (flat top-k over the score row, then the
    block pass with maxima taken on the fly)."""
    say("case: topk_hier k=512, max_blocks=%d (single-stage path)" % max_blocks)
    R_list = [1, 8, 9, 500, 511, 512, 513, 8 * max_blocks - 1, 8 * max_blocks, 8 * max_blocks + 1, 20000, 65536]
    stride = 65536
    for ties in (None, 2.0):
        rows, cache, scores = _topk_inputs(57 + max_blocks, R_list, stride, ties)
        idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8,
                                     max_blocks)
        ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, max_blocks)
        assert np.array_equal(nblocks.cpu().numpy(), rn)
        assert np.array_equal(blocks.cpu().numpy(), rb)
        assert np.array_equal(idx.cpu().numpy(), ri)


@pytest.mark.parametrize("max_blocks", [2048, 64])
def test_topk_hier_all_equal(orc, max_blocks):
    """Every score equal: the pool is the lowest block ids plus the newest block, and the
    flat top-k is the k lowest positions (ties go to the lowest index)."""
    say("case: topk_hier with all scores equal, max_blocks=%d" % max_blocks)
    R_list = [5, 16384, 16385, 30001, 65536]
    stride = 65536
    n = len(R_list)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([R - 1 for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(n, np.int64))
    scores = np.full((n, stride), 3.0, np.float32)
    idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8,
                                 max_blocks)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, max_blocks)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)
    for i, R in enumerate(R_list):
        nb = (R + 7) // 8
        want = list(range(nb)) if nb <= max_blocks else list(range(max_blocks - 1)) + [nb - 1]
        assert rb[i, :len(want)].tolist() == want
        assert ri[i, :min(R, 512)].tolist() == list(range(min(R, 512)))


def test_topk_hier_stride_below_reach(orc):
    """score_stride smaller than R and not a multiple of 8: only the columns that exist are
    candidates, and the newest block is the one holding column score_stride - 1."""
    say("case: topk_hier with score_stride < R, stride % 8 != 0")
    stride = 40003
    R_list = [50000, 40003, 40001, 39999, 16390]
    rows, cache, scores = _topk_inputs(59, R_list, stride)
    for mb in (2048, 64):
        idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8, mb)
        ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, mb)
        assert np.array_equal(nblocks.cpu().numpy(), rn)
        assert np.array_equal(blocks.cpu().numpy(), rb)
        assert np.array_equal(idx.cpu().numpy(), ri)


# ----------------------------------------- merge levels at their largest candidate counts
@pytest.mark.parametrize("stride", [262152, 524288])
def test_topk_merge_capacity_k2048(orc, stride):
    """k = 2048 over rows long enough that a merge level gathers more than 8 lists: every
    merge workgroup must hold all of its lists' candidates."""
    say("case: topk k=2048 at score_stride %d (merge-level capacity)" % stride)
    R_list = [stride, stride - 5, 300001 if stride > 300001 else 200001]
    rows, cache, scores = _topk_inputs(61 + stride % 97, R_list, stride)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 2048).cpu().numpy()
    ref = orc.topk(rows, cache, scores, 2048)
    assert np.array_equal(got, ref)


def test_topk_pool_merge_capacity(orc):
    """Pool top-k with k = 2048 over a pool of 32,768 blocks of 8 (262,144 candidates)."""
    say("case: pool topk k=2048 over 262144 pool columns")
    rng = np.random.default_rng(63)
    B_, NB = 8, 32768
    R_list = [400000, 262144]
    n = len(R_list)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([R - 1 for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(n, np.int64))
    blocks = np.full((n, NB), -1, np.int32)
    nb_ = np.zeros(n, np.int32)
    for i, R in enumerate(R_list):
        nb = (R + B_ - 1) // B_
        pick = sorted(set(rng.choice(nb - 1, NB - 1, replace=False).tolist()) | {nb - 1}) if nb > NB \
            else list(range(nb))
        blocks[i, :len(pick)] = pick
        nb_[i] = len(pick)
    scores = rng.standard_normal((n, NB * B_)).astype(np.float32)
    pool_o = dict(blocks=blocks, nblocks=nb_, block=B_, max_blocks=NB)
    pool_d = B.Pool(i32(blocks).to(DEV), i32(nb_).to(DEV), B_)
    got = _topk(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 2048, pool=pool_d).cpu().numpy()
    ref = orc.topk(rows, cache, scores, 2048, pool=pool_o)
    assert np.array_equal(got, ref)


def test_topk_hier_4096_blocks_long_row(orc):
    """max_blocks = 4096 on rows of more than 524,288 entries (block maxima merged over
    several levels with 4,095 kept per list)."""
    say("case: topk_hier max_blocks=4096 on 600000-entry rows")
    R_list = [600000, 590001]
    rows, cache, scores = _topk_inputs(65, R_list, 600000)
    idx, blocks, nblocks = _hier(dev_rows(rows), dev_cache(cache), torch.from_numpy(scores).to(DEV), 512, 8, 4096)
    ri, rb, rn = orc.topk_hier(rows, cache, scores, 512, 8, 4096)
    assert np.array_equal(nblocks.cpu().numpy(), rn)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(idx.cpu().numpy(), ri)


# ----------------------------------------------------------------- attention sink
@pytest.mark.parametrize("shift", [0.0, 6.0])
def test_attn_bf16_sink(orc, shift):
    """The sink adds exp(sink_h - max) to each head's denominator (one more key of value
    zero); sinks around and above the logits, bf16 path."""
    say("case: bf16 attention with a sink, shift %g" % shift)
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(71, (2600, 700), 2, 32, 512, 6)
    sink = (np.random.default_rng(72).standard_normal(32) * 2.0 + shift).astype(np.float32)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 32, 1 / math.sqrt(512),
                                            sink=sink)
    _check_bf16_attn(got, ref, lse_g, lse_r)


def test_attn_f32_sink(orc):
    say("case: fp32 attention (C0 shapes) with a sink")
    cfg = synth.config(0)
    g = cfg.geom
    rows_t = synth.prefill_rows(g)
    rows = {k: v.numpy() for k, v in rows_t.items()}
    n = len(rows["req_of_row"])
    cache = dict(ratio_m=2, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    q = synth.normal((n, 8, 64), 0, "q") * 3.0   # logits spread wide: the max shift matters
    kv = synth.normal((g.total_entries, 64), 0, "kv")
    win = synth.window_cache_geometry(g, 128, rows_held=g.seq_len)
    swa_data = synth.normal((win["rows"], 64), 0, "swa")
    rng = np.random.default_rng(5)
    sel = np.full((n, 64), -1, np.int32)
    for i in range(n):
        R = min((rows["pos_of_row"][i] + 1) // 2, 512)
        take = min(R, 64)
        sel[i, :take] = np.sort(rng.choice(R, size=take, replace=False)) if take else []
    sink = (rng.standard_normal(8) * 3.0 + 4.0).astype(np.float32)
    scale = 1.0 / 8.0
    wd = B.Window(swa_data.to(DEV), None, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    wo = dict(data=swa_data.numpy(), dtype=0, scale=None, row_start=win["row_start"].numpy(),
              pos_start=win["pos_start"].numpy(), window=128)
    out_d, lse_d = B.sparse_swa_attn(dev_rows(rows), dev_cache(cache), q.to(DEV), kv.to(DEV), i32(sel).to(DEV), wd,
                                     scale, sink=torch.from_numpy(sink).to(DEV), out=poison((n, 8, 64), torch.float32),
                                     lse=poison((n, 8), torch.float32))
    out_o, lse_o = orc.sparse_swa_attn(rows, cache, q.numpy(), 0, kv.numpy(), 0, sel, wo, heads=8, dim=64,
                                       sm_scale=scale, sink=sink)
    nb, emax, _ = allclose_report(out_d.cpu().numpy(), out_o, 1e-4, 1e-4)
    assert nb == 0, (nb, emax)
    assert allclose_report(lse_d.cpu().numpy(), lse_o, 1e-4, 1e-4)[0] == 0


# ------------------------------------------------------------- FP4 main KV
def test_quant_fp4s16_all_bf16_patterns(orc):
    say("case: main KV FP4 quantizer over every finite bf16 pattern, bf16 and fp32 input")
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals)]
    vals = vals[: (vals.numel() // 16) * 16]
    g = torch.Generator().manual_seed(5)
    for rep in range(3):
        x = vals[torch.randperm(vals.numel(), generator=g)].reshape(-1, 16).contiguous()
        quant_fp4_both(orc, x)
        quant_fp4_both(orc, x.to(torch.bfloat16))
    # blocks of similar magnitude (sorted patterns), where every element matters
    x = vals[torch.argsort(vals.abs())].reshape(-1, 16).contiguous()
    quant_fp4_both(orc, x)


def test_quant_fp4s16_ties_and_ranges(orc):
    say("case: main KV FP4 quantizer at E4M3 / E2M1 tie points, saturation, underflow, zeros")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4096, 16)).astype(np.float32)
    x *= (2.0 ** rng.integers(-40, 20, size=(4096, 1))).astype(np.float32)
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    # amax / 6 exactly at every E4M3 tie point (midpoints of consecutive codes)
    mids = (e4[1:] + e4[:-1]) / 2.0
    for i, t in enumerate(mids):
        x[i] = 0.0
        x[i, i % 16] = 6.0 * t
        x[i, (i + 1) % 16] = -6.0 * t * 0.5
    row = len(mids)
    # elements exactly at the E2M1 midpoints times the scale, for a few scales
    for sc in (0x38, 0x01, 0x07, 0x4B, 0x7E):
        s = e4[sc]
        x[row] = 0.0
        x[row, 0] = 6.0 * s
        x[row, 1:8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * s
        x[row, 8:15] = -x[row, 1:8]
        row += 1
    x[row] = 0.0
    x[row + 1] = -0.0
    x[row + 2, :] = 6.0 * 2.0 ** -11          # scale rounds to zero
    x[row + 3, 0] = 6.0 * 500.0                # scale saturates at 448
    x[row + 4, :] = 6.0 * 2.0 ** -10           # exactly half the smallest subnormal: ties to 0
    x[row + 5, :] = 6.0 * 2.0 ** -10 * 1.0001  # just above: the smallest subnormal
    quant_fp4_both(orc, torch.from_numpy(x))


@pytest.mark.parametrize("H,k,swa_fp8,tail", [(64, 512, True, False), (16, 64, True, True), (32, 512, False, False),
                                              (64, 0, True, False), (16, 2048, True, False), (128, 512, True, True),
                                              (80, 96, False, True)])
def test_attn_fp4_kv(orc, H, k, swa_fp8, tail):
    say("case: sparse+window attention, FP4 main KV, H=%d k=%d fp8=%s tail=%s" % (H, k, swa_fp8, tail))
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(130 + H + k, (2600, 700), 2 if k != 2048 else 1, H, k, 6,
                                                            win_lo_tail=tail)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, H, 1 / math.sqrt(512),
                                            swa_fp8=swa_fp8, kv_fp4=True)
    _check_bf16_attn(got, ref, lse_g, lse_r)


def test_attn_fp4_kv_equals_bf16_path_on_decoded_values(orc):
    """Every decoded FP4 value is exact in bf16, so the FP4 path must give bit for bit what
    the bf16 path gives on a cache holding the decoded values (same MFMA operands, same
    order); the decode here is torch's (E2M1 table times float8_e4m3fn)."""
    say("case: FP4 main KV path == bf16 path on the decoded cache, bitwise")
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(141, (2600, 700), 2, 32, 512, 6, win_lo_tail=True)
    n = len(rows["req_of_row"])
    codes, scales = B.quant_mx(B.FP4_S16, kv.to(DEV))
    dec = fp4_decode_torch(codes.cpu(), scales.cpu())
    assert torch.equal(dec.to(torch.bfloat16).float(), dec)
    (cd, sd), _ = quant_both(orc, B.MXFP8_E4M3, orc.E4M3, swa_raw)
    wd = B.Window(cd, sd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    args = (dev_rows(rows), dev_cache(cache), q.to(DEV))
    a, la = B.sparse_swa_attn(*args, codes, i32(sel).to(DEV), wd, 0.044, want_lse=True, kv_scale=scales)
    b, lb = B.sparse_swa_attn(*args, dec.to(torch.bfloat16).to(DEV), i32(sel).to(DEV), wd, 0.044, want_lse=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    assert a.shape == (n, 32, 512)


@pytest.mark.parametrize("sm_scale", [1.0, 3.0])
def test_attn_fp4_kv_wide_logits(orc, sm_scale):
    say("case: FP4 main KV attention with the redo pass (logits wider than the reference), scale %g" % sm_scale)
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(161, (2600, 700), 2, 16, 512, 6)
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, sel, 16, sm_scale, kv_fp4=True)
    _check_bf16_attn(got, ref, lse_g, lse_r)


def test_attn_fp4_kv_reuse_row_map(orc):
    say("case: FP4 main KV, Reuse layer through sel_row_map, bf16 window")
    rows, cache, q, kv, win, swa_raw, sel = _attn_bf16_case(188, (1500,), 2, 16, 512, 10)
    n = len(rows["req_of_row"])
    rng = np.random.default_rng(2)
    table = np.full((3 * n, 512), -1, np.int32)
    row_map = rng.permutation(3 * n)[:n].astype(np.int32)
    table[row_map] = sel
    got, lse_g, ref, lse_r = _run_attn_bf16(orc, rows, cache, q, kv, win, swa_raw, table, 16, 0.05,
                                            sel_row_map=row_map, swa_fp8=False, kv_fp4=True)
    _check_bf16_attn(got, ref, lse_g, lse_r)
