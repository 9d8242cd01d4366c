"""GPU parity of the index-K / main-KV producer (csa2_kv_produce) against the oracle.

Every cache byte (main KV in bf16 or the FP4 storage format, MXFP4 index codes and
scales, rows the call leaves alone included) and the pending state must match bit for
bit: the producer's rounding is fixed step by step (as include/csa2.h states it, the same
on both sides), so the quantized codes it decides are reproducible.  Then the caches
a decode sequence builds one token at a time must equal those of one prefill call, and a
Full layer reading the produced caches must match the oracle reading its own."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B
from compressed_sparse_attention_fp4_amd import synth

from gpu_util import DEV, bits, check_attn, check_scores, dev_cache, i32, i64, say

pytestmark = pytest.mark.gpu

KV, IDX, ROPE = 512, 128, 64
FILL = 0xEE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _rope_table(max_pos, base=10000.0):
    i = np.arange(ROPE // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * i / ROPE)[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


class _Stream:
    """Requests r with positions [prefix_r, prefix_r + len_r) for one call; seeded inputs."""

    def __init__(self, seed, lens, prefix, m, max_pos=None):
        self.m = m
        self.req = np.concatenate([np.full(L, r) for r, L in enumerate(lens)]).astype(np.int32)
        self.pos = np.concatenate([np.arange(p0, p0 + L) for p0, L in zip(prefix, lens)]).astype(np.int32)
        n = len(self.req)
        self.comp = synth.normal((n, KV), seed, "comp")
        self.pending = synth.normal((len(lens), KV), seed, "pending")
        self.wb = synth.normal_bf16((IDX, KV), seed, "w_index") * 0.05
        self.wb = self.wb.to(torch.bfloat16)
        ends = [p0 + L for p0, L in zip(prefix, lens)]
        self.n_ent = [e // m for e in ends]
        self.row_start = np.cumsum([0] + self.n_ent[:-1]).astype(np.int64)
        self.rows_cache = int(sum(self.n_ent))
        self.rope = _rope_table(max_pos or (max(ends) + 2))

    def rows(self, sel=slice(None)):
        return dict(req_of_row=self.req[sel], pos_of_row=self.pos[sel])


def _dev_caches(nrows, fp4):
    """Cache buffers filled with the sentinel the oracle's buffers start with."""
    if fp4:
        kv = torch.full((nrows, KV // 2), FILL, dtype=torch.uint8, device=DEV)
    else:
        kv = torch.full((nrows, KV), FILL * 0x101 - 0x10000, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    kvs = torch.full((nrows, KV // 16), FILL, dtype=torch.uint8, device=DEV) if fp4 else None
    ic = torch.full((nrows, IDX // 2), FILL, dtype=torch.uint8, device=DEV)
    isc = torch.full((nrows, IDX // 32), FILL, dtype=torch.uint8, device=DEV)
    return kv, kvs, ic, isc


def _run_dev(st, sel, pending_d, caches):
    kv, kvs, ic, isc = caches
    rows = st.rows(sel)
    rd = B.Rows(i32(rows["req_of_row"]).to(DEV), i32(rows["pos_of_row"]).to(DEV))
    cd = B.Cache(st.m, i32(st.n_ent).to(DEV), i64(st.row_start).to(DEV))
    B.kv_produce(rd, cd, st.comp[sel].contiguous().to(DEV), pending_d, st.wb.to(DEV), torch.from_numpy(st.rope).to(DEV),
                 kv, ic, isc, kv_scale=kvs)


def _compare(caches, o, fp4):
    kv, kvs, ic, isc = caches
    if fp4:
        assert np.array_equal(kv.cpu().numpy(), o["kv"]), "FP4 main KV codes"
        assert np.array_equal(kvs.cpu().numpy(), o["kv_scale"]), "FP4 main KV scales"
    else:
        assert np.array_equal(bits(kv), o["kv"]), "bf16 main KV"
    assert np.array_equal(ic.cpu().numpy(), o["index_codes"]), "index codes"
    assert np.array_equal(isc.cpu().numpy(), o["index_scales"]), "index scales"


@pytest.mark.parametrize("m,fp4,wide", [(2, True, False), (2, False, False), (1, True, False), (1, False, False),
                                        (2, True, True), (2, False, True), (1, True, True), (1, False, True)])
def test_kv_produce_one_call(orc, m, fp4, wide):
    """Short calls give each workgroup one row; calls of more than 4096 rows give it 8 m
    rows, processed in rounds of 8 closing rows."""
    say("case: kv producer, one call, m=%d fp4=%s wide=%s" % (m, fp4, wide))
    lens, prefix = [37, 20, 1, 300, 64, 9], [0, 5, 100, 2048, 7, 1001]
    if wide:
        lens, prefix = [3001, 20, 1, 1500, 64, 9], [0, 5, 100, 2049, 7, 1001]
    st = _Stream(600 + m, lens, prefix, m)
    caches = _dev_caches(st.rows_cache, fp4)
    pend = st.pending.clone().to(DEV)
    _run_dev(st, slice(None), pend if m == 2 else None, caches)
    o = orc.kv_produce(st.rows(), m, st.row_start, st.rows_cache, st.comp.numpy(), st.pending.numpy(), bits(st.wb),
                       st.rope, kv_dt=orc.DT_FP4S16 if fp4 else orc.DT_BF16, fill=FILL)
    _compare(caches, o, fp4)
    if m == 2:
        assert np.array_equal(pend.cpu().numpy(), o["pending"]), "pending state"


def test_kv_produce_decode_steps_equal_one_call(orc):
    """Nine requests fed one token per call (decode), the caches built across the calls
    equal one call over the whole stream, on the device, byte for byte."""
    say("case: kv producer, 40 decode steps vs one call")
    lens, prefix = [40] * 9, [0, 1, 2, 3, 100, 101, 4095, 4096, 12345]
    st = _Stream(611, lens, prefix, 2)
    whole = _dev_caches(st.rows_cache, True)
    p1 = st.pending.clone().to(DEV)
    _run_dev(st, slice(None), p1, whole)
    steps = _dev_caches(st.rows_cache, True)
    p2 = st.pending.clone().to(DEV)
    starts = np.cumsum([0] + lens[:-1])
    for u in range(40):
        _run_dev(st, starts + u, p2, steps)
    for a, b in zip(whole, steps):
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a, b.view(torch.uint8) if b.dtype != torch.uint8 else b)


@pytest.mark.parametrize("seed", range(6))
def test_kv_produce_random_call_splits(orc, seed):
    """Each request's tokens cut at random points into several calls (chunked prefill
    followed by shorter extends, pairs left open across calls): the caches and the
    pending state after the last call equal the oracle's single call, byte for byte."""
    rng = np.random.default_rng(4800 + seed)
    nreq = int(rng.integers(1, 6))
    lens = [int(rng.integers(1, 400)) for _ in range(nreq)]
    prefix = [int(rng.integers(0, 3000)) for _ in range(nreq)]
    m = int(rng.choice([1, 2]))
    fp4 = bool(rng.random() < 0.5)
    ncalls = int(rng.integers(2, 6))
    say("case: kv producer, random call splits seed=%d m=%d fp4=%s calls=%d lens=%s prefix=%s" %
        (seed, m, fp4, ncalls, lens, prefix))
    st = _Stream(4900 + seed, lens, prefix, m)
    o = orc.kv_produce(st.rows(), m, st.row_start, st.rows_cache, st.comp.numpy(), st.pending.numpy(), bits(st.wb),
                       st.rope, kv_dt=orc.DT_FP4S16 if fp4 else orc.DT_BF16, fill=FILL)
    caches = _dev_caches(st.rows_cache, fp4)
    pend = st.pending.clone().to(DEV)
    starts = np.cumsum([0] + lens[:-1])
    cuts = [[0] + sorted(rng.integers(0, L + 1, size=ncalls - 1).tolist()) + [L] for L in lens]
    for c in range(ncalls):
        sel = [i for r in range(nreq) for i in range(starts[r] + cuts[r][c], starts[r] + cuts[r][c + 1])]
        if sel:
            _run_dev(st, np.array(sel, dtype=np.int64), pend if m == 2 else None, caches)
    _compare(caches, o, fp4)
    if m == 2:
        # a request whose stream ends at an even position leaves that token pending; one
        # that ends on a closed pair keeps whatever its last open pair left (not compared)
        open_pair = [r for r in range(nreq) if (prefix[r] + lens[r] - 1) % 2 == 0]
        assert np.array_equal(pend.cpu().numpy()[open_pair], o["pending"][open_pair]), "pending state"


def test_produced_caches_feed_a_full_layer(orc):
    """The producer fills an owner's caches (m = 2, FP4 main KV) over a 2000-token prefill
    of two requests; a Full layer (scores, hierarchical top-k, attention over FP4 entries)
    then reads them; sampled rows match the oracle run on the oracle's own caches."""
    say("case: producer caches -> Full layer")
    lens = [2000, 1200]
    st = _Stream(620, lens, [0, 0], 2)
    caches = _dev_caches(st.rows_cache, True)
    _run_dev(st, slice(None), st.pending.clone().to(DEV), caches)
    o = orc.kv_produce(st.rows(), 2, st.row_start, st.rows_cache, st.comp.numpy(), st.pending.numpy(), bits(st.wb),
                       st.rope, fill=FILL)
    _compare(caches, o, True)
    kv, kvs, ic, isc = caches
    geom = synth.Geometry(lens, 2)
    cache = dict(ratio_m=2, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    assert np.array_equal(cache["row_start"], st.row_start)
    cd = dev_cache(cache)
    rows = dict(req_of_row=np.array([0] * 6 + [1] * 4, np.int32),
                pos_of_row=np.array([1, 2, 127, 128, 1000, 1999, 0, 129, 700, 1199], np.int32))
    rd = B.Rows(i32(rows["req_of_row"]).to(DEV), i32(rows["pos_of_row"]).to(DEV))
    n = 10
    qi = synth.normal_bf16((n, 64, IDX), 620, "index_q", device=DEV)
    w = synth.uniform((n, 64), 620, "index_w", device=DEV)
    C = max(geom.n_entries)
    sc = B.index_score(rd, cd, qi, w, B.IndexKeys(ic, isc, IDX), score_stride=C)
    idx, pb, pn = B.topk_hier(rd, cd, sc, 128, 8, 64)
    win = synth.window_cache_geometry(geom, 128, rows_held=lens)
    raw = synth.normal((win["rows"], KV), 620, "swa", device=DEV)
    scd, ssd = B.quant_mx(B.MXFP8_E4M3, raw)
    wd = B.Window(scd, ssd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    q = synth.normal_bf16((n, 16, KV), 620, "q", device=DEV)
    out = B.sparse_swa_attn(rd, cd, q, kv, idx, wd, 1 / math.sqrt(KV), kv_scale=kvs)
    torch.cuda.synchronize()
    s_o, bad = orc.index_score(rows, cache, qi.float().cpu().numpy(), w.cpu().numpy(), o["index_codes"],
                               key_scales=o["index_scales"], heads=64, dim=IDX, score_stride=C)
    assert bad == 0
    check_scores(sc.cpu().numpy(), s_o, [min((p + 1) // 2, geom.n_entries[r]) for r, p in
                                         zip(rows["req_of_row"], rows["pos_of_row"])])
    i_o, _, _ = orc.topk_hier(rows, cache, s_o, 128, 8, 64)
    assert np.array_equal(idx.cpu().numpy(), i_o)
    co, so = orc.mx_quant(orc.E4M3, raw.cpu().numpy())
    wo = dict(data=co, dtype=3, scale=so, row_start=win["row_start"].numpy(), pos_start=win["pos_start"].numpy(),
              window=128)
    a_o, _ = orc.sparse_swa_attn(rows, cache, bits(q), 1, o["kv"], orc.DT_FP4S16, i_o, wo, heads=16, dim=KV,
                                 sm_scale=1 / math.sqrt(KV), kv_scale=o["kv_scale"])
    check_attn(out.float().cpu().numpy(), a_o)
