"""GPU parity of the bounded-replay layouts and of the path run over the batches they
describe: mixed prefill + decode batches ("DeepSeek V4.1 Flash modeling", section
"Decoder Bounded Replay"), chunked extends ("SGLang: how DeepSeek V4.1 Flash late layers
only process tail tokens", section 2.5) and the encoder-side replay ("SGLang and Miles
Day-0 support for DeepSeek-V4.1", sections 4.1 and 4.3).

Layouts must match the oracle bit for bit on every row (outputs poisoned first).  The
flows run index scoring, selection and attention over the layouts' rows with the library
and recompute sampled rows with the oracle: scores and index sets bit for bit, attention
within |g - r| <= 2e-2 + 1e-2 |r| and a row relative L2 error <= 1e-2."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B
from compressed_sparse_attention_fp4_amd import synth

from gpu_util import DEV, bits, check_attn, check_scores, dev_cache, i32, poison, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _tail_dev(ext, seq, dec=None, borrow=False):
    nreq = len(ext)
    cap = 128 * nreq
    t = dict(tail_len=poison((nreq,), torch.int32), tail_row_start=poison((nreq + 1,), torch.int32))
    for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
        t[name] = poison((cap,), torch.int32)
    B.replay_tail_layout(i32(ext).to(DEV), i32(seq).to(DEV), 128, out=t,
                         is_decode=None if dec is None else i32(dec).to(DEV), borrow_prefix_window=borrow)
    return {k: v.cpu().numpy() for k, v in t.items()}


def _enc_dev(pre, ext):
    nreq = len(ext)
    cap = 128 * nreq + int(sum(ext))
    t = dict(row_start=poison((nreq + 1,), torch.int32))
    for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
        t[name] = poison((max(cap, 1),), torch.int32)
    B.encoder_replay_layout(i32(pre).to(DEV), i32(ext).to(DEV), int(sum(ext)), 128, out=t)
    return {k: v.cpu().numpy() for k, v in t.items()}


def _same_rows(d, o, start_key):
    tot = int(o[start_key][-1])
    assert d[start_key].tolist() == o[start_key].tolist()
    for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
        assert np.array_equal(d[name][:tot], o[name]), name


# ------------------------------------------------------------------- layouts
def test_tail_layout_mixed_batches_and_borrow(orc):
    say("case: tail layout with decode requests and the borrow flag, page examples and 700 random requests")
    rng = np.random.default_rng(21)
    e = rng.integers(0, 400, size=700)
    dec = (rng.random(700) < 0.4).astype(np.int32)
    e[dec == 1] = rng.integers(1, 9, size=int(dec.sum()))
    s = e + rng.integers(0, 1000, size=700)
    cases = [([8192, 1, 40, 3], [8192, 9000, 5000, 700], [0, 1, 0, 1]), ([64], [8256], None),
             (e.tolist(), s.tolist(), dec.tolist())]
    for ext, seq, dc in cases:
        for borrow in (False, True):
            d = _tail_dev(ext, seq, dc, borrow)
            o = orc.replay_tail_layout(ext, seq, 128, is_decode=dc, borrow_prefix_window=borrow)
            assert d["tail_len"].tolist() == o["tail_len"].tolist()
            _same_rows(d, o, "tail_row_start")


def test_encoder_replay_layout(orc):
    say("case: encoder replay layout, page example and 700 random requests")
    rng = np.random.default_rng(22)
    pre = rng.integers(0, 600, size=700)
    pre[rng.random(700) < 0.2] = 0
    ext = rng.integers(0, 300, size=700)
    for p, e in (([8192], [100]), ([0, 1, 127, 128, 129, 5000, 0, 40], [10, 0, 1, 200, 128, 3, 0, 7]),
                 (pre.tolist(), ext.tolist())):
        _same_rows(_enc_dev(p, e), orc.encoder_replay_layout(p, e), "row_start")


# --------------------------------------------------------------------- flows
H, HI, DI, D, K, BLK, NB = 16, 64, 128, 512, 128, 8, 256


class _Layer:
    """Per-layer inputs of a flow: index q and weights, attention q and an MXFP8 window
    (quantized on both sides from the same rows, bytes compared)."""

    def __init__(self, orc, tag, seed, nrows, win):
        self.qi = synth.normal_bf16((nrows, HI, DI), seed, "index_q/" + tag, device=DEV)
        self.w = synth.uniform((nrows, HI), seed, "index_w/" + tag, device=DEV)
        self.q = synth.normal_bf16((nrows, H, D), seed, "q/" + tag, device=DEV)
        raw = synth.normal((win["rows"], D), seed, "swa/" + tag, device=DEV)
        cd, sd = B.quant_mx(B.MXFP8_E4M3, raw)
        co, so = orc.mx_quant(orc.E4M3, raw.cpu().numpy())
        assert np.array_equal(co, cd.cpu().numpy()) and np.array_equal(so, sd.cpu().numpy())
        self.win_d = B.Window(cd, sd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
        self.win_o = dict(data=co, dtype=3, scale=so, row_start=win["row_start"].numpy(),
                          pos_start=win["pos_start"].numpy(), window=128)


class _Owner:
    """One KV owner (m = 1, the decoder's): MXFP4 index keys and bf16 main KV, quantized on
    both sides and compared."""

    def __init__(self, orc, seq, seed):
        self.geom = synth.Geometry(list(seq), 1)
        g = self.geom
        self.cache = dict(ratio_m=1, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
        self.cd = dev_cache(self.cache)
        raw = synth.normal((g.total_entries, DI), seed, "index_keys", device=DEV)
        kd, ksd = B.quant_mx(B.MXFP4, raw)
        self.ko, self.kso = orc.mx_quant(orc.E2M1, raw.cpu().numpy())
        assert np.array_equal(self.ko, kd.cpu().numpy()) and np.array_equal(self.kso, ksd.cpu().numpy())
        self.keys = B.IndexKeys(kd, ksd, DI)
        self.kv = synth.normal_bf16((g.total_entries, D), seed, "kv", device=DEV)
        self.kvb = bits(self.kv)
        self.C = max(g.n_entries)


def _full_layer(orc, own, rows, L, sample):
    """Source layer over `rows` (dict of host arrays): library on every row, oracle on the
    sampled rows.  Returns the device outputs and the oracle's sampled index sets / pools."""
    rd = B.Rows(i32(rows["req_of_row"]).to(DEV), i32(rows["pos_of_row"]).to(DEV),
                None if rows.get("win_lo") is None else i32(rows["win_lo"]).to(DEV))
    n = len(rows["req_of_row"])
    sc = B.index_score(rd, own.cd, L.qi, L.w, own.keys, score_stride=own.C)
    ws = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, n, own.C, K, NB)), dtype=torch.uint8, device=DEV)
    idx, pb, pn = B.topk_hier(rd, own.cd, sc, K, BLK, NB, workspace=ws)
    out = B.sparse_swa_attn(rd, own.cd, L.q, own.kv, idx, L.win_d, synth.sm_scale(D))
    torch.cuda.synchronize()
    rs = {k: np.asarray(v)[sample] for k, v in rows.items() if v is not None}
    s_o, bad = orc.index_score(rs, own.cache, L.qi[sample].float().cpu().numpy(), L.w[sample].cpu().numpy(), own.ko,
                               key_scales=own.kso, heads=HI, dim=DI, score_stride=own.C)
    assert bad == 0
    reach = [min(p + 1, own.geom.n_entries[r]) for r, p in zip(rs["req_of_row"], rs["pos_of_row"])]
    check_scores(sc[sample].cpu().numpy(), s_o, reach)
    i_o, b_o, n_o = orc.topk_hier(rs, own.cache, s_o, K, BLK, NB)
    assert np.array_equal(idx[sample].cpu().numpy(), i_o)
    assert np.array_equal(pn[sample].cpu().numpy(), n_o) and np.array_equal(pb[sample].cpu().numpy(), b_o)
    a_o, _ = orc.sparse_swa_attn(rs, own.cache, bits(L.q[sample]), 1, own.kvb, 1, i_o, L.win_o, heads=H, dim=D,
                                 sm_scale=synth.sm_scale(D))
    check_attn(out[sample].float().cpu().numpy(), a_o)
    return dict(rd=rd, idx=idx, pb=pb, pn=pn), dict(idx=i_o, pb=b_o, pn=n_o)


def _late_layers(orc, own, rows_t, src_map, src_dev, src_o, Lr, Lu, sample, src_sample_pos):
    """Reindex (own q, scores over the source pools through the row map) and Reuse (the
    source index sets through the row map) on the late-layer rows; sampled rows checked.
    src_sample_pos[i] is the position, within the source layer's sample, of the source
    row that sampled late row i reads."""
    rt = B.Rows(i32(rows_t["req_of_row"]).to(DEV), i32(rows_t["pos_of_row"]).to(DEV), i32(rows_t["win_lo"]).to(DEV))
    nt = len(rows_t["req_of_row"])
    smap = i32(src_map).to(DEV)
    pool = B.Pool(src_dev["pb"], src_dev["pn"], BLK, smap)
    sc = B.index_score(rt, own.cd, Lr.qi, Lr.w, own.keys, pool=pool, score_stride=NB * BLK)
    wsd = torch.empty(max(1, B.workspace_size(B.OP_TOPK, nt, NB * BLK, K)), dtype=torch.uint8, device=DEV)
    idx_r = B.topk(rt, own.cd, sc, K, pool=pool, workspace=wsd)
    out_r = B.sparse_swa_attn(rt, own.cd, Lr.q, own.kv, idx_r, Lr.win_d, synth.sm_scale(D))
    out_u = B.sparse_swa_attn(rt, own.cd, Lu.q, own.kv, src_dev["idx"], Lu.win_d, synth.sm_scale(D), sel_row_map=smap)
    torch.cuda.synchronize()
    rs = {k: np.asarray(v)[sample] for k, v in rows_t.items()}
    ns = len(sample)
    pool_o = dict(blocks=src_o["pb"][src_sample_pos], nblocks=src_o["pn"][src_sample_pos], block=BLK, max_blocks=NB,
                  row_map=np.arange(ns))
    s_o, bad = orc.index_score(rs, own.cache, Lr.qi[sample].float().cpu().numpy(), Lr.w[sample].cpu().numpy(),
                               own.ko, key_scales=own.kso, heads=HI, dim=DI, score_stride=NB * BLK, pool=pool_o)
    assert bad == 0
    check_scores(sc[sample].cpu().numpy(), s_o, (pool_o["nblocks"] * BLK).tolist())
    i_o = orc.topk(rs, own.cache, s_o, K, pool=pool_o)
    assert np.array_equal(idx_r[sample].cpu().numpy(), i_o)
    for L, sel_o, out in ((Lr, i_o, out_r), (Lu, src_o["idx"][src_sample_pos], out_u)):
        a_o, _ = orc.sparse_swa_attn(rs, own.cache, bits(L.q[sample]), 1, own.kvb, 1, sel_o, L.win_o, heads=H,
                                     dim=D, sm_scale=synth.sm_scale(D))
        check_attn(out[sample].float().cpu().numpy(), a_o)


def test_mixed_prefill_decode_flow(orc):
    """A batch of prefill extends (cached prefixes, one short extend) and decode requests
    (one and four new tokens): source layer over every extend row, tail layout with the
    decode flags, then Reindex and Reuse over the tail rows; decode rows keep full windows."""
    say("case: mixed prefill + decode batch through the source layer, tail layout, Reindex and Reuse")
    ext = [300, 1, 2000, 64, 4, 1]
    seq = [3000, 2500, 2000, 900, 1700, 130]
    dec = [0, 1, 0, 0, 1, 1]
    own = _Owner(orc, seq, 501)
    held = [min(s, e + 127) for s, e in zip(seq, ext)]
    win = synth.window_cache_geometry(own.geom, 128, rows_held=held)
    ext_req = np.concatenate([np.full(e, r) for r, e in enumerate(ext)]).astype(np.int32)
    ext_pos = np.concatenate([np.arange(s - e, s) for s, e in zip(seq, ext)]).astype(np.int32)
    rows = dict(req_of_row=ext_req, pos_of_row=ext_pos)
    Ls = _Layer(orc, "src", 501, len(ext_req), win)
    t = _tail_dev(ext, seq, dec)
    t_o = orc.replay_tail_layout(ext, seq, 128, is_decode=dec)
    _same_rows(t, t_o, "tail_row_start")
    nt = int(t_o["tail_row_start"][-1])
    st = t_o["tail_row_start"]
    # decode rows: every one of them, and the first and last tail row of every request
    late_sample = sorted(set(sum([list(range(st[r], st[r + 1])) for r in range(len(ext)) if dec[r]], [])
                             + [int(st[r]) for r in range(len(ext)) if st[r + 1] > st[r]]
                             + [int(st[r + 1]) - 1 for r in range(len(ext)) if st[r + 1] > st[r]]))
    src_rows = t_o["src_row"][late_sample]
    src_sample = sorted(set(src_rows.tolist()) | {0, 299, 1500})
    src_pos_of = {r: i for i, r in enumerate(src_sample)}
    src_dev, src_o = _full_layer(orc, own, rows, Ls, src_sample)
    rows_t = dict(req_of_row=t_o["req_of_row"], pos_of_row=t_o["abs_pos"], win_lo=t_o["win_lo"])
    assert np.all(t_o["win_lo"][st[1]:st[2]] == 0) and np.all(t_o["win_lo"][st[3]:st[4]] == 900 - 64)
    Lr = _Layer(orc, "reindex", 501, nt, win)
    Lu = _Layer(orc, "reuse", 501, nt, win)
    _late_layers(orc, own, rows_t, t_o["src_row"], src_dev, src_o, Lr, Lu, late_sample,
                 [src_pos_of[r] for r in src_rows])


def test_chunked_extends_flow(orc):
    """A 4096-token prompt scheduled as four 1024-token extends ([P2] section 2.5, scaled
    down): each chunk runs the source layer over its own rows and the late layers over its
    own tail (window cut at each chunk's tail start), the cache growing chunk by chunk."""
    say("case: chunked prefill, four 1024-token extends, tails per chunk")
    S_all = 4096
    own = _Owner(orc, [S_all], 502)
    win = synth.window_cache_geometry(own.geom, 128, rows_held=[S_all])
    for c in range(4):
        S = 1024 * (c + 1)
        t_o = orc.replay_tail_layout([1024], [S], 128)
        t = _tail_dev([1024], [S])
        _same_rows(t, t_o, "tail_row_start")
        assert t_o["abs_pos"][0] == S - 128 and np.all(t_o["win_lo"] == S - 128)
        # the cache as it stands after this chunk: S entries (m = 1)
        cache_c = dict(own.cache, n_entries=np.array([S]))
        own_c = own
        saved = (own.cache, own.cd)
        own_c.cache, own_c.cd = cache_c, dev_cache(cache_c)
        try:
            rows = dict(req_of_row=np.zeros(1024, np.int32), pos_of_row=np.arange(S - 1024, S, dtype=np.int32))
            Ls = _Layer(orc, "src%d" % c, 502, 1024, win)
            sample_src = [0, 1023 - 127, 1023]
            src_dev, src_o = _full_layer(orc, own_c, rows, Ls, sample_src)
            rows_t = dict(req_of_row=t_o["req_of_row"], pos_of_row=t_o["abs_pos"], win_lo=t_o["win_lo"])
            Lr = _Layer(orc, "reindex%d" % c, 502, 128, win)
            Lu = _Layer(orc, "reuse%d" % c, 502, 128, win)
            _late_layers(orc, own_c, rows_t, t_o["src_row"], src_dev, src_o, Lr, Lu, [0, 127], [1, 2])
        finally:
            own.cache, own.cd = saved


def test_encoder_replay_flow(orc):
    """Encoder-side replay: requests with cached prefixes (one of 8192 tokens, as on the
    page) and new extends; the rows of the encoder layout (replayed prefix rows, then the
    extend) run scoring, selection and attention with windows cut at R0."""
    say("case: encoder-side replay rows through scoring, selection and attention")
    pre = [8192, 50, 0, 700]
    ext = [100, 30, 200, 1]
    seq = [p + e for p, e in zip(pre, ext)]
    own = _Owner(orc, seq, 503)
    held = [min(s, e + 128) for s, e in zip(seq, ext)]
    win = synth.window_cache_geometry(own.geom, 128, rows_held=held)
    lay = _enc_dev(pre, ext)
    lay_o = orc.encoder_replay_layout(pre, ext)
    _same_rows(lay, lay_o, "row_start")
    n = int(lay_o["row_start"][-1])
    rows = dict(req_of_row=lay_o["req_of_row"], pos_of_row=lay_o["abs_pos"], win_lo=lay_o["win_lo"])
    rs = lay_o["row_start"]
    sample = sorted(set([int(rs[r]) for r in range(4)] + [int(rs[r + 1]) - 1 for r in range(4)]
                        + [int(rs[0]) + 127, int(rs[0]) + 128, int(rs[1]) + 49, int(rs[1]) + 50]))
    L = _Layer(orc, "enc", 503, n, win)
    _full_layer(orc, own, rows, L, sample)


def test_multi_token_decode_rows(orc):
    """Decode steps with several query rows per request (verify rows at consecutive
    positions sharing one cache): 6 requests x 4 rows at S - 4 .. S - 1 (m = 2), through
    full-range scores, the hierarchical selection, attention with FP4 main KV, and a
    Reindex layer through the fused pool top-k; every row checked against the oracle."""
    say("case: multi-token decode rows (6 requests x 4 verify rows)")
    seq = [9000, 20001, 33333, 4097, 16384, 65536]
    T = 4
    geom = synth.Geometry(seq, 2)
    cache = dict(ratio_m=2, n_entries=np.array(geom.n_entries), row_start=np.array(geom.row_start))
    cd = dev_cache(cache)
    req = np.repeat(np.arange(len(seq)), T).astype(np.int32)
    pos = np.concatenate([np.arange(s - T, s) for s in seq]).astype(np.int32)
    rows = dict(req_of_row=req, pos_of_row=pos)
    n = len(req)
    rd = B.Rows(i32(req).to(DEV), i32(pos).to(DEV))
    raw = synth.normal((geom.total_entries, DI), 504, "index_keys", device=DEV)
    kd, ksd = B.quant_mx(B.MXFP4, raw)
    ko, kso = orc.mx_quant(orc.E2M1, raw.cpu().numpy())
    keys = B.IndexKeys(kd, ksd, DI)
    kv = synth.normal_bf16((geom.total_entries, D), 504, "kv", device=DEV)
    kv4, kv4s = B.quant_mx(B.FP4_S16, kv)
    kv4o, kv4so = orc.fp4s16_quant(kv.float().cpu().numpy())
    assert np.array_equal(kv4o, kv4.cpu().numpy()) and np.array_equal(kv4so, kv4s.cpu().numpy())
    win = synth.window_cache_geometry(geom, 128, rows_held=[128 + T] * len(seq))
    C = max(geom.n_entries)
    kk, nbk = 512, 2048
    sm = synth.sm_scale(D)
    lay = [_Layer(orc, "mt%d" % l, 504, n, win) for l in range(2)]
    # source layer
    sc = B.index_score(rd, cd, lay[0].qi, lay[0].w, keys, score_stride=C)
    idx, pb, pn = B.topk_hier(rd, cd, sc, kk, BLK, nbk)
    out0 = B.sparse_swa_attn(rd, cd, lay[0].q, kv4, idx, lay[0].win_d, sm, kv_scale=kv4s)
    # Reindex layer through the fused pool top-k
    pool = B.Pool(pb, pn, BLK)
    idx1 = B.index_topk_pool(rd, cd, lay[1].qi, lay[1].w, keys, pool, kk)
    out1 = B.sparse_swa_attn(rd, cd, lay[1].q, kv4, idx1, lay[1].win_d, sm, kv_scale=kv4s)
    torch.cuda.synchronize()
    s_o, bad = orc.index_score(rows, cache, lay[0].qi.float().cpu().numpy(), lay[0].w.cpu().numpy(), ko,
                               key_scales=kso, heads=HI, dim=DI, score_stride=C)
    assert bad == 0
    check_scores(sc.cpu().numpy(), s_o, [min((p + 1) // 2, geom.n_entries[r]) for r, p in zip(req, pos)])
    i_o, b_o, n_o = orc.topk_hier(rows, cache, s_o, kk, BLK, nbk)
    assert np.array_equal(idx.cpu().numpy(), i_o)
    assert np.array_equal(pb.cpu().numpy(), b_o) and np.array_equal(pn.cpu().numpy(), n_o)
    pool_o = dict(blocks=b_o, nblocks=n_o, block=BLK, max_blocks=nbk)
    s1, bad = orc.index_score(rows, cache, lay[1].qi.float().cpu().numpy(), lay[1].w.cpu().numpy(), ko,
                              key_scales=kso, heads=HI, dim=DI, score_stride=BLK * nbk, pool=pool_o)
    assert bad == 0
    i1 = orc.topk(rows, cache, s1, kk, pool=pool_o)
    assert np.array_equal(idx1.cpu().numpy(), i1)
    for L, sel_o, out in ((lay[0], i_o, out0), (lay[1], i1, out1)):
        a_o, _ = orc.sparse_swa_attn(rows, cache, bits(L.q), 1, kv4o, orc.DT_FP4S16, sel_o, L.win_o, heads=H, dim=D,
                                     sm_scale=sm, kv_scale=kv4so)
        check_attn(out.float().cpu().numpy(), a_o)
