"""GPU parity at the workloads' full sizes.

Each test runs the HIP path on a whole workload (the decode step exactly as the
benchmark launches it for C3; C1 prefill with its full 8192-token requests; the C2
bounded-replay flow; C4 long-context decode) and recomputes a sample of rows with the
oracle, row by row: index scores and index sets bit for bit, attention outputs within
|g - r| <= 2e-2 + 1e-2 |r| and a per-row relative L2 error <= 1e-2.  Sampled rows
include the boundary positions (0, 126..129, 510..512, S - 1).  Every oracle input is
regenerated from the seeded generator and quantized by the oracle's own quantizer; its
bytes are checked against the library's before use.  Every row is checked as well: each
row's selection against its definition evaluated over the device's scores (C1, C2, C3,
C4), and each row's attention against the oracle over a compact cache of the rows it
selected (C2's tail rows, C3, C4)."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B
from compressed_sparse_attention_fp4_amd import synth

from gpu_util import DEV, bits, check_attn, check_scores, dev_cache, dev_rows, i32, i64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def oracle_window(orc, raw_rows, nreq_rows, pos_start, window=128):
    """Window rows (float32 host) -> the oracle's MXFP8 window dict."""
    codes, scales = orc.mx_quant(orc.E4M3, raw_rows)
    return codes, scales, dict(data=codes, dtype=3, scale=scales,
                               row_start=np.arange(nreq_rows, dtype=np.int64) * window,
                               pos_start=np.asarray(pos_start, dtype=np.int32), window=window)


# ------------------------------------------------------------------------- C3
@pytest.fixture(scope="module")
def c3_step():
    """The benchmark's input set 0 after one decode step, launched as bench.py times it."""
    import bench
    x = bench.InputSet(0, DEV)
    bench.step(x)
    torch.cuda.synchronize()
    return x


def order_keys(v):
    """float32 -> the selection's order-preserving uint32 keys (larger key = larger value)."""
    b = np.asarray(v, np.float32).view(np.uint32)
    return np.where(b >> 31, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def top_positions(keys, pos, k):
    """The k best (key desc, position asc) positions, ascending."""
    order = np.lexsort((pos, -keys.astype(np.int64)))
    return np.sort(pos[order[:k]])


def check_hier_by_definition(scores, reach, pb, pn, idx, k, nb, blk):
    """Hierarchical selection of every row, by its definition over the given score rows: the
    pool is the nb - 1 best non-newest blocks by maximum score (ties to the lower block id)
    plus the newest block, or every block when they fit; the index set is the k best pool
    positions below the reach (ties to the lower position), ascending."""
    for r, R in enumerate(reach):
        sk = order_keys(scores[r, :R])
        nblk = (R + blk - 1) // blk
        if nblk <= nb:
            pool = np.arange(nblk)
        else:
            full = (R // blk) * blk
            bmax = sk[:full].reshape(-1, blk).max(axis=1)[:nblk - 1]
            pool = np.sort(np.concatenate([top_positions(bmax, np.arange(nblk - 1), nb - 1), [nblk - 1]]))
        assert pn[r] == len(pool) and np.array_equal(pb[r, :pn[r]], pool), r
        assert np.all(pb[r, pn[r]:] == -1), r
        cand = (pool[:, None] * blk + np.arange(blk)[None, :]).ravel()
        cand = cand[cand < R]
        want = top_positions(sk[cand], cand, k)
        assert np.array_equal(idx[r, :len(want)], want) and np.all(idx[r, len(want):] == -1), r


def check_attn_compact(orc, kv, kv_base, sel, q, wo, pos, ratio_m, heads, dim, win_lo=None):
    """Attention of every row against the oracle over a compact cache: row r's selected
    main-KV rows (kv[kv_base[r] + sel[r, i]]) gathered to rows r * k + i (-1 slots stay
    -1), row r being request r of the compact cache (so `wo` gives each row's window by
    row: row_start / pos_start indexed by the row's own request)."""
    n, k = sel.shape
    valid = sel >= 0
    src = kv_base.to(torch.int64)[:, None] + torch.where(valid, sel, torch.zeros_like(sel)).to(torch.int64)
    kv_c = bits(kv[src.reshape(-1)])
    rows_o = dict(req_of_row=np.arange(n), pos_of_row=np.asarray(pos))
    if win_lo is not None:
        rows_o["win_lo"] = np.asarray(win_lo)
    cache_o = dict(ratio_m=ratio_m, n_entries=np.full(n, k), row_start=np.arange(n, dtype=np.int64) * k)
    sel_o = np.where(valid.cpu().numpy(), np.arange(k, dtype=np.int32)[None, :], -1).astype(np.int32)
    out_o, _ = orc.sparse_swa_attn(rows_o, cache_o, bits(q), 1, kv_c, 1, sel_o, wo, heads=heads, dim=dim,
                                   sm_scale=synth.sm_scale(dim))
    return out_o


def check_flat_topk_torch(scores, reach, idx, k):
    """Every row's flat top-k (score desc, position asc, among positions below its reach),
    ascending and -1 padded, evaluated on the device with a composite key (the selection's
    order key, then the complement of the position) in chunks of rows."""
    n, cols = scores.shape
    col = torch.arange(cols, device=scores.device, dtype=torch.int64)
    with torch.no_grad():
        for r0 in range(0, n, 4096):
            b = scores[r0:r0 + 4096].contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
            key = torch.where(b >= 0x80000000, 0xFFFFFFFF - b, b | 0x80000000)
            comp = key * cols + (cols - 1 - col)
            comp = torch.where(col[None, :] < reach[r0:r0 + 4096, None], comp, torch.full_like(comp, -1))
            top = torch.topk(comp, k, dim=1).values
            big = 1 << 40
            want = torch.where(top >= 0, cols - 1 - (top % cols), torch.full_like(top, big))
            want = torch.sort(want, dim=1).values
            want = torch.where(want == big, torch.full_like(want, -1), want)
            assert torch.equal(want.to(torch.int32), idx[r0:r0 + 4096]), r0


def test_c3_decode_step_sampled(orc, c3_step):
    """The benchmark's decode step (64 requests x 1 query, S=131072, m=2, source layer
    with hierarchical selection, then 7 Reindex layers through the fused pool scoring +
    top-k), launched exactly as bench.py times it; the source layer and the last Reindex
    layer checked on sampled rows (that layer's pool scores from the two-launch path's
    scoring call on the same inputs)."""
    import bench
    say("case: C3 full decode step (bench input set 0), oracle on sampled rows")
    x = c3_step
    seed, C, S, W = 3000, bench.C, bench.SEQ, bench.W
    sample = [0, 45]
    ns = len(sample)
    # index keys of the sampled requests, regenerated (1M-row chunks hold 16 requests)
    raw = []
    for r in sample:
        c0 = (r * C) // (1 << 20) * (1 << 20)
        chunk = synth.normal((min(1 << 20, bench.NREQ * C - c0), bench.DI), seed, "index_keys/%d" % c0, device=DEV)
        raw.append(chunk[r * C - c0:r * C - c0 + C].cpu())
        del chunk
    raw = torch.cat(raw).numpy()
    ko, kso = orc.mx_quant(orc.E2M1, raw)
    for s_i, r in enumerate(sample):
        assert np.array_equal(ko[s_i * C:(s_i + 1) * C], x.kcodes[r * C:(r + 1) * C].cpu().numpy())
        assert np.array_equal(kso[s_i * C:(s_i + 1) * C], x.kscale[r * C:(r + 1) * C].cpu().numpy())
    rows_o = dict(req_of_row=np.arange(ns), pos_of_row=np.full(ns, S - 1))
    cache_o = dict(ratio_m=bench.M, n_entries=np.full(ns, C), row_start=np.arange(ns, dtype=np.int64) * C)
    kv_o = np.concatenate([bits(x.kv[r * C:(r + 1) * C]) for r in sample])
    sm = synth.sm_scale(bench.D)

    def window_for(l):
        full = synth.normal((bench.NREQ * W, bench.D), seed, "swa/%d" % l, device=DEV)
        rw = torch.cat([full[r * W:(r + 1) * W] for r in sample]).cpu().numpy()
        codes, scales, wo = oracle_window(orc, rw, ns, [S - W] * ns, W)
        wd = x.layers[l]["window"]
        for s_i, r in enumerate(sample):
            assert np.array_equal(codes[s_i * W:(s_i + 1) * W], wd.data[r * W:(r + 1) * W].cpu().numpy())
            assert np.array_equal(scales[s_i * W:(s_i + 1) * W], wd.scale[r * W:(r + 1) * W].cpu().numpy())
        return wo

    # source layer: full-range scores, hierarchical selection, attention
    L0 = x.layers[0]
    s_o, bad = orc.index_score(rows_o, cache_o, L0["qi"][sample].float().cpu().numpy(), L0["w"][sample].cpu().numpy(),
                               ko, key_scales=kso, heads=bench.HI, dim=bench.DI, score_stride=C)
    assert bad == 0
    say("  source scores")
    check_scores(x.scores_full[sample].cpu().numpy(), s_o, [C] * ns)
    ri, rb, rn = orc.topk_hier(rows_o, cache_o, s_o, bench.K, bench.BLK, bench.NB)
    say("  hierarchical selection")
    assert np.array_equal(x.idx[0][sample].cpu().numpy(), ri)
    assert np.array_equal(x.pool_n[sample].cpu().numpy(), rn)
    assert np.array_equal(x.pool_blocks[sample].cpu().numpy(), rb)
    out_o, _ = orc.sparse_swa_attn(rows_o, cache_o, bits(L0["q"][sample]), 1, kv_o, 1, ri, window_for(0),
                                   heads=bench.H, dim=bench.D, sm_scale=sm)
    say("  source attention")
    check_attn(x.out[0][sample].float().cpu().numpy(), out_o)

    # the last Reindex layer: pool scores, pool top-k, attention
    L7 = x.layers[bench.LAYERS - 1]
    pool_o = dict(blocks=rb, nblocks=rn, block=bench.BLK, max_blocks=bench.NB)
    s7, bad = orc.index_score(rows_o, cache_o, L7["qi"][sample].float().cpu().numpy(), L7["w"][sample].cpu().numpy(),
                              ko, key_scales=kso, heads=bench.HI, dim=bench.DI, score_stride=bench.NB * bench.BLK,
                              pool=pool_o)
    assert bad == 0
    say("  Reindex scores")
    s7_d = B.index_score(x.rows, x.cache, L7["qi"], L7["w"], x.keys, pool=x.pool,
                         scores=torch.full_like(x.scores_pool, float("nan")))
    check_scores(s7_d[sample].cpu().numpy(), s7, (rn * bench.BLK).tolist())
    i7 = orc.topk(rows_o, cache_o, s7, bench.K, pool=pool_o)
    say("  Reindex selection")
    assert np.array_equal(x.idx[bench.LAYERS - 1][sample].cpu().numpy(), i7)
    out7, _ = orc.sparse_swa_attn(rows_o, cache_o, bits(L7["q"][sample]), 1, kv_o, 1, i7,
                                  window_for(bench.LAYERS - 1), heads=bench.H, dim=bench.D, sm_scale=sm)
    say("  Reindex attention")
    check_attn(x.out[bench.LAYERS - 1][sample].float().cpu().numpy(), out7)


def test_c3_decode_step_every_row(orc, c3_step):
    """Every row of every layer of the decode step.  Selections: the source layer's pools and
    index sets, and each Reindex layer's index set, equal their definitions evaluated on the
    host over the device's own scores (full-range scores from the step; pool scores from the
    scoring call, bit-exact to the oracle on the sampled rows above).  Attention: all 64 rows
    of all 8 layers against the oracle, each row's selected main-KV rows gathered into a
    compact cache (attention depends on the selected rows only), the FP8 window regenerated
    and quantized by the oracle."""
    import bench
    say("case: C3 full decode step, every row of every layer")
    x = c3_step
    seed, C, S, W, K, NB, BLK, n = 3000, bench.C, bench.SEQ, bench.W, bench.K, bench.NB, bench.BLK, bench.NREQ
    R = min(S // bench.M, C)
    # source layer: block maxima, the pool (NB - 1 best non-newest blocks plus the newest), top-K
    pb, pn = x.pool_blocks.cpu().numpy(), x.pool_n.cpu().numpy()
    check_hier_by_definition(x.scores_full.cpu().numpy(), [R] * n, pb, pn, x.idx[0].cpu().numpy(), K, NB, BLK)
    say("  source pools and index sets: %d rows" % n)
    # Reindex layers: top-K over the pool positions by the pool scores
    for l in range(1, bench.LAYERS):
        L = x.layers[l]
        sp = B.index_score(x.rows, x.cache, L["qi"], L["w"], x.keys, pool=x.pool,
                           scores=torch.full_like(x.scores_pool, float("nan"))).cpu().numpy()
        got = x.idx[l].cpu().numpy()
        for r in range(n):
            cols = np.arange(pn[r] * BLK)
            posn = pb[r, cols // BLK] * BLK + cols % BLK
            ok = posn < R
            assert np.array_equal(got[r], top_positions(order_keys(sp[r, cols[ok]]), posn[ok], K)), (l, r)
    say("  Reindex index sets: %d layers x %d rows" % (bench.LAYERS - 1, n))
    # attention of every row and layer, over a compact cache of the selected rows
    for l in range(bench.LAYERS):
        raw = synth.normal((n * W, bench.D), seed, "swa/%d" % l, device=DEV).cpu().numpy()
        codes, scales, wo = oracle_window(orc, raw, n, [S - W] * n, W)
        wd = x.layers[l]["window"]
        assert np.array_equal(codes, wd.data.cpu().numpy()) and np.array_equal(scales, wd.scale.cpu().numpy())
        out_o = check_attn_compact(orc, x.kv, x.cache.row_start, x.idx[l], x.layers[l]["q"], wo, [S - 1] * n, bench.M,
                                   bench.H, bench.D)
        check_attn(x.out[l].float().cpu().numpy(), out_o)
    say("  attention: %d layers x %d rows" % (bench.LAYERS, n))


# ------------------------------------------------------------------------- C1
def test_c1_prefill_sampled(orc):
    """C1 Full-layer prefill (m=1, 8 requests of 8192 tokens, top-512, fp8 window): scores,
    flat top-512 and attention for every row on the GPU; sampled rows of every request
    checked against the oracle, and every row's top-512 against its definition over the
    device's scores."""
    cfg = synth.config(1)
    g = cfg.geom
    say("case: %s (every row on the GPU)" % cfg.name)
    rows = synth.prefill_rows(g)
    n = rows["req_of_row"].numel()
    cache = dict(ratio_m=1, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    keys_raw = synth.normal((g.total_entries, cfg.index_dim), cfg.seed, "index_keys", device=DEV)
    kd, ksd = B.quant_mx(B.MXFP4, keys_raw)
    qi = synth.normal_bf16((n, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q", device=DEV)
    w = synth.uniform((n, cfg.index_heads), cfg.seed, "index_w", device=DEV)
    rd, cd = dev_rows(rows), dev_cache(cache)
    scores = B.index_score(rd, cd, qi, w, B.IndexKeys(kd, ksd, cfg.index_dim), score_stride=g.n_entries[0])
    idx = B.topk(rd, cd, scores, cfg.topk, workspace=torch.empty(
        max(1, B.workspace_size(B.OP_TOPK, n, g.n_entries[0], cfg.topk)), dtype=torch.uint8, device=DEV))
    q = synth.normal_bf16((n, cfg.heads, cfg.dim), cfg.seed, "q", device=DEV)
    kv = synth.normal_bf16((g.total_entries, cfg.dim), cfg.seed, "kv", device=DEV)
    win = synth.window_cache_geometry(g, 128, rows_held=g.seq_len)
    swa_raw = synth.normal((win["rows"], cfg.dim), cfg.seed, "swa", device=DEV)
    scd, ssd = B.quant_mx(B.MXFP8_E4M3, swa_raw)
    wd = B.Window(scd, ssd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    out = B.sparse_swa_attn(rd, cd, q, kv, idx, wd, synth.sm_scale(cfg.dim))
    torch.cuda.synchronize()

    # every row: the top-512 by its definition over the device's scores
    S = g.seq_len[0]
    check_flat_topk_torch(scores, rd.pos_of_row.to(torch.int64) + 1, idx, cfg.topk)
    say("  every row's top-512")
    rng = np.random.default_rng(11)
    sample = []
    for r in range(g.nreq):
        pos = {0, 1, 127, 128, 511, 512, S - 1} | set(rng.choice(S, size=2, replace=False).tolist())
        sample += [r * S + p for p in sorted(pos)]
    req = rows["req_of_row"].numpy()[sample]
    pos = rows["pos_of_row"].numpy()[sample]
    rows_o = dict(req_of_row=req, pos_of_row=pos)
    ko, kso = orc.mx_quant(orc.E2M1, keys_raw.cpu().numpy())
    assert np.array_equal(ko, kd.cpu().numpy()) and np.array_equal(kso, ksd.cpu().numpy())
    s_o, bad = orc.index_score(rows_o, cache, qi[sample].float().cpu().numpy(), w[sample].cpu().numpy(), ko,
                               key_scales=kso, heads=cfg.index_heads, dim=cfg.index_dim, score_stride=S)
    assert bad == 0
    say("  scores")
    check_scores(scores[sample].cpu().numpy(), s_o, (pos + 1).tolist())
    i_o = orc.topk(rows_o, cache, s_o, cfg.topk)
    say("  top-512")
    assert np.array_equal(idx[sample].cpu().numpy(), i_o)
    codes, scales = orc.mx_quant(orc.E4M3, swa_raw.cpu().numpy())
    assert np.array_equal(codes, scd.cpu().numpy()) and np.array_equal(scales, ssd.cpu().numpy())
    wo = dict(data=codes, dtype=3, scale=scales, row_start=win["row_start"].numpy(), pos_start=win["pos_start"].numpy(),
              window=128)
    out_o, _ = orc.sparse_swa_attn(rows_o, cache, bits(q[sample]), 1, bits(kv), 1, i_o, wo, heads=cfg.heads,
                                   dim=cfg.dim, sm_scale=synth.sm_scale(cfg.dim))
    say("  attention")
    check_attn(out[sample].float().cpu().numpy(), out_o)


# ------------------------------------------------------------------------- C2
def test_c2_replay_flow_sampled(orc):
    """C2 bounded replay: a Full layer over the extends of 8 requests (S=8192 each) gives
    top-512 and pools; the tail layout picks each request's last min(128, E) rows; a
    Reindex layer rescoring the source pools (through the tail->extend row map) with its
    own q, then a Reuse layer attending to the source layer's indices through the same
    map.  Tail layout checked whole, everything else on sampled tail rows."""
    cfg = synth.config(2)
    g = cfg.geom
    E = synth.C2_EXTENDS
    say("case: %s" % cfg.name)
    ext_req = np.concatenate([np.full(e, r) for r, e in enumerate(E)]).astype(np.int32)
    ext_pos = np.concatenate([np.arange(s - e, s) for s, e in zip(g.seq_len, E)]).astype(np.int32)
    n_ext = len(ext_req)
    cache = dict(ratio_m=1, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    cd = dev_cache(cache)
    keys_raw = synth.normal((g.total_entries, cfg.index_dim), cfg.seed, "index_keys", device=DEV)
    kd, ksd = B.quant_mx(B.MXFP4, keys_raw)
    keys = B.IndexKeys(kd, ksd, cfg.index_dim)
    C = g.n_entries[0]
    # source (Full) layer over every extend row
    rows_ext = dict(req_of_row=ext_req, pos_of_row=ext_pos)
    re_d = dev_rows(rows_ext)
    qi_s = synth.normal_bf16((n_ext, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q/src", device=DEV)
    w_s = synth.uniform((n_ext, cfg.index_heads), cfg.seed, "index_w/src", device=DEV)
    sc_s = B.index_score(re_d, cd, qi_s, w_s, keys, score_stride=C)
    ws = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, n_ext, C, cfg.topk, cfg.max_blocks)), dtype=torch.uint8,
                     device=DEV)
    idx_s, pb, pn = B.topk_hier(re_d, cd, sc_s, cfg.topk, cfg.block, cfg.max_blocks, workspace=ws)
    # tail rows
    t = B.replay_tail_layout(i32(E).to(DEV), i32(g.seq_len).to(DEV), 128)
    t_o = orc.replay_tail_layout(E, g.seq_len, 128)
    nt = int(t_o["tail_row_start"][-1])
    assert nt == 960
    for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
        assert np.array_equal(t[name][:nt].cpu().numpy(), t_o[name]), name
    rows_t = dict(req_of_row=t_o["req_of_row"], pos_of_row=t_o["abs_pos"], win_lo=t_o["win_lo"])
    rt_d = B.Rows(t["req_of_row"][:nt], t["abs_pos"][:nt], t["win_lo"][:nt])
    src_map = t["src_row"][:nt].contiguous()
    pool_d = B.Pool(pb, pn, cfg.block, src_map)
    qi_t = synth.normal_bf16((nt, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q/reindex", device=DEV)
    w_t = synth.uniform((nt, cfg.index_heads), cfg.seed, "index_w/reindex", device=DEV)
    sc_t = B.index_score(rt_d, cd, qi_t, w_t, keys, pool=pool_d, score_stride=cfg.max_blocks * cfg.block)
    idx_t = B.topk(rt_d, cd, sc_t, cfg.topk, pool=pool_d, workspace=torch.empty(
        max(1, B.workspace_size(B.OP_TOPK, nt, cfg.max_blocks * cfg.block, cfg.topk)), dtype=torch.uint8,
        device=DEV))
    # the fused Reindex call (960 rows: one workgroup per whole pool) gives the same sets
    ws_f = torch.empty(max(1, B.workspace_size(B.OP_TOPK_POOL_FUSED, nt, cfg.max_blocks * cfg.block, cfg.topk)),
                       dtype=torch.uint8, device=DEV)
    idx_f = B.index_topk_pool(rt_d, cd, qi_t, w_t, keys, pool_d, cfg.topk, workspace=ws_f,
                              out=torch.full((nt, cfg.topk), -7, dtype=torch.int32, device=DEV))
    assert torch.equal(idx_f, idx_t)
    kv = synth.normal_bf16((g.total_entries, cfg.dim), cfg.seed, "kv", device=DEV)
    win = synth.window_cache_geometry(g, 128)
    outs = {}
    windows = {}
    for layer, sel, smap in (("reindex", idx_t, None), ("reuse", idx_s, src_map)):
        raw = synth.normal((win["rows"], cfg.dim), cfg.seed, "swa/" + layer, device=DEV)
        scd, ssd = B.quant_mx(B.MXFP8_E4M3, raw)
        windows[layer] = (raw.cpu().numpy(), scd.cpu().numpy(), ssd.cpu().numpy())
        q = synth.normal_bf16((nt, cfg.heads, cfg.dim), cfg.seed, "q/" + layer, device=DEV)
        wd = B.Window(scd, ssd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
        outs[layer] = (q, B.sparse_swa_attn(rt_d, cd, q, kv, sel, wd, synth.sm_scale(cfg.dim), sel_row_map=smap))
    torch.cuda.synchronize()

    # sampled tail rows: first and last of every request's tail plus a few more
    rng = np.random.default_rng(12)
    st = t_o["tail_row_start"]
    sample = sorted(set([int(st[r]) for r in range(len(E))] + [int(st[r + 1]) - 1 for r in range(len(E))]
                        + rng.choice(nt, size=8, replace=False).tolist()))
    ns = len(sample)
    src = t_o["src_row"][sample]
    ko, kso = orc.mx_quant(orc.E2M1, keys_raw.cpu().numpy())
    assert np.array_equal(ko, kd.cpu().numpy()) and np.array_equal(kso, ksd.cpu().numpy())
    # the source layer on the extend rows the sample reads
    rows_src = dict(req_of_row=ext_req[src], pos_of_row=ext_pos[src])
    s_src, bad = orc.index_score(rows_src, cache, qi_s[src].float().cpu().numpy(), w_s[src].cpu().numpy(), ko,
                                 key_scales=kso, heads=cfg.index_heads, dim=cfg.index_dim, score_stride=C)
    assert bad == 0
    check_scores(sc_s[src].cpu().numpy(), s_src, (ext_pos[src] + 1).tolist())
    ri, rb, rn = orc.topk_hier(rows_src, cache, s_src, cfg.topk, cfg.block, cfg.max_blocks)
    say("  source layer on the sampled tail rows' extend rows")
    assert np.array_equal(idx_s[src].cpu().numpy(), ri)
    assert np.array_equal(pn[src].cpu().numpy(), rn)
    assert np.array_equal(pb[src].cpu().numpy(), rb)
    # Reindex on the sampled tail rows, pools read through the row map
    rows_ts = {k: v[sample] for k, v in rows_t.items()}
    pool_o = dict(blocks=rb, nblocks=rn, block=cfg.block, max_blocks=cfg.max_blocks, row_map=np.arange(ns))
    s_t, bad = orc.index_score(rows_ts, cache, qi_t[sample].float().cpu().numpy(), w_t[sample].cpu().numpy(), ko,
                               key_scales=kso, heads=cfg.index_heads, dim=cfg.index_dim,
                               score_stride=cfg.max_blocks * cfg.block, pool=pool_o)
    assert bad == 0
    check_scores(sc_t[sample].cpu().numpy(), s_t, (rn * cfg.block).tolist())
    i_t = orc.topk(rows_ts, cache, s_t, cfg.topk, pool=pool_o)
    say("  Reindex scores and selection")
    assert np.array_equal(idx_t[sample].cpu().numpy(), i_t)
    kvb = bits(kv)
    for layer, sel_o in (("reindex", i_t), ("reuse", ri)):
        raw, scd, ssd = windows[layer]
        codes, scales = orc.mx_quant(orc.E4M3, raw)
        assert np.array_equal(codes, scd) and np.array_equal(scales, ssd)
        wo = dict(data=codes, dtype=3, scale=scales, row_start=win["row_start"].numpy(),
                  pos_start=win["pos_start"].numpy(), window=128)
        q, out = outs[layer]
        out_o, _ = orc.sparse_swa_attn(rows_ts, cache, bits(q[sample]), 1, kvb, 1, sel_o, wo, heads=cfg.heads,
                                       dim=cfg.dim, sm_scale=synth.sm_scale(cfg.dim))
        say("  %s attention" % layer)
        check_attn(out[sample].float().cpu().numpy(), out_o)

    # every row.  Source layer: 8192 positions are 1024 blocks of 8, within the 2048 a pool
    # holds, so every pool is all blocks of its row and the index set is the flat top-512.
    reach_s = torch.minimum(re_d.pos_of_row.to(torch.int64) + 1, torch.tensor(C, device=DEV))
    check_flat_topk_torch(sc_s, reach_s, idx_s, cfg.topk)
    nblk = (reach_s + cfg.block - 1) // cfg.block
    assert torch.equal(pn.to(torch.int64), nblk)
    ar = torch.arange(cfg.max_blocks, device=DEV, dtype=torch.int64)[None, :]
    assert torch.equal(pb.to(torch.int64), torch.where(ar < nblk[:, None], ar, torch.full_like(ar, -1)))
    say("  every source row's pool and top-512 (%d rows)" % n_ext)
    # Reindex: every tail row's top-512 over its pool by the pool scores
    sct, pbn, pnn, it = sc_t.cpu().numpy(), pb.cpu().numpy(), pn.cpu().numpy(), idx_t.cpu().numpy()
    srcs = t_o["src_row"]
    for i in range(nt):
        p_r, R = srcs[i], min(int(t_o["abs_pos"][i]) + 1, C)
        cols = np.arange(pnn[p_r] * cfg.block)
        posn = pbn[p_r, cols // cfg.block] * cfg.block + cols % cfg.block
        ok = posn < R
        want = top_positions(order_keys(sct[i, cols[ok]]), posn[ok], cfg.topk)
        assert np.array_equal(it[i, :len(want)], want) and np.all(it[i, len(want):] == -1), i
    say("  every tail row's Reindex top-512 (%d rows)" % nt)
    # attention of every tail row in both layers, over compact caches
    kv_base = cd.row_start.to(torch.int64)[t["req_of_row"][:nt].to(torch.int64)]
    req_t = t_o["req_of_row"]
    for layer, sel in (("reindex", idx_t), ("reuse", idx_s[src_map.to(torch.int64)])):
        raw, scd_l, ssd_l = windows[layer]
        codes, scales = orc.mx_quant(orc.E4M3, raw)
        wo_rows = dict(data=codes, dtype=3, scale=scales, row_start=win["row_start"].numpy()[req_t],
                       pos_start=win["pos_start"].numpy()[req_t], window=128)
        q, out = outs[layer]
        out_o = check_attn_compact(orc, kv, kv_base, sel, q, wo_rows, t_o["abs_pos"], 1, cfg.heads, cfg.dim,
                                   win_lo=t_o["win_lo"])
        check_attn(out.float().cpu().numpy(), out_o)
        say("  every tail row's %s attention (%d rows)" % (layer, nt))


# ------------------------------------------------------------------------- C4
@pytest.mark.parametrize("nreq", [1, 32])
def test_c4_long_decode_sampled(orc, nreq):
    """C4 long-context decode (S=524288, m=2: 262144 reachable entries per row): full
    scan, hierarchical selection and attention for every row; one row checked against the
    oracle end to end, every row's selection by its definition over the device scores and
    every row's attention against the oracle."""
    cfg = synth.config(4, nreq=nreq)
    g = cfg.geom
    say("case: %s" % cfg.name)
    C = g.n_entries[0]
    rows = synth.decode_rows(g)
    cache = dict(ratio_m=2, n_entries=np.array(g.n_entries), row_start=np.array(g.row_start))
    rd, cd = dev_rows(rows), dev_cache(cache)
    sample_r = nreq - 1
    kd = torch.empty((g.total_entries, cfg.index_dim // 2), dtype=torch.uint8, device=DEV)
    ksd = torch.empty((g.total_entries, cfg.index_dim // 32), dtype=torch.uint8, device=DEV)
    raw_sample = None
    for r in range(nreq):
        raw = synth.normal((C, cfg.index_dim), cfg.seed, "index_keys/%d" % r, device=DEV)
        kd[r * C:(r + 1) * C], ksd[r * C:(r + 1) * C] = B.quant_mx(B.MXFP4, raw)
        if r == sample_r:
            raw_sample = raw.cpu().numpy()
        del raw
    qi = synth.normal_bf16((nreq, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q", device=DEV)
    w = synth.uniform((nreq, cfg.index_heads), cfg.seed, "index_w", device=DEV)
    scores = B.index_score(rd, cd, qi, w, B.IndexKeys(kd, ksd, cfg.index_dim), score_stride=C)
    ws = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, nreq, C, cfg.topk, cfg.max_blocks)), dtype=torch.uint8,
                     device=DEV)
    idx, pb, pn = B.topk_hier(rd, cd, scores, cfg.topk, cfg.block, cfg.max_blocks, workspace=ws)
    q = synth.normal_bf16((nreq, cfg.heads, cfg.dim), cfg.seed, "q", device=DEV)
    kv = synth.normal_bf16((g.total_entries, cfg.dim), cfg.seed, "kv", device=DEV, chunk_rows=1 << 19)
    win = synth.window_cache_geometry(g, 128)
    swa_raw = synth.normal((win["rows"], cfg.dim), cfg.seed, "swa", device=DEV)
    scd, ssd = B.quant_mx(B.MXFP8_E4M3, swa_raw)
    wd = B.Window(scd, ssd, win["row_start"].to(DEV), win["pos_start"].to(DEV), 128)
    out = B.sparse_swa_attn(rd, cd, q, kv, idx, wd, synth.sm_scale(cfg.dim))
    torch.cuda.synchronize()

    i = sample_r
    ko, kso = orc.mx_quant(orc.E2M1, raw_sample)
    assert np.array_equal(ko, kd[i * C:(i + 1) * C].cpu().numpy())
    assert np.array_equal(kso, ksd[i * C:(i + 1) * C].cpu().numpy())
    S = g.seq_len[0]
    rows_o = dict(req_of_row=np.zeros(1), pos_of_row=np.full(1, S - 1))
    cache_o = dict(ratio_m=2, n_entries=np.full(1, C), row_start=np.zeros(1, dtype=np.int64))
    s_o, bad = orc.index_score(rows_o, cache_o, qi[i:i + 1].float().cpu().numpy(), w[i:i + 1].cpu().numpy(), ko,
                               key_scales=kso, heads=cfg.index_heads, dim=cfg.index_dim, score_stride=C)
    assert bad == 0
    say("  scores")
    check_scores(scores[i:i + 1].cpu().numpy(), s_o, [C])
    ri, rb, rn = orc.topk_hier(rows_o, cache_o, s_o, cfg.topk, cfg.block, cfg.max_blocks)
    say("  hierarchical selection")
    assert np.array_equal(idx[i:i + 1].cpu().numpy(), ri)
    assert np.array_equal(pn[i:i + 1].cpu().numpy(), rn)
    assert np.array_equal(pb[i:i + 1].cpu().numpy(), rb)
    W = 128
    rw = swa_raw[i * W:(i + 1) * W].cpu().numpy()
    codes, scales, wo = oracle_window(orc, rw, 1, [S - W], W)
    assert np.array_equal(codes, scd[i * W:(i + 1) * W].cpu().numpy())
    out_o, _ = orc.sparse_swa_attn(rows_o, cache_o, bits(q[i:i + 1]), 1, bits(kv[i * C:(i + 1) * C]), 1, ri, wo,
                                   heads=cfg.heads, dim=cfg.dim, sm_scale=synth.sm_scale(cfg.dim))
    say("  attention")
    check_attn(out[i:i + 1].float().cpu().numpy(), out_o)
    # every row: selection by its definition over the device scores, attention over a
    # compact cache of its selected rows
    check_hier_by_definition(scores.cpu().numpy(), [C] * nreq, pb.cpu().numpy(), pn.cpu().numpy(),
                             idx.cpu().numpy(), cfg.topk, cfg.max_blocks, cfg.block)
    say("  every row's selection")
    codes, scales, wo = oracle_window(orc, swa_raw.cpu().numpy(), nreq, [S - W] * nreq, W)
    assert np.array_equal(codes, scd.cpu().numpy()) and np.array_equal(scales, ssd.cpu().numpy())
    out_all = check_attn_compact(orc, kv, cd.row_start, idx, q, wo, [S - 1] * nreq, 2, cfg.heads, cfg.dim)
    check_attn(out.float().cpu().numpy(), out_all)
    say("  every row's attention")
