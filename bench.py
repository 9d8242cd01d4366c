#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

Workload (default): hierarchical-indexer decode -- 64 requests x 1 query token at
context S = 131072 with m = 2 (65536 compressed entries each).  One step is a decode
step through 8 CSA2 layers sharing one KV owner:
  layer 0 (source, Full):  index scores over all 65536 entries (MXFP4 keys, 64 index
                           heads x 128) -> flat top-512 + candidate pool of 2048 blocks
                           of 8 -> sparse + window attention (64 bf16 heads x 512,
                           FP8 window of 128)
  layers 1..7 (Reindex):   own index q / weights, scores over the 16384-position pool
                           -> top-512 inside the pool (one fused scoring + selection,
                           no score row written) -> attention with own q and window.
Metric: sparse-attention queries per second = query rows x layers completed per second
(64 x 8 = 512 per step).  Inputs are seeded N(0,1) (weights U(0,1)) drawn on the GPU;
4 independent input sets rotate across steps so that no step finds the previous
step's data in the 256 MiB last-level cache.

Also reported: the dominant kernel's roofline (algorithmic bytes / average launch time,
HIP events on the launch stream), the two-launch Reindex path (pool scores written, then
selected) beside the fused one, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from compressed_sparse_attention_fp4_amd import binding as B  # noqa: E402
from compressed_sparse_attention_fp4_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0  # dense FP4 MFMA, MI355X
FP32_VALU_TFLOPS = 157.3   # fp32 vector, MI355X
NREQ, SEQ, M = 64, 131072, 2
C = SEQ // M
HI, DI = 64, 128
H, D = 64, 512
K, BLK, NB, W = 512, 8, 2048, 128
LAYERS = 8
NSETS = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------ inputs
class InputSet:
    def __init__(self, s: int, dev):
        seed = 3 * 1000 + s
        g = synth.Geometry([SEQ] * NREQ, M)
        self.rows = B.Rows(torch.arange(NREQ, dtype=torch.int32, device=dev),
                           torch.full((NREQ,), SEQ - 1, dtype=torch.int32, device=dev))
        self.cache = B.Cache(M, torch.tensor(g.n_entries, dtype=torch.int32, device=dev),
                             torch.tensor(g.row_start, dtype=torch.int64, device=dev))
        # index keys: N(0,1) -> MXFP4 by the library quantizer, chunk by chunk
        self.kcodes = torch.empty((g.total_entries, DI // 2), dtype=torch.uint8, device=dev)
        self.kscale = torch.empty((g.total_entries, DI // 32), dtype=torch.uint8, device=dev)
        step = 1 << 20
        for c0 in range(0, g.total_entries, step):
            raw = synth.normal((min(step, g.total_entries - c0), DI), seed, "index_keys/%d" % c0, device=dev)
            cd, sd = B.quant_mx(B.MXFP4, raw)
            self.kcodes[c0:c0 + raw.shape[0]] = cd
            self.kscale[c0:c0 + raw.shape[0]] = sd
            del raw
        self.keys = B.IndexKeys(self.kcodes, self.kscale, DI)
        self.kv = synth.normal_bf16((g.total_entries, D), seed, "kv", device=dev, chunk_rows=1 << 19)
        # the same main KV in the pages' FP4 storage format (E2M1 + one E4M3 scale per 16)
        self.kv4, self.kv4s = B.quant_mx(B.FP4_S16, self.kv)
        win = synth.window_cache_geometry(g, W)
        self.layers = []
        for l in range(LAYERS):
            qi = synth.normal_bf16((NREQ, HI, DI), seed, "index_q/%d" % l, device=dev)
            w = synth.uniform((NREQ, HI), seed, "index_w/%d" % l, device=dev)
            q = synth.normal_bf16((NREQ, H, D), seed, "q/%d" % l, device=dev)
            sraw = synth.normal((win["rows"], D), seed, "swa/%d" % l, device=dev)
            scd, ssd = B.quant_mx(B.MXFP8_E4M3, sraw)
            del sraw
            window = B.Window(scd, ssd, win["row_start"].to(dev), win["pos_start"].to(dev), W)
            self.layers.append(dict(qi=qi, w=w, q=q, window=window))
        # outputs and workspaces (allocated once)
        self.scores_full = torch.empty((NREQ, C), dtype=torch.float32, device=dev)
        self.scores_pool = torch.empty((NREQ, NB * BLK), dtype=torch.float32, device=dev)
        self.idx = [torch.empty((NREQ, K), dtype=torch.int32, device=dev) for _ in range(LAYERS)]
        self.pool_blocks = torch.empty((NREQ, NB), dtype=torch.int32, device=dev)
        self.pool_n = torch.empty((NREQ,), dtype=torch.int32, device=dev)
        self.out = [torch.empty((NREQ, H, D), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
        self.ws_hier = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, NREQ, C, K, NB)), dtype=torch.uint8,
                                   device=dev)
        self.ws_fused = torch.empty(max(1, B.workspace_size(B.OP_TOPK_POOL_FUSED, NREQ, NB * BLK, K)),
                                    dtype=torch.uint8, device=dev)
        self.ws_topk = torch.empty(max(1, B.workspace_size(B.OP_TOPK, NREQ, NB * BLK, K)), dtype=torch.uint8,
                                   device=dev)
        self.pool = B.Pool(self.pool_blocks, self.pool_n, BLK)


# ----------------------------------------------------------------- one decode step
STAGES = ["score_full", "topk_hier", "attn", "reindex"]
# the two-launch Reindex path (pool score rows written, then selected): same index sets
TWO_LAUNCH = ["score_pool", "topk_pool"]
ONE_KERNEL_STAGES = ["score_full", "attn"]


def step(x: InputSet, only: str | None = None):
    """One pass of the hot path over one input set; with `only`, just that stage's calls
    (their inputs are the previous full pass's outputs, so a repeat recomputes the same).
    The Reindex layers select through the fused pool scoring + top-k; `only` set to a
    TWO_LAUNCH stage runs that launch of the two-launch path instead."""
    def run(stage, fn):
        if only == stage or (only is None and stage not in TWO_LAUNCH):
            fn()

    sm = synth.sm_scale(D)
    L0 = x.layers[0]
    run("score_full", lambda: B.index_score(x.rows, x.cache, L0["qi"], L0["w"], x.keys, scores=x.scores_full))
    run("topk_hier", lambda: B.topk_hier(x.rows, x.cache, x.scores_full, K, BLK, NB, workspace=x.ws_hier,
                                         out=(x.idx[0], x.pool_blocks, x.pool_n)))
    run("attn", lambda: B.sparse_swa_attn(x.rows, x.cache, L0["q"], x.kv, x.idx[0], L0["window"], sm,
                                          out=x.out[0]))
    for l in range(1, LAYERS):
        Ll = x.layers[l]
        run("score_pool", lambda: B.index_score(x.rows, x.cache, Ll["qi"], Ll["w"], x.keys, pool=x.pool,
                                                scores=x.scores_pool))
        run("topk_pool", lambda: B.topk(x.rows, x.cache, x.scores_pool, K, pool=x.pool, out=x.idx[l],
                                        workspace=x.ws_topk))
        run("reindex", lambda: B.index_topk_pool(x.rows, x.cache, Ll["qi"], Ll["w"], x.keys, x.pool, K,
                                                 out=x.idx[l], workspace=x.ws_fused))
        run("attn", lambda: B.sparse_swa_attn(x.rows, x.cache, Ll["q"], x.kv, x.idx[l], Ll["window"], sm,
                                              out=x.out[l]))


STAGE_LAUNCHES = {"score_full": 1, "topk_hier": 1, "attn": LAYERS, "reindex": LAYERS - 1, "score_pool": LAYERS - 1,
                  "topk_pool": LAYERS - 1}


def attn_fp4kv(x: InputSet):
    """The step's 8 attention launches with the main KV in the FP4 storage format (same
    index sets, q and windows as the bf16 step)."""
    sm = synth.sm_scale(D)
    for l in range(LAYERS):
        Ll = x.layers[l]
        B.sparse_swa_attn(x.rows, x.cache, Ll["q"], x.kv4, x.idx[l], Ll["window"], sm, out=x.out[l],
                          kv_scale=x.kv4s)


def launch_ms_of(fn, sets, reps: int, per: int) -> float:
    """Average launch duration of fn's calls over every input set, as in stage_launch_ms."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x in sets:
            fn(x)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * len(sets) * per)


def stage_launch_ms(sets, reps: int) -> dict:
    """Average duration of one launch of each stage: the stage's calls for every input set
    captured in one HIP graph, replayed back to back between two HIP events on the stream
    the kernels run on (the GPU never waits for the host inside the timed replays)."""
    res = {}
    for s in STAGES + TWO_LAUNCH:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x in sets:
                step(x, only=s)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        res[s] = a.elapsed_time(b) / (reps * len(sets) * STAGE_LAUNCHES[s])
    return res


# Algorithmic bytes per launch (what the step must move at least once).
ATTN_BYTES_PER_QUERY = K * D * 2 + W * (D + D // 32) + H * D * 2 * 2 + K * 4     # 724,992
ATTN_FP4KV_BYTES_PER_QUERY = K * (D // 2 + D // 16) + W * (D + D // 32) + H * D * 2 * 2 + K * 4  # 348,160
STAGE_BYTES = {
    "score_full": NREQ * C * (DI // 2 + DI // 32) + NREQ * HI * DI * 2 + NREQ * HI * 4 + NREQ * C * 4,
    "topk_hier": 2 * NREQ * C * 4 + NREQ * (K + NB + 1) * 4,
    "attn": NREQ * ATTN_BYTES_PER_QUERY,
    "score_pool": NREQ * NB * BLK * (DI // 2 + DI // 32) + NREQ * (NB + 1) * 4 + NREQ * HI * DI * 2
    + NREQ * HI * 4 + NREQ * NB * BLK * 4,
    "topk_pool": NREQ * NB * BLK * 4 + NREQ * (NB + 1) * 4 + NREQ * K * 4,
    "reindex": NREQ * NB * BLK * (DI // 2 + DI // 32) + NREQ * (NB + 1) * 4 + NREQ * HI * DI * 2 + NREQ * HI * 4
    + NREQ * K * 4,
}
# Kernel (as rocprofv3 names it, with its workgroup count) and source file behind each
# stage, for the measured HBM traffic recorded under profiles/.
STAGE_PROFILE = {"attn": ("csa2::k_attn_bf16<false>", 256, "compressed_sparse_attention_fp4_amd/csrc/k_attn.hip"),
                 "attn_fp4kv": ("csa2::k_attn_bf16<true>", 256, "compressed_sparse_attention_fp4_amd/csrc/k_attn.hip")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c3_decode_hbm_traffic.txt")


def measured_traffic(stage: str):
    """HBM bytes per launch of the stage's kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is none or the
    kernel's source has changed since the counters were taken."""
    if stage not in STAGE_PROFILE or not os.path.exists(TRAFFIC_FILE):
        return None
    name, wgs, src = STAGE_PROFILE[stage]
    digest = hashlib.sha1(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) == 5 and not line.startswith("#") and f[0] == name and int(f[1]) == wgs:
            return float(f[3]) if f[4] == digest else None
    return None


# The 7 Reindex launches of a step rescore the same 71 MB of pool keys, which fit the 256
# MiB last-level cache; the counters (FETCH_SIZE) show what leaves L2, not whether the
# last-level cache or HBM answers, so these rates are not quoted as HBM bandwidth.
STAGE_NOTES = {"reindex": {"served_from": "HBM or last-level cache (pool keys reread by 7 launches)"},
               "score_pool": {"served_from": "HBM or last-level cache (pool keys reread by 7 launches)"},
               "topk_pool": {"served_from": "L2 / last-level cache (scores written by the previous launch)"}}

STAGE_KERNEL = {"score_full": "k_score_mxfp4", "topk_hier": "k_block_max + k_select (2 launches)",
                "attn": "k_attn_bf16", "reindex": "k_score_topk_pool + k_merge_segment_lists",
                "score_pool": "k_score_mxfp4 (pool)", "topk_pool": "k_select"}


# ------------------------------------------------------------------ cpu baseline
def _host():
    """What the host offers: CPUs this process may run on, all CPUs, and the CPU model."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), os.cpu_count(), model


def cpu_baseline(x: InputSet, nrows: int):
    """The oracle on a bounded sample: nrows requests through the source layer and one
    Reindex layer, timed per layer; the rate is scaled to the step's mix (1 source +
    7 Reindex layers per query row).  Then the same for one row on one thread (the
    per-core rate)."""
    import oracle as orc
    threads = orc.max_threads()
    nrows = max(1, min(nrows, NREQ))
    rows = dict(req_of_row=np.arange(nrows), pos_of_row=np.full(nrows, SEQ - 1))
    cache = dict(ratio_m=M, n_entries=np.full(nrows, C), row_start=np.arange(nrows, dtype=np.int64) * C)
    # the same inputs (first nrows requests), copied to the host; the oracle quantizes the keys itself
    seed = 3 * 1000 + 0
    keys_raw = []
    step_rows = 1 << 20
    for c0 in range(0, nrows * C, step_rows):
        keys_raw.append(synth.normal((min(step_rows, NREQ * C - c0), DI), seed, "index_keys/%d" % c0,
                                     device="cuda")[: max(0, nrows * C - c0)].cpu())
    keys_raw = torch.cat(keys_raw)[: nrows * C].numpy()
    kc, ks = orc.mx_quant(orc.E2M1, keys_raw)
    del keys_raw
    kv = x.kv[: nrows * C].view(torch.int16).cpu().numpy().view(np.uint16)
    lay = []
    for l in (0, 1):
        L = x.layers[l]
        wn = L["window"]
        lay.append(dict(qi=L["qi"][:nrows].float().cpu().numpy(), w=L["w"][:nrows].cpu().numpy(),
                        q=L["q"][:nrows].view(torch.int16).cpu().numpy().view(np.uint16),
                        swa=dict(data=wn.data[: nrows * W].cpu().numpy(), dtype=3,
                                 scale=wn.scale[: nrows * W].cpu().numpy(),
                                 row_start=wn.row_start[:nrows].cpu().numpy(),
                                 pos_start=wn.pos_start[:nrows].cpu().numpy(), window=W)))
    sm = synth.sm_scale(D)

    def layers(nr):
        """Seconds of the source layer and of one Reindex layer for the first nr rows."""
        rw = {k: v[:nr] for k, v in rows.items()}
        ly = [{k: (v[:nr] if k in ("qi", "w", "q") else v) for k, v in L.items()} for L in lay]
        t0 = time.perf_counter()
        s, _ = orc.index_score(rw, cache, ly[0]["qi"], ly[0]["w"], kc, key_scales=ks, heads=HI, dim=DI,
                               score_stride=C)
        idx, pb, pn = orc.topk_hier(rw, cache, s, K, BLK, NB)
        orc.sparse_swa_attn(rw, cache, ly[0]["q"], 1, kv, 1, idx, ly[0]["swa"], heads=H, dim=D, sm_scale=sm)
        t_src = time.perf_counter() - t0
        pool = dict(blocks=pb, nblocks=pn, block=BLK, max_blocks=NB)
        t0 = time.perf_counter()
        s2, _ = orc.index_score(rw, cache, ly[1]["qi"], ly[1]["w"], kc, key_scales=ks, heads=HI, dim=DI,
                                score_stride=NB * BLK, pool=pool)
        idx2 = orc.topk(rw, cache, s2, K, pool=pool)
        orc.sparse_swa_attn(rw, cache, ly[1]["q"], 1, kv, 1, idx2, ly[1]["swa"], heads=H, dim=D, sm_scale=sm)
        return t_src, time.perf_counter() - t0

    t_src, t_re = layers(nrows)
    rate = nrows * LAYERS / (t_src + (LAYERS - 1) * t_re)
    used = min(threads, nrows)  # the oracle parallelizes over query rows
    orc.set_threads(1)
    t1_src, t1_re = layers(1)
    orc.set_threads(threads)
    rate1 = LAYERS / (t1_src + (LAYERS - 1) * t1_re)
    avail, ncpu, model = _host()
    return {"value": rate, "unit": "queries/s", "cores": used, "threads_used": used, "kind": "oracle",
            "host_cpus_available": avail, "host_cpus_total": ncpu, "cpu_model": model,
            "single_thread_value": rate1,
            "sample": "%d of 64 query rows through the source layer (%.1f s) and one Reindex layer (%.1f s) on "
                      "%d host threads; rate = rows x 8 layers / (source + 7 x Reindex); single-thread rate from "
                      "1 row (%.2f s + %.2f s)" % (nrows, t_src, t_re, used, t1_src, t1_re)}


# ---------------------------------------------------------------------- main
def c1_scoring(steps: int, warmup: int, dev) -> dict:
    """FP4 MFMA rate of the index scoring alone on the C1 prefill workload (8 requests x 8192
    rows, m = 1: row p scores the p + 1 entries it reaches, 64 heads x 128 dims, MXFP4 keys).
    Algorithmic work: 2 x 64 x 128 flop per (row, reachable entry)."""
    cfg = synth.config(1)
    g = cfg.geom
    rows = synth.prefill_rows(g)
    n = rows["req_of_row"].numel()
    rd = B.Rows(rows["req_of_row"].to(dev), rows["pos_of_row"].to(dev))
    cd = B.Cache(1, torch.tensor(g.n_entries, dtype=torch.int32, device=dev),
                 torch.tensor(g.row_start, dtype=torch.int64, device=dev))
    kd, ksd = B.quant_mx(B.MXFP4, synth.normal((g.total_entries, cfg.index_dim), cfg.seed, "index_keys", device=dev))
    keys = B.IndexKeys(kd, ksd, cfg.index_dim)
    qi = synth.normal_bf16((n, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q", device=dev)
    w = synth.uniform((n, cfg.index_heads), cfg.seed, "index_w", device=dev)
    scores = torch.empty((n, max(g.seq_len)), dtype=torch.float32, device=dev)
    reach = int(((rows["pos_of_row"].to(torch.int64) + 1) // g.ratio_m).clamp(max=max(g.n_entries)).sum())
    flop = 2.0 * cfg.index_heads * cfg.index_dim * reach
    for _ in range(max(1, warmup)):
        B.index_score(rd, cd, qi, w, keys, scores=scores)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        B.index_score(rd, cd, qi, w, keys, scores=scores)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    tflops = flop / (ms * 1e-3) / 1e12
    return {"measurement": "C1 prefill index scoring, MXFP4 x MXFP4 MFMA", "rows": n, "row_entries": reach,
            "ms_per_launch": ms, "TFLOP/s": tflops, "peak_TFLOP/s": FP4_PEAK_TFLOPS,
            "frac": tflops / FP4_PEAK_TFLOPS}


C4_SEQ, C4_SETS = 524288, 24


def c4_decode(steps: int, warmup: int, dev, nreq: int = 32) -> dict:
    """C4 long-context decode: nreq requests x 1 query at S = 524,288, m = 2 (262,144
    reachable entries per row): full-range index scores, hierarchical top-k (32,768 blocks
    of 8 -> a pool of 2,048), attention over the top-512 and the 128-row window.  One KV
    cache; C4_SETS layers of index q, weights, q and window, so the attention timing
    rotates over C4_SETS different index sets (about 557 MB of gathered rows for 32
    requests, more than the 256 MiB MALL holds).  Each stage's launches for all sets are
    captured in one HIP graph and replayed between two HIP events."""
    seed = 4 * 1000 + nreq
    c = C4_SEQ // M
    g = synth.Geometry([C4_SEQ] * nreq, M)
    rows = B.Rows(torch.arange(nreq, dtype=torch.int32, device=dev),
                  torch.full((nreq,), C4_SEQ - 1, dtype=torch.int32, device=dev))
    cache = B.Cache(M, torch.tensor(g.n_entries, dtype=torch.int32, device=dev),
                    torch.tensor(g.row_start, dtype=torch.int64, device=dev))
    kcodes = torch.empty((g.total_entries, DI // 2), dtype=torch.uint8, device=dev)
    kscale = torch.empty((g.total_entries, DI // 32), dtype=torch.uint8, device=dev)
    for c0 in range(0, g.total_entries, 1 << 20):
        raw = synth.normal((min(1 << 20, g.total_entries - c0), DI), seed, "index_keys/%d" % c0, device=dev)
        kcodes[c0:c0 + raw.shape[0]], kscale[c0:c0 + raw.shape[0]] = B.quant_mx(B.MXFP4, raw)
        del raw
    keys = B.IndexKeys(kcodes, kscale, DI)
    kv = synth.normal_bf16((g.total_entries, D), seed, "kv", device=dev, chunk_rows=1 << 19)
    win = synth.window_cache_geometry(g, W)
    lay = []
    for l in range(C4_SETS):
        sraw = synth.normal((win["rows"], D), seed, "swa/%d" % l, device=dev)
        scd, ssd = B.quant_mx(B.MXFP8_E4M3, sraw)
        del sraw
        lay.append(dict(qi=synth.normal_bf16((nreq, HI, DI), seed, "index_q/%d" % l, device=dev),
                        w=synth.uniform((nreq, HI), seed, "index_w/%d" % l, device=dev),
                        q=synth.normal_bf16((nreq, H, D), seed, "q/%d" % l, device=dev),
                        window=B.Window(scd, ssd, win["row_start"].to(dev), win["pos_start"].to(dev), W),
                        idx=torch.empty((nreq, K), dtype=torch.int32, device=dev),
                        out=torch.empty((nreq, H, D), dtype=torch.bfloat16, device=dev)))
    scores = torch.empty((nreq, c), dtype=torch.float32, device=dev)
    pool_blocks = torch.empty((nreq, NB), dtype=torch.int32, device=dev)
    pool_n = torch.empty((nreq,), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, nreq, c, K, NB)), dtype=torch.uint8, device=dev)
    sm = synth.sm_scale(D)
    calls = {
        "score_full": lambda L: B.index_score(rows, cache, L["qi"], L["w"], keys, scores=scores),
        "topk_hier": lambda L: B.topk_hier(rows, cache, scores, K, BLK, NB, workspace=ws,
                                           out=(L["idx"], pool_blocks, pool_n)),
        "attn": lambda L: B.sparse_swa_attn(rows, cache, L["q"], kv, L["idx"], L["window"], sm, out=L["out"]),
    }
    for L in lay:  # eager pass: every set's index list
        for f in calls.values():
            f(L)
    torch.cuda.synchronize()
    nbytes = {
        "score_full": nreq * c * (DI // 2 + DI // 32) + nreq * HI * DI * 2 + nreq * HI * 4 + nreq * c * 4,
        "topk_hier": 2 * nreq * c * 4 + nreq * (K + NB + 1) * 4,
        "attn": nreq * ATTN_BYTES_PER_QUERY,
    }
    stages = {}
    for name, f in calls.items():
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for L in lay:
                f(L)
        for _ in range(max(1, warmup)):
            gr.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (steps * len(lay))
        stages[name] = {"us_per_launch": round(us, 2), "alg_bytes": nbytes[name],
                        "alg_GBs": round(nbytes[name] / (us * 1e-6) / 1e9, 1)}
    step_us = sum(v["us_per_launch"] for v in stages.values())
    att = stages["attn"]
    return {"measurement": "C4 long-context decode, %d requests x 1 query, S=524288, m=2 (262144 entries), "
                           "top-512 + hierarchical pool of 2048 blocks of 8" % nreq,
            "queries_per_s": nreq / (step_us * 1e-6), "us_per_layer": round(step_us, 2), "stages": stages,
            "attn_roofline": {"bound": "hbm", "achieved": att["alg_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": att["alg_GBs"] / HBM_PEAK_GBS}}


def kv_produce_rates(steps: int, warmup: int, dev) -> dict:
    """The index-K / main-KV producer (csa2_kv_produce, m = 2, FP4 main KV) on two shapes:
    the decode step's 64 new tokens (each closing a pair) and an 8 x 8192-token prefill
    chunk (32,768 entries).  Algorithmic bytes: compressor rows read (2 KiB per token, plus
    the pending row of a decode token) and 356 B of cache written per entry; work: the
    128 x 512 fma projection per entry on fp32 VALU (the bound of the prefill shape)."""
    out = {}
    rope_rows = SEQ + 2
    i = torch.arange(32, device=dev, dtype=torch.float64)
    ang = torch.arange(rope_rows, device=dev, dtype=torch.float64)[:, None] * 10000.0 ** (-2.0 * i / 64)[None, :]
    rope = torch.stack([ang.cos(), ang.sin()], dim=1).to(torch.float32).contiguous()
    del ang
    w_index = (synth.normal_bf16((128, D), 7, "w_index", device=dev) * 0.05).to(torch.bfloat16)
    for name, nreq, ntok in (("decode_64", NREQ, 1), ("prefill_8x8192", 8, 8192)):
        n = nreq * ntok
        pos0 = SEQ - ntok
        req = torch.arange(nreq, dtype=torch.int32, device=dev).repeat_interleave(ntok)
        pos = (torch.arange(ntok, dtype=torch.int32, device=dev) + pos0).repeat(nreq)
        rows = B.Rows(req, pos)
        cache = B.Cache(M, torch.full((nreq,), SEQ // M, dtype=torch.int32, device=dev),
                        torch.arange(nreq, dtype=torch.int64, device=dev) * (SEQ // M))
        comp = synth.normal((n, D), 7, "comp/" + name, device=dev)
        pending = synth.normal((nreq, D), 7, "pending/" + name, device=dev)
        nrows = nreq * (SEQ // M)
        kv = torch.empty((nrows, D // 2), dtype=torch.uint8, device=dev)
        kvs = torch.empty((nrows, D // 16), dtype=torch.uint8, device=dev)
        ic = torch.empty((nrows, DI // 2), dtype=torch.uint8, device=dev)
        isc = torch.empty((nrows, DI // 32), dtype=torch.uint8, device=dev)
        fn = lambda: B.kv_produce(rows, cache, comp, pending, w_index, rope, kv, ic, isc, kv_scale=kvs)  # noqa: E731
        us = _time_graph(fn, steps, warmup, 1)
        entries = n // M if ntok > 1 else nreq
        nbytes = n * D * 4 + (nreq * D * 4 if ntok == 1 else 0) + entries * (D // 2 + D // 16 + DI // 2 + DI // 32)
        flop = 2.0 * entries * DI * D
        out[name] = {"us_per_launch": round(us, 2), "entries": entries, "alg_bytes": nbytes,
                     "alg_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "projection_TFLOP/s": round(flop / (us * 1e-6) / 1e12, 2),
                     "fp32_valu_frac": round(flop / (us * 1e-6) / 1e12 / FP32_VALU_TFLOPS, 4)}
        del comp, kv, kvs, ic, isc
    return out


def _time_graph(fn, steps: int, warmup: int, per: int) -> float:
    """Microseconds per call of fn's launches: captured once in a HIP graph, replayed
    back to back between two HIP events (per = calls inside fn)."""
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    for _ in range(max(1, warmup)):
        gr.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        gr.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (steps * per)


def c2_replay(steps: int, warmup: int, dev) -> dict:
    """C2 decoder bounded replay: 8 requests of S = 8192 (m = 1) with extends
    8192, 8192, 4096, 4096, 2048, 512, 128, 64.  A Full layer scores every extend row
    (27,328 rows) and selects top-512 plus pools; the tail layout keeps each request's last
    min(128, E) rows (960); a Reindex layer rescored over the source pools (through the
    tail -> extend row map) with its own top-512 and attention; a Reuse layer attending to
    the source layer's top-512 through the same map.  Each stage timed by graph replay."""
    cfg = synth.config(2)
    g = cfg.geom
    E = synth.C2_EXTENDS
    ext_req = torch.cat([torch.full((e,), r, dtype=torch.int32) for r, e in enumerate(E)])
    ext_pos = torch.cat([torch.arange(sq - e, sq, dtype=torch.int32) for sq, e in zip(g.seq_len, E)])
    n_ext = ext_req.numel()
    cd = B.Cache(1, torch.tensor(g.n_entries, dtype=torch.int32, device=dev),
                 torch.tensor(g.row_start, dtype=torch.int64, device=dev))
    kd, ksd = B.quant_mx(B.MXFP4, synth.normal((g.total_entries, cfg.index_dim), cfg.seed, "index_keys", device=dev))
    keys = B.IndexKeys(kd, ksd, cfg.index_dim)
    c = g.n_entries[0]
    re_d = B.Rows(ext_req.to(dev), ext_pos.to(dev))
    qi_s = synth.normal_bf16((n_ext, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q/src", device=dev)
    w_s = synth.uniform((n_ext, cfg.index_heads), cfg.seed, "index_w/src", device=dev)
    sc_s = torch.empty((n_ext, c), dtype=torch.float32, device=dev)
    ws_h = torch.empty(max(1, B.workspace_size(B.OP_TOPK_HIER, n_ext, c, cfg.topk, cfg.max_blocks)),
                       dtype=torch.uint8, device=dev)
    idx_s = torch.empty((n_ext, cfg.topk), dtype=torch.int32, device=dev)
    pb = torch.empty((n_ext, cfg.max_blocks), dtype=torch.int32, device=dev)
    pn = torch.empty((n_ext,), dtype=torch.int32, device=dev)
    ext_len = torch.tensor(E, dtype=torch.int32, device=dev)
    seq_len = torch.tensor(g.seq_len, dtype=torch.int32, device=dev)
    t = B.replay_tail_layout(ext_len, seq_len, 128)
    torch.cuda.synchronize()
    nt = int(t["tail_row_start"][-1])
    rt_d = B.Rows(t["req_of_row"][:nt], t["abs_pos"][:nt], t["win_lo"][:nt])
    src_map = t["src_row"][:nt].contiguous()
    pool_d = B.Pool(pb, pn, cfg.block, src_map)
    qi_t = synth.normal_bf16((nt, cfg.index_heads, cfg.index_dim), cfg.seed, "index_q/reindex", device=dev)
    w_t = synth.uniform((nt, cfg.index_heads), cfg.seed, "index_w/reindex", device=dev)
    sc_t = torch.empty((nt, cfg.max_blocks * cfg.block), dtype=torch.float32, device=dev)
    idx_t = torch.empty((nt, cfg.topk), dtype=torch.int32, device=dev)
    ws_t = torch.empty(max(1, B.workspace_size(B.OP_TOPK, nt, cfg.max_blocks * cfg.block, cfg.topk)),
                       dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(1, B.workspace_size(B.OP_TOPK_POOL_FUSED, nt, cfg.max_blocks * cfg.block, cfg.topk)),
                       dtype=torch.uint8, device=dev)
    kv = synth.normal_bf16((g.total_entries, cfg.dim), cfg.seed, "kv", device=dev)
    win = synth.window_cache_geometry(g, 128)
    lay = {}
    for layer in ("reindex", "reuse"):
        scd, ssd = B.quant_mx(B.MXFP8_E4M3, synth.normal((win["rows"], cfg.dim), cfg.seed, "swa/" + layer, device=dev))
        lay[layer] = dict(q=synth.normal_bf16((nt, cfg.heads, cfg.dim), cfg.seed, "q/" + layer, device=dev),
                          window=B.Window(scd, ssd, win["row_start"].to(dev), win["pos_start"].to(dev), 128),
                          out=torch.empty((nt, cfg.heads, cfg.dim), dtype=torch.bfloat16, device=dev))
    sm = synth.sm_scale(cfg.dim)
    calls = {
        "score_src": lambda: B.index_score(re_d, cd, qi_s, w_s, keys, scores=sc_s),
        "topk_hier_src": lambda: B.topk_hier(re_d, cd, sc_s, cfg.topk, cfg.block, cfg.max_blocks, workspace=ws_h,
                                             out=(idx_s, pb, pn)),
        "tail_layout": lambda: B.replay_tail_layout(ext_len, seq_len, 128),
        "reindex": lambda: B.index_topk_pool(rt_d, cd, qi_t, w_t, keys, pool_d, cfg.topk, out=idx_t, workspace=ws_f),
        "attn_reindex": lambda: B.sparse_swa_attn(rt_d, cd, lay["reindex"]["q"], kv, idx_t, lay["reindex"]["window"],
                                                  sm, out=lay["reindex"]["out"]),
        "attn_reuse": lambda: B.sparse_swa_attn(rt_d, cd, lay["reuse"]["q"], kv, idx_s, lay["reuse"]["window"], sm,
                                                sel_row_map=src_map, out=lay["reuse"]["out"]),
    }
    # the same Reindex selection as two launches (scores written, then selected), timed
    # for comparison only
    two = {"score_reindex": lambda: B.index_score(rt_d, cd, qi_t, w_t, keys, pool=pool_d, scores=sc_t),
           "topk_reindex": lambda: B.topk(rt_d, cd, sc_t, cfg.topk, pool=pool_d, out=idx_t, workspace=ws_t)}
    for f in calls.values():  # eager pass in flow order
        f()
    torch.cuda.synchronize()
    reach = int((ext_pos.to(torch.int64) + 1).clamp(max=c).sum())
    nbytes = {
        "score_src": reach * (cfg.index_dim // 2 + cfg.index_dim // 32 + 4) + n_ext * cfg.index_heads * (cfg.index_dim * 2 + 4),
        "topk_hier_src": 2 * reach * 4 + n_ext * (cfg.topk + cfg.max_blocks + 1) * 4,
        "reindex": int(pn[src_map.long()].sum()) * cfg.block * (cfg.index_dim // 2 + cfg.index_dim // 32 + 4)
        + nt * cfg.index_heads * (cfg.index_dim * 2 + 4),
        "attn_reindex": nt * ATTN_BYTES_PER_QUERY,
        "attn_reuse": nt * ATTN_BYTES_PER_QUERY,
    }
    # scoring: the keys of a request are shared by all its rows and stay in cache, so the
    # FP4 MFMA rate (2 x heads x dim flop per scored pair) is the bound, not bytes
    flop = {"score_src": 2.0 * cfg.index_heads * cfg.index_dim * reach,
            "reindex": 2.0 * cfg.index_heads * cfg.index_dim * int(pn[src_map.long()].sum()) * cfg.block}
    nbytes["score_reindex"], flop["score_reindex"] = nbytes["reindex"], flop["reindex"]
    stages = {}
    for name, f in calls.items():
        us = _time_graph(f, steps, warmup, 1)
        st = {"us_per_launch": round(us, 2)}
        if name in nbytes:
            st["alg_bytes"] = nbytes[name]
            st["alg_GBs"] = round(nbytes[name] / (us * 1e-6) / 1e9, 1)
        if name in flop:
            st["TFLOP/s"] = round(flop[name] / (us * 1e-6) / 1e12, 1)
            st["fp4_frac"] = round(flop[name] / (us * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)
        stages[name] = st
    total = sum(v["us_per_launch"] for v in stages.values())
    two_launch = {}
    for name, f in two.items():
        us = _time_graph(f, steps, warmup, 1)
        two_launch[name] = {"us_per_launch": round(us, 2)}
        if name in nbytes:
            two_launch[name]["alg_GBs"] = round(nbytes[name] / (us * 1e-6) / 1e9, 1)
    two_launch["us_total"] = round(sum(v["us_per_launch"] for v in two_launch.values()), 2)
    att = stages["attn_reindex"]
    return {"measurement": "C2 decoder bounded replay: Full layer over 27,328 extend rows, 960 tail rows through "
                           "Reindex and Reuse (8 requests, S=8192, m=1, top-512, pools of 2048 blocks of 8)",
            "us_per_flow": round(total, 2), "stages": stages, "reindex_two_launch": two_launch,
            "attn_roofline": {"bound": "hbm", "achieved": att["alg_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": att["alg_GBs"] / HBM_PEAK_GBS, "note": "nominal 724,992 B per tail row"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c2", action="store_true", help="skip the C2 replay-tail prefill stages")
    ap.add_argument("--cpu-rows", type=int, default=int(os.environ.get("OMP_NUM_THREADS", "0") or 16))
    ap.add_argument("--c1-scoring", action="store_true",
                    help="instead of the decode step: time the C1 prefill index scoring alone (FP4 MFMA rate)")
    ap.add_argument("--c4-decode", type=int, default=0, metavar="NREQ",
                    help="instead of the decode step: time the C4 long-context decode stages for NREQ "
                         "requests (1 or 32)")
    ap.add_argument("--c2-replay", action="store_true",
                    help="instead of the decode step: time the C2 bounded-replay flow stage by stage")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the CSA2 path is built and timed on a single MI355X; "
              "multi-GPU sharding is designed but not run (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()
    if args.c1_scoring:
        print(json.dumps(c1_scoring(args.steps, args.warmup, dev)), flush=True)
        return
    if args.c2_replay:
        print(json.dumps(c2_replay(args.steps, args.warmup, dev)), flush=True)
        return
    if args.c4_decode:
        print(json.dumps(c4_decode(args.steps, args.warmup, dev, args.c4_decode)), flush=True)
        return
    log("building %d input sets ..." % NSETS)
    sets = [InputSet(s, dev) for s in range(NSETS)]
    torch.cuda.synchronize()
    log("warmup %d eager steps" % args.warmup)
    for i in range(max(args.warmup, NSETS)):
        step(sets[i % NSETS])
    torch.cuda.synchronize()

    # one HIP graph per input set: the step is launch-bound in Python otherwise
    graphs = []
    for x in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(x)
        graphs.append(g)
    torch.cuda.synchronize()
    # replays must reproduce the eager results bit for bit, replay after replay
    x = sets[0]
    step(x)
    torch.cuda.synchronize()
    ref = [t.clone() for t in x.idx] + [t.clone() for t in x.out] + [x.pool_blocks.clone(), x.pool_n.clone()]
    for rep in range(2):
        for t in x.idx + x.out + [x.pool_blocks, x.pool_n]:
            t.zero_()
        graphs[0].replay()
        torch.cuda.synchronize()
        got = x.idx + x.out + [x.pool_blocks, x.pool_n]
        assert all(torch.equal(a, b) for a, b in zip(ref, got)), "graph replay differs from the eager step"
        step(x)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % NSETS].replay()

    # timed region: exactly K steps (graph replays), synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % NSETS].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log("timed %d steps in %.3f ms" % (args.steps, elapsed * 1e3))
    # A/A: the same timed region again, for the run-to-run noise band (not the value)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % NSETS].replay()
    torch.cuda.synchronize()
    elapsed_aa = time.perf_counter() - t0

    # per-launch durations of each stage (HIP events around back-to-back graph replays)
    launch_ms = stage_launch_ms(sets, reps=max(3, args.steps // 4))
    per_step_ms = {s: launch_ms[s] * STAGE_LAUNCHES[s] for s in STAGES}
    # the roofline is the dominant kernel's: the one-kernel stage with the most time per
    # step (topk_hier and reindex launch two kernels each, every one of them shorter)
    dominant = max(ONE_KERNEL_STAGES, key=lambda s: per_step_ms[s])
    avg_launch_ms = launch_ms[dominant]
    achieved = STAGE_BYTES[dominant] / (avg_launch_ms * 1e-3) / 1e9
    stages = {s: {"ms_per_launch": launch_ms[s], "launches_per_step": STAGE_LAUNCHES[s],
                  "alg_GBs": STAGE_BYTES[s] / (launch_ms[s] * 1e-3) / 1e9} for s in STAGES}
    log(json.dumps(stages, indent=1))
    log("graph step %.3f ms; sum of stage launches %.3f ms" % (elapsed * 1e3 / args.steps, sum(per_step_ms.values())))

    # the FP4 main KV variant of the attention launches (the pages' storage format)
    fp4_ms = launch_ms_of(attn_fp4kv, sets, max(3, args.steps // 4), LAYERS)
    fp4_bytes = NREQ * ATTN_FP4KV_BYTES_PER_QUERY
    fp4_gbs = fp4_bytes / (fp4_ms * 1e-3) / 1e9
    fp4 = {"kernel": "k_attn_bf16<FP4 main KV>", "us_per_launch": round(fp4_ms * 1e3, 2),
           "alg_bytes_per_launch": fp4_bytes, "achieved": round(fp4_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": fp4_gbs / HBM_PEAK_GBS, "traffic": measured_traffic("attn_fp4kv"),
           "step_ms_with_fp4_kv": (sum(per_step_ms.values()) - per_step_ms["attn"] + LAYERS * fp4_ms)}
    log("FP4 main KV attention: %.2f us per launch (%.1f GB/s algorithmic)" % (fp4_ms * 1e3, fp4_gbs))
    two = {s: dict({"us_per_launch": round(launch_ms[s] * 1e3, 2), "kernel": STAGE_KERNEL[s],
                    "alg_GBs": round(STAGE_BYTES[s] / (launch_ms[s] * 1e-3) / 1e9, 1)}, **STAGE_NOTES.get(s, {}))
           for s in TWO_LAUNCH}
    two_launch = dict(two, us_per_layer=round((launch_ms["score_pool"] + launch_ms["topk_pool"]) * 1e3, 2),
                      fused_us_per_layer=round(launch_ms["reindex"] * 1e3, 2),
                      step_ms_with_two_launch_reindex=sum(per_step_ms.values()) + (LAYERS - 1) * (
                          launch_ms["score_pool"] + launch_ms["topk_pool"] - launch_ms["reindex"]))
    log("two-launch Reindex: %.2f us per layer (fused %.2f)" % (two_launch["us_per_layer"],
                                                                 two_launch["fused_us_per_layer"]))

    # spread of single steps: each replay alone between two HIP events (outside the timed
    # region above, which is the reported value)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        graphs[i % NSETS].replay()
        b.record()
    torch.cuda.synchronize()
    single = np.array([a.elapsed_time(b) for a, b in ev])
    spread = {"p10": round(float(np.percentile(single, 10)), 4), "p50": round(float(np.percentile(single, 50)), 4),
              "p90": round(float(np.percentile(single, 90)), 4)}

    queries = NREQ * LAYERS * args.steps
    value = queries / elapsed
    # one plain copy of known size, for scaling rocprof FETCH/WRITE counters
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()

    log("kv producer ...")
    producer = kv_produce_rates(max(5, args.steps // 2), args.warmup, dev)

    c2 = None
    if not args.no_c2:
        log("C2 replay-tail prefill flow ...")
        c2 = c2_replay(max(5, args.steps // 2), args.warmup, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on %d rows ..." % args.cpu_rows)
        cpu = cpu_baseline(sets[0], args.cpu_rows)

    line = {
        "metric": "CSA2 sparse-attn queries/s (decode, hierarchical indexer)",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "step_ms_spread": spread,
        "aa_repeat": {"value": NREQ * LAYERS * args.steps / elapsed_aa, "ms_per_step": elapsed_aa * 1e3 / args.steps,
                      "rel_diff": (elapsed_aa - elapsed) / elapsed},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+bf16",
        "data": "synthetic (seeded N(0,1) q/keys/KV/window, U(0,1) index weights)",
        "config": {"workload": "C3 hierarchical-indexer decode: 64 requests x 1 query, S=131072, m=2 "
                               "(65536 entries), 1 source + 7 Reindex layers per step",
                   "requests": NREQ, "context": SEQ, "ratio_m": M, "index_heads": HI, "index_dim": DI,
                   "topk": K, "pool_blocks": NB, "block": BLK, "heads": H, "dim": D, "window": W,
                   "layers_per_step": LAYERS, "queries_per_step": NREQ * LAYERS, "input_sets": NSETS},
        "roofline": {"bound": "hbm", "kernel": STAGE_KERNEL[dominant], "stage": dominant,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dominant), "alg_bytes_per_launch": STAGE_BYTES[dominant],
                     "avg_launch_us": avg_launch_ms * 1e3},
        "stages": {s: dict({"us_per_launch": round(v["ms_per_launch"] * 1e3, 2),
                            "launches_per_step": v["launches_per_step"], "alg_GBs": round(v["alg_GBs"], 1)},
                           **STAGE_NOTES.get(s, {}))
                   for s, v in stages.items()},
        "c2_replay_tail_prefill": c2,
        "fp4_main_kv_attn": fp4,
        "reindex_two_launch": two_launch,
        "kv_produce": producer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
