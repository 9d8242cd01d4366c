"""numpy front end of the C oracle (test infrastructure only).

Each wrapper names the section of the pages that its C function follows; the
citations are repeated in ``csa2_oracle.c``.  Every function is pinned by tests in
``tests/test_oracle_*.py``.  The attention sink is a reading (the pages only mention
that a sink exists, [P4] section 6): an extra key of value zero, pinned against torch
SDPA with an appended zero row.  Parity unpinned: V = K including the RoPE dimensions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

E2M1 = 0
E4M3 = 1
# attention data-type codes understood by the C oracle
DT_F32, DT_BF16, DT_MXFP8, DT_FP4S16 = 0, 1, 3, 4


def build(force: bool = False) -> str:
    """Compile csa2_oracle.c with gcc (-O2, no fp contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-D_GNU_SOURCE", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # CSA2_ORACLE_LIBRARY names another build of csa2_oracle.c (a sanitized one, say)
            path = os.environ.get("CSA2_ORACLE_LIBRARY") or build()
            _lib = ctypes.CDLL(path)
            _lib.orc_e2m1_value.restype = ctypes.c_double
            _lib.orc_e4m3_value.restype = ctypes.c_double
            _lib.orc_e8m0_value.restype = ctypes.c_double
            _lib.orc_reach.restype = ctypes.c_int64
            _lib.orc_reach.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64]
            _lib.orc_index_score_mxfp4.restype = ctypes.c_long
            _lib.orc_replay_tail_layout.restype = ctypes.c_int
    return _lib


def _p(a):
    """Pointer to a numpy array's data (None stays NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)  # the pointer object keeps the array alive


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _i64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def set_threads(n: int) -> None:
    """Host threads used by the oracle's OpenMP loops."""
    _load().orc_set_threads(ctypes.c_int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(ctypes.c_int(code))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(ctypes.c_int(code))


def e8m0_value(b: int) -> float:
    return _load().orc_e8m0_value(ctypes.c_int(b))


def mx_quant(fmt: int, x: np.ndarray):
    """OCP MX quantization of the last axis of x (a multiple of 32) ([P1] "Mixed
    precision": index Q/K MXFP4 with 32-element groups; SWA FP8 with block-32 scales).

    Returns (codes, scales): E2M1 codes packed two per byte (element 2i in the low
    nibble), E4M3 one per byte; one E8M0 byte per 32 elements."""
    x = _f32(x)
    assert x.shape[-1] % 32 == 0
    nblocks = x.size // 32
    lead = x.shape[:-1]
    d = x.shape[-1]
    codes = np.empty(lead + ((d // 2) if fmt == E2M1 else d,), dtype=np.uint8)
    scales = np.empty(lead + (d // 32,), dtype=np.uint8)
    _load().orc_mx_quant(ctypes.c_int(fmt), _p(x), ctypes.c_int64(nblocks), _p(codes), _p(scales))
    return codes, scales


def mx_dequant(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Value of every element of an MX tensor, in float64."""
    if fmt == E2M1:
        lo = codes & 15
        hi = codes >> 4
        c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
        table = np.array([e2m1_value(i) for i in range(16)])
    else:
        c = codes
        table = np.array([e4m3_value(i) for i in range(256)])
    v = table[c]
    s = np.array([e8m0_value(i) for i in range(256)])[scales]
    return v * np.repeat(s, 32, axis=-1)


def fp4s16_quant(x: np.ndarray):
    """Main KV storage format ([P1] "Mixed precision", per-entry bytes table): E2M1
    elements, one E4M3 scale per 16 channels, no global scale.  Rounding reading:
    s = RNE_E4M3(amax / 6), element = RNE_E2M1(|x| / s) with x's sign bit.

    Returns (codes packed two per byte, element 2i low nibble; scales, one E4M3 byte
    per 16 elements)."""
    x = _f32(x)
    assert x.shape[-1] % 16 == 0
    d = x.shape[-1]
    codes = np.empty(x.shape[:-1] + (d // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 16,), dtype=np.uint8)
    _load().orc_fp4s16_quant(_p(x), ctypes.c_int64(x.size // 16), _p(codes), _p(scales))
    return codes, scales


def fp4s16_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Value of every element of a main-KV-format tensor, in float64."""
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    v = np.array([e2m1_value(i) for i in range(16)])[c]
    s = np.array([e4m3_value(i) for i in range(256)])[scales]
    return v * np.repeat(s, 16, axis=-1)


# ----------------------------------------------------------------------- reachability
def reach(p: int, m: int, n_entries: int) -> int:
    """Number of compressed entries visible to the query at absolute position p
    ([P1] "CSA2" non-overlapping groups; only complete groups are entries)."""
    return int(_load().orc_reach(p, m, n_entries))


# ----------------------------------------------------------------------------- score
def index_score(rows, cache, q, w, keys, *, heads, dim, key_scales=None, w_row_stride=None,
                pool=None, score_stride):
    """Index scores s_j = sum_h w_h ReLU(q_h . k_j) in the canonical fp32 order.

    rows  = dict(req_of_row, pos_of_row); cache = dict(ratio_m, n_entries, row_start)
    q     = float32 [n, heads, dim] (bf16-representable values for the MXFP4 path)
    keys  = MXFP4 codes [rows, dim/2] with key_scales [rows, dim/32], or float32 [rows, dim]
    pool  = None or dict(blocks [prow, max_blocks], nblocks [prow], block, max_blocks, row_map)
    Returns (scores [n, score_stride] float32 with NaN in unwritten columns, inexact_count)."""
    lib = _load()
    req = _i32(rows["req_of_row"])
    pos = _i32(rows["pos_of_row"])
    n = len(req)
    ne = _i32(cache["n_entries"])
    rs = _i64(cache["row_start"])
    q = _f32(q).reshape(n, heads, dim)
    w = _f32(w)
    if w_row_stride is None:
        w_row_stride = heads if w.size == n * heads else 0
    scores = np.full((n, score_stride), np.nan, dtype=np.float32)
    pb = pn = pm = None
    block = max_blocks = 0
    if pool is not None:
        pb, pn = _i32(pool["blocks"]), _i32(pool["nblocks"])
        pm = _i32(pool.get("row_map"))
        block, max_blocks = int(pool["block"]), int(pool["max_blocks"])
    if key_scales is None:
        kf = _f32(keys)
        lib.orc_index_score_f32(
            ctypes.c_int(n), _p(req), _p(pos), ctypes.c_int(cache["ratio_m"]), _p(ne), _p(rs),
            ctypes.c_int(heads), ctypes.c_int(dim), _p(q), _p(w), ctypes.c_int64(w_row_stride), _p(kf),
            _p(pb), _p(pn), ctypes.c_int(block), ctypes.c_int(max_blocks), _p(pm), _p(scores),
            ctypes.c_int64(score_stride))
        return scores, 0
    kc = np.ascontiguousarray(keys, dtype=np.uint8)
    ks = np.ascontiguousarray(key_scales, dtype=np.uint8)
    bad = lib.orc_index_score_mxfp4(
        ctypes.c_int(n), _p(req), _p(pos), ctypes.c_int(cache["ratio_m"]), _p(ne), _p(rs),
        ctypes.c_int(heads), ctypes.c_int(dim), _p(q), _p(w), ctypes.c_int64(w_row_stride), _p(kc), _p(ks),
        _p(pb), _p(pn), ctypes.c_int(block), ctypes.c_int(max_blocks), _p(pm), _p(scores),
        ctypes.c_int64(score_stride))
    return scores, int(bad)


# ------------------------------------------------------------------------------ top-k
def topk(rows, cache, scores, k, pool=None):
    """Top-k per row by (score desc, position asc); ascending output, -1 padded."""
    lib = _load()
    req = _i32(rows["req_of_row"])
    pos = _i32(rows["pos_of_row"])
    n = len(req)
    scores = _f32(scores)
    out = np.empty((n, k), dtype=np.int32)
    pb = pn = pm = None
    block = max_blocks = 0
    if pool is not None:
        pb, pn = _i32(pool["blocks"]), _i32(pool["nblocks"])
        pm = _i32(pool.get("row_map"))
        block, max_blocks = int(pool["block"]), int(pool["max_blocks"])
    lib.orc_topk(ctypes.c_int(n), _p(req), _p(pos), ctypes.c_int(cache["ratio_m"]), _p(_i32(cache["n_entries"])),
                 _p(scores), ctypes.c_int64(scores.shape[1]), _p(pb), _p(pn), ctypes.c_int(block),
                 ctypes.c_int(max_blocks), _p(pm), ctypes.c_int(k), _p(out))
    return out


def topk_hier(rows, cache, scores, k, block=8, max_blocks=2048):
    """Flat top-k over all reachable positions plus the candidate pool of blocks."""
    lib = _load()
    req = _i32(rows["req_of_row"])
    pos = _i32(rows["pos_of_row"])
    n = len(req)
    scores = _f32(scores)
    out = np.empty((n, k), dtype=np.int32)
    ob = np.empty((n, max_blocks), dtype=np.int32)
    on = np.empty((n,), dtype=np.int32)
    lib.orc_topk_hier(ctypes.c_int(n), _p(req), _p(pos), ctypes.c_int(cache["ratio_m"]),
                      _p(_i32(cache["n_entries"])), _p(scores), ctypes.c_int64(scores.shape[1]), ctypes.c_int(k),
                      ctypes.c_int(block), ctypes.c_int(max_blocks), _p(out), _p(ob), _p(on))
    return out, ob, on


# -------------------------------------------------------------------------- attention
def _attn_operand(x, dt):
    if dt == DT_F32:
        return _f32(x)
    if dt == DT_BF16:
        return np.ascontiguousarray(x, dtype=np.uint16)
    return np.ascontiguousarray(x, dtype=np.uint8)


def sparse_swa_attn(rows, cache, q, q_dt, kv, kv_dt, sel_idx, swa, *, heads, dim, sm_scale,
                    sel_row_map=None, sink=None, dense=False, kv_scale=None):
    """Joint softmax over selected compressed entries and the row's window, in float64.

    q: [n, heads, dim] (f32 values or bf16 bit patterns); kv: [rows, dim] (f32, bf16
    bits) or, with kv_dt = DT_FP4S16, packed codes [rows, dim / 2] with kv_scale
    [rows, dim / 16];
    sel_idx: [*, k] int32 (-1 skipped); swa = dict(data, dtype, scale, row_start,
    pos_start, window).  Returns (out float64 [n, heads, dim], lse float64 [n, heads]).
    dense=True ignores sel_idx and attends to every reachable entry."""
    lib = _load()
    req = _i32(rows["req_of_row"])
    pos = _i32(rows["pos_of_row"])
    lo = _i32(rows.get("win_lo"))
    n = len(req)
    qa = _attn_operand(q, q_dt)
    kva = _attn_operand(kv, kv_dt)
    sw = _attn_operand(swa["data"], swa["dtype"])
    ss = None if swa.get("scale") is None else np.ascontiguousarray(swa["scale"], dtype=np.uint8)
    out = np.empty((n, heads, dim), dtype=np.float64)
    lse = np.empty((n, heads), dtype=np.float64)
    sk = _f32(sink)
    ks = None if kv_scale is None else np.ascontiguousarray(kv_scale, dtype=np.uint8)
    assert (kv_dt == DT_FP4S16) == (ks is not None), "kv_scale goes with the main KV storage format only"
    common = [ctypes.c_int(n), _p(req), _p(pos), _p(lo), ctypes.c_int(cache["ratio_m"]),
              _p(_i32(cache["n_entries"])), _p(_i64(cache["row_start"])), _p(qa), ctypes.c_int(q_dt),
              ctypes.c_int(heads), ctypes.c_int(dim), _p(kva), ctypes.c_int(kv_dt), _p(ks)]
    swa_args = [_p(sw), ctypes.c_int(swa["dtype"]), _p(ss), _p(_i64(swa["row_start"])),
                _p(_i32(swa["pos_start"])), ctypes.c_int(swa["window"]), ctypes.c_double(sm_scale), _p(sk),
                _p(out), _p(lse)]
    if dense:
        lib.orc_dense_attn(*common, *swa_args)
    else:
        sel = _i32(sel_idx)
        srm = _i32(sel_row_map)
        lib.orc_sparse_swa_attn(*common, _p(sel), ctypes.c_int(sel.shape[1]), ctypes.c_int64(sel.shape[1]),
                                _p(srm), *swa_args)
    return out, lse


# ------------------------------------------------------------------------ KV producer
KV_DIM, IDX_DIM, ROPE_DIM = 512, 128, 64


def kv_produce(rows, ratio_m, row_start, n_rows_cache, comp, pending, w_index_bits, rope, kv_dt=DT_FP4S16,
               fill=0xEE):
    """Index-K / main-KV producer ([P1] "CSA2"; [P4] sections 1 and 5; readings in
    csa2_oracle.c).  comp: float32 [n, 512] compressor outputs of the rows; pending:
    float32 [nreq, 512] (copied, the updated copy is returned); w_index_bits: uint16
    [128, 512] bf16 patterns; rope: float32 [max_pos, 2, 32] (cos, sin).  Cache buffers of
    n_rows_cache rows are created filled with `fill` (bf16: the pattern fill * 0x101), so
    rows the call does not produce keep it.  Returns a dict of the caches and the state."""
    lib = _load()
    req = _i32(rows["req_of_row"])
    pos = _i32(rows["pos_of_row"])
    n = len(req)
    comp = _f32(comp)
    assert comp.shape == (n, KV_DIM)
    pend = np.array(pending, dtype=np.float32, copy=True, order="C")
    w = np.ascontiguousarray(w_index_bits, dtype=np.uint16)
    assert w.shape == (IDX_DIM, KV_DIM)
    rope = _f32(rope)
    max_pos = rope.shape[0]
    assert rope.shape[1:] == (2, ROPE_DIM // 2)
    if kv_dt == DT_FP4S16:
        kv = np.full((n_rows_cache, KV_DIM // 2), fill, np.uint8)
        kvs = np.full((n_rows_cache, KV_DIM // 16), fill, np.uint8)
    else:
        kv = np.full((n_rows_cache, KV_DIM), fill * 0x101, np.uint16)
        kvs = None
    ic = np.full((n_rows_cache, IDX_DIM // 2), fill, np.uint8)
    isc = np.full((n_rows_cache, IDX_DIM // 32), fill, np.uint8)
    rc = lib.orc_kv_produce(ctypes.c_int(n), _p(req), _p(pos), ctypes.c_int(ratio_m), _p(_i64(row_start)), _p(comp),
                            _p(pend), _p(w), _p(rope), ctypes.c_int64(max_pos), ctypes.c_int(kv_dt), _p(kv), _p(kvs),
                            _p(ic), _p(isc))
    if rc != 0:
        raise ValueError("kv producer argument not supported (rc=%d)" % rc)
    return dict(kv=kv, kv_scale=kvs, index_codes=ic, index_scales=isc, pending=pend)


# ------------------------------------------------------------------------- tail layout
def replay_tail_layout(ext_len, seq_len, budget=128, capacity=None, is_decode=None, borrow_prefix_window=False):
    """Decoder bounded-replay tail layout ([P2] sections 2.1, 2.3); decode requests of a
    mixed batch keep all their rows uncut ([P1] "Decoder Bounded Replay"); the optional
    short-extend reading of [P2] section 2.6 lowers the window bound to S - budget."""
    lib = _load()
    e = _i32(ext_len)
    s = _i32(seq_len)
    nreq = len(e)
    dec = None if is_decode is None else _i32(is_decode)
    if capacity is None:
        capacity = budget * nreq
    tail_len = np.empty(nreq, np.int32)
    start = np.empty(nreq + 1, np.int32)
    bufs = [np.full(max(capacity, 1), -1, np.int32) for _ in range(4)]
    rc = lib.orc_replay_tail_layout(ctypes.c_int(nreq), _p(e), _p(s), _p(dec), ctypes.c_int(budget),
                                    ctypes.c_int(1 if borrow_prefix_window else 0), _p(tail_len), _p(start),
                                    *[_p(b) for b in bufs], ctypes.c_int(capacity))
    if rc != 0:
        raise ValueError("tail layout precondition violated (rc=%d)" % rc)
    tot = int(start[nreq])
    src_row, abs_pos, win_lo, req_of_row = (b[:tot] for b in bufs)
    return dict(tail_len=tail_len, tail_row_start=start, src_row=src_row, abs_pos=abs_pos, win_lo=win_lo,
                req_of_row=req_of_row)


def encoder_replay_layout(prefix_len, ext_len, budget=128, capacity=None):
    """Encoder-side bounded replay ([P4] sections 4.1, 4.3): per request the last
    min(P, budget) cached prefix positions are recomputed before the extend; every row's
    window stops at R0 = max(0, P - budget); src_row is -1 for replayed prefix rows."""
    lib = _load()
    p = _i32(prefix_len)
    e = _i32(ext_len)
    nreq = len(e)
    if capacity is None:
        capacity = budget * nreq + int(e.sum())
    start = np.empty(nreq + 1, np.int32)
    bufs = [np.full(max(capacity, 1), -7, np.int32) for _ in range(4)]
    rc = lib.orc_encoder_replay_layout(ctypes.c_int(nreq), _p(p), _p(e), ctypes.c_int(budget), _p(start),
                                       *[_p(b) for b in bufs], ctypes.c_int(capacity))
    if rc != 0:
        raise ValueError("encoder replay layout precondition violated (rc=%d)" % rc)
    tot = int(start[nreq])
    src_row, abs_pos, win_lo, req_of_row = (b[:tot] for b in bufs)
    return dict(row_start=start, src_row=src_row, abs_pos=abs_pos, win_lo=win_lo, req_of_row=req_of_row)
