"""ctypes binding of libcsa2.so: the same entry points as include/csa2.h, taking torch
tensors.  Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, outputs and workspaces are allocated with torch (device
memory plumbing).  Every step of the path runs in the library's HIP kernels; when the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIBRARY names another build of the same library (a sanitized host build, say)
LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(_HERE, "libcsa2.so")

CSA2_OK, CSA2_E_ARG, CSA2_E_UNSUPPORTED, CSA2_E_WORKSPACE, CSA2_E_LAUNCH = 0, 1, 2, 3, 4
F32, BF16, MXFP4, MXFP8_E4M3, FP4_S16 = 0, 1, 2, 3, 4
OP_TOPK, OP_TOPK_HIER, OP_ATTN, OP_TOPK_POOL_FUSED = 1, 2, 3, 4

# Every symbol include/csa2.h declares.
EXPORTS = ["csa2_index_score", "csa2_topk", "csa2_topk_hier", "csa2_topk_hier_noalloc", "csa2_sparse_swa_attn",
           "csa2_replay_tail_layout", "csa2_encoder_replay_layout", "csa2_workspace_size", "csa2_last_error",
           "csa2_version", "csa2_quant_mx", "csa2_kv_produce", "csa2_index_topk_pool", "csa2_check_inputs"]
BAD_REQ, BAD_POS, BAD_WIN_LO, BAD_CACHE, BAD_POOL_MAP, BAD_POOL, BAD_SEL_MAP, BAD_SEL = 1, 2, 4, 8, 16, 32, 64, 128
TAIL_BORROW_PREFIX_WINDOW = 1


class Csa2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("csa2 error %d: %s" % (code, msg))
        self.code = code


class _Rows(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("req_of_row", ctypes.c_void_p), ("pos_of_row", ctypes.c_void_p),
                ("win_lo", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("nreq", ctypes.c_int32), ("ratio_m", ctypes.c_int32), ("n_entries", ctypes.c_void_p),
                ("row_start", ctypes.c_void_p)]


class _IndexKeys(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("dim", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scale", ctypes.c_void_p)]


class _Pool(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("blocks", ctypes.c_void_p),
                ("nblocks", ctypes.c_void_p), ("row_map", ctypes.c_void_p)]


class _Swa(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("data", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("row_start", ctypes.c_void_p), ("pos_start", ctypes.c_void_p), ("window", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcsa2.so is not built (%s); run __graft_entry__.build() or "
                               "python -m compressed_sparse_attention_fp4_amd.build_lib" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_workspace_size.restype = ctypes.c_size_t
        L.csa2_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_contiguous(), "tensors passed to libcsa2 must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int):
    if rc != CSA2_OK:
        raise Csa2Error(rc, lib().csa2_last_error().decode())


# ------------------------------------------------------------------ descriptors
@dataclass
class Rows:
    req_of_row: torch.Tensor           # int32 [n]
    pos_of_row: torch.Tensor           # int32 [n]
    win_lo: Optional[torch.Tensor] = None

    def c(self):
        return _Rows(self.req_of_row.numel(), _ptr(self.req_of_row), _ptr(self.pos_of_row), _ptr(self.win_lo))

    @property
    def n(self):
        return self.req_of_row.numel()


@dataclass
class Cache:
    ratio_m: int
    n_entries: torch.Tensor            # int32 [nreq]
    row_start: torch.Tensor            # int64 [nreq]

    def c(self):
        return _Cache(self.n_entries.numel(), self.ratio_m, _ptr(self.n_entries), _ptr(self.row_start))


@dataclass
class IndexKeys:
    data: torch.Tensor                 # uint8 [rows, dim/2] (MXFP4) or float32 [rows, dim]
    scale: Optional[torch.Tensor]      # uint8 [rows, dim/32] or None
    dim: int

    def c(self):
        dt = MXFP4 if self.scale is not None else F32
        return _IndexKeys(dt, self.dim, _ptr(self.data), _ptr(self.scale))


@dataclass
class Pool:
    blocks: torch.Tensor               # int32 [prows, max_blocks]
    nblocks: torch.Tensor              # int32 [prows]
    block: int = 8
    row_map: Optional[torch.Tensor] = None

    @property
    def max_blocks(self):
        return self.blocks.shape[1]

    def c(self):
        return _Pool(self.block, self.max_blocks, _ptr(self.blocks), _ptr(self.nblocks), _ptr(self.row_map))


@dataclass
class Window:
    data: torch.Tensor                 # [rows, dim]: uint8 codes (MXFP8), bfloat16 or float32
    scale: Optional[torch.Tensor]      # uint8 [rows, dim/32] for MXFP8
    row_start: torch.Tensor            # int64 [nreq]
    pos_start: torch.Tensor            # int32 [nreq]
    window: int = 128

    @property
    def dtype(self):
        if self.scale is not None:
            return MXFP8_E4M3
        return BF16 if self.data.dtype == torch.bfloat16 else F32

    def c(self):
        return _Swa(self.dtype, _ptr(self.data), _ptr(self.scale), _ptr(self.row_start), _ptr(self.pos_start),
                    self.window)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported tensor dtype %s" % t.dtype)


# ---------------------------------------------------------------- entry points
def _index_q(q_idx: torch.Tensor, q_scale: Optional[torch.Tensor]):
    """(dtype code, q_scale pointer): MXFP4 when the E8M0 scale plane comes with the codes."""
    if q_scale is None:
        return _dtype_code(q_idx), None
    if q_idx.dtype != torch.uint8 or q_scale.dtype != torch.uint8:
        raise TypeError("MXFP4 index q: uint8 codes [n, heads, dim / 2] and uint8 scales [n, heads, dim / 32]")
    return MXFP4, _ptr(q_scale)


def index_score(rows: Rows, cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, keys: IndexKeys,
                pool: Optional[Pool] = None, score_stride: Optional[int] = None, scores: Optional[torch.Tensor] = None,
                q_scale: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """csa2_index_score.  q_idx [n, heads, dim] (bf16 / fp32), or with q_scale the MXFP4 q as
    quant_mx writes it (codes [n, heads, dim / 2], scales [n, heads, dim / 32]); w [n, heads]
    or [heads] (shared)."""
    n, heads = q_idx.shape[0], q_idx.shape[1]
    qdt, qsp = _index_q(q_idx, q_scale)
    if scores is None:
        if score_stride is None:
            raise ValueError("score_stride or scores is required")
        scores = torch.empty((n, score_stride), dtype=torch.float32, device=q_idx.device)
    w_stride = 0 if w.dim() == 1 else w.stride(0)
    rc = lib().csa2_index_score(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(q_idx), ctypes.c_int(qdt), qsp,
                                ctypes.c_int32(heads), _ptr(w),
                                ctypes.c_int64(w_stride), ctypes.byref(keys.c()),
                                ctypes.byref(pool.c()) if pool is not None else None, _ptr(scores),
                                ctypes.c_int64(scores.stride(0)), _stream(stream))
    _check(rc)
    return scores


def index_topk_pool(rows: Rows, cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, keys: IndexKeys, pool: Pool,
                    k: int, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    q_scale: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """csa2_index_topk_pool: the pool top-k of csa2_index_score + csa2_topk without the score
    rows; int32 [n, k] ascending positions, -1 padded.  q_idx / q_scale as for index_score."""
    n, heads = q_idx.shape[0], q_idx.shape[1]
    qdt, qsp = _index_q(q_idx, q_scale)
    if out is None:
        out = torch.empty((n, k), dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        workspace = _workspace(workspace_size(OP_TOPK_POOL_FUSED, n, pool.block * pool.max_blocks, k), q_idx.device)
    w_stride = 0 if w.dim() == 1 else w.stride(0)
    rc = lib().csa2_index_topk_pool(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(q_idx), ctypes.c_int(qdt),
                                    qsp, ctypes.c_int32(heads), _ptr(w),
                                    ctypes.c_int64(w_stride), ctypes.byref(keys.c()), ctypes.byref(pool.c()),
                                    ctypes.c_int32(k), _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                    _stream(stream))
    _check(rc)
    return out


def check_inputs(rows: Rows, cache: Cache, pool: Optional[Pool] = None, sel: Optional[torch.Tensor] = None,
                 sel_row_map: Optional[torch.Tensor] = None, word: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """csa2_check_inputs: a device uint32 word (as int32 [1]) of CSA2_BAD_* bits; 0 when
    every checked precondition holds.  sel: int32 [sel_rows, k] index sets."""
    if word is None:
        word = torch.empty(1, dtype=torch.int32, device=rows.req_of_row.device)
    k = sel.shape[1] if sel is not None else 0
    rc = lib().csa2_check_inputs(ctypes.byref(rows.c()), ctypes.byref(cache.c()),
                                 ctypes.byref(pool.c()) if pool is not None else None,
                                 ctypes.c_int32(pool.blocks.shape[0] if pool is not None else 0), _ptr(sel),
                                 ctypes.c_int32(k), ctypes.c_int64(sel.stride(0) if sel is not None else 0),
                                 _ptr(sel_row_map), ctypes.c_int32(sel.shape[0] if sel is not None else 0),
                                 _ptr(word), _stream(stream))
    _check(rc)
    return word


def workspace_size(op: int, n: int, cols: int, k: int, max_blocks: int = 0) -> int:
    return int(lib().csa2_workspace_size(op, n, cols, k, max_blocks))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def topk(rows: Rows, cache: Cache, scores: torch.Tensor, k: int, pool: Optional[Pool] = None,
         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """csa2_topk: int32 [n, k] ascending positions, -1 padded."""
    n = rows.n
    if out is None:
        out = torch.empty((n, k), dtype=torch.int32, device=scores.device)
    cols = pool.block * pool.max_blocks if pool is not None else scores.stride(0)
    if workspace is None:
        workspace = _workspace(workspace_size(OP_TOPK, n, cols, k), scores.device)
    rc = lib().csa2_topk(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(scores),
                         ctypes.c_int64(scores.stride(0)), ctypes.byref(pool.c()) if pool is not None else None,
                         ctypes.c_int32(k), _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                         _stream(stream))
    _check(rc)
    return out


def topk_hier(rows: Rows, cache: Cache, scores: torch.Tensor, k: int, block: int = 8, max_blocks: int = 2048,
              workspace: Optional[torch.Tensor] = None, out=None, stream=None):
    """csa2_topk_hier: (flat top-k [n, k], pool blocks [n, max_blocks], pool nblocks [n]).
    out: optional preallocated (idx, blocks, nblocks)."""
    n = rows.n
    dev = scores.device
    if out is None:
        out = (torch.empty((n, k), dtype=torch.int32, device=dev),
               torch.empty((n, max_blocks), dtype=torch.int32, device=dev),
               torch.empty((n,), dtype=torch.int32, device=dev))
    idx, blocks, nblocks = out
    if workspace is None:
        workspace = _workspace(workspace_size(OP_TOPK_HIER, n, scores.stride(0), k, max_blocks), dev)
    rc = lib().csa2_topk_hier(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(scores),
                              ctypes.c_int64(scores.stride(0)), ctypes.c_int32(k), ctypes.c_int32(block),
                              ctypes.c_int32(max_blocks), _ptr(idx), _ptr(blocks), _ptr(nblocks), _ptr(workspace),
                              ctypes.c_size_t(workspace.numel()), _stream(stream))
    _check(rc)
    return idx, blocks, nblocks


def topk_hier_noalloc(rows: Rows, cache: Cache, scores: torch.Tensor, k: int, block: int = 8,
                      max_blocks: int = 2048, out=None, stream=None):
    """csa2_topk_hier_noalloc: csa2_topk_hier with the library's own per-device scratch (no
    workspace argument).  out: optional preallocated (idx, blocks, nblocks)."""
    n = rows.n
    dev = scores.device
    if out is None:
        out = (torch.empty((n, k), dtype=torch.int32, device=dev),
               torch.empty((n, max_blocks), dtype=torch.int32, device=dev),
               torch.empty((n,), dtype=torch.int32, device=dev))
    idx, blocks, nblocks = out
    rc = lib().csa2_topk_hier_noalloc(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(scores),
                                      ctypes.c_int64(scores.stride(0)), ctypes.c_int32(k), ctypes.c_int32(block),
                                      ctypes.c_int32(max_blocks), _ptr(idx), _ptr(blocks), _ptr(nblocks),
                                      _stream(stream))
    _check(rc)
    return idx, blocks, nblocks


def sparse_swa_attn(rows: Rows, cache: Cache, q: torch.Tensor, kv: torch.Tensor, sel_idx: Optional[torch.Tensor],
                    window: Window, sm_scale: float, sel_row_map: Optional[torch.Tensor] = None,
                    sink: Optional[torch.Tensor] = None, want_lse: bool = False, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, kv_scale: Optional[torch.Tensor] = None, stream=None):
    """csa2_sparse_swa_attn: out [n, heads, dim] (q's dtype), and lse [n, heads] if asked
    (or given: a preallocated lse implies want_lse).  kv is float32 / bfloat16 [rows, dim],
    or with kv_scale the FP4 main KV format: uint8 codes [rows, dim / 2] and E4M3 scales
    uint8 [rows, dim / 16]."""
    n, heads, dim = q.shape
    if out is None:
        out = torch.empty_like(q)
    want_lse = want_lse or lse is not None
    if want_lse and lse is None:
        lse = torch.empty((n, heads), dtype=torch.float32, device=q.device)
    k = 0 if sel_idx is None else sel_idx.shape[1]
    sel_stride = 0 if sel_idx is None else sel_idx.stride(0)
    rc = lib().csa2_sparse_swa_attn(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(q),
                                    ctypes.c_int(_dtype_code(q)), ctypes.c_int32(heads), ctypes.c_int32(dim), _ptr(kv),
                                    ctypes.c_int(FP4_S16 if kv_scale is not None else _dtype_code(kv)),
                                    _ptr(kv_scale), _ptr(sel_idx), ctypes.c_int32(k),
                                    ctypes.c_int64(sel_stride), _ptr(sel_row_map), ctypes.byref(window.c()),
                                    ctypes.c_float(sm_scale), _ptr(sink), _ptr(out), ctypes.c_int(_dtype_code(out)),
                                    _ptr(lse), None, ctypes.c_size_t(0), _stream(stream))
    _check(rc)
    return (out, lse) if want_lse else out


def replay_tail_layout(ext_len: torch.Tensor, seq_len: torch.Tensor, budget: int = 128, out: Optional[dict] = None,
                       is_decode: Optional[torch.Tensor] = None, borrow_prefix_window: bool = False,
                       stream=None) -> dict:
    """csa2_replay_tail_layout; returns device tensors sized for budget * nreq rows (or
    fills `out`, a dict of the same int32 tensors).  is_decode (int32 [nreq]) marks the
    decode requests of a mixed batch."""
    nreq = ext_len.numel()
    dev = ext_len.device
    cap = budget * nreq
    if out is not None:
        t = out
        cap = min(t[name].numel() for name in ("src_row", "abs_pos", "win_lo", "req_of_row"))
    else:
        t = dict(tail_len=torch.empty(nreq, dtype=torch.int32, device=dev),
                 tail_row_start=torch.empty(nreq + 1, dtype=torch.int32, device=dev))
        for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
            t[name] = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    flags = TAIL_BORROW_PREFIX_WINDOW if borrow_prefix_window else 0
    rc = lib().csa2_replay_tail_layout(ctypes.c_int32(nreq), _ptr(ext_len), _ptr(seq_len), _ptr(is_decode),
                                       ctypes.c_int32(budget), ctypes.c_int32(flags), _ptr(t["tail_len"]),
                                       _ptr(t["tail_row_start"]), _ptr(t["src_row"]), _ptr(t["abs_pos"]),
                                       _ptr(t["win_lo"]), _ptr(t["req_of_row"]), ctypes.c_int32(cap),
                                       _stream(stream))
    _check(rc)
    return t


def encoder_replay_layout(prefix_len: torch.Tensor, ext_len: torch.Tensor, n_ext: int, budget: int = 128,
                          out: Optional[dict] = None, stream=None) -> dict:
    """csa2_encoder_replay_layout; device tensors sized for budget * nreq + n_ext rows (or
    fills `out`).  n_ext must equal ext_len.sum()."""
    nreq = ext_len.numel()
    dev = ext_len.device
    cap = budget * nreq + n_ext
    if out is not None:
        t = out
        cap = min(t[name].numel() for name in ("src_row", "abs_pos", "win_lo", "req_of_row"))
    else:
        t = dict(row_start=torch.empty(nreq + 1, dtype=torch.int32, device=dev))
        for name in ("src_row", "abs_pos", "win_lo", "req_of_row"):
            t[name] = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    rc = lib().csa2_encoder_replay_layout(ctypes.c_int32(nreq), _ptr(prefix_len), _ptr(ext_len),
                                          ctypes.c_int64(n_ext), ctypes.c_int32(budget), _ptr(t["row_start"]),
                                          _ptr(t["src_row"]), _ptr(t["abs_pos"]), _ptr(t["win_lo"]),
                                          _ptr(t["req_of_row"]), ctypes.c_int32(cap), _stream(stream))
    _check(rc)
    return t


def quant_mx(fmt: int, x: torch.Tensor, stream=None):
    """csa2_quant_mx over the last axis of x: (codes uint8, scales uint8).  MXFP4 / MXFP8_E4M3
    take 32-element blocks; FP4_S16 (the main KV format) takes 16-element blocks."""
    blk = 16 if fmt == FP4_S16 else 32
    assert x.shape[-1] % blk == 0
    d = x.shape[-1]
    nblocks = x.numel() // blk
    codes = torch.empty(x.shape[:-1] + ((d // 2) if fmt in (MXFP4, FP4_S16) else d,), dtype=torch.uint8,
                        device=x.device)
    scales = torch.empty(x.shape[:-1] + (d // blk,), dtype=torch.uint8, device=x.device)
    rc = lib().csa2_quant_mx(ctypes.c_int(fmt), _ptr(x), ctypes.c_int(_dtype_code(x)), ctypes.c_int64(nblocks),
                             _ptr(codes), _ptr(scales), _stream(stream))
    _check(rc)
    return codes, scales


def kv_produce(rows: Rows, cache: Cache, comp: torch.Tensor, pending: Optional[torch.Tensor], w_index: torch.Tensor,
               rope: torch.Tensor, kv: torch.Tensor, index_codes: torch.Tensor, index_scales: torch.Tensor,
               kv_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """csa2_kv_produce: writes the entries the rows complete into kv (bf16 [rows, 512], or
    FP4 codes uint8 [rows, 256] with kv_scale [rows, 32]) and the MXFP4 index caches; updates
    pending (float32 [nreq, 512], m = 2).  comp float32 [n, 512]; w_index bf16 [128, 512];
    rope float32 [max_pos, 2, 32]."""
    kv_dt = FP4_S16 if kv_scale is not None else BF16
    rc = lib().csa2_kv_produce(ctypes.byref(rows.c()), ctypes.byref(cache.c()), _ptr(comp), _ptr(pending),
                               _ptr(w_index), _ptr(rope), ctypes.c_int64(rope.shape[0]), ctypes.c_int(kv_dt),
                               _ptr(kv), _ptr(kv_scale), _ptr(index_codes), _ptr(index_scales), _stream(stream))
    _check(rc)

