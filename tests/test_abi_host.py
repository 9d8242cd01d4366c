"""Host-side checks of the C ABI (no GPU): libcsa2.so loads, exports every symbol that
include/csa2.h declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_fp4_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libcsa2.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(csa2_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.csa2_version() == 4


def _rows(n=4):
    return B._Rows(n, ctypes.c_void_p(16), ctypes.c_void_p(32), None)


def _cache(nreq=1, m=2):
    return B._Cache(nreq, m, ctypes.c_void_p(64), ctypes.c_void_p(128))


def _err():
    return B.lib().csa2_last_error().decode()


P = ctypes.c_void_p(4096)  # a non-null pointer that is never dereferenced on these paths
M = ctypes.c_void_p(4104)  # the same, not on a 16-byte boundary


def test_index_score_arg_errors():
    L = B.lib()
    keys = B._IndexKeys(B.MXFP4, 128, P, P)
    args = lambda **kw: dict(dict(rows=ctypes.byref(_rows()), cache=ctypes.byref(_cache()), q=P, qdt=B.BF16, qs=None,
                                  heads=64, w=P, ws=64, keys=ctypes.byref(keys), pool=None, scores=P, stride=512), **kw)

    def call(a):
        return L.csa2_index_score(a["rows"], a["cache"], a["q"], a["qdt"], a["qs"], a["heads"], a["w"],
                                  ctypes.c_int64(a["ws"]), a["keys"], a["pool"], a["scores"], ctypes.c_int64(a["stride"]),
                                  None)

    assert call(args(rows=None)) == B.CSA2_E_ARG
    assert call(args(q=None)) == B.CSA2_E_ARG
    assert call(args(stride=0)) == B.CSA2_E_ARG
    assert call(args(heads=8)) == B.CSA2_E_UNSUPPORTED and "heads" in _err()
    assert call(args(qdt=B.F32)) == B.CSA2_E_UNSUPPORTED
    # MXFP4 index q: codes plus the E8M0 plane; a scale plane only with MXFP4 q
    assert call(args(qdt=B.MXFP4)) == B.CSA2_E_ARG and "q_scale" in _err()
    assert call(args(qs=P)) == B.CSA2_E_ARG and "q_scale" in _err()
    assert call(args(qdt=B.MXFP4, qs=P, q=M)) == B.CSA2_E_ARG and "16-byte" in _err()
    assert call(args(qdt=B.MXFP4, qs=P, rows=ctypes.byref(B._Rows(0, None, None, None)))) == B.CSA2_OK
    assert call(args(cache=ctypes.byref(_cache(m=3)))) == B.CSA2_E_UNSUPPORTED
    bad_dim = B._IndexKeys(B.MXFP4, 64, P, P)
    assert call(args(keys=ctypes.byref(bad_dim))) == B.CSA2_E_UNSUPPORTED
    no_scale = B._IndexKeys(B.MXFP4, 128, P, None)
    assert call(args(keys=ctypes.byref(no_scale))) == B.CSA2_E_ARG
    pool = B._Pool(8, 2048, P, P, None)
    assert call(args(pool=ctypes.byref(pool), stride=1000)) == B.CSA2_E_ARG and "score_stride" in _err()
    assert call(args(q=M)) == B.CSA2_E_ARG and "16-byte" in _err()
    odd_keys = B._IndexKeys(B.MXFP4, 128, M, P)
    assert call(args(keys=ctypes.byref(odd_keys))) == B.CSA2_E_ARG and "16-byte" in _err()
    f32 = B._IndexKeys(B.F32, 64, P, None)
    assert call(args(keys=ctypes.byref(f32), qdt=B.F32, heads=6)) == B.CSA2_E_UNSUPPORTED
    assert call(args(keys=ctypes.byref(f32), qdt=B.F32, heads=8, qs=P)) == B.CSA2_E_ARG and "q_scale" in _err()
    # zero rows: valid and a no-op
    zero = B._Rows(0, None, None, None)
    assert call(args(rows=ctypes.byref(zero))) == B.CSA2_OK


def test_topk_arg_errors():
    L = B.lib()

    def call(k=512, stride=8192, ws=None, nbytes=0, rows=None, pool=None):
        return L.csa2_topk(ctypes.byref(rows or _rows()), ctypes.byref(_cache()), P, ctypes.c_int64(stride), pool,
                           ctypes.c_int32(k), P, ws, ctypes.c_size_t(nbytes), None)

    assert call(k=0) == B.CSA2_E_ARG
    assert call(k=2049) == B.CSA2_E_ARG
    # a 262144-column row needs merge workspace (workspace_size is the pool-source bound)
    need = B.workspace_size(B.OP_TOPK, 4, 262144, 512)
    assert need > 0
    assert call(stride=262144) == B.CSA2_E_WORKSPACE
    assert call(stride=262144, ws=P, nbytes=64) == B.CSA2_E_WORKSPACE
    assert B.workspace_size(B.OP_TOPK, 4, 8192, 512) == 0


def test_topk_hier_arg_errors():
    L = B.lib()

    def call(k=512, block=8, maxb=2048):
        return L.csa2_topk_hier(ctypes.byref(_rows()), ctypes.byref(_cache()), P, ctypes.c_int64(1024),
                                ctypes.c_int32(k), ctypes.c_int32(block), ctypes.c_int32(maxb), P, P, P, None,
                                ctypes.c_size_t(0), None)

    assert call(block=16) == B.CSA2_E_UNSUPPORTED
    assert call(maxb=0) == B.CSA2_E_ARG
    assert call(k=0) == B.CSA2_E_ARG


def test_attn_arg_errors():
    L = B.lib()
    swa = B._Swa(B.MXFP8_E4M3, P, P, P, P, 128)

    def call(qdt=B.BF16, kvdt=B.BF16, odt=B.BF16, heads=64, dim=512, k=512, stride=512, sel=P, w=None, scale=0.04,
             q=P, kv=P, out=P, kvs=None):
        s = w or swa
        return L.csa2_sparse_swa_attn(ctypes.byref(_rows()), ctypes.byref(_cache()), q, qdt, ctypes.c_int32(heads),
                                      ctypes.c_int32(dim), kv, kvdt, kvs, sel, ctypes.c_int32(k),
                                      ctypes.c_int64(stride), None,
                                      ctypes.byref(s), ctypes.c_float(scale), None, out, odt, None, None,
                                      ctypes.c_size_t(0), None)

    assert call(dim=256) == B.CSA2_E_UNSUPPORTED
    assert call(heads=40) == B.CSA2_E_UNSUPPORTED
    assert call(kvdt=B.F32) == B.CSA2_E_UNSUPPORTED
    assert call(k=600) == B.CSA2_E_ARG            # k > sel_stride
    assert call(sel=None) == B.CSA2_E_ARG         # k > 0 without indices
    assert call(k=4096, stride=4096) == B.CSA2_E_ARG
    assert call(scale=0.0) == B.CSA2_E_ARG
    noscale = B._Swa(B.MXFP8_E4M3, P, None, P, P, 128)
    assert call(w=noscale) == B.CSA2_E_ARG
    for kw in (dict(q=M), dict(kv=M), dict(out=M), dict(w=B._Swa(B.MXFP8_E4M3, M, P, P, P, 128)),
               dict(w=B._Swa(B.MXFP8_E4M3, P, M, P, P, 128))):
        assert call(**kw) == B.CSA2_E_ARG and "16-byte" in _err(), kw
    f32win = B._Swa(B.F32, P, None, P, P, 128)
    assert call(qdt=B.F32, kvdt=B.F32, odt=B.F32, dim=300, w=f32win) == B.CSA2_E_UNSUPPORTED
    # FP4 main KV: codes with their E4M3 scale plane, bf16 q / out, dim 512 only
    assert call(kvdt=B.FP4_S16) == B.CSA2_E_ARG and "kv_scale" in _err()
    assert call(kvdt=B.BF16, kvs=P) == B.CSA2_E_ARG and "kv_scale" in _err()
    assert call(kvdt=B.FP4_S16, kvs=M) == B.CSA2_E_ARG and "16-byte" in _err()
    assert call(kvdt=B.FP4_S16, kvs=P, dim=256) == B.CSA2_E_UNSUPPORTED
    assert call(kvdt=B.FP4_S16, kvs=P, qdt=B.F32, odt=B.F32, w=f32win, dim=64) == B.CSA2_E_UNSUPPORTED


def test_tail_layout_arg_errors():
    L = B.lib()

    def call(nreq=8, budget=128, cap=1024, flags=0):
        return L.csa2_replay_tail_layout(ctypes.c_int32(nreq), P, P, None, ctypes.c_int32(budget),
                                         ctypes.c_int32(flags), P, P, P, P, P, P, ctypes.c_int32(cap), None)

    assert call(cap=1023) == B.CSA2_E_ARG and "capacity" in _err()
    assert call(budget=0) == B.CSA2_E_ARG
    assert call(nreq=-1) == B.CSA2_E_ARG
    assert call(flags=2) == B.CSA2_E_ARG and "flags" in _err()


def test_encoder_replay_layout_arg_errors():
    L = B.lib()

    def call(nreq=8, budget=128, cap=1024 + 500, n_ext=500, pre=P):
        return L.csa2_encoder_replay_layout(ctypes.c_int32(nreq), pre, P, ctypes.c_int64(n_ext),
                                            ctypes.c_int32(budget), P, P, P, P, P, ctypes.c_int32(cap), None)

    assert call(cap=1024 + 499) == B.CSA2_E_ARG and "capacity" in _err()
    assert call(n_ext=-1) == B.CSA2_E_ARG
    assert call(budget=0) == B.CSA2_E_ARG
    assert call(pre=None) == B.CSA2_E_ARG


def test_quant_arg_errors():
    L = B.lib()
    assert L.csa2_quant_mx(B.BF16, P, B.F32, ctypes.c_int64(4), P, P, None) == B.CSA2_E_UNSUPPORTED
    assert L.csa2_quant_mx(B.MXFP4, P, B.MXFP4, ctypes.c_int64(4), P, P, None) == B.CSA2_E_UNSUPPORTED
    assert L.csa2_quant_mx(B.MXFP4, None, B.F32, ctypes.c_int64(4), P, P, None) == B.CSA2_E_ARG
    assert L.csa2_quant_mx(B.MXFP4, None, B.F32, ctypes.c_int64(0), None, None, None) == B.CSA2_OK
    assert L.csa2_quant_mx(B.MXFP4, M, B.F32, ctypes.c_int64(4), P, P, None) == B.CSA2_E_ARG and "16-byte" in _err()
    assert L.csa2_quant_mx(B.MXFP4, P, B.F32, ctypes.c_int64(4), M, P, None) == B.CSA2_E_ARG
    assert L.csa2_quant_mx(B.FP4_S16, M, B.BF16, ctypes.c_int64(4), P, P, None) == B.CSA2_E_ARG
    assert L.csa2_quant_mx(B.FP4_S16, None, B.BF16, ctypes.c_int64(0), None, None, None) == B.CSA2_OK


def test_topk_hier_block_is_8_only():
    """The header documents block 8 only; every other block size is refused before launch."""
    L = B.lib()
    for block in (1, 2, 4, 16, 64, 0, -8):
        rc = L.csa2_topk_hier(ctypes.byref(_rows()), ctypes.byref(_cache()), P, ctypes.c_int64(1024),
                              ctypes.c_int32(512), ctypes.c_int32(block), ctypes.c_int32(2048), P, P, P, None,
                              ctypes.c_size_t(0), None)
        assert rc == B.CSA2_E_UNSUPPORTED and "block" in _err(), block


def test_f32_index_dim_range():
    """F32 index keys take dim 1..1024 (the header's range); 0 and 1025 are refused."""
    L = B.lib()

    def call(dim):
        keys = B._IndexKeys(B.F32, dim, P, None)
        return L.csa2_index_score(ctypes.byref(_rows()), ctypes.byref(_cache()), P, B.F32, None, 8, P,
                                  ctypes.c_int64(8), ctypes.byref(keys), None, P, ctypes.c_int64(512), None)

    for dim in (0, 1025):
        assert call(dim) == B.CSA2_E_UNSUPPORTED and "dim" in _err()
    for dim in (1, 7, 1024):
        rc = call(dim)
        assert not (rc == B.CSA2_E_UNSUPPORTED and "dim" in _err()), dim


def test_workspace_grows_with_merge_levels():
    """Rows long enough for several merge levels need workspace for each level's lists
    (k = 2048 at 524,288 columns: 32 segments of 16,384, then groups of 8 lists)."""
    a = B.workspace_size(B.OP_TOPK, 3, 262152, 2048)
    b = B.workspace_size(B.OP_TOPK, 3, 524288, 2048)
    assert 0 < a < b
    assert B.workspace_size(B.OP_TOPK_HIER, 2, 600000, 512, 4096) > 0


def test_topk_hier_noalloc_refuses_oversized_scratch():
    """The allocation-free hierarchy holds at most 32 MiB of scratch per device; a size that
    needs more is refused before anything touches the device."""
    L = B.lib()
    need = B.workspace_size(B.OP_TOPK_HIER, 2048, 65536, 512, 2048)
    assert need > (32 << 20)
    rc = L.csa2_topk_hier_noalloc(ctypes.byref(_rows(2048)), ctypes.byref(_cache()), P, ctypes.c_int64(65536),
                                  ctypes.c_int32(512), ctypes.c_int32(8), ctypes.c_int32(2048), P, P, P, None)
    assert rc == B.CSA2_E_WORKSPACE and "scratch" in _err()
    rc = L.csa2_topk_hier_noalloc(ctypes.byref(_rows()), ctypes.byref(_cache()), P, ctypes.c_int64(1024),
                                  ctypes.c_int32(512), ctypes.c_int32(16), ctypes.c_int32(2048), P, P, P, None)
    assert rc == B.CSA2_E_UNSUPPORTED


def test_kv_produce_arg_errors():
    L = B.lib()

    def call(m=2, pend=P, kvdt=B.FP4_S16, kvs=P, comp=P, max_pos=1000, kv=P):
        c = B._Cache(1, m, ctypes.c_void_p(64), ctypes.c_void_p(128))
        return L.csa2_kv_produce(ctypes.byref(_rows()), ctypes.byref(c), comp, pend, P, P, ctypes.c_int64(max_pos),
                                 kvdt, kv, kvs, P, P, None)

    assert call(pend=None) == B.CSA2_E_ARG and "pending" in _err()
    assert call(kvdt=B.MXFP8_E4M3) == B.CSA2_E_UNSUPPORTED
    assert call(kvdt=B.BF16) == B.CSA2_E_ARG and "kv_scale" in _err()
    assert call(kvs=None) == B.CSA2_E_ARG and "kv_scale" in _err()
    assert call(comp=None) == B.CSA2_E_ARG
    assert call(max_pos=0) == B.CSA2_E_ARG
    assert call(comp=M) == B.CSA2_E_ARG and "16-byte" in _err()
    assert call(kv=M) == B.CSA2_E_ARG and "16-byte" in _err()
    assert call(m=3) == B.CSA2_E_UNSUPPORTED


def test_index_topk_pool_arg_errors():
    L = B.lib()
    keys = B._IndexKeys(B.MXFP4, 128, P, P)

    def call(heads=64, block=8, maxb=2048, k=512, ws=P, nbytes=1 << 30, qdt=B.BF16, kk=None, qs=None):
        pool = B._Pool(block, maxb, P, P, None)
        return L.csa2_index_topk_pool(ctypes.byref(_rows()), ctypes.byref(_cache()), P, qdt, qs, ctypes.c_int32(heads),
                                      P, ctypes.c_int64(64), ctypes.byref(kk or keys), ctypes.byref(pool),
                                      ctypes.c_int32(k), P, ws, ctypes.c_size_t(nbytes), None)

    assert call(heads=48) == B.CSA2_E_UNSUPPORTED
    assert call(block=16) == B.CSA2_E_UNSUPPORTED
    assert call(maxb=4096) == B.CSA2_E_UNSUPPORTED
    assert call(k=0) == B.CSA2_E_ARG and call(k=2049) == B.CSA2_E_ARG
    assert call(qdt=B.F32) == B.CSA2_E_UNSUPPORTED
    assert call(qdt=B.MXFP4) == B.CSA2_E_ARG and "q_scale" in _err()
    assert call(qs=P) == B.CSA2_E_ARG and "q_scale" in _err()
    assert call(kk=B._IndexKeys(B.F32, 128, P, None)) == B.CSA2_E_UNSUPPORTED
    assert call(kk=B._IndexKeys(B.MXFP4, 128, P, ctypes.c_void_p(4098))) == B.CSA2_E_ARG and "keys->scale" in _err()
    need = B.workspace_size(B.OP_TOPK_POOL_FUSED, 4, 8 * 2048, 512)
    assert need == 4 * 4 * 512 * 8
    assert B.workspace_size(B.OP_TOPK_POOL_FUSED, 4, 8 * 512, 512) == 0   # one segment: no lists
    assert B.workspace_size(B.OP_TOPK_POOL_FUSED, 128, 8 * 2048, 512) == 0  # whole pools: no lists
    assert B.workspace_size(B.OP_TOPK_POOL_FUSED, 127, 8 * 2048, 512) == 127 * 4 * 512 * 8
    assert call(ws=None) == B.CSA2_E_WORKSPACE
    assert call(nbytes=need - 1) == B.CSA2_E_WORKSPACE


def test_check_inputs_arg_errors():
    L = B.lib()
    W = ctypes.c_void_p(4096)

    def call(rows=None, pool=None, prows=4, sel=None, k=8, stride=8, smap=None, srows=4, word=W):
        return L.csa2_check_inputs(ctypes.byref(rows or _rows()), ctypes.byref(_cache()),
                                   ctypes.byref(pool) if pool is not None else None, ctypes.c_int32(prows), sel,
                                   ctypes.c_int32(k), ctypes.c_int64(stride), smap, ctypes.c_int32(srows), word, None)

    assert call(word=None) == B.CSA2_E_ARG and "error_word" in _err()
    assert call(word=ctypes.c_void_p(4098)) == B.CSA2_E_ARG and "4-byte" in _err()
    assert call(rows=B._Rows(-1, P, P, None)) == B.CSA2_E_ARG
    assert call(pool=B._Pool(8, 64, P, P, None), prows=0) == B.CSA2_E_ARG and "pool_rows" in _err()
    assert call(pool=B._Pool(3, 64, P, P, None)) == B.CSA2_E_ARG and "block" in _err()
    assert call(sel=P, k=-1) == B.CSA2_E_ARG
    assert call(sel=P, k=8, stride=4) == B.CSA2_E_ARG and "sel_stride" in _err()
    assert call(sel=P, smap=P, srows=0) == B.CSA2_E_ARG and "sel_rows" in _err()
    assert call(smap=P) == B.CSA2_E_ARG and "sel_row_map without sel" in _err()
