"""The built device code never touches a register whose vector memory load is in flight,
and never accesses LDS while an earlier group of LDS-DMA copies may still be landing.

The attention kernel copies its KV tiles into LDS with inline-assembly
global_load_lds_dwordx4 and waits for them with hand-placed s_waitcnt vmcnt(N); this
compiles every HIP source of the library to gfx950 assembly with the library's own flags
and replays the vector-memory counter over each kernel's control flow
(tests/asm_waitcheck.py).  The checker itself is pinned on small hand-written listings
first: a use before the wait, a use after it, a wait that leaves the needed load in
flight, a loop whose back edge carries a load, and double-buffered copy groups whose wait
is right or one group short.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

import asm_waitcheck as W

from compressed_sparse_attention_fp4_amd import build_lib

HIP_SOURCES = [s for s in build_lib.SOURCES if s.endswith(".hip")]


def _kernel(body: str) -> str:
    return "\t.type\tk,@function\nk:\n" + body + "\n.Lfunc_end0:\n"


def test_checker_flags_use_before_wait():
    asm = _kernel("""
\tglobal_load_dwordx4 v[6:9], v[60:61], off
\tv_xor_b32_e32 v1, v6, v7
\ts_waitcnt vmcnt(0)
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "v6" in hits[0] and "v7" in hits[0]


def test_checker_accepts_use_after_wait():
    asm = _kernel("""
\tglobal_load_dwordx4 v[6:9], v[60:61], off
\tglobal_load_dword v10, v[60:61], off offset:16
\ts_waitcnt vmcnt(1)
\tv_xor_b32_e32 v1, v6, v9
\ts_waitcnt vmcnt(0)
\tv_mov_b32_e32 v2, v10
\ts_endpgm""")
    assert W.check_asm(asm) == {"k": []}


def test_checker_counts_stores_and_in_order_completion():
    # vmcnt(1) after load A, store, load B leaves only B in flight; vmcnt(2) would
    # leave A's successor store and B, so A is complete but reading B is not allowed
    asm = _kernel("""
\tglobal_load_dword v1, v[60:61], off
\tglobal_store_dword v[62:63], v5, off
\tglobal_load_dword v2, v[60:61], off offset:4
\ts_waitcnt vmcnt(2)
\tv_mov_b32_e32 v3, v1
\tv_mov_b32_e32 v4, v2
\ts_waitcnt vmcnt(0)
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "v4, v2" in hits[0]


def test_checker_follows_loop_back_edge():
    # the load at the loop's end is still in flight at the loop's head, so the next
    # iteration's add reads it early (its reload of the same register is allowed: loads
    # complete in order)
    asm = _kernel("""
\tglobal_load_dword v1, v[60:61], off
\ts_waitcnt vmcnt(0)
.LBB0_1:
\tv_add_u32_e32 v3, v1, v3
\tglobal_load_dword v1, v[60:61], off
\ts_cbranch_scc1 .LBB0_1
\ts_waitcnt vmcnt(0)
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "v_add_u32" in hits[0]


def test_checker_flags_load_address_in_flight():
    # a load whose address register is still being loaded (a pointer chase without a wait)
    asm = _kernel("""
\tglobal_load_dwordx2 v[2:3], v[60:61], off
\tglobal_load_dword v4, v[2:3], off
\ts_waitcnt vmcnt(0)
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "global_load_dword v4" in hits[0]


def test_checker_branch_merge_and_lds_dma():
    # a load on one path only is pending after the join; an LDS-DMA load writes no VGPR
    asm = _kernel("""
\ts_cbranch_scc0 .LBB0_2
\tglobal_load_dword v1, v[60:61], off
.LBB0_2:
\tglobal_load_lds_dwordx4 v[60:61], off
\tv_mov_b32_e32 v2, v1
\ts_waitcnt vmcnt(0)
\tv_mov_b32_e32 v3, v60
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "v2, v1" in hits[0]


def test_checker_atomics_and_lds_modifier():
    # gfx940-style returning atomic (sc0) writes its first operand; one without sc0 or glc
    # does not; a buffer load with the lds modifier writes LDS only
    asm = _kernel("""
\tglobal_atomic_add v5, v[60:61], v6, off sc0
\tv_mov_b32_e32 v1, v5
\tglobal_atomic_add v[60:61], v7, off
\tv_mov_b32_e32 v2, v7
\tbuffer_load_dword v9, s[4:7], 0 offen lds
\tv_mov_b32_e32 v3, v9
\ts_waitcnt vmcnt(0)
\ts_endpgm""")
    (hits,) = W.check_asm(asm).values()
    assert len(hits) == 1 and "v1, v5" in hits[0]


def _copies(n, base=0):
    return "\n".join("\tglobal_load_lds_dwordx4 v%d, s[4:5] offset:%d" % (10 + i % 4, base + 1072 * i)
                     for i in range(n))


def test_checker_lds_copy_groups():
    # double buffer: group A (4 copies), read of the index list, group B, wait that keeps
    # only B in flight, operand reads: clean.  With vmcnt(6) two copies of A may still land
    # when the operands are read: flagged.  Reads while only the newest group lands: clean.
    body = """
%s
\tds_read_b128 v[20:23], v1
%s
\ts_waitcnt vmcnt(%%d)
\tds_read_b128 v[24:27], v2
\ts_endpgm""" % (_copies(4), _copies(4, 8192))
    (ok,) = W.check_asm(_kernel(body % 4)).values()
    assert ok == []
    (hits,) = W.check_asm(_kernel(body % 6)).values()
    assert len(hits) == 1 and "ds_read_b128 v[24:27]" in hits[0] and "earlier LDS copy" in hits[0]
    # a loop: each iteration starts the next group, then waits for all but it; with the
    # wait the previous iteration's group has landed when the loop body reads LDS again
    loop = """
%s
.LBB0_1:
\tds_read_b64_tr_b16 v[30:31], v3
%s
\ts_waitcnt vmcnt(%%d)
\tds_read_b128 v[24:27], v2
\ts_cbranch_scc0 .LBB0_1
\ts_endpgm""" % (_copies(4), _copies(4, 8192))
    (ok,) = W.check_asm(_kernel(loop % 4)).values()
    assert ok == []
    (hits,) = W.check_asm(_kernel(loop % 8)).values()
    assert hits and all("earlier LDS copy" in h for h in hits)


def test_checker_groups_span_lgkmcnt_waits():
    # the row addresses of a tile come from scalar loads, so the copies of one group are
    # separated by lgkmcnt waits; they still form one group (a wait for all but that group
    # is clean), and leaving two copies of the previous group in flight is still flagged
    def tile(base):
        return "%s\n\ts_waitcnt lgkmcnt(0)\n%s" % (_copies(2, base), _copies(2, base + 4096))
    body = """
%s
\tds_read_b128 v[20:23], v1
%s
\ts_waitcnt vmcnt(%%d)
\tds_read_b128 v[24:27], v2
\ts_endpgm""" % (tile(0), tile(8192))
    (ok,) = W.check_asm(_kernel(body % 4)).values()
    assert ok == []
    (hits,) = W.check_asm(_kernel(body % 6)).values()
    assert len(hits) == 1 and "ds_read_b128 v[24:27]" in hits[0]


def test_checker_keeps_paths_apart():
    # one path drains the copies, the other starts the next group without a wait; an LDS
    # read after the join is clean on both paths.  Joining them (a wait seen on one path,
    # an earlier group in flight on the other) would report it: the exact replay does not,
    # the replay forced to join every state at once (a budget of 0 exact states) does
    body = """
%s
\ts_cbranch_scc0 .LBB0_2
\ts_waitcnt vmcnt(0)
\ts_branch .LBB0_3
.LBB0_2:
\tds_read_b128 v[20:23], v1
%s
.LBB0_3:
\tds_read_b128 v[24:27], v2
\ts_waitcnt vmcnt(0)
\ts_endpgm""" % (_copies(4), _copies(4, 8192))
    ((name, fbody),) = W.split_functions(_kernel(body)).items()
    assert W.check_function(fbody) == []
    joined = W.check_function(fbody, exact_per_block=0)
    assert len(joined) == 1 and "ds_read_b128 v[24:27]" in joined[0]


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = ([build_lib.hipcc()] + build_lib.COMMON + build_lib.EXTRA.get(src, [])
           + ["--cuda-device-only", "-S", os.path.join(build_lib.CSRC, src), "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-4000:]))
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        build_lib.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(len(HIP_SOURCES)) as ex:
        return dict(zip(HIP_SOURCES, ex.map(lambda s: _device_asm(s, d), HIP_SOURCES)))


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_access_to_registers_in_flight(device_asm, src):
    res = W.check_asm(device_asm[src])
    assert res, "no kernels found in %s" % src
    bad = {k: v[:5] for k, v in res.items() if v}
    assert not bad, "\n".join("%s:\n  %s" % (k, "\n  ".join(v)) for k, v in bad.items())
