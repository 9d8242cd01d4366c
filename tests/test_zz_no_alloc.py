"""csa2_topk_hier_noalloc (the allocation-free variant of csa2_topk_hier, for callers that
cannot allocate device memory) against csa2_topk_hier with a caller workspace: two calls
in a row through the C ABI, the second on a smaller input, both bit-exact against the
workspace entry point and against the oracle.  Also run alone in a fresh process."""
import ctypes

import numpy as np
import pytest
import torch

from compressed_sparse_attention_fp4_amd import binding as B

from gpu_util import DEV, dev_cache, dev_rows, poison, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _inputs(seed, R_list, stride):
    rng = np.random.default_rng(seed)
    n = len(R_list)
    rows = dict(req_of_row=np.arange(n), pos_of_row=np.array([max(R - 1, 0) for R in R_list]))
    cache = dict(ratio_m=1, n_entries=np.array(R_list), row_start=np.zeros(n, np.int64))
    scores = np.full((n, stride), np.nan, np.float32)
    for i, R in enumerate(R_list):
        scores[i, :min(R, stride)] = (rng.standard_normal(min(R, stride)) * 30 + 150).astype(np.float32)
    return rows, cache, scores


def _call_noalloc(rows_d, cache_d, scores_d, k, block, max_blocks, out):
    idx, blocks, nblocks = out
    L = B.lib()
    rc = L.csa2_topk_hier_noalloc(ctypes.byref(rows_d.c()), ctypes.byref(cache_d.c()),
                                  ctypes.c_void_p(scores_d.data_ptr()), ctypes.c_int64(scores_d.stride(0)),
                                  ctypes.c_int32(k), ctypes.c_int32(block), ctypes.c_int32(max_blocks),
                                  ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(blocks.data_ptr()),
                                  ctypes.c_void_p(nblocks.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == B.CSA2_OK, L.csa2_last_error().decode()


def test_noalloc_matches_workspace_entry_point(orc):
    # first call: the decode shape (64 rows of 65,536 columns); second: fewer, shorter rows
    # with another k and max_blocks, so stale scratch from the first call would show
    cases = [(list(range(65536, 65536 - 64 * 37, -37)), 65536, 512, 2048),
             ([1, 9, 100, 16385, 30001, 40000], 40000, 256, 1024)]
    for step, (R_list, stride, k, mb) in enumerate(cases):
        say("case: noalloc call %d: %d rows x %d columns, k=%d, max_blocks=%d" % (step, len(R_list), stride, k, mb))
        rows, cache, scores = _inputs(900 + step, R_list, stride)
        rd, cd = dev_rows(rows), dev_cache(cache)
        sd = torch.from_numpy(scores).to(DEV)
        n = len(R_list)
        got = (poison((n, k), torch.int32), poison((n, mb), torch.int32), poison((n,), torch.int32))
        _call_noalloc(rd, cd, sd, k, 8, mb, got)
        ref = B.topk_hier(rd, cd, sd, k, 8, mb)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        ri, rb, rn = orc.topk_hier(rows, cache, scores, k, 8, mb)
        assert np.array_equal(got[0].cpu().numpy(), ri)
        assert np.array_equal(got[1].cpu().numpy(), rb)
        assert np.array_equal(got[2].cpu().numpy(), rn)


def test_noalloc_refuses_oversized_scratch():
    # 2,048 rows of 65,536 columns need 64 MiB of block maxima: refused before any launch
    L = B.lib()
    rows = B.Rows(torch.zeros(2048, dtype=torch.int32, device=DEV), torch.zeros(2048, dtype=torch.int32, device=DEV))
    cache = B.Cache(1, torch.ones(1, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int64, device=DEV))
    p = ctypes.c_void_p(rows.req_of_row.data_ptr())
    rc = L.csa2_topk_hier_noalloc(ctypes.byref(rows.c()), ctypes.byref(cache.c()), p, ctypes.c_int64(65536),
                                  ctypes.c_int32(512), ctypes.c_int32(8), ctypes.c_int32(2048), p, p, p, None)
    assert rc == B.CSA2_E_WORKSPACE and "scratch" in L.csa2_last_error().decode()
