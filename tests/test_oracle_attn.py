"""Pins of the oracle's sparse + sliding-window attention (CPU only).

Pages: "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 1 (each query
attends to its own 128-position window and to at most 512 compressed positions
chosen by the indexer); "DeepSeek V4.1 Flash modeling", section "Mixed precision"
(the 512-d main entry is one shared latent, so key = value; the window cache is
FP8); "SGLang: how DeepSeek V4.1 Flash late layers only process tail tokens",
section 2.3 (the window of a tail row is cut at the replay lower bound).

Pins: the dense routine against torch's scaled_dot_product_attention in float64
(a library routine) on explicitly listed key sets; sparse attention with every
reachable entry selected equals the dense routine (the equivalence the problem
statement asks for); k = 0 is plain sliding-window attention; one key gives its
value; identical keys give the mean of the values; FP8 window rows dequantize
like torch's float8_e4m3fn times the block scale.
"""
import numpy as np
import pytest
import torch


def _case(rng, S=(40, 25), m=2, H=4, D=32, W=8, lo=None):
    nreq = len(S)
    ne = [s // m for s in S]
    rs = np.cumsum([0] + ne[:-1])
    req, pos = [], []
    for r in range(nreq):
        for p in sorted(rng.choice(S[r], size=7, replace=False).tolist()):
            req.append(r)
            pos.append(p)
    n = len(req)
    rows = dict(req_of_row=np.array(req), pos_of_row=np.array(pos))
    if lo is not None:
        rows["win_lo"] = np.array([max(0, p - lo) for p in pos])
    cache = dict(ratio_m=m, n_entries=np.array(ne), row_start=rs)
    kv = rng.standard_normal((sum(ne), D)).astype(np.float32)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    swa_rows = sum(S)
    swa = dict(data=rng.standard_normal((swa_rows, D)).astype(np.float32), dtype=0, scale=None,
               row_start=np.cumsum([0] + list(S[:-1])), pos_start=np.zeros(nreq, np.int64), window=W)
    return rows, cache, kv, q, swa


def _keyset(rows, cache, kv, swa, i, sel=None):
    r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
    lo = int(rows["win_lo"][i]) if "win_lo" in rows else 0
    R = min((p + 1) // cache["ratio_m"], int(cache["n_entries"][r]))
    js = list(range(R)) if sel is None else [j for j in sel if j >= 0]
    main = [kv[int(cache["row_start"][r]) + j] for j in js]
    t0 = max(lo, p - swa["window"] + 1, int(swa["pos_start"][r]))
    win = [swa["data"][int(swa["row_start"][r]) + t - int(swa["pos_start"][r])] for t in range(t0, p + 1)]
    return np.array(main + win, dtype=np.float64).reshape(-1, kv.shape[1])


def _sdpa(qh, keys, scale):
    qt = torch.from_numpy(qh).reshape(1, 1, -1, qh.shape[-1])
    kt = torch.from_numpy(keys).reshape(1, 1, -1, keys.shape[-1])
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("lo", [None, 3])
def test_dense_vs_torch_sdpa(orc, lo):
    rng = np.random.default_rng(41)
    H, D = 4, 32
    rows, cache, kv, q, swa = _case(rng, H=H, D=D, lo=lo)
    scale = 0.3
    out, lse = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, None, swa, heads=H, dim=D, sm_scale=scale, dense=True)
    for i in range(len(rows["req_of_row"])):
        keys = _keyset(rows, cache, kv, swa, i)
        ref = _sdpa(q[i].astype(np.float64), keys, scale)
        assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-12)
        lref = np.log(np.exp(scale * q[i].astype(np.float64) @ keys.T).sum(-1))
        assert np.allclose(lse[i], lref, rtol=1e-12)


def test_sparse_with_all_entries_equals_dense(orc):
    rng = np.random.default_rng(42)
    H, D = 4, 32
    rows, cache, kv, q, swa = _case(rng, H=H, D=D)
    n = len(rows["req_of_row"])
    k = 24
    sel = np.full((n, k), -1, np.int32)
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // 2, int(cache["n_entries"][r]))
        perm = rng.permutation(R)               # order of the index set does not matter
        sel[i, :R] = perm
    a, la = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, sel, swa, heads=H, dim=D, sm_scale=0.2)
    b, lb = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, None, swa, heads=H, dim=D, sm_scale=0.2, dense=True)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13) and np.allclose(la, lb, rtol=1e-12)


def test_k0_is_sliding_window_attention(orc):
    rng = np.random.default_rng(43)
    H, D = 4, 32
    rows, cache, kv, q, swa = _case(rng, H=H, D=D)
    n = len(rows["req_of_row"])
    sel = np.zeros((n, 0), np.int32)
    out, _ = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, sel, swa, heads=H, dim=D, sm_scale=0.25)
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        base = int(swa["row_start"][r])
        seq = swa["data"][base:base + p + 1].astype(np.float64)           # positions 0..p of request r
        qt = torch.from_numpy(q[i].astype(np.float64)).reshape(1, H, 1, D)
        kt = torch.from_numpy(seq).reshape(1, 1, -1, D).expand(1, H, -1, D)
        mask = torch.zeros(1, 1, 1, p + 1, dtype=torch.bool)
        mask[..., max(0, p - swa["window"] + 1):] = True                  # band of width W ending at p
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=0.25)
        assert np.allclose(out[i], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_single_key_and_identical_keys(orc):
    rng = np.random.default_rng(44)
    H, D = 2, 32
    # query at p = 0 with m = 2: no compressed entry reachable, window holds one row
    rows = dict(req_of_row=np.array([0]), pos_of_row=np.array([0]))
    cache = dict(ratio_m=2, n_entries=np.array([0]), row_start=np.array([0]))
    kv = np.zeros((1, D), np.float32)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    swa = dict(data=rng.standard_normal((1, D)).astype(np.float32), dtype=0, scale=None,
               row_start=np.array([0]), pos_start=np.array([0]), window=128)
    out, lse = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, np.zeros((1, 4), np.int32) - 1, swa, heads=H, dim=D,
                                   sm_scale=1.0)
    assert np.allclose(out[0], swa["data"][0].astype(np.float64)[None], rtol=0, atol=0)
    # identical keys everywhere -> uniform weights -> the mean (= that key)
    kv2 = np.tile(rng.standard_normal((1, D)).astype(np.float32), (10, 1))
    rows2 = dict(req_of_row=np.array([0]), pos_of_row=np.array([19]))
    cache2 = dict(ratio_m=2, n_entries=np.array([10]), row_start=np.array([0]))
    swa2 = dict(data=np.tile(kv2[:1], (20, 1)), dtype=0, scale=None, row_start=np.array([0]),
                pos_start=np.array([0]), window=4)
    out2, lse2 = orc.sparse_swa_attn(rows2, cache2, q, 0, kv2, 0, np.arange(10, dtype=np.int32)[None], swa2,
                                     heads=H, dim=D, sm_scale=0.5)
    assert np.allclose(out2[0], kv2[0].astype(np.float64)[None], rtol=1e-14, atol=1e-14)
    logit = 0.5 * (q[0].astype(np.float64) @ kv2[0].astype(np.float64))
    assert np.allclose(lse2[0], logit + np.log(14.0), rtol=1e-13)


def test_fp8_window_and_bf16_operands(orc):
    """MXFP8 window rows and bf16 q / KV decode like torch's float8 / bfloat16."""
    rng = np.random.default_rng(45)
    H, D = 2, 64
    rows, cache, kv, q, swa = _case(rng, S=(30,), H=H, D=D, W=16)
    codes, scales = orc.mx_quant(orc.E4M3, swa["data"])
    deq = (torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
           * np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1))
    q_bf = torch.from_numpy(q).to(torch.bfloat16)
    kv_bf = torch.from_numpy(kv).to(torch.bfloat16)
    qb = q_bf.view(torch.int16).numpy().view(np.uint16)
    kvb = kv_bf.view(torch.int16).numpy().view(np.uint16)
    swa8 = dict(swa, data=codes, dtype=3, scale=scales)
    a, _ = orc.sparse_swa_attn(rows, cache, qb, 1, kvb, 1, None, swa8, heads=H, dim=D, sm_scale=0.1, dense=True)
    swaf = dict(swa, data=deq.astype(np.float32))  # fp8 values are exact in float32
    b, _ = orc.sparse_swa_attn(rows, cache, q_bf.float().numpy(), 0, kv_bf.float().numpy(), 0, None, swaf,
                               heads=H, dim=D, sm_scale=0.1, dense=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("shift", [0.0, 40.0])
def test_sink_is_an_extra_zero_value_key(orc, shift):
    """A sink of logit sink_h is one more key whose value is the zero vector: torch SDPA over
    the key set with a zero row appended (its logit set to sink_h through an additive mask)
    gives the output, and log-sum-exp over the logits together with sink_h gives lse.  With
    shift 40 every logit is moved 40 up (one extra dimension: 1 in every key, shift/scale in
    q), so that a sink added without the max shift, or added to the numerator, fails."""
    rng = np.random.default_rng(46)
    H, D = 4, 32
    rows, cache, kv, q, swa = _case(rng, H=H, D=D)
    n = len(rows["req_of_row"])
    scale = 0.3
    kv = np.concatenate([kv, np.ones((kv.shape[0], 1), np.float32)], axis=1)
    swa = dict(swa, data=np.concatenate([swa["data"], np.ones((swa["data"].shape[0], 1), np.float32)], axis=1))
    q = np.concatenate([q, np.full((n, H, 1), shift / scale, np.float32)], axis=2)
    D += 1
    sink = (rng.standard_normal(H) * 2.0 + shift).astype(np.float32)
    out, lse = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, None, swa, heads=H, dim=D, sm_scale=scale, sink=sink,
                                   dense=True)
    for i in range(n):
        keys = _keyset(rows, cache, kv, swa, i)
        nk = keys.shape[0]
        aug = np.concatenate([keys, np.zeros((1, D))], axis=0)
        qt = torch.from_numpy(q[i].astype(np.float64)).reshape(1, H, 1, D)
        kt = torch.from_numpy(aug).reshape(1, 1, nk + 1, D).expand(1, H, nk + 1, D)
        bias = torch.zeros(1, H, 1, nk + 1, dtype=torch.float64)
        bias[0, :, 0, nk] = torch.from_numpy(sink.astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=bias, scale=scale)
        assert np.allclose(out[i], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)
        logits = scale * (q[i].astype(np.float64) @ keys.T)
        lref = torch.logsumexp(torch.from_numpy(np.concatenate([logits, sink[:, None].astype(np.float64)], axis=1)),
                               dim=1).numpy()
        assert np.allclose(lse[i], lref, rtol=1e-12, atol=1e-12)


def test_fp4_main_kv_attends_like_its_dequantized_values(orc):
    """Main KV in its storage format ("DeepSeek V4.1 Flash modeling", section "Mixed
    precision": dequantized before attention): the oracle's result with FP4 entries is
    the same as with the fp32 values that the format's decode gives (exactly: each
    decoded value is an E2M1 value times an E4M3 scale, representable in fp32), and
    both match torch's SDPA on the dequantized key sets."""
    rng = np.random.default_rng(47)
    H, D = 4, 32
    rows, cache, kv, q, swa = _case(rng, H=H, D=D)
    codes, scales = orc.fp4s16_quant(kv)
    deq = orc.fp4s16_dequant(codes, scales)
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    n = len(rows["req_of_row"])
    sel = np.full((n, 6), -1, np.int32)
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // 2, int(cache["n_entries"][r]))
        sel[i, :min(R, 6)] = rng.permutation(R)[:6]
    a, la = orc.sparse_swa_attn(rows, cache, q, 0, codes, orc.DT_FP4S16, sel, swa, heads=H, dim=D, sm_scale=0.2,
                                kv_scale=scales)
    b, lb = orc.sparse_swa_attn(rows, cache, q, 0, deq.astype(np.float32), 0, sel, swa, heads=H, dim=D, sm_scale=0.2)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    for i in range(n):
        keys = _keyset(rows, cache, deq, swa, i, sel[i])
        assert np.allclose(a[i], _sdpa(q[i].astype(np.float64), keys, 0.2), rtol=1e-12, atol=1e-12)
    # and the FP4 result differs from the unquantized one (the format is lossy)
    c, _ = orc.sparse_swa_attn(rows, cache, q, 0, kv, 0, sel, swa, heads=H, dim=D, sm_scale=0.2)
    assert not np.allclose(a, c, atol=1e-6)
