"""Pins of the oracle's reachability and index score (CPU only).

Pages: "DeepSeek V4.1 Flash modeling" (pages.haorui.li), sections "CSA2" (non-
overlapping compression, complete groups only) and "Mixed precision" (index Q/K
MXFP4, 32-element groups); "SGLang and Miles Day-0 support for DeepSeek-V4.1"
(theainews.cc), section 5 (FP4 index scoring in MQA form).  The score formula
s_j = sum_h w_h ReLU(q_h . k_j) comes from the workload definition (the pages say only "MQA form").

Pins: reachability against its closed form and the C0 count; the MXFP4 score
against exact rational arithmetic (a dropped term, a wrong sign, a transposed
operand or an unquantized q all exceed the fp32 rounding bound); the fp32 score
against float64; pool columns against the full-range columns.
"""
from fractions import Fraction

import numpy as np
import pytest

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_reach_closed_form(orc):
    for m in (1, 2, 3):
        for C in (0, 1, 5, 64):
            for p in range(0, 3 * C + 4):
                assert orc.reach(p, m, C) == min((p + 1) // m, C), (p, m, C)
    # C0: S = 1024 tokens at m = 2 -> 512 compressed entries, all visible to the last token.
    assert orc.reach(1023, 2, 512) == 512
    assert orc.reach(0, 2, 512) == 0       # the first pair is incomplete at p = 0
    assert orc.reach(1, 2, 512) == 1       # ... and complete at p = 1


def _decode_e2m1(codes, scales):
    """Independent decode of packed MXFP4 into exact Fractions (test-side)."""
    n, half = codes.shape
    out = []
    for i in range(n):
        row = []
        for c in range(half * 2):
            b = int(codes[i, c // 2])
            code = (b >> 4) if c & 1 else (b & 15)
            mag = Fraction(E2M1_TABLE[code & 7])
            v = -mag if code & 8 else mag
            e = int(scales[i, c // 32]) - 127
            row.append(v * (Fraction(2) ** e))
        out.append(row)
    return out


def _small_case(rng, nreq=2, S=(40, 29), m=2, H=8, D=64):
    ne = [s // m for s in S]
    rs = [0, ne[0]]
    rows_req, rows_pos = [], []
    for r in range(nreq):
        for p in rng.choice(S[r], size=6, replace=False):
            rows_req.append(r)
            rows_pos.append(int(p))
    n = len(rows_req)
    rows = dict(req_of_row=np.array(rows_req), pos_of_row=np.array(rows_pos))
    cache = dict(ratio_m=m, n_entries=np.array(ne), row_start=np.array(rs))
    keys = rng.standard_normal((sum(ne), D)).astype(np.float32)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    w = rng.random((n, H)).astype(np.float32)
    return rows, cache, keys, q, w


def test_mxfp4_score_exact_reference(orc):
    rng = np.random.default_rng(5)
    H, D = 8, 64
    rows, cache, keys_raw, q, w = _small_case(rng, H=H, D=D)
    # give some heads negative weights so that the ReLU and the sign of w both matter
    w[:, ::3] *= -1.0
    kc, ks = orc.mx_quant(orc.E2M1, keys_raw)
    scores, bad = orc.index_score(rows, cache, q, w, kc, key_scales=ks, heads=H, dim=D, score_stride=32)
    assert bad == 0
    qc, qs = orc.mx_quant(orc.E2M1, q.reshape(-1, D))
    qv = _decode_e2m1(qc, qs)
    kv = _decode_e2m1(kc, ks)
    n = len(rows["req_of_row"])
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // cache["ratio_m"], int(cache["n_entries"][r]))
        assert np.all(np.isnan(scores[i, R:]))
        for j in range(R):
            krow = kv[int(cache["row_start"][r]) + j]
            exact = Fraction(0)
            mag = Fraction(0)
            for h in range(H):
                d = sum(a * b for a, b in zip(qv[i * H + h], krow))
                t = Fraction(float(w[i, h])) * max(d, Fraction(0))
                exact += t
                mag += abs(t)
            got = Fraction(float(scores[i, j]))
            # fp32 fma chain over H/4 terms plus 2 levels of adds: <= (H/4 + 2) ulp-ish
            bound = mag * Fraction(H // 4 + 2, 2 ** 24)
            assert abs(got - exact) <= bound, (i, j, float(got), float(exact))


def test_mxfp4_score_uses_quantized_q(orc):
    """Scoring with raw q would differ far beyond rounding: the pin above detects it."""
    rng = np.random.default_rng(6)
    H, D = 8, 64
    rows, cache, keys_raw, q, w = _small_case(rng, H=H, D=D)
    kc, ks = orc.mx_quant(orc.E2M1, keys_raw)
    s_q, _ = orc.index_score(rows, cache, q, w, kc, key_scales=ks, heads=H, dim=D, score_stride=32)
    qc, qs = orc.mx_quant(orc.E2M1, q.reshape(-1, D))
    qdeq = orc.mx_dequant(orc.E2M1, qc, qs).astype(np.float32).reshape(q.shape)
    s_qq, _ = orc.index_score(rows, cache, qdeq, w, kc, key_scales=ks, heads=H, dim=D, score_stride=32)
    # quantization is idempotent: scoring already-quantized q gives identical bits
    assert np.array_equal(np.nan_to_num(s_q, nan=-7), np.nan_to_num(s_qq, nan=-7))


def test_f32_score_vs_float64(orc):
    rng = np.random.default_rng(7)
    H, D = 8, 64
    rows, cache, keys, q, w = _small_case(rng, H=H, D=D)
    scores, _ = orc.index_score(rows, cache, q, w, keys, heads=H, dim=D, score_stride=32)
    n = len(rows["req_of_row"])
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // 2, int(cache["n_entries"][r]))
        kr = keys[int(cache["row_start"][r]):int(cache["row_start"][r]) + R].astype(np.float64)
        d = q[i].astype(np.float64) @ kr.T                      # [H, R]
        ref = (w[i].astype(np.float64)[:, None] * np.maximum(d, 0)).sum(0)
        mag = (np.abs(w[i]).astype(np.float64)[:, None] * (np.abs(q[i]).astype(np.float64) @ np.abs(kr).T)).sum(0)
        assert np.all(np.abs(scores[i, :R] - ref) <= mag * (D + H) * 2.0 ** -23)
        assert np.all(np.isnan(scores[i, R:]))


def test_pool_columns_match_full_range(orc):
    rng = np.random.default_rng(8)
    H, D, B = 8, 64, 8
    S = (160, 120)
    rows, cache, keys_raw, q, w = _small_case(rng, S=S, H=H, D=D)
    kc, ks = orc.mx_quant(orc.E2M1, keys_raw)
    full, _ = orc.index_score(rows, cache, q, w, kc, key_scales=ks, heads=H, dim=D, score_stride=80)
    n = len(rows["req_of_row"])
    maxb = 4
    blocks = np.full((n, maxb), -1, np.int32)
    nblocks = np.zeros(n, np.int32)
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // 2, int(cache["n_entries"][r]))
        nb = (R + B - 1) // B
        if nb == 0:
            continue
        pick = sorted(set(rng.choice(nb, size=min(maxb - 1, nb), replace=False).tolist()) | {nb - 1})[:maxb]
        blocks[i, :len(pick)] = pick
        nblocks[i] = len(pick)
    pool = dict(blocks=blocks, nblocks=nblocks, block=B, max_blocks=maxb)
    ps, _ = orc.index_score(rows, cache, q, w, kc, key_scales=ks, heads=H, dim=D, score_stride=maxb * B, pool=pool)
    for i in range(n):
        r, p = int(rows["req_of_row"][i]), int(rows["pos_of_row"][i])
        R = min((p + 1) // 2, int(cache["n_entries"][r]))
        for c in range(nblocks[i] * B):
            j = blocks[i, c // B] * B + c % B
            if j < R:
                assert ps[i, c] == full[i, j]
            else:
                assert ps[i, c] == -np.inf
        assert np.all(np.isnan(ps[i, nblocks[i] * B:]))
