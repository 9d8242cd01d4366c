"""Pins of the oracle's element formats and MX quantizer (CPU only).

The formats are the OCP Microscaling (MX) v1.0 ones named by the pages ("DeepSeek
V4.1 Flash modeling", section "Mixed precision": index Q/K are MXFP4 with 32-element
groups; the window cache stays FP8).  Pins:
  * E2M1 decode against the value table of the format definition;
  * E4M3 decode of all 256 codes against torch.float8_e4m3fn (a library routine);
  * E4M3 element rounding against torch's float8_e4m3fn cast;
  * E2M1 element rounding against a brute-force nearest search, ties to even code;
  * the shared exponent against its defining property (amax / 2^e in [2^emax, 2^(emax+1))).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table(orc):
    for c in range(16):
        v = orc.e2m1_value(c)
        mag = E2M1_TABLE[c & 7]
        assert v == (-mag if c & 8 else mag) or (mag == 0 and v == 0)
        if c == 8:
            assert math.copysign(1.0, v) == -1.0


def test_e4m3_decode_all_codes_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[c])


def test_e8m0_values(orc):
    assert orc.e8m0_value(127) == 1.0
    assert orc.e8m0_value(0) == 2.0 ** -127
    assert orc.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(orc.e8m0_value(255))


def _blocks(rng, nblk, spread=True):
    x = rng.standard_normal((nblk, 32)).astype(np.float32)
    if spread:
        x *= (2.0 ** rng.integers(-20, 20, size=(nblk, 1))).astype(np.float32)
    return x


def _check_scale(x, scales, emax):
    for b in range(x.shape[0]):
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        e = int(scales[b, 0]) - 127
        if amax == 0:
            assert e == -127
            continue
        r = amax / 2.0 ** e
        if -127 < e < 127:
            assert 2.0 ** emax <= r < 2.0 ** (emax + 1), (b, amax, e)


def _nearest_even(y, grid_codes, grid_vals):
    """Brute force: nearest grid value to y; on a tie the code with LSB 0."""
    best = None
    for c, v in zip(grid_codes, grid_vals):
        d = abs(y - v)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def test_mx_e2m1_rounding_brute_force(orc):
    rng = np.random.default_rng(11)
    x = _blocks(rng, 400)
    codes, scales = orc.mx_quant(orc.E2M1, x)
    _check_scale(x, scales, 2)
    unpacked = np.stack([codes & 15, codes >> 4], axis=-1).reshape(x.shape)
    grid_codes = list(range(8))
    grid_vals = E2M1_TABLE
    for b in range(x.shape[0]):
        e = int(scales[b, 0]) - 127
        for i in range(32):
            y = abs(float(x[b, i])) / 2.0 ** e
            want = _nearest_even(y, grid_codes, grid_vals)
            if np.signbit(x[b, i]):
                want |= 8
            assert unpacked[b, i] == want, (b, i, float(x[b, i]), e)


def test_mx_e2m1_tie_table(orc):
    # amax 6 gives e = floor(log2 6) - 2 = 0, so the elements are rounded as given.
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0
    x[0, 1:8] = ties
    x[0, 8:15] = [-t for t in ties]
    x[0, 15] = 7.5 / 8  # 0.9375 -> 1.0
    codes, scales = orc.mx_quant(orc.E2M1, x)
    assert scales[0, 0] == 127
    deq = orc.mx_dequant(orc.E2M1, codes, scales)[0]
    assert deq[0] == 6.0
    assert list(deq[1:8]) == want
    assert list(deq[8:15]) == [-w for w in want]
    assert deq[15] == 1.0


def test_mx_e2m1_saturates_and_zero_block(orc):
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 7.5          # e = floor(log2 7.5) - 2 = 0 -> 7.5 saturates to 6
    x[0, 1] = -7.9
    codes, scales = orc.mx_quant(orc.E2M1, x)
    deq = orc.mx_dequant(orc.E2M1, codes, scales)
    assert scales[0, 0] == 127 and deq[0, 0] == 6.0 and deq[0, 1] == -6.0
    assert scales[1, 0] == 0 and np.all(codes[1] == 0) and np.all(deq[1] == 0)


def test_mx_e4m3_rounding_vs_torch(orc):
    rng = np.random.default_rng(12)
    x = _blocks(rng, 500)
    codes, scales = orc.mx_quant(orc.E4M3, x)
    _check_scale(x, scales, 8)
    e = scales.astype(np.int64).reshape(-1, 1) - 127
    y = x.astype(np.float64) / np.exp2(e.astype(np.float64))
    y = np.clip(y, -448.0, 448.0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_mx_e4m3_saturation(orc):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 511.0        # e = floor(log2 511) - 8 = 0 -> 511 saturates to 448
    x[0, 1] = 460.0        # rounds to 448 (nearest of 448 / 480 -> 448), no saturation needed
    x[0, 2] = 470.0        # rounds to 480 -> saturates to 448
    codes, scales = orc.mx_quant(orc.E4M3, x)
    deq = orc.mx_dequant(orc.E4M3, codes, scales)
    assert scales[0, 0] == 127
    assert deq[0, 0] == 448.0 and deq[0, 1] == 448.0 and deq[0, 2] == 448.0


def test_mx_quant_error_bound(orc):
    """Every non-saturated element is within half a quantum of its input."""
    rng = np.random.default_rng(13)
    x = _blocks(rng, 300, spread=False)
    for fmt, mbits, emin in ((orc.E2M1, 1, 0), (orc.E4M3, 3, -6)):
        codes, scales = orc.mx_quant(fmt, x)
        deq = orc.mx_dequant(fmt, codes, scales)
        e = scales.astype(np.float64).reshape(-1, 1) - 127
        y = np.abs(x.astype(np.float64)) / np.exp2(e)
        E = np.floor(np.log2(np.maximum(y, 1e-300)))
        q = np.exp2(np.maximum(E, emin) - mbits) * np.exp2(e)
        maxv = 6.0 if fmt == orc.E2M1 else 448.0
        ok = y <= maxv
        assert np.all(np.abs(deq - x)[ok] <= 0.5 * q[ok] + 1e-30)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cache_bytes.json")


def test_index_entry_bytes_golden(orc):
    """[P1] "Mixed precision": an index K entry is 128 x (0.5 + 1/32) = 68 B (the page's
    number, tests/golden/cache_bytes.json); the oracle's MXFP4 quantizer writes exactly
    that many bytes per 128-d entry."""
    g = json.load(open(GOLDEN))["index_entry_bytes"]
    x = np.random.default_rng(1).standard_normal((3, g["dim"])).astype(np.float32)
    codes, scales = orc.mx_quant(orc.E2M1, x)
    assert codes.shape[1] + scales.shape[1] == g["bytes"] == 68
