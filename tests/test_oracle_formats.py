"""Pins of the oracle's element formats and MX quantizer (CPU only).

The formats are the OCP Microscaling (MX) v1.0 ones named by the pages ("DeepSeek
V4.1 Flash modeling", section "Mixed precision": index Q/K are MXFP4 with 32-element
groups; the window cache stays FP8).  Pins:
  * E2M1 decode against the value table of the format definition;
  * E4M3 decode of all 256 codes against torch.float8_e4m3fn (a library routine);
  * E4M3 element rounding against torch's float8_e4m3fn cast;
  * E2M1 element rounding against a brute-force nearest search, ties to even code;
  * the shared exponent against its defining property (amax / 2^e in [2^emax, 2^(emax+1))).
The main KV storage format (same section: E2M1 data, one E4M3 scale per 16 channels, no
global scale) is pinned by its byte count, by decode against torch's float8_e4m3fn table
times the E2M1 table, and by brute-force nearest searches for its scale and elements.
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


def test_index_and_main_entry_bytes_calculator(orc):
    """The page's cache calculator: C(N) entries x (288 + 68) B plus the saturated 2.5 MiB
    window payload is 892.50 MiB at 2,621,440 entries; both entry sizes come out of the
    oracle's quantizers."""
    g = json.load(open(GOLDEN))
    x = np.random.default_rng(2).standard_normal((1, 512)).astype(np.float32)
    mc, ms = orc.fp4s16_quant(x)
    main = mc.shape[1] + ms.shape[1]
    assert main == g["main_entry_bytes_fp4"]["bytes"] == 288
    ic, isc = orc.mx_quant(orc.E2M1, x[:, :128])
    index = ic.shape[1] + isc.shape[1]
    c = g["calculator"]
    assert c["entries"] == c["tokens"] // 2 * c["owners_m2"] + c["tokens"] * c["owners_m1"]
    mib = (c["entries"] * (main + index)) / 2.0 ** 20 + g["swa_payload_mib_saturated"]
    assert mib == c["mib"] == 892.5


E4M3_POS = [(c, float(v)) for c, v in
            enumerate(torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist())]


def _fp4s16_blocks(rng, nblk, lo=-14):
    x = rng.standard_normal((nblk, 16))
    x *= 2.0 ** rng.integers(lo, 8, size=(nblk, 1))
    return x.astype(np.float32)


def test_fp4s16_decode_vs_torch_tables(orc):
    """Every (code, scale) pair: element value = E2M1 table value x torch's E4M3 decode."""
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    codes = np.array([[(2 * i) % 16 | (((2 * i + 1) % 16) << 4) for i in range(8)]], np.uint8)
    for sb in list(range(0, 127)) + [128, 200, 254]:
        deq = orc.fp4s16_dequant(codes, np.array([[sb]], np.uint8))[0]
        for c in range(16):
            elem = -E2M1_TABLE[c & 7] if c & 8 else E2M1_TABLE[c & 7]
            assert deq[c] == elem * e4[sb], (sb, c, deq[c])


def test_fp4s16_scale_and_elements_brute_force(orc):
    """Scale byte = nearest positive E4M3 value to amax / 6 (ties to the even code,
    saturating at 448); element = nearest E2M1 value to |x| / s (ties to even code,
    saturating at 6) with x's sign bit; searched over the whole grids."""
    rng = np.random.default_rng(21)
    x = _fp4s16_blocks(rng, 300)
    codes, scales = orc.fp4s16_quant(x)
    assert codes.shape == (300, 8) and scales.shape == (300, 1)
    un = np.stack([codes & 15, codes >> 4], axis=-1).reshape(300, 16)
    for b in range(300):
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        sc = _nearest_even(min(amax / 6.0, 448.0), [c for c, _ in E4M3_POS], [v for _, v in E4M3_POS])
        assert scales[b, 0] == sc, (b, amax)
        s = E4M3_POS[sc][1]
        for i in range(16):
            want = _nearest_even(min(abs(float(x[b, i])) / s, 6.0), list(range(8)), E2M1_TABLE) if s > 0 else 0
            if np.signbit(x[b, i]):
                want |= 8
            assert un[b, i] == want, (b, i)


def test_fp4s16_ties_and_saturation(orc):
    """amax 6 gives scale 1.0 (E4M3 code 0x38), so elements round as given and the E2M1
    tie points go to the even code.  amax 6.3: 6.3 / 6 = 1.05 rounds to the E4M3 value
    1.0 (the next one is 1.125), so 6.3 itself saturates to 6."""
    x = np.zeros((2, 16), np.float32)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x[0, 0] = 6.0
    x[0, 1:8] = ties
    x[0, 8:15] = [-t for t in ties]
    x[1, 0] = 6.3
    x[1, 1] = -6.2
    codes, scales = orc.fp4s16_quant(x)
    assert scales[0, 0] == 0x38 and scales[1, 0] == 0x38
    deq = orc.fp4s16_dequant(codes, scales)
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert deq[0, 0] == 6.0 and list(deq[0, 1:8]) == want and list(deq[0, 8:15]) == [-w for w in want]
    assert deq[1, 0] == 6.0 and deq[1, 1] == -6.0


def test_fp4s16_zero_and_underflow_blocks(orc):
    """An all-zero block, and a block whose amax / 6 rounds below the smallest E4M3
    subnormal (2^-9), store scale 0 and zero magnitudes; a block at the top saturates the
    scale at 448."""
    x = np.zeros((3, 16), np.float32)
    x[1, :] = 6.0 * 2.0 ** -11      # amax / 6 = 2^-11 < half of 2^-9 -> scale 0
    x[1, 3] = -x[1, 3]
    x[2, 0] = 6.0 * 1000.0          # amax / 6 = 1000 -> scale saturates at 448, element at 6
    codes, scales = orc.fp4s16_quant(x)
    deq = orc.fp4s16_dequant(codes, scales)
    assert scales[0, 0] == 0 and np.all(codes[0] == 0)
    assert scales[1, 0] == 0 and np.all(deq[1] == 0) and (codes[1, 1] >> 4) == 8
    assert scales[2, 0] == 0x7E and deq[2, 0] == 6.0 * 448.0


def test_fp4s16_error_bound(orc):
    """The scale is within half an E4M3 quantum of amax / 6, and non-saturated elements lie
    within half an E2M1 quantum (times the scale) of their input."""
    rng = np.random.default_rng(22)
    x = _fp4s16_blocks(rng, 400, lo=-5)   # scales stay positive (no block underflows)
    codes, scales = orc.fp4s16_quant(x)
    deq = orc.fp4s16_dequant(codes, scales)
    s = np.array([v for _, v in E4M3_POS] + [0.0])[scales.astype(np.int64).clip(max=127)]
    assert np.all(s > 0)
    t = np.abs(x.astype(np.float64)).max(axis=1, keepdims=True) / 6.0
    qs = np.exp2(np.maximum(np.floor(np.log2(t)), -6) - 3)
    assert np.all(np.abs(s - t) <= 0.5 * qs)
    y = np.abs(x.astype(np.float64)) / s
    E = np.floor(np.log2(np.maximum(y, 1e-300)))
    q = np.exp2(np.maximum(E, 0) - 1) * s
    ok = y <= 6.0
    assert ok.mean() > 0.9
    assert np.all(np.abs(deq - x)[ok] <= 0.5 * q[ok])
