"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from the seeded generator; each side prepares its own copy: the HIP side
quantizes on the device with csa2_quant_mx, the oracle on the host with its own
quantizer, and the tests check that both produce the same bytes before comparing
anything downstream.
"""
import sys

import numpy as np
import torch

from compressed_sparse_attention_fp4_amd import binding as B

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def i32(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32)


def i64(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int64)


def dev_rows(rows):
    return B.Rows(i32(rows["req_of_row"]).to(DEV), i32(rows["pos_of_row"]).to(DEV),
                  None if rows.get("win_lo") is None else i32(rows["win_lo"]).to(DEV))


def dev_cache(cache):
    return B.Cache(cache["ratio_m"], i32(cache["n_entries"]).to(DEV), i64(cache["row_start"]).to(DEV))


def np_rows(rows):
    return {k: (None if v is None else np.asarray(v)) for k, v in rows.items()}


def quant_both(orc, fmt_hip, fmt_orc, x_f32: torch.Tensor):
    """Quantize x (float32, host) on both sides; assert identical bytes; return both."""
    codes_d, scales_d = B.quant_mx(fmt_hip, x_f32.to(DEV))
    codes_o, scales_o = orc.mx_quant(fmt_orc, x_f32.numpy())
    cd, sd = codes_d.cpu().numpy(), scales_d.cpu().numpy()
    assert np.array_equal(sd, scales_o), "scale bytes differ"
    assert np.array_equal(cd, codes_o), "code bytes differ"
    return (codes_d, scales_d), (codes_o, scales_o)


def quant_fp4_both(orc, x: torch.Tensor):
    """Main KV storage format on both sides (x float32 or bfloat16, host): the device
    quantizer takes x as it is, the oracle its float32 values; identical bytes asserted."""
    codes_d, scales_d = B.quant_mx(B.FP4_S16, x.to(DEV))
    codes_o, scales_o = orc.fp4s16_quant(x.float().numpy())
    cd, sd = codes_d.cpu().numpy(), scales_d.cpu().numpy()
    assert np.array_equal(sd, scales_o), ("E4M3 scale bytes differ", int((sd != scales_o).sum()))
    assert np.array_equal(cd, codes_o), ("E2M1 code bytes differ", int((cd != codes_o).sum()))
    return (codes_d, scales_d), (codes_o, scales_o)


E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def fp4_decode_torch(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """Decoded values of main-KV-format rows (host tensors), from the E2M1 value table and
    torch's float8_e4m3fn decode of the scale bytes; float32 (every value is exact)."""
    table = torch.tensor(E2M1_VALUES, dtype=torch.float32)
    c = torch.stack([codes & 15, codes >> 4], dim=-1).reshape(codes.shape[0], -1).long()
    s = scales.view(torch.float8_e4m3fn).float().repeat_interleave(16, dim=-1)
    return table[c] * s


def allclose_report(got, ref, atol, rtol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    return int(bad.sum()), float(err.max(initial=0.0)), float((err / (np.abs(ref) + 1e-30)).max(initial=0.0))


def bits(t):
    """bf16 tensor -> its 16-bit patterns as a host uint16 array (the oracle's bf16 input)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_scores(got, ref, ncols):
    """Scores bit for bit on the first ncols[i] columns of every sampled row."""
    for i, n in enumerate(ncols):
        if not np.array_equal(got[i, :n], ref[i, :n]):
            bad = np.nonzero(got[i, :n] != ref[i, :n])[0]
            raise AssertionError("sample row %d: %d of %d score columns differ, first %s" % (i, len(bad), n, bad[:6]))


def check_attn(got, ref):
    """bf16 attention tolerance: |g - r| <= 2e-2 + 1e-2 |r| and a row relative L2 error <= 1e-2."""
    nb, emax, _ = allclose_report(got, ref, 2e-2, 1e-2)
    assert nb == 0, ("attention elements out of tolerance", nb, emax)
    n, h, d = ref.shape
    rel = np.linalg.norm((got - ref).reshape(n * h, d), axis=1) / (np.linalg.norm(ref.reshape(n * h, d), axis=1)
                                                                   + 1e-30)
    assert rel.max() <= 1e-2, ("row relative L2", rel.max())


POISON_I32 = 0x7FFFFFFF


def poison(shape, dtype, device=DEV):
    """An output buffer filled with a sentinel no kernel writes (NaN for floating point,
    0x7fffffff for int32), so that elements a kernel leaves unwritten are caught."""
    if dtype == torch.int32:
        return torch.full(shape, POISON_I32, dtype=dtype, device=device)
    return torch.full(shape, float("nan"), dtype=dtype, device=device)
