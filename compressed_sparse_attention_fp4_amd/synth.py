"""Seeded synthetic inputs for the CSA2 hot path.

This module serves both the HIP path and the CPU oracle.  It holds none of the
method's arithmetic: it draws random numbers (torch generators, one stream per
tensor and chunk, seeded from the configuration's seed and the tensor's name),
casts them to the input dtypes (float32, or bfloat16 by torch's round-to-nearest
-even cast) and lays out the per-configuration geometry (requests, positions,
cache row offsets).  MX quantization of index keys and window KV is left to each
side: the library quantizes on the device, the oracle on the host.

Value recipe (same for every configuration): q, index q, index keys, main KV and
window KV are iid N(0,1); index head weights are U(0,1).

Configurations (numbered as in the workload list):
  C0  tiny fp32 Full layer: 1 request, S=1024, m=2 (512 entries), index 8x64,
      top-64, 8 query heads x 64, window 128.
  C1  decoder-style Full-layer prefill, m=1: 8 requests x 8192 tokens, index 64x128
      MXFP4 keys, top-512, 64 bf16 query heads x 512 over one shared KV head, fp8 window.
  C2  decoder bounded-replay tail: extends {8192,8192,4096,4096,2048,512,128,64} on
      sequences of S=8192; one Reindex then one Reuse layer on the tail rows.
  C3  hierarchical decode: 64 requests x 1 query, S=131072, m=2 (65536 entries);
      source pass (flat top-512 + pool of 2048 blocks of 8) then 7 Reindex passes.
  C4  long-context decode: {1, 32} requests x 1 query, S=524288, m=2 (262144 entries).
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import torch


def _seed(seed: int, tag: str, chunk: int = 0) -> int:
    return (seed * 1_000_003 + zlib.crc32(tag.encode()) * 7919 + chunk * 104_729) & 0x7FFF_FFFF_FFFF


def _gen(device, seed, tag, chunk=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, chunk))
    return g


def normal(shape, seed: int, tag: str, device="cpu", chunk_rows: int = 0) -> torch.Tensor:
    """iid N(0,1) float32.  With chunk_rows > 0 the leading axis is drawn in
    chunks of that many rows, each chunk from its own stream (bounded temporaries)."""
    shape = tuple(int(s) for s in shape)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        return torch.randn(shape, generator=_gen(device, seed, tag), device=device, dtype=torch.float32)
    out = torch.empty(shape, device=device, dtype=torch.float32)
    for c, r0 in enumerate(range(0, shape[0], chunk_rows)):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=_gen(device, seed, tag, c + 1),
                                 device=device, dtype=torch.float32)
    return out


def normal_bf16(shape, seed: int, tag: str, device="cpu", chunk_rows: int = 0) -> torch.Tensor:
    """iid N(0,1) drawn in float32 and cast to bfloat16 (round to nearest even),
    chunk by chunk so that no full-size float32 temporary exists."""
    shape = tuple(int(s) for s in shape)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        return normal(shape, seed, tag, device).to(torch.bfloat16)
    out = torch.empty(shape, device=device, dtype=torch.bfloat16)
    for c, r0 in enumerate(range(0, shape[0], chunk_rows)):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=_gen(device, seed, tag, c + 1),
                                 device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def uniform(shape, seed: int, tag: str, device="cpu") -> torch.Tensor:
    """iid U(0,1) float32."""
    return torch.rand(tuple(int(s) for s in shape), generator=_gen(device, seed, tag), device=device,
                      dtype=torch.float32)


def bf16_bits(t: torch.Tensor):
    """Raw 16-bit patterns of a bfloat16 tensor as a numpy uint16 array (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def bf16_values(t: torch.Tensor):
    """float32 values of a bfloat16 tensor as numpy (exact widening)."""
    return t.detach().cpu().float().numpy()


# --------------------------------------------------------------------------- geometry
@dataclass
class Geometry:
    """Requests of one layer call: per request the total length S, the compressed
    ratio m and the entry count C = S // m of its KV owner; cache rows of request r
    start at row_start[r] (requests packed back to back)."""
    seq_len: list
    ratio_m: int
    n_entries: list = field(init=False)
    row_start: list = field(init=False)

    def __post_init__(self):
        self.n_entries = [s // self.ratio_m for s in self.seq_len]
        acc, rs = 0, []
        for c in self.n_entries:
            rs.append(acc)
            acc += c
        self.row_start = rs

    @property
    def nreq(self):
        return len(self.seq_len)

    @property
    def total_entries(self):
        return sum(self.n_entries)


@dataclass
class Config:
    name: str
    seed: int
    geom: Geometry
    index_heads: int
    index_dim: int
    index_fp4: bool
    topk: int
    heads: int
    dim: int
    window: int = 128
    block: int = 8
    max_blocks: int = 2048


def config(i: int, nreq: int | None = None) -> Config:
    """The five workload configurations; nreq overrides the request count of the
    decode configurations (C3, C4) and of C1 (a prefix of its requests)."""
    if i == 0:
        return Config("C0 tiny fp32 Full layer", 0, Geometry([1024], 2), 8, 64, False, 64, 8, 64)
    if i == 1:
        n = nreq or 8
        return Config("C1 Full-layer prefill 8x8192 m=1", 1, Geometry([8192] * n, 1), 64, 128, True, 512, 64, 512)
    if i == 2:
        return Config("C2 bounded-replay tail", 2, Geometry([8192] * 8, 1), 64, 128, True, 512, 64, 512)
    if i == 3:
        n = nreq or 64
        return Config("C3 hierarchical decode 64x131072 m=2", 3, Geometry([131072] * n, 2), 64, 128, True, 512,
                      64, 512)
    if i == 4:
        n = nreq or 32
        return Config("C4 long-context decode %dx524288 m=2" % n, 4, Geometry([524288] * n, 2), 64, 128, True,
                      512, 64, 512)
    raise ValueError(i)


C2_EXTENDS = [8192, 8192, 4096, 4096, 2048, 512, 128, 64]


def prefill_rows(geom: Geometry):
    """Every token of every request as a query row (a Full-layer prefill)."""
    req, pos = [], []
    for r, s in enumerate(geom.seq_len):
        req += [r] * s
        pos += list(range(s))
    return dict(req_of_row=torch.tensor(req, dtype=torch.int32), pos_of_row=torch.tensor(pos, dtype=torch.int32))


def decode_rows(geom: Geometry):
    """One new token per request at position S-1 (S counts the new token)."""
    return dict(req_of_row=torch.arange(geom.nreq, dtype=torch.int32),
                pos_of_row=torch.tensor([s - 1 for s in geom.seq_len], dtype=torch.int32))


def window_cache_geometry(geom: Geometry, window: int, rows_held=None):
    """A window KV buffer holding, per request, the positions [S - held, S) where
    held = min(window, S) unless rows_held gives it; requests packed back to back."""
    pos_start, row_start, acc = [], [], 0
    for r, s in enumerate(geom.seq_len):
        held = min(window, s) if rows_held is None else rows_held[r]
        pos_start.append(s - held)
        row_start.append(acc)
        acc += held
    return dict(pos_start=torch.tensor(pos_start, dtype=torch.int32),
                row_start=torch.tensor(row_start, dtype=torch.int64), rows=acc)


def sm_scale(dim: int) -> float:
    return 1.0 / math.sqrt(dim)
