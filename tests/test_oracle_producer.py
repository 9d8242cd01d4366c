"""Pins of the oracle's index-K / main-KV producer (CPU only).

Pages: "DeepSeek V4.1 Flash modeling", section "CSA2" (non-overlapping compression; index K
projected from the compressed main KV) and "Mixed precision" (main KV quantized after
RoPE); "SGLang and Miles Day-0 support for DeepSeek-V4.1", section 1 (incomplete pairs are
kept across decode steps) and section 5 (BF16 projection weights with FP32 accumulation;
ratio-2 pooling of each completed pair; RoPE, FP4 quantization and cache write fused
without changing the intermediate rounding).

Pins, each against numpy float64 arithmetic written here from the definitions, not the
oracle's fp32 steps:
  * bf16 main KV = the RoPE'd mean of each completed pair (m = 2) or the token itself
    (m = 1), rotated in interleaved pairs over the last 64 dims at the group's last
    position, within bf16 rounding;
  * the MXFP4 index key dequantizes to W . bf16(latent), rotated the same way on its last
    64 dims, within the MXFP4 rounding bound of its block;
  * the FP4 main KV dequantizes to the same RoPE'd latent within its block's scale;
  * splitting the token stream into calls of any size (decode steps, odd chunks) gives the
    same caches and the same pending state: incomplete pairs wait for their partner;
  * rows that complete no entry leave the cache untouched.
"""
import numpy as np
import pytest

KV, IDX, ROPE = 512, 128, 64
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _rope_table(max_pos, base=10000.0):
    i = np.arange(ROPE // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * i / ROPE)[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32), ang


def _bf16(x):
    """float64 -> nearest-even bf16 values (float64)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def _rotate(v, table, P):
    """float64 rotation of the last 64 dims in interleaved pairs with the table's values."""
    v = v.astype(np.float64).copy()
    c = table[P, 0].astype(np.float64)
    s = table[P, 1].astype(np.float64)
    a, b = v[-ROPE::2].copy(), v[-ROPE + 1::2].copy()
    v[-ROPE::2] = a * c - b * s
    v[-ROPE + 1::2] = a * s + b * c
    return v


def _case(seed, lens, m, prefix=None):
    """Token rows of one call: request r covers positions [prefix_r, prefix_r + len_r)."""
    rng = np.random.default_rng(seed)
    prefix = prefix or [0] * len(lens)
    req = np.concatenate([np.full(L, r) for r, L in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(p0, p0 + L) for p0, L in zip(prefix, lens)]).astype(np.int32)
    comp = rng.standard_normal((len(req), KV)).astype(np.float32)
    w = rng.standard_normal((IDX, KV)).astype(np.float32) * 0.05
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)          # truncate to bf16 patterns
    ends = [p0 + L for p0, L in zip(prefix, lens)]
    n_ent = [e // m for e in ends]
    row_start = np.cumsum([0] + n_ent[:-1]).astype(np.int64)
    return dict(req_of_row=req, pos_of_row=pos), comp, wb, row_start, int(sum(n_ent))


def _wfloat(wb):
    return (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("m", [1, 2])
def test_bf16_main_kv_is_rope_of_pooled_latent(orc, m):
    rows, comp, wb, rs, nrows = _case(1, [37, 20], m)
    table, _ = _rope_table(64)
    out = orc.kv_produce(rows, m, rs, nrows, comp, np.zeros((2, KV), np.float32), wb, table, kv_dt=orc.DT_BF16)
    kv = (out["kv"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r, L in enumerate([37, 20]):
        base = 0 if r == 0 else 37
        for j in range(L // m):
            toks = comp[base + j * m: base + j * m + m].astype(np.float64)
            ref = _rotate(toks.mean(axis=0), table, j * m + m - 1)
            got = kv[rs[r] + j]
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6), (r, j)
        # the lone last token of an odd-length request (m = 2) produced nothing
        if m == 2 and L % 2:
            assert np.array_equal(out["pending"][r], comp[base + L - 1])


def test_rope_position_and_pairing_matter(orc):
    """The same latent at two different entry positions gives different rotations, and the
    first 448 dims are never rotated."""
    rows, comp, wb, rs, nrows = _case(2, [8], 2)
    table, _ = _rope_table(16)
    out = orc.kv_produce(rows, 2, rs, nrows, comp, np.zeros((1, KV), np.float32), wb, table, kv_dt=orc.DT_BF16)
    kv = (out["kv"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for j in range(4):
        mean = comp[2 * j: 2 * j + 2].astype(np.float64).mean(axis=0)
        assert np.array_equal(kv[j, :KV - ROPE], _bf16(mean[:KV - ROPE]))
        wrong_pos = _rotate(mean, table, 2 * j)                 # the group's first position
        right = _rotate(mean, table, 2 * j + 1)
        assert np.max(np.abs(kv[j] - right)) < np.max(np.abs(kv[j] - wrong_pos))


def test_index_key_is_rope_of_projection(orc):
    rows, comp, wb, rs, nrows = _case(3, [30, 11], 2)
    table, _ = _rope_table(64)
    out = orc.kv_produce(rows, 2, rs, nrows, comp, np.zeros((2, KV), np.float32), wb, table)
    codes, scales = out["index_codes"], out["index_scales"]
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(nrows, IDX)
    val = np.where(c & 8, -1.0, 1.0) * E2M1[c & 7] * np.exp2(np.repeat(scales.astype(np.float64) - 127, 32, axis=1))
    W = _wfloat(wb)
    refs, got = [], []
    for r, L in enumerate([30, 11]):
        base = 0 if r == 0 else 30
        for j in range(L // 2):
            latent = comp[base + 2 * j: base + 2 * j + 2].astype(np.float64).mean(axis=0)
            k = _rotate(W @ _bf16(latent), table, 2 * j + 1)
            e = np.repeat(scales[rs[r] + j].astype(np.float64) - 127, 32)
            assert np.all(np.abs(val[rs[r] + j] - k) <= np.exp2(e + 1) * 1.0001), (r, j)
            refs.append(k)
            got.append(rs[r] + j)
    # and the codes are those of the float64 key, except where fp32 accumulation moved a
    # value across a rounding boundary (rare)
    rc, rsc = orc.mx_quant(orc.E2M1, np.array(refs, np.float32))
    assert np.mean(rsc == scales[got]) > 0.98
    assert np.mean(rc == codes[got]) > 0.99


def test_fp4_main_kv_within_block_scale(orc):
    rows, comp, wb, rs, nrows = _case(4, [24], 2)
    table, _ = _rope_table(32)
    out = orc.kv_produce(rows, 2, rs, nrows, comp, np.zeros((1, KV), np.float32), wb, table)
    deq = orc.fp4s16_dequant(out["kv"], out["kv_scale"])
    s = np.repeat(np.array([orc.e4m3_value(int(b)) for b in out["kv_scale"].ravel()]).reshape(nrows, KV // 16), 16,
                  axis=1)
    for j in range(12):
        ref = _rotate(comp[2 * j: 2 * j + 2].astype(np.float64).mean(axis=0), table, 2 * j + 1)
        assert np.all(np.abs(deq[j] - ref) <= s[j] * 1.0001 + 1e-9), j


@pytest.mark.parametrize("kv_dt", ["fp4", "bf16"])
def test_call_split_invariance(orc, kv_dt):
    """One call over the whole stream == decode steps of one token == odd-sized chunks, for
    two interleaved requests; the pending state of a request left with an incomplete pair
    is the same too (for the others it holds a consumed token and is never read)."""
    dt = orc.DT_FP4S16 if kv_dt == "fp4" else orc.DT_BF16
    lens = [23, 16]
    rows, comp, wb, rs, nrows = _case(5, lens, 2)
    table, _ = _rope_table(64)
    whole = orc.kv_produce(rows, 2, rs, nrows, comp, np.zeros((2, KV), np.float32), wb, table, kv_dt=dt)
    starts = [0, lens[0]]
    for sizes in ([1] * 23, [3, 5, 1, 7, 2, 5]):
        pend = np.zeros((2, KV), np.float32)
        acc = None
        done = [0, 0]
        k = 0
        while done[0] < lens[0] or done[1] < lens[1]:
            step = sizes[k % len(sizes)]
            k += 1
            idx = []
            for r in (1, 0):            # request order inside a call does not matter
                take = min(step, lens[r] - done[r])
                idx += list(range(starts[r] + done[r], starts[r] + done[r] + take))
                done[r] += take
            if not idx:
                continue
            idx = np.array(idx)
            part = orc.kv_produce({k2: v[idx] for k2, v in rows.items()}, 2, rs, nrows, comp[idx], pend, wb, table,
                                  kv_dt=dt)
            pend = part["pending"]
            if acc is None:
                acc = part
            else:
                for name in ("kv", "kv_scale", "index_codes", "index_scales"):
                    if part[name] is None:
                        continue
                    fill = 0xEE if part[name].dtype == np.uint8 else 0xEEEE
                    written = np.any(part[name] != fill, axis=1)
                    acc[name][written] = part[name][written]
        for name in ("kv", "kv_scale", "index_codes", "index_scales"):
            if whole[name] is not None:
                assert np.array_equal(acc[name], whole[name]), (sizes, name)
        # pending is meaningful only for a request whose last pair is incomplete
        for r in range(2):
            if lens[r] % 2:
                assert np.array_equal(pend[r], whole["pending"][r])


def test_only_completed_groups_are_written(orc):
    """Rows [5, 9) of a request (m = 2): entries 2 and 3 complete (positions 5 and 7); the
    lone 8 waits in pending; entry 2 takes its first half (position 4) from pending."""
    rng = np.random.default_rng(6)
    comp = rng.standard_normal((4, KV)).astype(np.float32)
    pend = rng.standard_normal((1, KV)).astype(np.float32)
    wb = (rng.standard_normal((IDX, KV)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    table, _ = _rope_table(16)
    rows = dict(req_of_row=np.zeros(4, np.int32), pos_of_row=np.arange(5, 9, dtype=np.int32))
    out = orc.kv_produce(rows, 2, np.array([0]), 6, comp, pend, wb, table, kv_dt=orc.DT_BF16)
    written = np.any(out["kv"] != 0xEEEE, axis=1)
    assert written.tolist() == [False, False, True, True, False, False]
    kv = (out["kv"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref2 = _rotate((pend[0].astype(np.float64) + comp[0]) / 2, table, 5)
    assert np.all(np.abs(kv[2] - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-6)
    assert np.array_equal(out["pending"][0], comp[3])
