"""Pins of the oracle's bounded-replay layouts (CPU only).

Every expected value comes from the worked examples of "SGLang: how DeepSeek V4.1
Flash late layers only process tail tokens" (lab.ttaoai.cn), of "SGLang and Miles Day-0
support for DeepSeek-V4.1" section 4 (encoder-side replay) and of "DeepSeek V4.1 Flash
modeling", section "Decoder Bounded Replay" (mixed batches), stored with their section
citations in tests/golden/replay_tail_examples.json; the rest are invariants that hold
for any batch.
"""
import json
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "replay_tail_examples.json")))


def test_single_8192_extend(orc):
    g = GOLD["single_8192"]
    t = orc.replay_tail_layout(g["ext_len"], g["seq_len"])
    assert t["tail_len"].tolist() == [128]
    assert t["abs_pos"][0] == g["tail_first"] and t["abs_pos"][-1] == g["tail_last"]
    assert np.all(t["win_lo"] == g["win_lo"])
    # rows keep their absolute positions and point at the matching extend rows
    assert t["src_row"].tolist() == list(range(8064, 8192))
    assert t["abs_pos"].tolist() == list(range(8064, 8192))


def test_window_table(orc):
    g = GOLD["window_table"]
    t = orc.replay_tail_layout([g["ext_len"]], [g["seq_len"]])
    W = g["window"]
    for row in g["rows"]:
        p = row["pos"]
        u = int(np.where(t["abs_pos"] == p)[0][0])
        lo = int(t["win_lo"][u])
        assert [max(0, p - W + 1), p] == row["normal"]
        assert [max(lo, p - W + 1), p] == row["bounded"]


def test_short_extend(orc):
    g = GOLD["short_extend"]
    t = orc.replay_tail_layout(g["ext_len"], g["seq_len"])
    assert t["tail_len"].tolist() == [g["tail_len"]]
    assert np.all(t["win_lo"] == g["win_lo"])
    first, last = int(t["abs_pos"][0]), int(t["abs_pos"][-1])
    assert [max(g["win_lo"], first - 127), first] == g["first_row_window"]
    assert [max(g["win_lo"], last - 127), last] == g["last_row_window"]
    a, b = g["invisible"]
    for p in t["abs_pos"]:
        assert max(g["win_lo"], int(p) - 127) > b  # cached 8128..8191 never visible


def test_chunked_32k(orc):
    g = GOLD["chunked_32k"]
    # each chunk is its own extend (one request per extend call)
    tails = []
    for e, s in zip(g["ext_len"], g["seq_len"]):
        t = orc.replay_tail_layout([e], [s])
        tails.append([int(t["abs_pos"][0]), int(t["abs_pos"][-1])])
    assert tails == g["tails"]
    # the same four extends batched as four requests: per-request tails, never a batch-wide 128
    t = orc.replay_tail_layout(g["ext_len"], g["seq_len"])
    assert int(t["tail_row_start"][-1]) == g["late_rows_total"]
    assert t["tail_row_start"].tolist() == [0, 128, 256, 384, 512]
    assert t["src_row"][128] == 8192 + 8064  # second request's extend rows start at 8192


@pytest.mark.parametrize("case", ["one_8192", "four_8k_chunks", "single_32k"])
def test_token_layer_counts(orc, case):
    g = GOLD["token_layer_counts"]
    c = g[case]
    rows_tail = 0
    for e in c["extends"]:
        t = orc.replay_tail_layout([e], [e])
        rows_tail += int(t["tail_row_start"][-1])
    total = g["layers_full"] * sum(c["extends"]) + g["layers_tail"] * rows_tail
    assert total == c["bounded"]
    if "full" in c:
        assert g["layers_total"] * sum(c["extends"]) * (1 if case == "one_8192" else 1) == c["full"]
    if "reduction_pct" in c:
        assert (c["full"] - total) / c["full"] * 100 == c["reduction_pct"]


def test_edge_lengths_and_mixed_batch(orc):
    ext = [0, 1, 127, 128, 129, 8192, 64]
    seq = [10, 50, 127, 1000, 129, 8192, 8256]
    t = orc.replay_tail_layout(ext, seq)
    assert t["tail_len"].tolist() == [0, 1, 127, 128, 128, 128, 64]
    starts = np.cumsum([0] + [0, 1, 127, 128, 128, 128, 64])
    assert t["tail_row_start"].tolist() == starts.tolist()
    ext_start = np.cumsum([0] + ext[:-1])
    for r in range(len(ext)):
        a, b = starts[r], starts[r + 1]
        T = b - a
        assert np.all(t["req_of_row"][a:b] == r)
        assert t["abs_pos"][a:b].tolist() == list(range(seq[r] - T, seq[r]))
        assert np.all(t["win_lo"][a:b] == seq[r] - T)
        assert t["src_row"][a:b].tolist() == list(range(ext_start[r] + ext[r] - T, ext_start[r] + ext[r]))


def test_precondition(orc):
    with pytest.raises(ValueError):
        orc.replay_tail_layout([10], [5])   # E > S


def test_mixed_batch_decode_rows_pass_whole(orc):
    """A decode request in a mixed batch keeps its new token(s) with an uncut window; the
    prefill requests beside it are cut as usual (golden: mixed_batch)."""
    g = GOLD["mixed_batch"]
    pf, dc = g["prefill"], g["decode"]
    ext = [pf["ext_len"], dc["ext_len"], 40, 3]
    seq = [pf["seq_len"], dc["seq_len"], 5000, 700]
    dec = [0, 1, 0, 1]
    t = orc.replay_tail_layout(ext, seq, is_decode=dec)
    s = t["tail_row_start"]
    assert t["tail_len"].tolist() == [128, 1, 40, 3]
    assert t["abs_pos"][s[0]:s[1]].tolist() == list(range(pf["tail"][0], pf["tail"][1] + 1))
    assert np.all(t["win_lo"][s[0]:s[1]] == pf["win_lo"])
    assert t["abs_pos"][s[1]:s[2]].tolist() == list(range(dc["rows"][0], dc["rows"][1] + 1))
    assert np.all(t["win_lo"][s[1]:s[2]] == dc["win_lo"])
    assert np.all(t["win_lo"][s[2]:s[3]] == 5000 - 40)          # a short prefill extend is still cut
    assert t["abs_pos"][s[3]:s[4]].tolist() == [697, 698, 699] and np.all(t["win_lo"][s[3]:s[4]] == 0)
    # every extend row of a decode request is kept, in order
    ext_start = np.cumsum([0] + ext[:-1])
    assert t["src_row"][s[1]:s[2]].tolist() == [ext_start[1]]
    assert t["src_row"][s[3]:s[4]].tolist() == list(range(ext_start[3], ext_start[3] + 3))
    # the same token as a one-token prefill extend would see only itself
    t1 = orc.replay_tail_layout([1], [9000])
    assert t1["win_lo"].tolist() == [8999]
    with pytest.raises(ValueError):
        orc.replay_tail_layout([200], [300], is_decode=[1])      # decode rows must fit the budget


def test_short_extend_borrowing_prefix_window(orc):
    """Reading of the short-extend proposal ([P2] section 2.6): with the flag the late
    layers' window of a 64-token extend after 8192 cached tokens starts at S - 128 = 8128,
    so the cached 8128..8191 become visible; extends of at least 128 are unchanged."""
    g = GOLD["short_extend"]
    t = orc.replay_tail_layout(g["ext_len"], g["seq_len"], borrow_prefix_window=True)
    assert t["tail_len"].tolist() == [g["tail_len"]]
    assert np.all(t["win_lo"] == g["invisible"][0])
    a = orc.replay_tail_layout([8192, 300, 20], [8192, 9000, 50], borrow_prefix_window=True)
    b = orc.replay_tail_layout([8192, 300, 20], [8192, 9000, 50])
    for key in ("abs_pos", "src_row", "req_of_row"):
        assert np.array_equal(a[key], b[key])
    assert a["win_lo"].tolist()[:256] == b["win_lo"].tolist()[:256]
    assert np.all(a["win_lo"][256:] == 0) and np.all(b["win_lo"][256:] == 30)


def test_encoder_replay_page_example(orc):
    """[P4] section 4.1: a prefix hit of 8192 cached tokens recomputes 8064..8191 before the
    100 new tokens; every row's window stops at the rebuild boundary 8064 (section 4.3)."""
    g = GOLD["encoder_replay_8192_hit"]
    t = orc.encoder_replay_layout([g["prefix_len"]], [g["ext_len"]])
    assert t["row_start"].tolist() == [0, g["rows"]]
    assert t["abs_pos"].tolist() == list(range(g["replay_first"], g["prefix_len"] + g["ext_len"]))
    assert np.all(t["win_lo"] == g["win_lo"])
    nrep = g["replay_last"] - g["replay_first"] + 1
    assert np.all(t["src_row"][:nrep] == -1) and t["src_row"][nrep:].tolist() == list(range(g["ext_len"]))


def test_encoder_replay_invariants(orc):
    """Per request: min(P, 128) replayed rows then E extend rows, contiguous absolute
    positions, no row below the boundary R0 = max(0, P - 128); the extend rows map one to
    one onto the flattened extend input in order; P = 0 is a plain prefill."""
    rng = np.random.default_rng(5)
    P = [0, 1, 127, 128, 129, 5000, 0, 40]
    E = [10, 0, 1, 200, 128, 3, 0, 7]
    t = orc.encoder_replay_layout(P, E)
    s = t["row_start"]
    ext_start = np.cumsum([0] + E[:-1])
    seen = []
    for r in range(len(P)):
        a, b = s[r], s[r + 1]
        rep = min(P[r], 128)
        assert b - a == rep + E[r]
        R0 = max(0, P[r] - 128)
        assert t["abs_pos"][a:b].tolist() == list(range(R0, P[r] + E[r]))
        assert np.all(t["win_lo"][a:b] == R0) and np.all(t["req_of_row"][a:b] == r)
        assert np.all(t["src_row"][a:a + rep] == -1)
        assert t["src_row"][a + rep:b].tolist() == list(range(ext_start[r], ext_start[r] + E[r]))
        seen += t["src_row"][a + rep:b].tolist()
    assert seen == list(range(sum(E)))
    p0 = orc.encoder_replay_layout([0], [50])
    assert p0["abs_pos"].tolist() == list(range(50)) and np.all(p0["win_lo"] == 0)
    assert p0["src_row"].tolist() == list(range(50))
    with pytest.raises(ValueError):
        orc.encoder_replay_layout([10, 10], [5, 5], capacity=20)
    del rng
