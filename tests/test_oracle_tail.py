"""Pins of the oracle's decoder bounded-replay tail layout (CPU only).

Every expected value comes from the worked examples of "SGLang: how DeepSeek V4.1
Flash late layers only process tail tokens" (lab.ttaoai.cn), stored with their
section citations in tests/golden/replay_tail_examples.json.
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
