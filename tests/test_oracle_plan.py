"""Pins of the oracle's plan (token counts, windows, cu_seqlens).

The plan is pinned three ways: the values the pages print
(tests/golden/pages_values.json), brute force against the output length of
torch's own Conv2d(3, stride 2, padding 1), and the closed form
13 * floor(L / 100) + ceil((L mod 100) / 8) (three ceiling halvings of r equal
ceil(r / 8)).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))
CFG = si.model_config("rag")


def torch_stem_len(h: int, w: int):
    """Output (H, W) of three stride-2 3x3 convolutions with padding 1, by
    running torch's conv2d on a zero image."""
    x = torch.zeros(1, 1, h, w, dtype=torch.float64)
    k = torch.zeros(1, 1, 3, 3, dtype=torch.float64)
    for _ in range(3):
        x = torch.nn.functional.conv2d(x, k, stride=2, padding=1)
    return x.shape[2], x.shape[3]


def test_page_values():
    assert oracle.chunk_frames(CFG) == GOLDEN["chunk_frames"]["value"]
    assert oracle.tokens_for_frames(100, CFG) == GOLDEN["tokens_per_full_chunk"]["value"]
    fb = CFG["num_mel_bins"]
    for _ in range(3):
        fb = oracle.conv_out_len(fb)
    assert fb == GOLDEN["mel_bins_after_stem"]["value"]
    assert oracle.window_tokens(CFG) == GOLDEN["window_tokens"]["value"]
    frames_8s = GOLDEN["window_seconds"]["value"] * 100
    assert oracle.tokens_for_frames(frames_8s, CFG) == GOLDEN["window_tokens"]["value"]
    d = GOLDEN["config_defaults"]["value"]
    assert 2 * d["n_window"] == GOLDEN["chunk_frames"]["value"]
    assert oracle.window_tokens(d) == 104


@pytest.mark.parametrize("r", range(0, 101))
def test_remainder_tokens_vs_torch_conv(r):
    # brute force: the time axis of a zero-padded-to-r image through torch's conv2d
    if r == 0:
        assert oracle.tokens_for_frames(0, CFG) == 0
        return
    h, w = torch_stem_len(128, r)
    assert h == 16
    assert oracle.tokens_for_frames(r, CFG) == w
    assert oracle.tokens_for_frames(r, CFG) == -(-r // 8)


@pytest.mark.parametrize("L", [0, 1, 7, 8, 9, 99, 100, 101, 799, 800, 801, 1737, 3000, 120000, 3499])
def test_closed_form(L):
    n = oracle.tokens_for_frames(L, CFG)
    assert n == 13 * (L // 100) + -(-(L % 100) // 8)
    wl = oracle.window_lengths(n, CFG)
    assert sum(wl) == n
    assert all(0 < x <= 104 for x in wl)
    assert all(x == 104 for x in wl[:-1])


def test_plan_invariants_all_workloads():
    for name in si.WORKLOADS:
        cfg = si.model_config(name)
        lens = si.feature_lens(name)
        pl = oracle.plan(lens, cfg)
        cu = pl["cu_seqlens"]
        assert cu[0] == 0 and cu[-1] == pl["total_tokens"]
        assert all(cu[i] < cu[i + 1] for i in range(len(cu) - 1))
        # windows never cross requests: every request's first row is a window start
        starts = np.cumsum([0] + pl["tokens_per_request"][:-1])
        assert set(int(s) for s in starts if s < cu[-1]).issubset(set(cu))
        # chunk table consistency
        assert sum(c[3] for c in pl["chunks"]) == pl["total_tokens"]
        for b, L in enumerate(lens):
            assert pl["tokens_per_request"][b] == 13 * (L // 100) + -(-(L % 100) // 8)


def test_known_workload_sizes():
    # 8 s -> one window of 104 (m-star summary); 1200 s -> 150 full windows
    pl = oracle.plan(si.feature_lens("tiny"), CFG)
    assert pl["cu_seqlens"] == [0, 104]
    pl = oracle.plan(si.feature_lens("long"), CFG)
    assert pl["total_tokens"] == 15600 and pl["window_lengths"] == [104] * 150
    # the ragged workload: per request 3 s, 8 s, 17.37 s, 30 s
    lens = si.feature_lens("rag")
    assert list(lens) == [300, 800, 1737, 3000]
    pl = oracle.plan(lens, CFG)
    toks = [13 * (L // 100) + -(-(L % 100) // 8) for L in lens]
    assert pl["tokens_per_request"] == toks
    wl = []
    for t in toks:
        wl += [104] * (t // 104) + ([t % 104] if t % 104 else [])
    assert pl["window_lengths"] == wl
    assert pl["cu_seqlens"] == list(np.cumsum([0] + wl))
    # the same values as literals, worked out by hand: 300 frames -> 39
    # tokens, 800 -> 104, 1737 -> 13 * 17 + ceil(37 / 8) = 226, 3000 -> 390;
    # windows 39 | 104 | 104, 104, 18 | 104, 104, 104, 78
    assert pl["tokens_per_request"] == [39, 104, 226, 390]
    assert pl["window_lengths"] == [39, 104, 104, 104, 18, 104, 104, 104, 78]
    assert pl["cu_seqlens"] == [0, 39, 143, 247, 351, 369, 473, 577, 681, 759]


def test_empty_requests_and_edges():
    pl = oracle.plan([0, 5, 0, 100, 0], CFG)
    assert pl["tokens_per_request"] == [0, 1, 0, 13, 0]
    assert pl["cu_seqlens"] == [0, 1, 14]
    pl = oracle.plan([0, 0], CFG)
    assert pl["cu_seqlens"] == [0] and pl["total_tokens"] == 0
    with pytest.raises(ValueError):
        oracle.plan([-1], CFG)
    bad = dict(CFG, n_window_infer=750)
    with pytest.raises(ValueError):
        oracle.window_tokens(bad)
