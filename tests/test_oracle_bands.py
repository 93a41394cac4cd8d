"""The band planner (page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs",
the bands section): the oracle's dependency-set `plan_band` against the
pages' own walk-back test, closed forms, and banded evaluation of a 1-D
integer decoder (bands computed from the planned rows only reproduce the
whole-frame rows exactly); then the library's interval planner against the
oracle's sets on random decoders."""

import json
import os
import random

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "band_walk_back_case.json")


def _levels(has_up):
    lvl, l = [], 0
    for u in has_up:
        lvl.append(l)
        l += 1 if u else 0
    return lvl, l


def test_walk_back_matches_the_pages_case():
    g = json.load(open(GOLDEN))
    inp, feed = O.plan_band(g["n_res"], g["has_up"], g["h0"], g["band_from"], tuple(g["keep"]))
    assert list(feed[0]) == g["expected_feed_block0"]
    assert list(inp) == g["expected_input"]
    # the clamp at the frame edge: three 3x3 convs (one resnet, then
    # conv_out) on a 12-row frame, keeping rows [0, 10), need all 12 rows
    e = g["edge_case"]
    inp, feed = O.plan_band([1], [0], e["h"], 0, tuple(e["rows"]))
    assert e["grow"] == 3 and list(inp) == e["expected"] and feed == {}


def test_plan_band_closed_forms():
    """Without upsamples the band grows by one row per 3x3 conv on each
    side, cut at the frame: [max(lo - n, 0), min(hi + n, h)) for n convs. An
    upsample then a 3x3 conv then conv_out (no resnets) needs
    [(lo - 2) // 2, (hi + 1) // 2 + 1) of the half-resolution rows, cut."""
    for h in (5, 9, 16):
        for n_res in (0, 1, 3):
            for lo in range(h):
                for hi in range(lo + 1, h + 1):
                    n = 2 * n_res + 1
                    inp, feed = O.plan_band([n_res], [0], h, 0, (lo, hi))
                    assert inp == (max(lo - n, 0), min(hi + n, h)) and feed == {}
    for h0 in (3, 8):
        for lo in range(2 * h0):
            for hi in range(lo + 1, 2 * h0 + 1):
                inp, feed = O.plan_band([0], [1], h0, 0, (lo, hi))
                want = (max((lo - 2) // 2, 0), min((hi + 1) // 2 + 1, h0))
                assert inp == want and feed == {0: want}


def _random_decoder(rng):
    n_up = rng.randint(1, 4)
    n_res = [rng.randint(0, 2) for _ in range(n_up)]
    has_up = [rng.random() < 0.7 for _ in range(n_up)]
    return n_res, has_up, rng.randint(3, 9)


def _conv3(x, taps):
    """3-tap conv along rows with zero padding, exact integers."""
    y = taps[1] * x
    y[1:] += taps[0] * x[:-1]
    y[:-1] += taps[2] * x[1:]
    return y


def _run_blocks(x, n_res, has_up, blocks, taps, feed=None, lo=0):
    """1-D stand-in for the decoder's up blocks on rows [lo, lo + len(x))
    of the level (integer taps; an upsample repeats rows)."""
    for i in blocks:
        for c in range(2 * n_res[i]):
            x = _conv3(x, taps[i][c])
        if has_up[i]:
            if feed is not None:
                f = feed[i]
                x = x[f[0] - lo:f[1] - lo]
                lo = f[0]
            x = _conv3(np.repeat(x, 2), taps[i][-1])
            lo *= 2
    return x, lo


def test_bands_from_the_planned_rows_reproduce_the_whole_frame():
    rng = random.Random(6)
    nprng = np.random.default_rng(6)
    for _ in range(200):
        n_res, has_up, h0 = _random_decoder(rng)
        lvl, lf = _levels(has_up)
        hf = h0 << lf
        s = rng.randint(0, len(n_res))
        taps = [[nprng.integers(-3, 4, 3) for _ in range(2 * n_res[i] + 1)] for i in range(len(n_res))]
        out_taps = nprng.integers(-3, 4, 3)
        hs = h0 << (lvl[s] if s < len(n_res) else lf)
        xs = nprng.integers(-9, 10, hs).astype(np.int64)  # block s's input, whole frame
        whole, _ = _run_blocks(xs.copy(), n_res, has_up, range(s, len(n_res)), taps)
        whole = _conv3(whole, out_taps)
        for _ in range(4):
            lo = rng.randrange(hf)
            keep = (lo, rng.randint(lo + 1, hf))
            inp, feed = O.plan_band(n_res, has_up, h0, s, keep)
            band, blo = _run_blocks(xs[inp[0]:inp[1]].copy(), n_res, has_up, range(s, len(n_res)), taps,
                                    feed, inp[0])
            band = _conv3(band, out_taps)
            got = band[keep[0] - blo:keep[1] - blo]
            assert np.array_equal(got, whole[keep[0]:keep[1]])


def test_library_band_planner_matches_the_oracle():
    ig = pytest.importorskip("implicit_gemm_conv_nhwc_amd")
    rng = random.Random(7)
    for _ in range(500):
        n_res, has_up, h0 = _random_decoder(rng)
        hf = h0 << sum(has_up)
        s = rng.randint(0, len(n_res))
        lo = rng.randrange(hf)
        keep = (lo, rng.randint(lo + 1, hf))
        inp, feed = O.plan_band(n_res, has_up, h0, s, keep)
        got_in, got_feed = ig.band_plan(n_res, has_up, h0, s, keep[0], keep[1])
        assert got_in == inp
        for i in range(len(n_res)):
            assert got_feed[i] == feed.get(i, (0, 0))
    # the pages' case through the library
    g = json.load(open(GOLDEN))
    got_in, got_feed = ig.band_plan(g["n_res"], g["has_up"], g["h0"], g["band_from"], *g["keep"])
    assert list(got_in) == g["expected_input"] and list(got_feed[0]) == g["expected_feed_block0"]


def test_library_band_planner_rejects_bad_rows():
    ig = pytest.importorskip("implicit_gemm_conv_nhwc_amd")
    with pytest.raises(ig.IgError):
        ig.band_plan([1], [1], 8, 0, 10, 10)  # empty keep
    with pytest.raises(ig.IgError):
        ig.band_plan([1], [1], 8, 0, 0, 17)  # past the 16-row frame
