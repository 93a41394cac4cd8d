"""The band planner (page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs",
the bands section): the oracle's `plan_band` against the pages' own
walk-back test, against an exact backward dependency analysis, and against
banded evaluation of a 1-D integer decoder (bands computed from the planned
rows only reproduce the whole-frame rows exactly); then the library's host
planner against the oracle's on random decoders."""

import json
import os
import random

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "band_walk_back_case.json")


def test_walk_back_matches_the_pages_case():
    g = json.load(open(GOLDEN))
    inp, feed = O.plan_band(g["n_res"], g["has_up"], g["h0"], g["band_from"], tuple(g["keep"]))
    assert list(feed[0]) == g["expected_feed_block0"]
    assert list(inp) == g["expected_input"]
    e = g["edge_case"]
    assert list(O.rows_grow(e["rows"][0], e["rows"][1], e["grow"], e["h"])) == e["expected"]


def test_half_rounds_outward():
    # output row r of a 2x upsample reads input row r // 2
    for lo in range(0, 9):
        for hi in range(lo + 1, 12):
            need = {r // 2 for r in range(lo, hi)}
            assert O.rows_half(lo, hi) == (min(need), max(need) + 1)


def _levels(has_up):
    lvl, l = [], 0
    for u in has_up:
        lvl.append(l)
        l += 1 if u else 0
    return lvl, l


def _needed(n_res, has_up, h0, band_from, keep):
    """Exact backward dependency as sets of rows."""
    lvl, lf = _levels(has_up)

    def conv_back(rows, h):
        return {r + d for r in rows for d in (-1, 0, 1) if 0 <= r + d < h}

    rows = conv_back(set(range(*keep)), h0 << lf)
    feed = {}
    for i in range(len(n_res) - 1, band_from - 1, -1):
        if has_up[i]:
            rows = {r // 2 for r in conv_back(rows, h0 << (lvl[i] + 1))}
            feed[i] = rows
        for _ in range(2 * n_res[i]):
            rows = conv_back(rows, h0 << lvl[i])
    return rows, feed


def _random_decoder(rng):
    n_up = rng.randint(1, 4)
    n_res = [rng.randint(0, 2) for _ in range(n_up)]
    has_up = [rng.random() < 0.7 for _ in range(n_up)]
    return n_res, has_up, rng.randint(3, 9)


def test_plan_band_equals_exact_dependencies():
    rng = random.Random(5)
    for _ in range(300):
        n_res, has_up, h0 = _random_decoder(rng)
        hf = h0 << sum(has_up)
        s = rng.randint(0, len(n_res))
        lo = rng.randrange(hf)
        keep = (lo, rng.randint(lo + 1, hf))
        inp, feed = O.plan_band(n_res, has_up, h0, s, keep)
        rows, need_feed = _needed(n_res, has_up, h0, s, keep)
        assert (min(rows), max(rows) + 1) == inp
        assert sorted(feed) == sorted(need_feed)
        for i, f in feed.items():
            assert (min(need_feed[i]), max(need_feed[i]) + 1) == f


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
