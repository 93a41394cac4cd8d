"""Pins of oracle.dupup, the DupUp shortcut of an up stage (page
"cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs", DUPUP_SRC and `run_blocks`),
against library routines that reach the same map another way (CPU only):

* in = out channels (repeats 4): every output channel reads its own
  channel at the source pixel -- the nearest 2x upsample (F.interpolate);
* in = 4 out (repeats 1): channel 4 o + 2 sy + sx goes to sub-pixel
  (sy, sx) of channel o -- depth-to-space (F.pixel_shuffle);
* in = 2 out (repeats 2): the channels repeated twice, then depth-to-space
  (Tensor.repeat_interleave, F.pixel_shuffle);
* a temporal factor ft > 1: the repeated channels grouped as
  [out][ft][4], chunk ft - 1 taken, then depth-to-space.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth


def _src(cin, h=3, w=5, idx=0):
    return synth.normal(7, idx, (cin, h, w), 1.0, np.float64)


def _shuffle(src, cout, ft=1):
    t = torch.from_numpy(src)
    cin, h, w = t.shape
    rep = cout * 4 * ft // cin
    e = t.repeat_interleave(rep, dim=0).reshape(cout, ft, 4, h, w)[:, ft - 1]
    return F.pixel_shuffle(e.reshape(1, 4 * cout, h, w), 2)[0].numpy()


def test_same_width_is_the_nearest_upsample():
    src = _src(8)
    want = F.interpolate(torch.from_numpy(src)[None], scale_factor=2, mode="nearest")[0].numpy()
    assert np.array_equal(O.dupup(src, 8), want)


def test_four_times_wider_input_is_depth_to_space():
    src = _src(16, idx=1)
    want = F.pixel_shuffle(torch.from_numpy(src)[None], 2)[0].numpy()
    assert np.array_equal(O.dupup(src, 4), want)


@pytest.mark.parametrize("cin,cout", [(8, 4), (128, 64), (512, 256)])
def test_twice_wider_input_repeats_then_moves_to_space(cin, cout):
    src = _src(cin, idx=2)
    got = O.dupup(src, cout)
    assert np.array_equal(got, _shuffle(src, cout))
    # spelled out for one pixel: output channel o at sub-pixel (sy, sx)
    # reads channel 2 o + sy (the repeat pairs sx = 0 and sx = 1)
    for o in (0, cout - 1):
        for sy in (0, 1):
            for sx in (0, 1):
                assert got[o, 2 * 1 + sy, 2 * 2 + sx] == src[2 * o + sy, 1, 2]


@pytest.mark.parametrize("cin,cout,ft", [(8, 4, 2), (4, 4, 2), (12, 3, 2)])
def test_temporal_factor_takes_its_chunk(cin, cout, ft):
    src = _src(cin, idx=3)
    assert np.array_equal(O.dupup(src, cout, ft), _shuffle(src, cout, ft))


def test_a_non_integer_repeat_is_refused():
    with pytest.raises(AssertionError):
        O.dupup(_src(12), 5)
