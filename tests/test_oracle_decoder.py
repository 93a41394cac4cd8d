"""The oracle's synthetic decoder: shapes, the guard's effect, and agreement
between its f16-emulating and pure-float64 modes. The pages print no decoder
output values; the composition itself (order, bias sites, shortcut, guard,
attention, DupUp, GroupNorm) is pinned in test_oracle_composition.py against
an independent float64 transcription of the recipe. These tests cover the
plumbing and the guard's behaviour (page "cortiq-engine 0.8.3,
src/gpu_wgpu/qi21_vae.rs", `guard`: unguarded f16 casts of a stream past the
f16 range turned most of an image into NaN)."""

import os
import sys

import numpy as np
import pytest

import oracle as O
import synth


def _small(gain=1.0):
    spec = synth.decoder_spec(small=True)
    return spec, synth.decoder_weights(spec, seed_config=4, conv_in_gain=gain)


def test_decoder_output_shape_and_range():
    spec, w = _small()
    z = synth.decoder_latent(4, 6, zc=spec.zc)
    y = O.decode(w, z, guard_log2=8, q_chunk=8)
    assert y.shape == (3, 32, 48)
    assert np.all(np.isfinite(y))
    # the f16 sites change the output only at the f16 rounding level
    y64 = O.decode(w, z, guard_log2=8, emulate_f16=False)
    assert O.psnr_u8(y, y64) > 45.0


def test_guard_keeps_a_large_stream_finite():
    spec, w = _small(gain=2.0 ** 11)
    z = synth.decoder_latent(4, 4, zc=spec.zc, scale=8.0)
    tr = O.Trace()
    y = O.decode(w, z, guard_log2=8, trace=tr)
    assert max(tr.guard_max) > 65504.0
    assert np.all(np.isfinite(y))
    y0 = O.decode(w, z, guard_log2=0)
    assert not np.all(np.isfinite(y0))


def test_guard_does_not_change_an_in_range_stream():
    spec, w = _small()
    z = synth.decoder_latent(4, 4, zc=spec.zc)
    tr = O.Trace()
    y8 = O.decode(w, z, guard_log2=8, trace=tr)
    assert max(tr.guard_max) < 2.0 ** 9
    # every guarded value sits in the f16 normal range for both g = 0 and
    # g = 8 except values below 2^-6, whose rounding differs slightly
    y0 = O.decode(w, z, guard_log2=0)
    assert O.psnr_u8(y0, y8) > 60.0


@pytest.mark.parametrize("size", [1024, 2048])
def test_stored_decode_rows_match_the_seeded_inputs(size):
    """The stored oracle rows of the full-size decode belong to the inputs the
    seeded generator draws today (a change to the generator would make them
    stale)."""
    import hashlib
    import json

    gdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    meta_path = os.path.join(gdir, "decode_%d_rows.json" % size)
    if not os.path.exists(meta_path):
        pytest.skip("no stored rows for %d^2" % size)
    sys.path.insert(0, gdir)
    import make_decode_golden as mg

    meta = json.load(open(meta_path))
    w, z = mg.inputs(size)
    assert meta["latent_digest"] == hashlib.sha256(z.tobytes()).hexdigest()[:16]
    assert meta["weights_digest"] == mg.weights_digest(w)
    assert max(meta["guard_max"]) > 65504.0
    with np.load(mg.golden_path(size)) as g:
        assert g["u8"].shape == (3, size // mg.STRIDE[size], size)
        assert g["f32"].shape == (3, size // (8 * mg.STRIDE[size]), size)
        assert np.array_equal(O.to_u8(g["f32"]), g["u8"][:, ::8, :].astype(np.float64))
