"""decoder_forward against the oracle's decoder on the same seeded weights
and latents: u8 PSNR >= 60 dB over the whole frame, plus the guard's effect
on a stream past the f16 range, query-chunk invariance and the workspace
contract."""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_nhwc_amd as ig
import oracle as O
import synth
from gpu_util import dev, host, nan_f32

pytestmark = pytest.mark.gpu

PSNR_MIN = 60.0


def _run(dd, z, guard_log2=8, q_chunk=0):
    zc, h0, w0 = z.shape
    out = dd.forward(dev(z), h0, w0, guard_log2=guard_log2, q_chunk=q_chunk)
    return host(out)


def _report(tag, got, ref):
    p = O.psnr_u8(got, ref)
    d = float(np.max(np.abs(got - ref)))
    clip = float(np.mean(np.abs(ref) > 1.0))
    print("%s: PSNR %.2f dB, max|d| %.3e, clipped %.3f" % (tag, p, d, clip), flush=True)
    return p


@pytest.mark.parametrize("h0,w0,q_chunk", [(4, 4, 0), (5, 7, 8), (8, 8, 24)])
def test_small_decoder(h0, w0, q_chunk):
    spec = synth.decoder_spec(small=True)
    w = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(h0, w0, zc=spec.zc)
    dd = ig.DeviceDecoder(w)
    got = _run(dd, z, q_chunk=q_chunk)
    ref = O.decode(w, z, guard_log2=8, q_chunk=q_chunk or None)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert _report("small %dx%d" % (h0, w0), got, ref) >= PSNR_MIN


@pytest.fixture(scope="module")
def full_decoder():
    spec = synth.decoder_spec()
    w = synth.decoder_weights(spec, seed_config=4)
    return w, ig.DeviceDecoder(w)


def test_config4_decode_256(full_decoder):
    w, dd = full_decoder
    z = synth.decoder_latent(32, 32, config=4)
    got = _run(dd, z, q_chunk=256)
    assert got.shape == (3, 256, 256)
    ref = O.decode(w, z, guard_log2=8, q_chunk=256)
    assert _report("config4 256^2", got, ref) >= PSNR_MIN


def test_decode_query_chunks_agree(full_decoder):
    _, dd = full_decoder
    z = synth.decoder_latent(32, 32, config=4)
    a = _run(dd, z, q_chunk=256)
    b = _run(dd, z, q_chunk=1024)
    c = _run(dd, z, q_chunk=100)
    # rows are independent: the chunking changes nothing
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_guard_on_a_stream_past_f16():
    spec = synth.decoder_spec()
    w = synth.decoder_weights(spec, seed_config=4, conv_in_gain=2.0 ** 11)
    z = synth.decoder_latent(16, 16, config=5, scale=8.0)
    dd = ig.DeviceDecoder(w)
    got = _run(dd, z, guard_log2=8)
    tr = O.Trace()
    ref = O.decode(w, z, guard_log2=8, trace=tr)
    print("stream max at guarded casts:", ["%.3g" % v for v in tr.guard_max])
    assert max(tr.guard_max) > 65504.0
    assert np.all(np.isfinite(got))
    assert _report("guarded 128^2", got, ref) >= PSNR_MIN
    # without the guard the f16 casts overflow, as the pages report
    bad = _run(dd, z, guard_log2=0)
    assert not np.all(np.isfinite(bad))


def test_workspace_too_small_leaves_output_untouched(full_decoder):
    _, dd = full_decoder
    z = dev(synth.decoder_latent(32, 32, config=4))
    need = dd.workspace_bytes(32, 32)
    ws = torch.empty(need // 2, dtype=torch.uint8, device="cuda")
    out = nan_f32((3, 256, 256))
    with pytest.raises(ig.IgError) as e:
        ig.decoder_forward(dd.desc, z, 32, 32, 8, 0, ws, need // 2, out)
    assert e.value.code == -3
    assert torch.isnan(out).all()
