"""decoder_forward against the oracle's decoder on the same seeded weights
and latents: u8 PSNR >= 60 dB over the whole frame, plus the guard's effect
on a stream past the f16 range, query-chunk invariance and the workspace
contract."""

import os
import sys

import numpy as np
import pytest
import torch

import implicit_gemm_conv_nhwc_amd as ig
import oracle as O
import synth
from gpu_util import dev, host, nan_f32

pytestmark = pytest.mark.gpu

PSNR_MIN = 60.0
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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


def test_decoder_256_wide_attention_pairs_q_and_k():
    """A decoder 256 channels wide at the latent: the attention's Q and K
    then come from one GEMM launch over both weight planes (each half one
    256-column tile), here on a ragged 6x10 latent (60 tokens)."""
    spec = synth.DecoderSpec(zc=4, c_in=256, stages=(256, 128, 64), n_res=1, out_c=3)
    w = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(6, 10, zc=spec.zc)
    got = _run(ig.DeviceDecoder(w), z)
    ref = O.decode(w, z, guard_log2=8)
    assert got.shape == ref.shape == (3, 48, 80)
    assert np.all(np.isfinite(got))
    assert _report("256-wide 6x10", got, ref) >= PSNR_MIN


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


def test_full_decoder_non_square_ragged(full_decoder):
    """The full-width decoder on a 20x28 latent (a 160x224 frame): ragged
    tiles at every level, 560 attention tokens (a partial key block), the
    single-pass attention, against the oracle's decode."""
    w, dd = full_decoder
    z = synth.decoder_latent(20, 28, config=4)
    got = _run(dd, z, q_chunk=0)
    assert got.shape == (3, 160, 224)
    ref = O.decode(w, z, guard_log2=8, q_chunk=None)
    assert np.all(np.isfinite(got))
    assert _report("full decoder 20x28", got, ref) >= PSNR_MIN


def test_config4_decode_256_single_pass_attention(full_decoder):
    w, dd = full_decoder
    z = synth.decoder_latent(32, 32, config=4)
    got = _run(dd, z, q_chunk=0)
    ref = O.decode(w, z, guard_log2=8, q_chunk=256)
    assert _report("config4 256^2, single-pass attention", got, ref) >= PSNR_MIN
    chunked = _run(dd, z, q_chunk=256)
    assert _report("single-pass vs chunked attention", got, chunked) >= PSNR_MIN


def test_decode_query_chunks_agree(full_decoder):
    _, dd = full_decoder
    z = synth.decoder_latent(32, 32, config=4)
    a = _run(dd, z, q_chunk=256)
    b = _run(dd, z, q_chunk=1024)
    c = _run(dd, z, q_chunk=100)
    # rows are independent: the chunking changes nothing
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("band_rows,band_from", [(64, 0), (94, 1), (100, 2), (37, 2), (256, 1), (8, 2)])
def test_banded_decode_is_bit_identical(full_decoder, band_rows, band_from):
    """Bands with exact halos (the pages' bands section): every kept row is
    computed by the same kernels on the same inputs as in the whole frame,
    so the banded output equals the whole-frame output bit for bit."""
    _, dd = full_decoder
    z = dev(synth.decoder_latent(32, 32, config=4))
    whole = dd.forward(z, 32, 32, q_chunk=0)
    banded = dd.forward_bands(z, 32, 32, band_rows, band_from, q_chunk=0)
    torch.cuda.synchronize()
    d = float((banded - whole).abs().max())
    print("bands of %d rows from block %d: max|d| %g" % (band_rows, band_from, d), flush=True)
    assert torch.equal(banded, whole)


def test_banded_decode_small_decoder_and_frame_edges():
    spec = synth.decoder_spec(small=True)
    w = synth.decoder_weights(spec, seed_config=4)
    dd = ig.DeviceDecoder(w)
    z = dev(synth.decoder_latent(5, 7, zc=spec.zc))
    whole = dd.forward(z, 5, 7, q_chunk=8)
    H = 5 << dd.n_up
    for band_rows in (1, 3, H - 1, H):
        for band_from in range(len(w["ups"])):
            banded = dd.forward_bands(z, 5, 7, band_rows, band_from, q_chunk=8)
            assert torch.equal(banded, whole), (band_rows, band_from)


def test_banded_workspace_is_bounded(full_decoder):
    _, dd = full_decoder
    whole = ig.decoder_workspace_bytes(dd.desc, 128, 128, 0)
    banded = ig.decoder_bands_workspace_bytes(dd.desc, 128, 128, 0, 128, 2)
    print("1024^2 workspace: whole %.2f GB, bands of 128 rows from block 2 %.2f GB" % (whole / 1e9, banded / 1e9))
    assert banded < whole


def test_banded_decode_full_size_1024(full_decoder):
    w, dd = full_decoder
    z = dev(synth.decoder_latent(128, 128, config=5, scale=8.0))
    whole = dd.forward(z, 128, 128, q_chunk=0)
    banded = dd.forward_bands(z, 128, 128, 373, 1, q_chunk=0)
    torch.cuda.synchronize()
    assert torch.equal(banded, whole)


@pytest.mark.parametrize("small,h0,w0,dupup", [(True, 8, 8, True), (False, 16, 16, False)])
def test_decode_replays_from_a_captured_graph(small, h0, w0, dupup):
    """decoder_forward allocates nothing, synchronises nothing and enqueues
    only kernels and device-to-device copies on its stream, so a caller can
    capture a decode into a HIP graph (torch.cuda.CUDAGraph) and replay it.
    Each replay, with new latents copied into the captured input and eager
    decodes on the same workspace between replays, equals the eager decode
    of that latent bit for bit."""
    spec = synth.decoder_spec(small=small, dupup=dupup)
    dd = ig.DeviceDecoder(synth.decoder_weights(spec, seed_config=4))
    ws = dd.alloc_workspace(h0, w0, 0)
    zs = [dev(synth.decoder_latent(h0, w0, zc=spec.zc, config=4 + i)) for i in range(3)]
    refs = [dd.forward(z, h0, w0, ws=ws).clone() for z in zs]
    zin = torch.empty_like(zs[0])
    out = torch.empty_like(refs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        zin.copy_(zs[0])
        dd.forward(zin, h0, w0, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dd.forward(zin, h0, w0, ws=ws, out=out)
    for i in (1, 0, 2, 1):
        zin.copy_(zs[i])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[i]), i
        other = dd.forward(zs[(i + 1) % 3], h0, w0, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, refs[(i + 1) % 3])
    print("graph replays equal the eager decodes (%s %dx%d)" % ("small" if small else "full", h0, w0), flush=True)


@pytest.mark.parametrize("small,h0,w0", [(True, 5, 7), (True, 8, 8), (False, 32, 32)])
def test_decoder_with_dupup(small, h0, w0):
    """Every up stage adds the DupUp shortcut of its input (the pages'
    `run_blocks`): stage widths (in, out) = (c, c) take repeats 4 and
    (2c, c) repeats 2; the last stage's norm_out is not fused into its up
    conv then. Against the oracle's decode, and banded == whole."""
    spec = synth.decoder_spec(small=small, dupup=True)
    w = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(h0, w0, zc=spec.zc, config=4)
    dd = ig.DeviceDecoder(w)
    qc = 8 if small else 256
    got = _run(dd, z, q_chunk=qc)
    ref = O.decode(w, z, guard_log2=8, q_chunk=qc)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert _report("DupUp %s %dx%d" % ("small" if small else "full", h0, w0), got, ref) >= PSNR_MIN
    zd = dev(z)
    whole = dd.forward(zd, h0, w0, q_chunk=qc)
    H = h0 << dd.n_up
    for band_rows, band_from in ((3, 0), (H // 3 + 1, 1), (H - 1, 2)):
        banded = dd.forward_bands(zd, h0, w0, band_rows, band_from, q_chunk=qc)
        assert torch.equal(banded, whole), (band_rows, band_from)


@pytest.mark.parametrize("small,h0,w0,dupup", [(True, 5, 7, False), (True, 8, 8, True), (False, 32, 32, False)])
def test_group_norm_decoder(small, h0, w0, dupup):
    """A FLUX-class decoder: GroupNorm(32, 1e-6) with betas at every norm
    site instead of RMS_norm (the conv kernels unchanged; the epilogue norm
    fusions are off, GroupNorm needs the frame's statistics). Against the
    oracle's decode of the same weights."""
    spec = synth.decoder_spec(small=small, dupup=dupup, norm="group")
    w = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(h0, w0, zc=spec.zc, config=4)
    dd = ig.DeviceDecoder(w)
    qc = 8 if small else 256
    got = _run(dd, z, q_chunk=qc)
    ref = O.decode(w, z, guard_log2=8, q_chunk=qc)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert _report("GroupNorm %s %dx%d%s" % ("small" if small else "full", h0, w0, " + DupUp" if dupup else ""),
                   got, ref) >= PSNR_MIN


def test_group_norm_decoder_refuses_bands():
    spec = synth.decoder_spec(small=True, norm="group")
    dd = ig.DeviceDecoder(synth.decoder_weights(spec, seed_config=4))
    with pytest.raises(ig.IgError) as e:
        dd.forward_bands(dev(synth.decoder_latent(4, 4, zc=spec.zc)), 4, 4, 8, 1, q_chunk=8)
    assert "GroupNorm" in str(e.value)


def test_decode_4096_in_bands_with_dupup():
    """A 4096x4096 frame (latent 512x512, 262144 attention tokens), the
    DupUp decoder with the guarded stream: up block 0 on the whole frame,
    the rest in bands (the pages' large-frame path). Two band sizes give the
    same frame bit for bit, and it is finite. No oracle at this size."""
    spec = synth.decoder_spec(dupup=True)
    w = synth.decoder_weights(spec, seed_config=4, conv_in_gain=2.0 ** 11)
    dd = ig.DeviceDecoder(w)
    z = dev(synth.decoder_latent(512, 512, zc=spec.zc, config=5, scale=8.0))
    a = dd.forward_bands(z, 512, 512, 373, 1, q_chunk=0)
    b = dd.forward_bands(z, 512, 512, 1024, 1, q_chunk=0)
    torch.cuda.synchronize()
    assert a.shape == (3, 4096, 4096)
    assert bool(torch.isfinite(a).all())
    d = float((a - b).abs().max())
    print("4096^2 in bands of 373 and 1024 rows: max|d| %g, mean |x| %.3f" % (d, float(a.abs().mean())), flush=True)
    assert torch.equal(a, b)


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


def _load_golden(size, norm="rms"):
    sys.path.insert(0, GOLDEN)
    import make_decode_golden as mg

    path = mg.golden_path(size, norm)
    if not os.path.exists(path):
        pytest.skip("no stored oracle rows for %d^2 (tests/golden/make_decode_golden.py)" % size)
    with np.load(path) as g:
        return mg, {k: g[k] for k in g.files}


@pytest.mark.parametrize("size,q_chunk,norm", [(1024, 0, "rms"), (1024, 16384, "rms"), (2048, 0, "rms"),
                                             (1024, 0, "group")])
def test_full_size_decode_against_stored_oracle_rows(size, q_chunk, norm):
    """The full-size decode, launched as the benchmark launches it (guard 8,
    latent N(0,1)*8, conv_in gain 2^11; q_chunk 0 = the single-pass
    attention, > 0 = the chunked path), against the oracle's stored rows:
    u8 PSNR >= 60 dB over every sampled row, plus the float rows' max |d|
    relative to their RMS (reported). norm "group": the GroupNorm decoder of
    the same seeds, its norms from the statistics the convs gather."""
    mg, g = _load_golden(size, norm)
    w, z = mg.inputs(size, norm)
    assert float(np.max(g["guard_max"])) > 65504.0  # the guard is exercised
    dd = ig.DeviceDecoder(w)
    h0 = size // 8
    out = dd.forward(dev(z), h0, h0, guard_log2=mg.GUARD_LOG2, q_chunk=q_chunk)
    rows = torch.from_numpy(g["rows"].astype(np.int64)).cuda()
    frows = torch.from_numpy(g["frows"].astype(np.int64)).cuda()
    got_rows = host(out.index_select(1, rows))
    got_f = host(out.index_select(1, frows))
    assert bool(torch.isfinite(out).all())
    del out, dd
    torch.cuda.empty_cache()
    d = O.to_u8(got_rows) - g["u8"].astype(np.float64)
    mse = float(np.mean(d * d))
    p = float("inf") if mse == 0 else 10.0 * np.log10(255.0 ** 2 / mse)
    ref_f = g["f32"].astype(np.float64)
    unclipped = np.abs(ref_f) <= 1.0
    p_unclipped = O.psnr_u8(got_f[unclipped], ref_f[unclipped])
    rel = float(np.max(np.abs(got_f - ref_f)) / np.sqrt(np.mean(ref_f ** 2)))
    print("%d^2 %s (q_chunk %d): sampled-row PSNR %.2f dB (unclipped float rows %.2f dB), max|d|/RMS %.3e, "
          "u8 levels off: %d of %d" % (size, norm, q_chunk, p, p_unclipped, rel, int(np.count_nonzero(d)), d.size),
          flush=True)
    assert p >= PSNR_MIN
    assert p_unclipped >= PSNR_MIN
