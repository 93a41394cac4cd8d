"""Per-kernel parity of the HIP path against the CPU oracle, through the C
ABI, on the seeded inputs of the per-kernel configurations (and smaller,
ragged and padded shapes). Every output buffer starts as NaN so a test
also proves the kernel wrote every element it owns."""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_nhwc_amd as ig
import oracle as O
import synth
from gpu_util import (CONV_TOL, conv_err, cpad, dev, f16_ulps, host, nan_f16, nan_f32,
                      nhwc_to_chw, packed, pad_last, padded_vec, sample_pixels)

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    print("device:", torch.cuda.get_device_name(0), flush=True)


# ---------------------------------------------------------------------------
# weight packing (a layout: exact)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cout,cin,k", [(128, 128, 3), (3, 128, 3), (288, 288, 3), (256, 512, 1)])
def test_pack_weights_layout(cout, cin, k):
    w = synth.normal(9, 1, (cout, cin, k, k), 1.0, np.float16)
    plane = host(packed(w)).reshape(-1)
    full = np.zeros((cpad(cout), cpad(cin), k * k), np.float16)
    full[:cout, :cin] = w.reshape(cout, cin, k * k)
    if k == 1:  # [cout_p][cin_p]
        want = full[:, :, 0]
    else:  # [cin_p/16][9][cout_p][16]
        want = full.reshape(cpad(cout), cpad(cin) // 16, 16, 9).transpose(1, 3, 0, 2)
    assert np.array_equal(plane.view(np.uint16), np.ascontiguousarray(want).reshape(-1).view(np.uint16))


# ---------------------------------------------------------------------------
# RMS_norm
# ---------------------------------------------------------------------------


def _norm_case(x_nhwc, gamma, c_real, cp, bias=None, silu=True):
    H, W, _ = x_nhwc.shape
    M = H * W
    xd = dev(pad_last(x_nhwc.reshape(M, -1), cp))
    g = padded_vec(gamma, cp)
    b = padded_vec(bias, cp) if bias is not None else None
    y = nan_f16((M, cp))
    ig.rmsnorm_silu_f16(xd, M, cp, c_real, b, g, int(silu), 1e-12, y)
    got = host(y)
    ref = O.f16(O.rmsnorm(x_nhwc.reshape(M, -1).T, gamma, bias=bias, silu=silu)).T
    return got, ref


def _assert_f16_close(got_real, ref):
    u = f16_ulps(got_real, ref.astype(np.float16))
    assert np.max(u) <= 1, "max ulp %d" % np.max(u)
    exact = float(np.mean(u == 0))
    assert exact >= 0.999, "exact fraction %.5f" % exact
    return exact


def test_rmsnorm_config1():
    d = synth.config1()
    got, ref = _norm_case(d["x"], d["gamma"], 128, 128)
    assert not np.isnan(got).any()
    _assert_f16_close(got, ref)


@pytest.mark.parametrize("c,cp,with_bias,silu", [(288, 320, True, True), (144, 192, False, True),
                                                 (128, 128, True, False), (64, 64, True, True),
                                                 (512, 512, False, True), (576, 576, True, True),
                                                 (700, 768, True, True), (1000, 1024, True, False)])
def test_rmsnorm_widths_bias_padding(c, cp, with_bias, silu):
    H, W = 7, 9  # M = 63, not a multiple of the 16-pixel block
    x = synth.normal(11, c, (H, W, c), 4.0)
    gamma = synth.uniform(11, c + 1, (c,), 0.5, 1.5)
    bias = synth.normal(11, c + 2, (c,), 0.02) if with_bias else None
    got, ref = _norm_case(x, gamma, c, cp, bias, silu)
    assert not np.isnan(got).any()
    assert np.all(got[:, c:] == 0), "padded channels must stay zero"
    _assert_f16_close(got[:, :c], ref)


def test_rmsnorm_zero_and_single_pixel():
    x = np.zeros((1, 1, 128), np.float32)
    got, _ = _norm_case(x, np.ones(128, np.float32), 128, 128)
    assert np.all(got == 0)
    x = synth.normal(12, 0, (1, 1, 128), 1.0)
    got, ref = _norm_case(x, np.ones(128, np.float32), 128, 128, silu=False)
    _assert_f16_close(got, ref)


# ---------------------------------------------------------------------------
# guarded cast
# ---------------------------------------------------------------------------


# ---------------------------------------------------------------------------
# GroupNorm (the variant for FLUX-class decoders)
# ---------------------------------------------------------------------------


def _gn_case(H, W, c, cp, groups, with_bias, silu, seed):
    M = H * W
    x = (synth.normal(18, seed, (M, c), 4.0) + synth.normal(18, seed + 1, (1, c), 9.0)).astype(np.float32)
    gamma = synth.uniform(18, seed + 2, (c,), 0.5, 1.5)
    beta = synth.normal(18, seed + 3, (c,), 0.1)
    bias = synth.normal(18, seed + 4, (c,), 0.02) if with_bias else None
    nbytes = ig.groupnorm_workspace_bytes(M, cp, groups)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = nan_f16((M, cp))
    ig.groupnorm_silu_f16(dev(pad_last(x, cp)), M, cp, c, groups, None if bias is None else padded_vec(bias, cp),
                          padded_vec(gamma, cp), padded_vec(beta, cp), int(silu), 1e-6, ws, nbytes, y)
    got = host(y)
    ref = O.group_norm(x.T, groups, gamma, beta, bias=bias, silu=silu).T
    return got, ref


@pytest.mark.parametrize("H,W,c,cp,groups,with_bias,silu", [
    (64, 64, 128, 128, 32, True, True), (7, 9, 288, 320, 32, False, True), (33, 17, 512, 512, 32, True, False),
    (1, 1, 64, 64, 32, False, True), (100, 90, 96, 128, 8, True, True), (512, 512, 128, 128, 32, True, True)])
def test_groupnorm(H, W, c, cp, groups, with_bias, silu):
    """GroupNorm on the GPU against the oracle (per-group statistics over
    all pixels; the chunked statistics merge exactly up to rounding)."""
    got, ref = _gn_case(H, W, c, cp, groups, with_bias, silu, seed=H + c)
    assert not np.isnan(got.astype(np.float32)).any()
    assert np.all(got[:, c:] == 0), "padded channels must be zero"
    u = f16_ulps(got[:, :c], ref.astype(np.float16))
    d = np.abs(got[:, :c].astype(np.float64) - ref)
    exact = float(np.mean(u == 0))
    print("groupnorm %dx%d c=%d g=%d: max ulp %d, exact %.5f" % (H, W, c, groups, u.max(), exact))
    assert np.all((u <= 1) | (d <= 1e-5)) and exact >= 0.999


def test_groupnorm_many_batches_per_workgroup():
    """A frame large enough that each of the statistics kernel's 1024
    workgroups folds many batches (with the next batch's loads in flight),
    a row count that leaves a ragged last batch, and a mean far from zero
    (the running merge must not lose the variance to cancellation).

    Tolerance: an f32 evaluation of (v - mean) * inv * gamma + beta carries
    the f32 rounding of the mean, up to 2^-24 |mean|, times inv * |gamma|;
    near zero that exceeds 1 f16 ulp, so each element must be within 1 ulp
    or within 1e-5 + 2^-21 |mean| inv |gamma| (8x that rounding), and 97%
    exact (98.3% measured at mean 100, std 1)."""
    H, W, c, groups = 701, 1499, 64, 16
    M = H * W
    x = (synth.normal(18, 77, (M, c), 1.0) + 100.0).astype(np.float32)
    gamma = synth.uniform(18, 78, (c,), 0.5, 1.5)
    beta = synth.normal(18, 79, (c,), 0.1)
    nbytes = ig.groupnorm_workspace_bytes(M, c, groups)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = nan_f16((M, c))
    ig.groupnorm_silu_f16(dev(x), M, c, c, groups, None, dev(gamma), dev(beta), 1, 1e-6, ws, nbytes, y)
    got = host(y)
    ref = O.group_norm(x.T, groups, gamma, beta, silu=True).T
    xg = x.astype(np.float64).reshape(M, groups, c // groups)
    mean = xg.mean(axis=(0, 2))
    inv = 1.0 / np.sqrt(xg.var(axis=(0, 2)) + 1e-6)
    bound = 1e-5 + 2.0 ** -21 * np.repeat(np.abs(mean) * inv, c // groups)[None, :] * np.abs(gamma)[None, :]
    u = f16_ulps(got, ref.astype(np.float16))
    d = np.abs(got.astype(np.float64) - ref)
    exact = float(np.mean(u == 0))
    print("groupnorm %dx%d c=%d g=%d (mean 100): max ulp %d, exact %.5f, max d/bound %.3f" % (
        H, W, c, groups, u.max(), exact, float(np.max(np.where(u <= 1, 0.0, d / bound)))))
    assert np.all((u <= 1) | (d <= bound)) and exact >= 0.97


def _merge_partials(part, groups, nchunk):
    """Per-group (count, mean, M2) from a conv's per-tile partials: the
    exact parallel combination (sums of counts, count-weighted means, M2s
    plus the spread of the tile means), in float64."""
    p = part.reshape(groups, nchunk, 3).astype(np.float64)
    n = p[..., 0].sum(axis=1)
    mean = (p[..., 0] * p[..., 1]).sum(axis=1) / n
    m2 = p[..., 2].sum(axis=1) + (p[..., 0] * (p[..., 1] - mean[:, None]) ** 2).sum(axis=1)
    return n, mean, m2


def _gn_stats_conv(H, W, cin, cout, groups, mode, acc, seed, offset=0.0):
    """A 3x3 conv that gathers its output's GroupNorm statistics; returns
    the stored f32 output, the partials, their chunk count and the oracle's
    conv of the same f16 input (plus the stream it was added to)."""
    d = {"x": synth.normal(20, 4 * seed, (H, W, cin), 1.0),
         "w": synth.normal(20, 4 * seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16),
         "b": synth.normal(20, 4 * seed + 2, (cout,), 0.02).astype(np.float32)}
    x16 = d["x"].astype(np.float16)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    y0 = (synth.normal(20, 4 * seed + 3, (Ho * Wo, cout), 1.0) + offset).astype(np.float32) if acc else None
    y = dev(y0) if acc else nan_f32((Ho * Wo, cout))
    nbytes = ig.conv_gn_partials_bytes(mode, H, W, groups)
    nchunk = nbytes // (12 * groups)
    part = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ig.conv3x3_gn_stats_nhwc(dev(x16.reshape(H * W, cin)), H, W, cin, mode, packed(d["w"]), cout, dev(d["b"]), 1.0,
                             acc, y, cout, groups, part, nbytes)
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    ref = (O.conv2d_up2 if mode == 2 else O.conv2d)(xc, d["w"], d["b"])
    ref = ref.transpose(1, 2, 0).reshape(Ho * Wo, cout)
    if acc:
        ref = ref + y0
    return host(y), host(part), nchunk, ref


@pytest.mark.parametrize("H,W,cin,cout,groups,mode,acc", [
    (40, 52, 128, 128, 32, 1, 0), (33, 70, 64, 256, 32, 1, 1), (12, 20, 128, 512, 32, 2, 0),
    (20, 36, 64, 128, 16, 2, 1), (16, 40, 64, 128, 2, 1, 0), (9, 150, 64, 256, 8, 1, 1)])
def test_conv_gathers_group_statistics(H, W, cin, cout, groups, mode, acc):
    """The conv's epilogue gathers per-tile GroupNorm statistics of what it
    stores (after adding into the stream). The output meets the per-conv
    bar against the oracle; the merged partials give every group's exact
    count, and mean and variance within f32 folding error of the float64
    statistics of the stored values (groups of 4 to 64 channels, ragged
    tiles, plain and upsampled, stored and accumulated)."""
    got, part, nchunk, ref = _gn_stats_conv(H, W, cin, cout, groups, mode, acc, seed=H + cout)
    err, rms, ratio = conv_err(got, ref)
    assert ratio <= CONV_TOL, (err, rms)
    assert np.all(np.isfinite(part))
    M, cpg = got.shape[0], cout // groups
    n, mean, m2 = _merge_partials(part, groups, nchunk)
    v = got.astype(np.float64).reshape(M, groups, cpg)
    rmean = v.mean(axis=(0, 2))
    rvar = v.var(axis=(0, 2))
    dm = np.abs(mean - rmean) / (np.abs(rmean) + np.sqrt(rvar))
    dv = np.abs(m2 / n - rvar) / rvar
    print("gn stats %dx%d %d->%d g=%d mode %d acc %d: %d tiles, mean rel %.2e, var rel %.2e" % (
        H, W, cin, cout, groups, mode, acc, nchunk, dm.max(), dv.max()))
    assert np.all(n == M * cpg)
    assert dm.max() <= 2e-6 and dv.max() <= 2e-5


@pytest.mark.parametrize("offset", [0.0, 100.0])
def test_groupnorm_from_conv_statistics(offset):
    """GroupNorm of a conv's output from the statistics its epilogue
    gathered (one read of the stream) against the oracle's GroupNorm of
    the same stored values, at the standalone GroupNorm's bars: 1 ulp or
    1e-5 and 99.9% exact; with the stream at mean 100 (the conv adds into
    it), the mean-dependent bound of the large-mean standalone case and
    97% exact."""
    H, W, cin, cout, groups = 48, 64, 64, 256, 32
    got, part, nchunk, _ = _gn_stats_conv(H, W, cin, cout, groups, 1, 1, seed=5, offset=offset)
    M = H * W
    gamma = synth.uniform(18, 90, (cout,), 0.5, 1.5)
    beta = synth.normal(18, 91, (cout,), 0.1)
    tab = torch.empty(3 * cout, dtype=torch.float32, device="cuda")
    y = nan_f16((M, cout))
    ig.groupnorm_silu_f16_from_partials(dev(got), M, cout, cout, groups, dev(gamma), dev(beta), 1, 1e-6,
                                        dev(part), nchunk, tab, tab.numel() * 4, y)
    gy = host(y)
    ref = O.group_norm(got.T.astype(np.float64), groups, gamma, beta, silu=True).T
    u = f16_ulps(gy, ref.astype(np.float16))
    d = np.abs(gy.astype(np.float64) - ref)
    exact = float(np.mean(u == 0))
    xg = got.astype(np.float64).reshape(M, groups, cout // groups)
    mean = xg.mean(axis=(0, 2))
    inv = 1.0 / np.sqrt(xg.var(axis=(0, 2)) + 1e-6)
    bound = 1e-5 + 2.0 ** -21 * np.repeat(np.abs(mean) * inv, cout // groups)[None, :] * np.abs(gamma)[None, :]
    print("groupnorm from conv statistics (stream mean %g): max ulp %d, exact %.5f" % (offset, u.max(), exact))
    if offset == 0.0:
        assert np.all((u <= 1) | (d <= 1e-5)) and exact >= 0.999
    else:
        assert np.all((u <= 1) | (d <= bound)) and exact >= 0.97


def test_groupnorm_workspace_too_small():
    M, cp = 64, 128
    y = nan_f16((M, cp))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    z = torch.zeros(cp, device="cuda")
    with pytest.raises(ig.IgError) as e:
        ig.groupnorm_silu_f16(torch.zeros((M, cp), device="cuda"), M, cp, cp, 32, None, z, z, 1, 1e-6, ws, 16, y)
    assert e.value.code == -3
    assert torch.isnan(y.float()).all()


def test_guard_cast_config2_is_exact():
    d = synth.config2()
    H, W, C = d["x"].shape
    M = H * W
    y = nan_f16((M, C))
    ig.guard_cast(dev(d["x"].reshape(M, C)), M, C, None, d["guard_log2"], y)
    got = host(y)
    ref = O.guard_cast(d["x"].reshape(M, C), d["guard_log2"])
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("g", [0, 8, 14])
def test_guard_cast_bias_and_range(g):
    M, C = 333, 64
    x = synth.normal(13, g, (M, C), 1.0e10)  # std 1e5: past the f16 range
    b = synth.normal(13, 100 + g, (C,), 0.02)
    y = nan_f16((M, C))
    ig.guard_cast(dev(x), M, C, dev(b), g, y)
    got = host(y)
    ref = O.guard_cast(x.T, g, bias=b).T  # the oracle is channel-first
    fin = np.isfinite(ref)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    _assert_f16_close(got[fin], ref[fin])
    if g == 8:
        assert fin.all()  # 2^-8 keeps |x| < 65504 * 256 finite


@pytest.mark.parametrize("c,cp,with_bias,g", [(256, 256, False, 8), (512, 512, False, 8), (288, 320, True, 4),
                                             (1000, 1024, True, 14)])
def test_rmsnorm_with_guarded_cast(c, cp, with_bias, g):
    """The norm of a resnet with a shortcut and the shortcut's guarded cast
    from one read of the stream: each output against the oracle's norm and
    cast of the same rows (and bit for bit against the separate kernels)."""
    M = 1000
    x = synth.normal(14, c, (M, c), 1.0e8)  # std 1e4: the guard matters
    gamma = synth.uniform(14, c + 1, (c,), 0.5, 1.5)
    bias = synth.normal(14, c + 2, (c,), 0.02) if with_bias else None
    xd = dev(pad_last(x, cp))
    gd = padded_vec(gamma, cp)
    bd = padded_vec(bias, cp) if bias is not None else None
    y, yg = nan_f16((M, cp)), nan_f16((M, cp))
    ig.rmsnorm_silu_guard_cast_f16(xd, M, cp, c, bd, gd, 1, 1e-12, y, g, yg)
    y1, yg1 = nan_f16((M, cp)), nan_f16((M, cp))
    ig.rmsnorm_silu_f16(xd, M, cp, c, bd, gd, 1, 1e-12, y1)
    ig.guard_cast(xd, M, cp, bd, g, yg1)
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(yg.view(torch.int16), yg1.view(torch.int16))
    got, gotg = host(y), host(yg)
    ref = O.f16(O.rmsnorm(x.T, gamma, bias=bias, silu=True)).T
    _assert_f16_close(got[:, :c], ref)
    assert np.all(got[:, c:] == 0)
    refg = O.guard_cast(x.T, g, bias=bias).T
    fin = np.isfinite(refg)
    assert np.array_equal(np.isinf(gotg[:, :c]), np.isinf(refg))
    _assert_f16_close(gotg[:, :c][fin], refg[fin])


# ---------------------------------------------------------------------------
# 3x3 convolution
# ---------------------------------------------------------------------------


def _conv_isolated(H, W, cin, cout, mode, seed, oscale=1.0, with_bias=True):
    """Seeded f16 input shared by both sides; returns (got, ref) as [C,H,W]."""
    x16 = synth.normal(14, seed, (H, W, cin), 1.0, np.float16)
    k = 1 if mode == 0 else 3
    w = synth.normal(14, seed + 1, (cout, cin, k, k), 1.0 / (k * k * cin), np.float16)
    b = synth.normal(14, seed + 2, (cout,), 0.02) if with_bias else None
    cin_p, cout_p = cpad(cin), cpad(cout)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    y = nan_f32((Ho * Wo, cout_p))
    bd = padded_vec(b, cout_p) if with_bias else None
    ig.conv_nhwc_ex(dev(pad_last(x16.reshape(H * W, cin), cin_p)), H, W, cin_p, mode, packed(w),
                    cout_p, bd, oscale, 0, y)
    got = host(y)
    assert not np.isnan(got).any(), "output not fully written"
    assert np.all(got[:, cout:] == 0), "padded output channels must be zero"
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    if mode == 2:
        ref = oscale * O.conv2d_up2(xc, w) + (0 if b is None else b[:, None, None])
    else:
        ref = oscale * O.conv2d(xc, w) + (0 if b is None else b[:, None, None])
    return nhwc_to_chw(got[:, :cout], Ho, Wo), ref


@pytest.mark.parametrize("H,W,cin,cout", [(64, 64, 128, 128), (13, 29, 64, 192), (1, 1, 64, 64),
                                          (5, 1, 128, 64), (1, 7, 64, 128), (33, 17, 320, 320),
                                          (9, 70, 256, 512)])
def test_conv3x3_isolated(H, W, cin, cout):
    got, ref = _conv_isolated(H, W, cin, cout, 1, seed=H * 7 + W)
    err, rms, ratio = conv_err(got, ref)
    print("conv3x3 %dx%d %d->%d: max|d| %.3e rms %.3e ratio %.2e" % (H, W, cin, cout, err, rms, ratio))
    assert ratio <= CONV_TOL
    assert ratio <= 1e-4  # identical f16 inputs: only f32 accumulation order differs


@pytest.mark.parametrize("H,W,cin,cout", [(9, 13, 64, 128), (1, 1, 64, 64), (16, 3, 128, 192)])
def test_conv3x3_up2_isolated(H, W, cin, cout):
    got, ref = _conv_isolated(H, W, cin, cout, 2, seed=100 + H, oscale=256.0)
    err, rms, ratio = conv_err(got, ref)
    print("up2 %dx%d %d->%d: ratio %.2e" % (H, W, cin, cout, ratio))
    assert ratio <= CONV_TOL and ratio <= 1e-4


@pytest.mark.parametrize("H,W,cin,cout,mode", [(300, 530, 64, 192, 1), (160, 270, 128, 128, 2),
                                               (272, 512, 128, 128, 1)])
def test_conv3x3_tile_walk_sampled(H, W, cin, cout, mode):
    """More 16x32x64 output tiles than the chip holds workgroups, so each
    workgroup walks several (the next tile's first stage loading under the
    current tile's last stage and epilogue), with ragged image edges and a
    tile count that splits unevenly over the 8 XCDs: every output written,
    the border pixels, one pixel of every tile and seeded picks against the
    oracle."""
    seed = 500 + H + mode
    x16 = synth.normal(14, seed, (H, W, cin), 1.0, np.float16)
    w = synth.normal(14, seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = synth.normal(14, seed + 2, (cout,), 0.02)
    cin_p, cout_p = cpad(cin), cpad(cout)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    assert ((Ho + 15) // 16) * ((Wo + 31) // 32) * (cout_p // 64) > 512
    y = nan_f32((Ho * Wo, cout_p))
    ig.conv_nhwc_ex(dev(pad_last(x16.reshape(H * W, cin), cin_p)), H, W, cin_p, mode, packed(w), cout_p,
                    padded_vec(b, cout_p), 1.0, 0, y)
    got = host(y)
    assert not np.isnan(got).any(), "a tile was not written"
    assert np.all(got[:, cout:] == 0)
    corners = np.array([r * Wo + c for r in range(0, Ho, 16) for c in range(0, Wo, 32)], np.int64)
    pix = np.unique(np.concatenate([sample_pixels(Ho, Wo, 512, seed=seed), corners, corners + 15 * Wo + 31]))
    pix = pix[pix < Ho * Wo]
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    ref = O.conv2d_at(xc, w, pix, b, up2=(mode == 2))
    err, rms, ratio = conv_err(got[pix, :cout], ref)
    print("tile walk %dx%d %d->%d mode %d (%d px): ratio %.2e" % (H, W, cin, cout, mode, len(pix), ratio))
    assert ratio <= CONV_TOL and ratio <= 1e-4


@pytest.mark.parametrize("H,W,cin,cout", [(11, 23, 256, 256), (1, 1, 64, 64), (32, 32, 512, 256)])
def test_conv1x1_isolated(H, W, cin, cout):
    got, ref = _conv_isolated(H, W, cin, cout, 0, seed=200 + H)
    assert conv_err(got, ref)[2] <= 1e-4


@pytest.mark.parametrize("H,W,cin,cout", [(17, 45, 128, 3), (8, 32, 64, 1), (40, 70, 192, 16), (33, 31, 128, 5),
                                          (1, 1, 64, 3), (64, 64, 128, 3), (9, 33, 256, 2), (24, 40, 128, 4)])
def test_output_conv_nchw(H, W, cin, cout):
    """The decoder's output conv: few output channels, NCHW frame + bias,
    against the oracle's convolution on the same f16 input (up to 3
    channels the nine taps' products side by side, 4 and more one tap per
    MFMA)."""
    seed = 300 + H + cout
    x16 = synth.normal(16, seed, (H, W, cin), 1.0, np.float16)
    w = synth.normal(16, seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = synth.normal(16, seed + 2, (cout,), 0.02)
    cin_p, cout_p = cpad(cin), cpad(cout)
    out = nan_f32((cout, H * W))
    ig.conv3x3_out_nchw(dev(pad_last(x16.reshape(H * W, cin), cin_p)), H, W, cin_p, packed(w), cout, cout_p,
                        padded_vec(b, cout_p), out)
    got = host(out).reshape(cout, H, W)
    assert not np.isnan(got).any(), "output not fully written"
    ref = O.conv2d(nhwc_to_chw(x16.astype(np.float64), H, W), w) + b[:, None, None]
    err, rms, ratio = conv_err(got, ref)
    print("output conv %dx%d %d->%d: ratio %.2e" % (H, W, cin, cout, ratio))
    assert ratio <= 1e-4


def test_output_conv_rejects_wide_output():
    with pytest.raises(ig.IgError) as e:
        ig.conv3x3_out_nchw(dev(np.zeros((4, 64), np.float16)), 2, 2, 64, dev(np.zeros(9 * 64 * 64, np.float16)),
                            17, 64, None, nan_f32((17, 4)))
    assert e.value.code == -2


@pytest.mark.parametrize("H,W,cin,cout,c_real,mode,silu,want_y", [
    (64, 64, 128, 128, 128, 1, 1, False), (13, 29, 64, 64, 50, 1, 0, True),
    (9, 13, 64, 128, 128, 2, 1, False), (40, 33, 192, 128, 100, 1, 1, True), (1, 1, 64, 64, 64, 2, 1, False)])
def test_conv_with_fused_norm(H, W, cin, cout, c_real, mode, silu, want_y):
    """A 3x3 conv whose epilogue emits f16(RMS_norm(conv + b) -> SiLU),
    against the oracle's norm of the oracle's convolution. The conv's f32
    accumulation moves v by ~1e-6 relative, which flips the f16 rounding of
    a few tenths of a percent of the outputs: <= 1 ulp (or <= 1e-5 absolute
    near zero, where the conv's error is several tiny ulps), >= 99.5% exact."""
    seed = 400 + H + cout
    x16 = synth.normal(17, seed, (H, W, cin), 1.0, np.float16)
    w = np.zeros((cout, cin, 3, 3), np.float16)
    w[:c_real] = synth.normal(17, seed + 1, (c_real, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = np.zeros(cout, np.float32)
    b[:c_real] = synth.normal(17, seed + 2, (c_real,), 0.02)
    gamma = np.zeros(cout, np.float32)
    gamma[:c_real] = synth.uniform(17, seed + 3, (c_real,), 0.5, 1.5)
    cin_p = cpad(cin)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    osc = 256.0 if mode == 2 else 1.0
    yn = nan_f16((Ho * Wo, cout))
    y = nan_f32((Ho * Wo, cout)) if want_y else None
    ig.conv3x3_norm_nhwc(dev(pad_last(x16.reshape(H * W, cin), cin_p)), H, W, cin_p, mode, packed(w), cout,
                         c_real, dev(b), osc, dev(gamma), silu, 1e-12, y, yn)
    got = host(yn)
    assert not np.isnan(got.astype(np.float32)).any()
    assert np.all(got[:, c_real:] == 0)
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    conv = osc * (O.conv2d_up2(xc, w) if mode == 2 else O.conv2d(xc, w)) + b[:, None, None]
    ref = O.rmsnorm(conv[:c_real].reshape(c_real, -1), gamma[:c_real], silu=bool(silu)).T
    u = f16_ulps(got[:, :c_real], ref.astype(np.float16))
    d = np.abs(got[:, :c_real].astype(np.float64) - ref)
    exact = float(np.mean(u == 0))
    print("conv+norm %dx%d %d->%d mode %d: max ulp %d, exact %.5f, max|d| %.2e" % (H, W, cin, cout, mode, u.max(),
                                                                               exact, d.max()))
    # near zero an ulp is tiny; there the bar is the conv's absolute error
    # carried through the norm (outputs have RMS ~1)
    assert np.all((u <= 1) | (d <= 1e-5)) and exact >= 0.995
    if want_y:
        gy = nhwc_to_chw(host(y)[:, :c_real], Ho, Wo)
        assert conv_err(gy, conv[:c_real])[2] <= 1e-4


@pytest.mark.parametrize("H,W,cin,cout,mode", [
    (400, 700, 64, 64, 1), (300, 530, 128, 128, 1), (150, 260, 128, 128, 2)])
def test_conv_with_fused_norm_tile_walk_sampled(H, W, cin, cout, mode):
    """The fused-norm conv with more tiles than the chip holds workgroups
    (each walks several; its f32 rows are staged in the last stage's buffer
    while the next tile's first stage loads into the other; at 128 channels
    two rows per staging pass), on ragged frames: every pixel written, the
    borders, one pixel of every tile and seeded picks against the oracle's
    norm of the oracle's convolution, to the bar of the full-image test."""
    seed = 900 + cout + mode
    x16 = synth.normal(17, seed, (H, W, cin), 1.0, np.float16)
    w = synth.normal(17, seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = synth.normal(17, seed + 2, (cout,), 0.02)
    gamma = synth.uniform(17, seed + 3, (cout,), 0.5, 1.5)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    osc = 256.0 if mode == 2 else 1.0
    assert ((Ho + 15) // 16) * ((Wo + 31) // 32) > (512 if cout == 64 else 256)
    yn = nan_f16((Ho * Wo, cout))
    ig.conv3x3_norm_nhwc(dev(x16.reshape(H * W, cin)), H, W, cin, mode, packed(w), cout, cout, dev(b), osc,
                         dev(gamma), 1, 1e-12, None, yn)
    got = host(yn)
    assert not np.isnan(got.astype(np.float32)).any(), "a tile was not written"
    corners = np.array([r * Wo + c for r in range(0, Ho, 16) for c in range(0, Wo, 32)], np.int64)
    edges = np.array([(Ho - 1) * Wo + c for c in range(Wo)] + [r * Wo + Wo - 1 for r in range(Ho)], np.int64)
    pix = np.unique(np.concatenate([sample_pixels(Ho, Wo, 512, seed=seed), corners, edges]))
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    conv = osc * O.conv2d_at(xc, w, pix, up2=(mode == 2)) + b[None, :]  # [npix, cout]
    ref = O.rmsnorm(conv.T, gamma, silu=True).T
    u = f16_ulps(got[pix], ref.astype(np.float16))
    d = np.abs(got[pix].astype(np.float64) - ref)
    exact = float(np.mean(u == 0))
    print("conv+norm tile walk %dx%d %d->%d mode %d (%d px): max ulp %d, exact %.5f" % (
        H, W, cin, cout, mode, len(pix), u.max(), exact))
    assert np.all((u <= 1) | (d <= 1e-5)) and exact >= 0.995


@pytest.mark.parametrize("H,W,cin,cout,mode,acc,write_y,g", [
    (64, 64, 128, 128, 1, 1, 0, 8), (13, 29, 64, 256, 1, 1, 1, 8), (9, 13, 128, 64, 2, 0, 1, 4),
    (40, 33, 192, 128, 1, 0, 0, 14), (128, 128, 512, 512, 1, 1, 0, 8)])
def test_conv_with_guarded_cast_output(H, W, cin, cout, mode, acc, write_y, g):
    """A 3x3 conv (or up conv) whose epilogue emits the guarded f16 cast of
    its (accumulated) result: bit for bit the separate conv then guard_cast
    (the same f32 value, the same scaling and rounding), and the f32 result
    against the oracle's conv."""
    seed = 500 + H + cout
    x16 = synth.normal(18, seed, (H, W, cin), 1.0, np.float16)
    w = synth.normal(18, seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = synth.normal(18, seed + 2, (cout,), 0.02)
    cin_p, cout_p = cpad(cin), cpad(cout)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    M = Ho * Wo
    xd = dev(pad_last(x16.reshape(H * W, cin), cin_p))
    pl = packed(w)
    y0 = synth.normal(18, seed + 3, (M, cout_p), 1.0e6).astype(np.float32)  # a stream past f16's range
    y = dev(y0)
    yg = nan_f16((M, cout_p))
    ig.conv3x3_guard_out_nhwc(xd, H, W, cin_p, mode, pl, cout_p, padded_vec(b, cout_p), 1.0, acc, y, write_y, g, yg)
    yref = dev(y0)
    ig.conv_nhwc_ex(xd, H, W, cin_p, mode, pl, cout_p, padded_vec(b, cout_p), 1.0, acc, yref)
    ygref = nan_f16((M, cout_p))
    ig.guard_cast(yref, M, cout_p, None, g, ygref)
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int16), ygref.view(torch.int16))
    if write_y:
        assert torch.equal(y, yref)
    else:
        assert torch.equal(y, dev(y0))  # the f32 result is not stored
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    conv = (O.conv2d_up2(xc, w) if mode == 2 else O.conv2d(xc, w)) + b[:, None, None]
    want = conv + (nhwc_to_chw(y0[:, :cout].astype(np.float64), Ho, Wo) if acc else 0.0)
    got = nhwc_to_chw(host(yref)[:, :cout].astype(np.float64), Ho, Wo)
    assert np.max(np.abs(got - want)) <= 2e-3 * np.sqrt(np.mean(conv ** 2)) + 1e-7 * np.max(np.abs(want))


def test_clock_probe_reads_the_conv_clock():
    """The measurement hook: the first wave's shader-clock and real-time
    counters around a 512x512x128 conv give a clock in the chip's range, and
    the conv's output is the same with the hook set."""
    H = W = 512
    C = 128
    M = H * W
    rng = np.random.default_rng(7)
    x = dev(rng.standard_normal((M, C)).astype(np.float16))
    plane = packed((rng.standard_normal((C, C, 3, 3)) / 34).astype(np.float16))
    b = dev((rng.standard_normal(C) * 0.02).astype(np.float32))
    y0, y1 = nan_f32((M, C)), nan_f32((M, C))
    ig.conv3x3_nhwc(x, H, W, C, plane, C, b, 1.0, y0)
    buf = torch.zeros(4, dtype=torch.int64, device="cuda")
    ig.set_clock_probe(buf)
    try:
        ig.conv3x3_nhwc(x, H, W, C, plane, C, b, 1.0, y1)
    finally:
        ig.set_clock_probe(None)
    torch.cuda.synchronize()
    ck0, rt0, ck1, rt1 = [int(v) for v in buf.cpu()]
    assert rt1 > rt0 and ck1 > ck0
    ghz = (ck1 - ck0) / ((rt1 - rt0) / 1e8) / 1e9
    print("clock during the conv: %.3f GHz over %.1f us" % (ghz, (rt1 - rt0) / 100.0))
    assert 0.3 < ghz < 3.5
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("H,W,mode,acc,write_y,g", [
    (258, 300, 1, 0, 1, 8), (258, 300, 1, 1, 1, 8), (259, 301, 1, 1, 0, 8),
    (130, 150, 2, 0, 1, 8), (131, 149, 2, 1, 0, 4)])
def test_conv_weights_in_registers_sampled(H, W, mode, acc, write_y, g):
    """128 -> 128 convs on frames large enough for the kernel that keeps the
    weights in registers (4-row tiles walked by one workgroup per CU, each
    tile's result staged in LDS and written out during the next tile's
    stages), ragged at the bottom and right: every pixel written; the f32
    result, plain or accumulated into a stream, at the borders, at a pixel
    of every tile and at seeded picks against the oracle; and the guarded
    f16 cast emitted by the same epilogue bit for bit the separate cast of
    the f32 result."""
    seed = 1100 + H + mode
    c = 128
    x16 = synth.normal(19, seed, (H, W, c), 1.0, np.float16)
    w = synth.normal(19, seed + 1, (c, c, 3, 3), 1.0 / (9 * c), np.float16)
    b = synth.normal(19, seed + 2, (c,), 0.02)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    M = Ho * Wo
    assert ((Ho + 3) // 4) * ((Wo + 31) // 32) >= 512
    osc = 256.0 if mode == 2 else 1.0
    xd = dev(x16.reshape(H * W, c))
    pl = packed(w)
    y0 = synth.normal(19, seed + 3, (M, c), 100.0).astype(np.float32)
    yref = dev(y0) if acc else nan_f32((M, c))
    ig.conv_nhwc_ex(xd, H, W, c, mode, pl, c, dev(b), osc, acc, yref)
    ygref = nan_f16((M, c))
    ig.guard_cast(yref, M, c, None, g, ygref)
    y = dev(y0)
    yg = nan_f16((M, c))
    ig.conv3x3_guard_out_nhwc(xd, H, W, c, mode, pl, c, dev(b), osc, acc, y, write_y, g, yg)
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int16), ygref.view(torch.int16))
    assert torch.equal(y, yref) if write_y else torch.equal(y, dev(y0))
    got = host(yref)
    assert not np.isnan(got).any(), "a tile was not written"
    corners = np.array([r * Wo + cc for r in range(0, Ho, 4) for cc in range(0, Wo, 32)], np.int64)
    edges = np.array([(Ho - 1) * Wo + cc for cc in range(Wo)] + [r * Wo + Wo - 1 for r in range(Ho)], np.int64)
    pix = np.unique(np.concatenate([sample_pixels(Ho, Wo, 512, seed=seed), corners, corners + 3 * Wo + 31, edges]))
    pix = pix[pix < M]
    xc = nhwc_to_chw(x16.astype(np.float64), H, W)
    conv = osc * O.conv2d_at(xc, w, pix, up2=(mode == 2)) + b[None, :]
    want = conv + (y0[pix].astype(np.float64) if acc else 0.0)
    err = float(np.max(np.abs(got[pix] - want)))
    rms = float(np.sqrt(np.mean(conv * conv)))
    print("weights in registers %dx%d mode %d acc %d (%d px): max|d| %.3e rms %.3e" % (H, W, mode, acc, len(pix), err, rms))
    assert err <= 1e-4 * rms + 1e-7 * float(np.max(np.abs(want)))


@pytest.mark.parametrize("mode,H,W,cin,cout", [(1, 2048, 4095, 128, 128), (1, 4096, 4095, 64, 64),
                                              (2, 2047, 4095, 128, 128)])
def test_conv_at_the_largest_input(mode, H, W, cin, cout):
    """The 3x3 kernels address their f16 input with 32-bit byte offsets:
    the largest input they take is just below 0x7fff0000 bytes. At that
    size (ragged width; the register-weight kernel at 128 channels, the
    patch kernel at 64; the upsampling form writes a 17 GB frame) the f32
    result at the borders, the last rows and columns and seeded picks
    equals the oracle's conv. The input repeats a seeded block of R rows,
    so the oracle sees each sampled pixel's 3x3 source window from it."""
    R = 64
    assert H * W * cin * 2 < 0x7fff0000 and H * W * cin * 2 > 0x7fff0000 - (W + 2) * cin * 4
    seed = 1300 + mode + cin
    blk = synth.normal(20, seed, (R, W, cin), 1.0, np.float16)
    w = synth.normal(20, seed + 1, (cout, cin, 3, 3), 1.0 / (9 * cin), np.float16)
    b = synth.normal(20, seed + 2, (cout,), 0.02)
    Ho, Wo = (2 * H, 2 * W) if mode == 2 else (H, W)
    osc = 256.0 if mode == 2 else 1.0
    xd = dev(blk.reshape(R * W, cin)).repeat((H + R - 1) // R, 1)[:H * W].contiguous()
    y = torch.empty((Ho * Wo, cout), dtype=torch.float32, device="cuda")
    y.fill_(float("nan"))
    ig.conv_nhwc_ex(xd, H, W, cin, mode, packed(w), cout, dev(b), osc, 0, y)
    torch.cuda.synchronize()
    # corners, the last row and column (strided), the tail of the row above
    # the last, and seeded picks
    pix = np.unique(np.concatenate([
        np.array([0, Wo - 1, (Ho - 1) * Wo, Ho * Wo - 1], np.int64),
        (Ho - 1) * Wo + np.arange(0, Wo, 97), np.arange(0, Ho, 61) * Wo + Wo - 1,
        (Ho - 2) * Wo + np.arange(Wo - 40, Wo), np.random.default_rng(seed).integers(0, Ho * Wo, 160)]))
    got = host(y[torch.from_numpy(pix).cuda()])
    assert not np.isnan(got).any()
    want = np.empty((pix.size, cout))
    for n, q in enumerate(pix):
        r, c = divmod(int(q), Wo)
        # the output pixel's source window in the input (rows and columns
        # clamped to the frame, whose edges are the conv's zero padding)
        sr = (lambda v: v >> 1) if mode == 2 else (lambda v: v)
        r0, r1 = max(0, sr(max(r - 1, 0))), min(H - 1, sr(min(r + 1, Ho - 1)))
        c0, c1 = max(0, sr(max(c - 1, 0))), min(W - 1, sr(min(c + 1, Wo - 1)))
        win = blk[np.arange(r0, r1 + 1) % R][:, c0:c1 + 1, :]
        xc = np.ascontiguousarray(win.transpose(2, 0, 1)).astype(np.float64)
        rl, cl = r - (2 * r0 if mode == 2 else r0), c - (2 * c0 if mode == 2 else c0)
        wl = (c1 - c0 + 1) * (2 if mode == 2 else 1)
        want[n] = osc * O.conv2d_at(xc, w, np.array([rl * wl + cl], np.int64), up2=(mode == 2))[0] + b
    err = float(np.max(np.abs(got - want)))
    rms = float(np.sqrt(np.mean(want * want)))
    print("largest input %dx%dx%d mode %d (%.3f GB in, %.2f GB out, %d px): max|d| %.3e rms %.3e" % (
        H, W, cin, mode, H * W * cin * 2 / 1e9, Ho * Wo * cout * 4 / 1e9, pix.size, err, rms), flush=True)
    assert err <= 1e-4 * rms
    del y, xd
    torch.cuda.empty_cache()


def test_conv_fused_norm_needs_one_tile_per_pixel():
    with pytest.raises(ig.IgError) as e:
        z = dev(np.zeros((4, 64), np.float16))
        ig.conv3x3_norm_nhwc(z, 2, 2, 64, 1, dev(np.zeros(9 * 64 * 192, np.float16)), 192, 192, None, 1.0,
                             dev(np.zeros(192, np.float32)), 1, 1e-12, None, nan_f16((4, 192)))
    assert e.value.code == -2


def test_conv_accumulate_epilogue():
    H, W, c = 10, 12, 64
    x16 = synth.normal(15, 0, (H * W, c), 1.0, np.float16)
    w = synth.normal(15, 1, (c, c, 3, 3), 1.0 / (9 * c), np.float16)
    b = synth.normal(15, 2, (c,), 0.02)
    y0 = synth.normal(15, 3, (H * W, c), 1.0)
    y = dev(y0)
    ig.conv_nhwc_ex(dev(x16), H, W, c, 1, packed(w), c, dev(b), 0.5, 1, y)
    got = nhwc_to_chw(host(y), H, W)
    ref = nhwc_to_chw(y0.astype(np.float64), H, W) + 0.5 * O.conv2d(nhwc_to_chw(x16.astype(np.float64), H, W), w) + b[:, None, None]
    assert conv_err(got, ref)[2] <= 1e-4


def test_config1_norm_then_conv():
    """The whole config-1 unit: RMS_norm + SiLU -> f16 -> 3x3 conv (+bias)."""
    d = synth.config1()
    H, W, C = d["x"].shape
    xn = nan_f16((H * W, C))
    ig.rmsnorm_silu_f16(dev(d["x"].reshape(H * W, C)), H * W, C, C, None, dev(d["gamma"]), 1, 1e-12, xn)
    y = nan_f32((H * W, C))
    ig.conv3x3_nhwc(xn, H, W, C, packed(d["w"]), C, dev(d["b"]), 1.0, y)
    got = nhwc_to_chw(host(y), H, W)
    xref = O.f16(O.rmsnorm(nhwc_to_chw(d["x"], H, W), d["gamma"], silu=True))
    ref = O.conv2d(xref, d["w"], d["b"])
    err, rms, ratio = conv_err(got, ref)
    print("config1: max|d| %.3e rms %.3e ratio %.2e" % (err, rms, ratio))
    assert ratio <= CONV_TOL


# ---------------------------------------------------------------------------
# config 2: guarded up conv + 1x1 shortcut, added in f32
# ---------------------------------------------------------------------------


@pytest.fixture(scope="module")
def cfg2_run():
    d = synth.config2()
    H, W, C = d["x"].shape
    M = H * W
    g = d["guard_log2"]
    gs = float(2 ** g)
    xg = nan_f16((M, C))
    ig.guard_cast(dev(d["x"].reshape(M, C)), M, C, None, g, xg)
    up = nan_f32((4 * M, C))
    ig.conv3x3_up2_nhwc(xg, H, W, C, packed(d["w_up"]), C, dev(d["b_up"]), gs, up)
    sc = nan_f32((M, C))
    plane_sc = packed(d["w_sc"])
    ig.gemm1x1(xg, M, C, C, plane_sc, C, C, dev(d["b_sc"]), gs, sc, C, 0)
    tot = up.clone()
    ig.dupup_add(sc, H, W, C, tot, C, C, 4, 4, 1)
    xq = nhwc_to_chw(O.guard_cast(d["x"].reshape(M, C), g), H, W)
    return d, host(up), host(sc), host(tot), xq


def test_config2_shortcut_gemm(cfg2_run):
    d, _, sc, _, xq = cfg2_run
    H, W, C = d["x"].shape
    ref = 2.0 ** d["guard_log2"] * O.conv2d(xq, d["w_sc"]) + d["b_sc"][:, None, None]
    err, rms, ratio = conv_err(nhwc_to_chw(sc, H, W), ref)
    print("config2 shortcut: ratio %.2e" % ratio)
    assert ratio <= CONV_TOL and ratio <= 1e-4


def test_config2_up_conv_sampled(cfg2_run):
    d, up, _, _, xq = cfg2_run
    H, W, C = d["x"].shape
    pix = sample_pixels(2 * H, 2 * W, 1024, seed=2)
    ref = 2.0 ** d["guard_log2"] * O.conv2d_at(xq, d["w_up"], pix, up2=True) + d["b_up"][None, :]
    err, rms, ratio = conv_err(up[pix], ref)
    print("config2 up conv (%d px): ratio %.2e" % (len(pix), ratio))
    assert not np.isnan(up).any()
    assert ratio <= CONV_TOL and ratio <= 1e-4


def test_config2_sum_sampled(cfg2_run):
    d, _, _, tot, xq = cfg2_run
    H, W, C = d["x"].shape
    gs = 2.0 ** d["guard_log2"]
    pix = sample_pixels(2 * H, 2 * W, 1024, seed=3)
    up = gs * O.conv2d_at(xq, d["w_up"], pix, up2=True) + d["b_up"][None, :]
    src = (pix // (2 * W)) // 2 * W + (pix % (2 * W)) // 2  # nearest-2x source pixel
    sc = gs * O.conv2d_at(xq, d["w_sc"], src) + d["b_sc"][None, :]
    err, rms, ratio = conv_err(tot[pix], up + sc)
    print("config2 up + shortcut: ratio %.2e" % ratio)
    assert ratio <= CONV_TOL


# ---------------------------------------------------------------------------
# config 3: the large-tile conv and its padded variants
# ---------------------------------------------------------------------------


def _cfg3(c, H, W, n_sample=None):
    d = synth.config3(c, H, W)
    cp = cpad(c)
    M = H * W
    xd = dev(pad_last(d["x"].reshape(M, c), cp))
    xn = nan_f16((M, cp))
    ig.rmsnorm_silu_f16(xd, M, cp, c, None, padded_vec(d["gamma"], cp), 0, 1e-12, xn)
    y = nan_f32((M, cp))
    ig.conv3x3_nhwc(xn, H, W, cp, packed(d["w"]), cp, padded_vec(d["b"], cp), 1.0, y)
    got = host(y)
    assert not np.isnan(got).any()
    assert np.all(got[:, c:] == 0), "padded output channels must be zero"
    xref = O.f16(O.rmsnorm(nhwc_to_chw(d["x"], H, W), d["gamma"]))
    if n_sample is None:
        ref = O.conv2d(xref, d["w"], d["b"])
        return conv_err(nhwc_to_chw(got[:, :c], H, W), ref)
    pix = sample_pixels(H, W, n_sample, seed=c)
    ref = O.conv2d_at(xref, d["w"], pix, d["b"])
    return conv_err(got[pix, :c], ref)


@pytest.mark.parametrize("c", [128, 288, 144])
def test_config3_small_full(c):
    err, rms, ratio = _cfg3(c, 48, 40)
    print("config3 %d @48x40: ratio %.2e" % (c, ratio))
    assert ratio <= CONV_TOL


@pytest.mark.parametrize("c", [128, 288, 144])
def test_config3_full_size_sampled(c):
    err, rms, ratio = _cfg3(c, 512, 512, n_sample=1024)
    print("config3 %d @512x512 (sampled): ratio %.2e" % (c, ratio))
    assert ratio <= CONV_TOL


# ---------------------------------------------------------------------------
# GEMM epilogues, softmax, combine, ingest, output
# ---------------------------------------------------------------------------


def test_gemm_f16_out_with_bias():
    M, K, N = 300, 512, 1024
    a = synth.normal(16, 0, (M, K), 1.0, np.float16)
    b = synth.normal(16, 1, (N, K), 1.0 / K, np.float16)
    bias = synth.normal(16, 2, (N,), 0.02)
    c = nan_f16((M, N))
    ig.gemm1x1(dev(a), M, K, K, dev(b), N, K, dev(bias), 1.0, c, N, 1)
    got = host(c)
    ref = O.f16(a.astype(np.float64) @ b.astype(np.float64).T + bias)
    # both sides round to f16; near zero the f32 accumulation error is
    # several f16 ulps of a tiny value, so the bar is one ulp of the value
    # or 1e-5 of the output RMS, whichever is larger
    rms = float(np.sqrt(np.mean(ref * ref)))
    ulp = np.abs(np.spacing(ref.astype(np.float16)).astype(np.float64))
    d = np.abs(got.astype(np.float64) - ref)
    assert np.all(d <= np.maximum(ulp, 1e-5 * rms))
    assert np.mean(d == 0) >= 0.99


def test_gemm_long_k_scaled():
    M, K, N = 200, 4096, 128
    a = synth.normal(17, 0, (M, K), 1.0, np.float16)
    b = synth.normal(17, 1, (N, K), 1.0, np.float16)
    c = nan_f32((M, N))
    ig.gemm1x1(dev(a), M, K, K, dev(b), N, K, None, 1.0 / 64, c, N, 0)
    ref = (a.astype(np.float64) @ b.astype(np.float64).T) / 64
    assert conv_err(host(c), ref)[2] <= 1e-4


def test_softmax_rows():
    rows, valid, ncols, ld = 37, 1000, 1024, 1024
    s = synth.normal(18, 0, (rows, ld), 9.0)
    p = nan_f16((rows, ld))
    ig.softmax_rows_f16(dev(s), rows, ld, valid, ncols, p, ld)
    got = host(p)
    ref = O.f16(O.softmax_rows(s[:, :valid]))
    assert np.all(got[:, valid:ncols] == 0)
    u = f16_ulps(got[:, :valid], ref.astype(np.float16))
    assert np.max(u) <= 2 and np.mean(u == 0) >= 0.99


def test_combine_modes():
    M, C = 77, 128
    x0 = synth.normal(19, 0, (M, C), 1.0)
    h = synth.normal(19, 1, (M, C), 1.0)
    s = synth.normal(19, 2, (M, C), 1.0)
    hb = synth.normal(19, 3, (C,), 1.0)
    sb = synth.normal(19, 4, (C,), 1.0)
    for mode, ref in ((0, x0 + h + hb), (1, s + sb + h + hb), (2, h + hb)):
        x = dev(x0)
        ig.combine(x, dev(h), dev(hb), dev(s), dev(sb), M, C, mode)
        assert np.allclose(host(x), ref, rtol=1e-6, atol=1e-6)


def test_latent_ingest_and_output():
    zc, H, W = 16, 5, 7
    z = synth.normal(20, 0, (zc, H, W), 1.0)
    y = nan_f16((H * W, 64))
    ig.latent_to_nhwc_f16(dev(z), zc, H * W, 64, y)
    got = host(y)
    assert np.array_equal(got[:, :zc].astype(np.float64), O.f16(z.reshape(zc, -1).T))
    assert np.all(got[:, zc:] == 0)
    yy = synth.normal(20, 1, (H * W, 64), 1.0)
    b = synth.normal(20, 2, (3,), 1.0)
    out = nan_f32((3, H * W))
    ig.nhwc_to_nchw(dev(yy), H * W, 64, 3, dev(b), out)
    assert np.allclose(host(out), yy[:, :3].T + b[:, None], rtol=1e-7, atol=1e-7)


def test_rejected_call_leaves_output_untouched():
    y = nan_f32((16, 64))
    x = torch.zeros((16, 100), dtype=torch.float16, device="cuda")
    w = torch.zeros((64, 9, 100), dtype=torch.float16, device="cuda")
    with pytest.raises(ig.IgError) as e:
        ig.conv3x3_nhwc(x, 4, 4, 100, w, 64, None, 1.0, y)
    assert e.value.code == -2
    assert torch.isnan(y).all()


# ---------------------------------------------------------------------------
# the single-pass attention core
# ---------------------------------------------------------------------------


def _attn_inputs(m, kind, seed, C=512):
    """q, k [m][C], V^T [C][m], bv: f16 operands with the decoder's
    scale (entries ~ N(0, 1): scores q.k / sqrt(C) ~ N(0, 1)).
    kind: 'flat'; 'growing' (key norms grow along the sequence, so later
    blocks' maxima pass the first block's, the kernel's reference); 'self' (k = q: each query's
    own key dominates by ~sqrt(C) in the exponent)."""
    q = synth.normal(7, seed, (m, C), 1.0, np.float16)
    k = synth.normal(7, seed + 1, (m, C), 1.0, np.float16)
    v = synth.normal(7, seed + 2, (m, C), 1.0, np.float16)
    bv = synth.normal(7, seed + 3, (C,), 0.02, np.float32)
    if kind == "growing":
        k = (k.astype(np.float64) * np.linspace(0.5, 6.0, m)[:, None]).astype(np.float16)
    elif kind == "self":
        k = q.copy()
    return q, k, np.ascontiguousarray(v.T), bv


def _attn_tol(o_ref, p, vt):
    """Per-element bound: f16 rounding of the output (half an ulp, 2^-11
    relative) and of every weight (2^-11 relative, the weights' f16 grid
    relative to the kernel's reference max or to the row sum), each doubled, plus f32
    accumulation slack."""
    pv = np.matmul(p, np.abs(vt.astype(np.float64)).T)
    return 2.0 ** -10 * (np.abs(o_ref) + pv) + 1e-6


def _run_flash(q, k, vt, bv, ld=None):
    m, C = q.shape
    ld = ld or (m + 63) // 64 * 64
    qd = torch.zeros((ld, C), dtype=torch.float16, device="cuda")
    kd = torch.zeros((ld, C), dtype=torch.float16, device="cuda")
    vd = torch.zeros((C, ld), dtype=torch.float16, device="cuda")
    qd[:m] = dev(q)
    kd[:m] = dev(k)
    vd[:, :m] = dev(vt)
    nb = ig.attention_workspace_bytes(m, C)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    out = nan_f16((m, C))
    ig.attention_f16(qd, kd, vd, m, ld, C, dev(bv), ws, nb, out)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


def _check_attn(got_rows, q_rows, k, vt, bv, tag):
    o, p = O.attention_core(q_rows, k, vt, bv)
    tol = _attn_tol(o, p, vt)
    err = np.abs(got_rows - o)
    rms = float(np.sqrt(np.mean(o ** 2)))
    print("%s: max|d| %.3e (RMS %.3e, max|d|/RMS %.2e), worst err/tol %.3f" % (
        tag, float(err.max()), rms, float(err.max()) / rms, float((err / tol).max())), flush=True)
    assert np.all(np.isfinite(got_rows))
    assert np.all(err <= tol)


@pytest.mark.parametrize("m,kind", [(1, "flat"), (100, "flat"), (1024, "flat"), (1500, "growing"),
                                    (4096, "self"), (2000, "self")])
def test_attention_single_pass(m, kind):
    q, k, vt, bv = _attn_inputs(m, kind, seed=10 + m % 7)
    got = _run_flash(q, k, vt, bv)
    rows = np.arange(m) if m <= 2048 else np.unique(np.r_[0:64, m - 64:m, np.linspace(0, m - 1, 128).astype(int)])
    _check_attn(got[rows], q[rows], k, vt, bv, "attention m=%d %s" % (m, kind))


@pytest.mark.parametrize("m", [16384, 32768, 40000])
def test_attention_single_pass_large(m):
    """16384 = the 1024^2 decode's tokens (two key ranges merged); 32768
    runs as one key range per workgroup (no merge); 40000 as three ranges
    (its 313 query blocks fill waves of 256 workgroups best that way)."""
    q, k, vt, bv = _attn_inputs(m, "flat", seed=3)
    got = _run_flash(q, k, vt, bv)
    rows = np.unique(np.r_[0:32, m - 32:m, np.linspace(0, m - 1, 64).astype(int)])
    _check_attn(got[rows], q[rows], k, vt, bv, "attention m=%d" % m)


@pytest.mark.parametrize("C,m,kind", [(128, 1, "flat"), (128, 333, "growing"), (128, 2000, "self"),
                                      (256, 100, "flat"), (256, 1500, "growing"), (256, 4096, "self"),
                                      (384, 64, "flat"), (384, 1000, "growing"), (384, 2048, "self")])
def test_attention_single_pass_other_widths(C, m, kind):
    """Head widths below 512: K rows packed (several per load) with their
    units swizzled in LDS, and the softmax steps spread over fewer P.V
    hooks; the same bound against the plain definition."""
    q, k, vt, bv = _attn_inputs(m, kind, seed=40 + C // 128 + m % 5, C=C)
    got = _run_flash(q, k, vt, bv)
    rows = np.arange(m) if m <= 2048 else np.unique(np.r_[0:64, m - 64:m, np.linspace(0, m - 1, 128).astype(int)])
    _check_attn(got[rows], q[rows], k, vt, bv, "attention C=%d m=%d %s" % (C, m, kind))


@pytest.mark.parametrize("C", [128, 256, 384])
def test_attention_other_widths_with_key_ranges(C):
    """16384 tokens: the keys split into ranges whose partial results the
    merge kernel (C / 4 threads) combines."""
    m = 16384
    assert ig.attention_workspace_bytes(m, C) > 0
    q, k, vt, bv = _attn_inputs(m, "flat", seed=5 + C // 128, C=C)
    got = _run_flash(q, k, vt, bv)
    rows = np.unique(np.r_[0:32, m - 32:m, np.linspace(0, m - 1, 64).astype(int)])
    _check_attn(got[rows], q[rows], k, vt, bv, "attention C=%d m=%d" % (C, m))


def test_attention_chunked_path_meets_the_same_bound():
    """The chunked path (statistics GEMM, row merge, probabilities GEMM,
    P.V) through the decoder's kernels: the same per-element bound against
    the plain definition."""
    m, C = 1000, 512
    q, k, vt, bv = _attn_inputs(m, "growing", seed=21)
    mp = 1024
    qd = torch.zeros((mp, C), dtype=torch.float16, device="cuda")
    kd = torch.zeros((mp, C), dtype=torch.float16, device="cuda")
    vd = torch.zeros((C, mp), dtype=torch.float16, device="cuda")
    qd[:m], kd[:m], vd[:, :m] = dev(q), dev(k), dev(vt)
    S = nan_f32((m, mp))
    ig.gemm1x1(qd, m, C, C, kd, mp, C, None, 1.0 / np.sqrt(C), S, mp, 0)
    P = torch.zeros((m, mp), dtype=torch.float16, device="cuda")
    ig.softmax_rows_f16(S, m, mp, m, mp, P, mp)
    o32 = nan_f32((m, C))
    ig.gemm1x1(P, m, mp, mp, vd, C, mp, None, 1.0, o32, C, 0)
    out = nan_f16((m, C))
    ig.guard_cast(o32, m, C, dev(bv), 0, out)
    _check_attn(host(out).astype(np.float64), q, k, vt, bv, "chunked m=%d" % m)


def test_attention_rejects_other_widths_and_short_workspace():
    for c in (192, 640):
        with pytest.raises(ig.IgError) as e:
            ig.attention_f16(None, None, None, 64, 64, c, None, None, 0, None)
        assert e.value.code == -2
    m = 16384
    need = ig.attention_workspace_bytes(m, 512)
    assert need > 0
    q = torch.zeros((m, 512), dtype=torch.float16, device="cuda")
    out = nan_f16((m, 512))
    with pytest.raises(ig.IgError) as e:
        ig.attention_f16(q, q, q, m, m, 512, None, None, 0, out)
    assert e.value.code == -3
    assert torch.isnan(out).all()
