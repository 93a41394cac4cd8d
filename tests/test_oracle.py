"""Pins of the CPU oracle against values it does not produce itself:
library routines (numpy's binary16 casts, torch's float64 conv2d, normalize,
interpolate, silu and scaled-dot-product attention), closed forms,
invariants, and the worked values the pages print (tests/golden/)."""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# f16 rounding
# ---------------------------------------------------------------------------


def test_f16_every_finite_half_is_a_fixed_point():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    v = h[np.isfinite(h)].astype(np.float64)
    r = O.f16(v)
    # bit-for-bit, so the sign of zero counts too
    assert np.array_equal(r.view(np.uint64), v.view(np.uint64))


@pytest.mark.parametrize("src", ["f32", "f64"])
def test_f16_matches_numpy_casts(src):
    g = np.random.default_rng(11)
    if src == "f32":
        bits = g.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
    else:
        # wide exponent spread around the binary16 range, plus exact ties
        e = g.integers(-30, 18, 1_000_000)
        m = g.random(1_000_000) + 1.0
        v = m * np.exp2(e.astype(np.float64)) * np.where(g.random(1_000_000) < 0.5, -1, 1)
        ties = (np.arange(1, 4097, dtype=np.float64) + 0.5) * 2.0 ** -10
        v = np.concatenate([v, ties, -ties, ties * 2.0 ** -14])
    v = v[~np.isnan(v)]
    ref = v.astype(np.float16).astype(np.float64)
    got = O.f16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_f16_closed_form_cases():
    u = 2.0 ** -10
    cases = [
        (1.0 + u / 2, 1.0),  # tie -> even
        (1.0 + 1.5 * u, 1.0 + 2 * u),  # tie -> even (up)
        (65504.0, 65504.0),
        (65519.0, 65504.0),
        (65520.0, math.inf),  # tie between 65504 and 2^16 -> overflow
        (-65520.0, -math.inf),
        (2.0 ** -25, 0.0),  # half the smallest subnormal -> even (0)
        (3 * 2.0 ** -25, 2.0 ** -23),
        (2.0 ** -24 * 1.25, 2.0 ** -24),
        (2.0 ** -14 - 2.0 ** -25, 2.0 ** -14),  # rounds up into the normals
    ]
    for v, want in cases:
        assert O.f16_scalar(v) == want, v


# ---------------------------------------------------------------------------
# convolution
# ---------------------------------------------------------------------------


def test_conv_hand_case_from_pages():
    g = _gold("conv_hand_case.json")
    x = np.array(g["x"], np.float64).reshape(1, g["h"], g["w"])
    w = np.array(g["weight"], np.float64).reshape(1, 1, 3, 3)
    y = O.conv2d(x, w, np.array([g["bias"]])).reshape(-1)
    for idx, val in g["expect"].items():
        assert y[int(idx)] == val


@pytest.mark.parametrize("k", [1, 3])
def test_conv_matches_torch_f64(k):
    g = np.random.default_rng(1)
    x = g.standard_normal((3, 6, 7))
    w = g.standard_normal((5, 3, k, k))
    b = g.standard_normal(5)
    y = O.conv2d(x, w, b)
    ref = F.conv2d(torch.from_numpy(x)[None], torch.from_numpy(w), torch.from_numpy(b),
                   padding=k // 2)[0].numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_conv_delta_and_shift_kernels():
    g = np.random.default_rng(2)
    x = g.standard_normal((4, 5, 6))
    w = np.zeros((4, 4, 3, 3))
    for i in range(4):
        w[i, i, 1, 1] = 1.0
    assert np.array_equal(O.conv2d(x, w), x)
    # tap (0, 0) reads the pixel up-left: y[r][c] = x[r-1][c-1], zero border
    w = np.zeros((1, 4, 3, 3))
    w[0, 2, 0, 0] = 1.0
    y = O.conv2d(x, w)[0]
    want = np.zeros((5, 6))
    want[1:, 1:] = x[2, :-1, :-1]
    assert np.array_equal(y, want)


def test_conv_constant_input_closed_form():
    g = np.random.default_rng(3)
    w = g.standard_normal((2, 3, 3, 3))
    b = np.array([0.25, -1.0])
    y = O.conv2d(np.ones((3, 4, 5)), w, b)
    s = w.sum(axis=1)  # [2, 3, 3]: per-tap weight sum over input channels
    for o in range(2):
        assert np.isclose(y[o, 2, 2], b[o] + s[o].sum(), rtol=1e-13)
        assert np.isclose(y[o, 0, 0], b[o] + s[o, 1:, 1:].sum(), rtol=1e-13)
        assert np.isclose(y[o, 3, 4], b[o] + s[o, :2, :2].sum(), rtol=1e-13)
        assert np.isclose(y[o, 0, 2], b[o] + s[o, 1:, :].sum(), rtol=1e-13)


def test_conv_zero_channel_padding_is_exact():
    g = np.random.default_rng(4)
    x = g.standard_normal((3, 5, 4))
    w = g.standard_normal((2, 3, 3, 3))
    b = g.standard_normal(2)
    xp = np.zeros((5, 5, 4))
    xp[:3] = x
    wp = np.zeros((4, 5, 3, 3))
    wp[:2, :3] = w
    bp = np.zeros(4)
    bp[:2] = b
    y = O.conv2d(x, w, b)
    yp = O.conv2d(xp, wp, bp)
    assert np.array_equal(yp[:2], y)
    assert np.array_equal(yp[2:], np.zeros_like(yp[2:]))


def test_conv_at_equals_full_conv():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 5, 7))
    w = g.standard_normal((4, 3, 3, 3))
    b = g.standard_normal(4)
    pix = np.array([0, 6, 17, 34, 28])
    full = O.conv2d(x, w, b).reshape(4, -1)
    assert np.array_equal(O.conv2d_at(x, w, pix, b), full[:, pix].T)
    fu = O.conv2d_up2(x, w, b).reshape(4, -1)
    pix2 = np.array([0, 13, 14, 27, 100, 139])
    assert np.array_equal(O.conv2d_at(x, w, pix2, b, up2=True), fu[:, pix2].T)


# ---------------------------------------------------------------------------
# upsample and the folded gather
# ---------------------------------------------------------------------------


def test_upsample_from_pages():
    g = _gold("upsample_nearest.json")
    x = np.array(g["x"], np.float64).reshape(g["c"], g["h"], g["w"])
    assert O.upsample2x(x).reshape(-1).tolist() == g["expect"]


def test_upsample_matches_torch_nearest():
    x = np.random.default_rng(6).standard_normal((3, 4, 5))
    ref = F.interpolate(torch.from_numpy(x)[None], scale_factor=2, mode="nearest")[0].numpy()
    assert np.array_equal(O.upsample2x(x), ref)


def test_folded_upsample_conv_equals_upsample_then_conv():
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 5, 4))
    w = g.standard_normal((2, 3, 3, 3))
    b = g.standard_normal(2)
    folded = O.conv2d_up2(x, w, b)
    explicit = O.conv2d(O.upsample2x(x), w, b)
    assert np.array_equal(folded, explicit)
    ref = F.conv2d(F.interpolate(torch.from_numpy(x)[None], scale_factor=2, mode="nearest"),
                   torch.from_numpy(w), torch.from_numpy(b), padding=1)[0].numpy()
    assert np.max(np.abs(folded - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------------------
# RMS_norm
# ---------------------------------------------------------------------------


def _torch_rms(x, gamma, bias=None, silu=False):
    v = torch.from_numpy(x)
    if bias is not None:
        v = v + torch.from_numpy(bias)[:, None]
    c = v.shape[0]
    y = F.normalize(v, p=2.0, dim=0, eps=1e-12) * math.sqrt(c) * torch.from_numpy(gamma)[:, None]
    if silu:
        y = F.silu(y)
    return y.numpy()


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_rmsnorm_matches_torch_normalize(silu, with_bias):
    g = np.random.default_rng(8)
    x = g.standard_normal((24, 50)) * 3
    gamma = g.uniform(0.5, 1.5, 24)
    b = g.standard_normal(24) if with_bias else None
    y = O.rmsnorm(x, gamma, bias=b, silu=silu)
    ref = _torch_rms(x, gamma, b, silu)
    assert np.max(np.abs(y - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


def test_rmsnorm_invariants():
    g = np.random.default_rng(9)
    c = 37
    x = g.standard_normal((c, 40)) * 5
    ones = np.ones(c)
    y = O.rmsnorm(x, ones)
    assert np.allclose(np.linalg.norm(y, axis=0), math.sqrt(c), rtol=1e-12)
    assert np.allclose(O.rmsnorm(x * 7.5, ones), y, rtol=1e-12)
    # an all-zero pixel normalises to zero; a tiny one hits the eps clamp
    x[:, 3] = 0.0
    x[:, 4] = 1e-20
    y = O.rmsnorm(x, ones)
    assert np.all(y[:, 3] == 0.0)
    assert np.allclose(y[:, 4], 1e-20 * math.sqrt(c) / 1e-12, rtol=1e-12)
    # one channel: sign(v) * gamma
    v = np.array([[-3.0, 0.5, 2.0]])
    assert np.array_equal(O.rmsnorm(v, np.array([1.5])), np.array([[-1.5, 1.5, 1.5]]))
    # the bias is added on read
    b = g.standard_normal(c)
    assert np.allclose(O.rmsnorm(x, ones, bias=b), O.rmsnorm(x + b[:, None], ones), rtol=1e-13)


# ---------------------------------------------------------------------------
# the range guard
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("gl2", [0, 8, 14])
def test_guard_is_exact_on_the_normal_range(gl2):
    g = np.random.default_rng(10)
    lo, hi = 2.0 ** (gl2 - 14), 65504.0
    x = np.exp(g.uniform(np.log(lo), np.log(hi), 200_000)) * np.where(g.random(200_000) < .5, -1, 1)
    assert np.array_equal(O.guard_cast(x, gl2) * 2.0 ** gl2, O.f16(x))


def test_guard_subnormal_error_and_overflow():
    g = np.random.default_rng(12)
    gl2 = 8
    x = g.uniform(-1, 1, 100_000) * 2.0 ** (gl2 - 14)
    err = np.abs(O.guard_cast(x, gl2) * 2.0 ** gl2 - x)
    assert np.max(err) <= 2.0 ** (gl2 - 25)
    big = np.array([7.0e4, -1.5e5, 65504.0 * 256])
    assert np.all(np.isinf(O.f16(big)))
    back = O.guard_cast(big, gl2) * 2.0 ** gl2
    assert np.all(np.isfinite(back))
    assert np.allclose(back, big, rtol=2.0 ** -11)
    bias = np.array([1.0, 2.0, 3.0])
    assert np.array_equal(O.guard_cast(big, gl2, bias), O.guard_cast(big + bias, gl2))


# ---------------------------------------------------------------------------
# GroupNorm (the NEXT variant for FLUX-class decoders)
# ---------------------------------------------------------------------------


def test_group_norm_hand_case_from_pages():
    g = _gold("group_norm_case.json")
    x = np.array(g["x"], np.float64).reshape(2, g["h"], g["w"])
    y = O.group_norm(x, g["groups"], np.array(g["weight"]), np.array(g["bias"])).ravel()
    for k, v in g["expect"].items():
        assert abs(y[int(k)] - v) < g["tol"][k], (k, y[int(k)], v)


@pytest.mark.parametrize("c,groups,with_bias,silu", [(64, 32, False, False), (128, 32, True, False),
                                                     (96, 8, True, True), (6, 3, False, True)])
def test_group_norm_matches_torch_f64(c, groups, with_bias, silu):
    rng = np.random.default_rng(c + groups)
    x = rng.standard_normal((c, 7, 9)) * 3 + rng.standard_normal((c, 1, 1)) * 5
    gamma = rng.uniform(0.5, 1.5, c)
    beta = rng.standard_normal(c) * 0.1
    b = rng.standard_normal(c) * 0.3 if with_bias else None
    got = O.group_norm(x, groups, gamma, beta, bias=b, silu=silu)
    xt = torch.from_numpy(x if b is None else x + b[:, None, None])[None]
    ref = F.group_norm(xt, groups, torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-6)
    if silu:
        ref = F.silu(ref)
    assert np.allclose(got, ref[0].numpy(), rtol=1e-12, atol=1e-12)


def test_group_norm_invariants():
    rng = np.random.default_rng(5)
    c, groups = 32, 4
    x = rng.standard_normal((c, 6, 5)) * 2 + 7
    one, zero = np.ones(c), np.zeros(c)
    y = O.group_norm(x, groups, one, zero).reshape(groups, -1)
    var = x.reshape(groups, -1).var(axis=1)
    # each group: mean 0, variance var / (var + eps)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + 1e-6), rtol=1e-12)
    # a per-group shift changes nothing
    shift = np.repeat(rng.standard_normal(groups) * 10, c // groups)[:, None, None]
    assert np.allclose(O.group_norm(x + shift, groups, one, zero), O.group_norm(x, groups, one, zero), atol=1e-10)
    # one group per channel is per-channel standardisation
    y1 = O.group_norm(x, c, one, zero)
    xr = x.reshape(c, -1)
    ref = (xr - xr.mean(axis=1, keepdims=True)) / np.sqrt(xr.var(axis=1, keepdims=True) + 1e-6)
    assert np.allclose(y1.reshape(c, -1), ref, atol=1e-12)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def _attn_weights(g, c):
    a = {"gamma": g.uniform(0.5, 1.5, c)}
    for n in ("q", "k", "v", "proj"):
        a[n] = {"w": g.standard_normal((c, c, 1, 1)) / math.sqrt(c), "b": g.standard_normal(c) * .1}
    return a


def test_attention_matches_torch_sdpa_without_f16():
    g = np.random.default_rng(13)
    c, m = 16, 40
    x = g.standard_normal((c, m)) * 2
    a = _attn_weights(g, c)
    got = O.attention(x, a, q_chunk=7, emulate_f16=False)
    xn = F.normalize(torch.from_numpy(x), dim=0, eps=1e-12) * math.sqrt(c) * torch.from_numpy(a["gamma"])[:, None]

    def lin(n):
        w = torch.from_numpy(a[n]["w"].reshape(c, c))
        return xn.T @ w.T + torch.from_numpy(a[n]["b"])  # [m, c]

    o = F.scaled_dot_product_attention(lin("q")[None], lin("k")[None], lin("v")[None])[0]
    wp = torch.from_numpy(a["proj"]["w"].reshape(c, c))
    ref = (torch.from_numpy(x) + (o @ wp.T + torch.from_numpy(a["proj"]["b"])).T).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_attention_closed_forms():
    g = np.random.default_rng(14)
    c, m = 8, 16
    a = _attn_weights(g, c)
    # identical keys (Wk = 0): P is uniform, 1/16 is exact in f16, so
    # O = mean of the V rows (before the deferred bias)
    a["k"]["w"] = np.zeros_like(a["k"]["w"])
    x = g.standard_normal((c, m))
    got = O.attention(x, a, emulate_f16=True)
    xn = O.f16(O.rmsnorm(x, a["gamma"]))
    vt = O.f16(a["v"]["w"].reshape(c, c) @ xn)
    o = O.f16(vt.mean(axis=1) + a["v"]["b"])
    h = a["proj"]["w"].reshape(c, c) @ o + a["proj"]["b"]
    assert np.allclose(got, x + h[:, None], rtol=1e-13, atol=1e-13)
    # one token: softmax of one score is 1, so O = V
    x1 = g.standard_normal((c, 1))
    a2 = _attn_weights(g, c)
    got = O.attention(x1, a2, emulate_f16=False)
    xn = O.rmsnorm(x1, a2["gamma"])
    v = a2["v"]["w"].reshape(c, c) @ xn[:, 0] + a2["v"]["b"]
    h = a2["proj"]["w"].reshape(c, c) @ v + a2["proj"]["b"]
    assert np.allclose(got[:, 0], x1[:, 0] + h, rtol=1e-13)


def test_attention_query_chunks_change_nothing():
    g = np.random.default_rng(15)
    c, m = 8, 33
    a = _attn_weights(g, c)
    x = g.standard_normal((c, m))
    ref = O.attention(x, a, q_chunk=None)
    for ch in (1, 5, 32):
        assert np.allclose(O.attention(x, a, q_chunk=ch), ref, rtol=0, atol=1e-13)


def test_attention_core_matches_torch_sdpa():
    g = np.random.default_rng(17)
    m, c = 37, 24
    q, k = g.standard_normal((m, c)) * 2, g.standard_normal((m, c)) * 2
    v = g.standard_normal((m, c))
    bv = g.standard_normal(c)
    o, p = O.attention_core(q, k, v.T, bv)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t)[None] for t in (q, k, v)))[0].numpy() + bv
    assert np.max(np.abs(o - ref)) <= 1e-13 * np.max(np.abs(ref))
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-14)


def test_attention_core_closed_forms():
    g = np.random.default_rng(18)
    m, c = 20, 8
    v = g.standard_normal((m, c))
    # identical keys: uniform weights, O = the mean of the V rows
    k = np.tile(g.standard_normal(c), (m, 1))
    o, p = O.attention_core(g.standard_normal((m, c)), k, v.T)
    assert np.allclose(o, np.tile(v.mean(axis=0), (m, 1)), rtol=0, atol=1e-14)
    # one key: O = V
    o1, _ = O.attention_core(g.standard_normal((1, c)), g.standard_normal((1, c)), v[:1].T)
    assert np.allclose(o1[0], v[0], rtol=0, atol=1e-15)
    # a dominant key (scores 60 apart after the scale): O is that key's row
    q = np.zeros((m, c))
    q[:, 0] = 1.0
    k = np.zeros((m, c))
    k[:, 0] = np.arange(m) * (60.0 * np.sqrt(c))
    o, _ = O.attention_core(q, k, v.T)
    assert np.allclose(o, np.tile(v[-1], (m, 1)), rtol=0, atol=1e-20 + 1e-12)
    # a common shift of the scores changes nothing (q gains a component
    # along a direction all keys share)
    q = g.standard_normal((m, c))
    k = g.standard_normal((m, c))
    k[:, -1] = 1.0
    q2 = q.copy()
    q2[:, -1] += 7.0
    assert np.allclose(O.attention_core(q2, k, v.T)[0], O.attention_core(q, k, v.T)[0], rtol=1e-12, atol=1e-13)


def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = np.random.default_rng(16).standard_normal((5, 9)) * 20
    p = O.softmax_rows(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-15)
    assert np.allclose(O.softmax_rows(s + 1000.0), p, rtol=1e-12)
    ref = torch.softmax(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(p, ref, rtol=1e-13)


# ---------------------------------------------------------------------------
# metrics
# ---------------------------------------------------------------------------


def test_psnr_closed_forms():
    a = np.linspace(-0.9, 0.9, 300).reshape(3, 10, 10)
    assert O.psnr_u8(a, a) == math.inf
    b = a + 1.0 / 127.5  # exactly one u8 level everywhere
    assert abs(O.psnr_u8(a, b) - 20 * math.log10(255.0)) < 1e-9
