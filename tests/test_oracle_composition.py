"""An independent pin of the oracle's decoder composition (CPU only).

The pages print the decoder's recipe -- page "cortiq-engine 0.8.3,
src/gpu_wgpu/qi21_vae.rs", `Rec::resnet` (norm, conv1, norm of conv1 + its
bias, conv2, then the shortcut's guarded cast and 1x1 conv and the combine),
`attention` (norm without SiLU, q and k cast with their biases, V^T without
its bias, per-chunk softmax into f16 P, P.V, the cast of O + bv, the
projection added with its bias), `run_blocks` (the guarded cast before each
up conv, undone in its epilogue) and `decode` -- but no values for this
synthetic decoder. This file writes that recipe out a second time, in torch
float64 with library routines only (F.conv2d, F.normalize, F.interpolate,
F.silu, torch.softmax, torch.matmul, F.scaled_dot_product_attention) and
numpy's own float64 -> float16 cast at the f16 sites; it imports nothing from
oracle/ for the transcription. oracle.decode must agree with it to 1e-12
relative, with and without the f16 sites, on the small decoder and on a
256-wide decoder whose up stages change width (1x1 shortcuts).

Each planted slip in the transcription (a bias dropped or added twice, an
f16 site skipped) must move its output by far more than that: the same slip
in the oracle would fail the comparison.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _h(t):
    """binary16 round-to-nearest-even of a float64 tensor (numpy's direct
    float64 -> float16 conversion), back in float64."""
    return torch.from_numpy(t.numpy().astype(np.float16).astype(np.float64))


def _same(t):
    return t


class Recipe:
    """The pages' decoder recipe in torch float64. `skip` names one step to
    get wrong on purpose (the sensitivity checks)."""

    def __init__(self, wts, guard_log2=8, emulate_f16=True, skip=None):
        self.w = wts
        self.g = int(guard_log2)
        self.rnd = _h if emulate_f16 else _same
        self.skip = skip

    def site(self, name, t):
        """An f16 site of the recipe, unless it is the one being skipped."""
        return t if self.skip == name else self.rnd(t)

    @staticmethod
    def conv(x, cw, with_bias=False):
        w = _t(cw["w"])
        b = _t(cw["b"]) if with_bias else None
        return F.conv2d(x[None], w, b, padding=w.shape[-1] // 2)[0]

    @staticmethod
    def rmsn(x, gamma, bias=None, silu=False):
        """RMS_norm over the channels (RMSN_SRC): v / max(|v|_2, 1e-12) *
        sqrt(C) * gamma, bias on read, optional SiLU. x: [C, H, W]."""
        v = x if bias is None else x + _t(bias)[:, None, None]
        y = F.normalize(v, dim=0, eps=1e-12) * math.sqrt(v.shape[0]) * _t(gamma)[:, None, None]
        return F.silu(y) if silu else y

    def norm(self, x, gamma, beta=None, bias=None, silu=False):
        """The decoder's norm site: RMS_norm, or for a decoder whose norm
        is "group" F.group_norm with the site's beta (vae.rs, GroupNorm;
        the device recipe adds the conv bias on read), optional SiLU."""
        nk = self.w.get("norm") or {"kind": "rms"}
        if nk["kind"] == "rms":
            return self.rmsn(x, gamma, bias, silu)
        v = x if bias is None else x + _t(bias)[:, None, None]
        bt = None if self.skip == "beta" else _t(beta)
        y = F.group_norm(v[None], nk["groups"], _t(gamma), bt, eps=nk["eps"])[0]
        return F.silu(y) if silu else y

    def resnet(self, x, r):
        xn = self.site("xn1", self.norm(x, r["g1"], r.get("beta1"), silu=True))
        h = self.conv(xn, r["c1"])
        b1 = None if self.skip == "b1" else r["c1"]["b"]
        xn = self.site("xn2", self.norm(h, r["g2"], r.get("beta2"), bias=b1, silu=True))
        h = self.conv(xn, r["c2"])
        b2 = _t(r["c2"]["b"])[:, None, None]
        if r.get("sc") is None:
            return x + h + b2
        gs = 2.0 ** self.g
        xs = self.site("xs", x / gs)
        s = gs * self.conv(xs, r["sc"])
        bsc = 0.0 if self.skip == "bsc" else _t(r["sc"]["b"])[:, None, None]
        return s + bsc + h + b2

    def attention(self, x):
        a = self.w["attn"]
        C, H, W = x.shape
        m = H * W
        xn = self.site("xna", self.norm(x, a["gamma"], a.get("beta"), silu=False)).reshape(C, m)

        def lin(name):
            return _t(a[name]["w"]).reshape(C, C), _t(a[name]["b"])

        wq, bq = lin("q")
        wk, bk = lin("k")
        wv, bv = lin("v")
        wp, bp = lin("proj")
        q = self.site("q", torch.matmul(wq, xn).T + bq)
        k = self.site("k", torch.matmul(wk, xn).T + bk)
        vt = self.site("vt", torch.matmul(wv, xn))
        p = self.site("p", torch.softmax(torch.matmul(q, k.T) / math.sqrt(C), dim=1))
        o = torch.matmul(p, vt.T)
        if self.rnd is _same and self.skip is None:
            # the same product by another library route
            o2 = F.scaled_dot_product_attention(q[None], k[None], vt.T.contiguous()[None])[0]
            assert torch.allclose(o, o2, rtol=1e-12, atol=1e-13)
        o16 = self.site("o", o + bv)
        h = torch.matmul(wp, o16.T) + bp[:, None]
        if self.skip == "bp2":
            h = h + bp[:, None]
        return x + h.reshape(C, H, W)

    @staticmethod
    def dupup(src, cout, ft):
        """The stage input's channels, each repeated cout 4 ft / cin times,
        grouped [cout][ft][4]; chunk ft - 1 moved to the 2x grid
        (depth-to-space)."""
        cin, h, w = src.shape
        rep = cout * 4 * ft // cin
        e = src.repeat_interleave(rep, dim=0).reshape(cout, ft, 4, h, w)[:, ft - 1]
        return F.pixel_shuffle(e.reshape(1, 4 * cout, h, w), 2)[0]

    def decode(self, z):
        w = self.w
        x = self.conv(self.site("z", _t(z)), w["conv_in"], with_bias=True)
        x = self.resnet(x, w["mid"][0])
        x = self.attention(x)
        x = self.resnet(x, w["mid"][1])
        gs = 2.0 ** self.g
        for st in w["ups"]:
            x_in = x
            for r in st["res"]:
                x = self.resnet(x, r)
            xg = self.site("xg", x / gs)
            u = F.interpolate(xg[None], scale_factor=2, mode="nearest")[0]
            x = gs * self.conv(u, st["up"]) + _t(st["up"]["b"])[:, None, None]
            if st.get("dupup") is not None and self.skip != "dupup":
                x = x + self.dupup(x_in, x.shape[0], st["dupup"]["ft"])
        xn = self.site("xno", self.norm(x, w["norm_out"], w.get("norm_out_beta"), silu=True))
        return self.conv(xn, w["conv_out"], with_bias=True)


def _wide_spec(dupup=False, norm="rms"):
    return synth.DecoderSpec(zc=4, c_in=256, stages=(256, 128, 64), n_res=2, out_c=3, dupup=dupup, norm=norm)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("norm", ["rms", "group"])
@pytest.mark.parametrize("dupup", [False, True])
@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("emulate", [False, True])
def test_decode_matches_the_recipe_transcription(wide, emulate, dupup, norm):
    spec = _wide_spec(dupup, norm) if wide else synth.decoder_spec(small=True, dupup=dupup, norm=norm)
    wts = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(4, 5 if wide else 6, zc=spec.zc)
    got = O.decode(wts, z, guard_log2=8, emulate_f16=emulate)
    want = Recipe(wts, 8, emulate).decode(z).numpy()
    assert got.shape == want.shape
    r = _rel(got, want)
    print("decode vs transcription (wide %s, f16 sites %s, DupUp %s, %s): %.2e" % (wide, emulate, dupup, norm, r))
    assert r <= 1e-12


def test_guarded_stream_matches_the_recipe_transcription():
    """With conv_in scaled by 2^11 the stream passes f16's range at the
    guarded casts; the guard keeps both sides finite and equal."""
    spec = synth.decoder_spec(small=True)
    wts = synth.decoder_weights(spec, seed_config=4, conv_in_gain=2.0 ** 11)
    z = synth.decoder_latent(4, 4, zc=spec.zc, scale=8.0)
    tr = O.Trace()
    got = O.decode(wts, z, guard_log2=8, trace=tr)
    assert max(tr.guard_max) > 65504.0
    want = Recipe(wts, 8, True).decode(z).numpy()
    assert np.all(np.isfinite(want))
    assert _rel(got, want) <= 1e-12


@pytest.mark.parametrize("emulate", [False, True])
def test_attention_matches_the_recipe_transcription(emulate):
    spec = synth.decoder_spec(small=True)
    wts = synth.decoder_weights(spec, seed_config=4)
    C = spec.attn_c
    x = synth.normal(4, 900, (C, 5, 7), 4.0, np.float64)
    got = O.attention(x.reshape(C, 35), wts["attn"], q_chunk=8, emulate_f16=emulate).reshape(C, 5, 7)
    want = Recipe(wts, 8, emulate).attention(_t(x)).numpy()
    assert _rel(got - x, want - x) <= 1e-12


@pytest.mark.parametrize("wide", [False, True])
def test_resnet_matches_the_recipe_transcription(wide):
    spec = _wide_spec() if wide else synth.decoder_spec(small=True)
    wts = synth.decoder_weights(spec, seed_config=4)
    # the first resnet of stage 1 changes the width: a 1x1 shortcut
    r = wts["ups"][1]["res"][0]
    assert r["sc"] is not None
    cin = r["c1"]["w"].shape[1]
    x = synth.normal(4, 901, (cin, 6, 9), 2.0e4, np.float64)
    got = O.resnet(x, r, 8)
    want = Recipe(wts, 8, True).resnet(_t(x), r).numpy()
    assert _rel(got, want) <= 1e-12


@pytest.mark.parametrize("skip", ["b1", "bsc", "bp2", "z", "xn1", "xn2", "xs", "xna", "q", "k", "vt", "p", "o",
                                  "xg", "xno"])
def test_a_slip_in_the_recipe_is_caught(skip):
    """A planted slip moves the decode far past the 1e-12 the oracle is held
    to: a dropped conv1 bias on the second norm's read, a dropped shortcut
    bias, the projection bias added twice, or any single f16 site skipped.
    (On a stream in f16's range: with the stream near 1e5 the attention's
    rounding changes are swallowed by the later f16 sites, so the
    attention's own sites are also checked on the attention alone.)"""
    spec = synth.decoder_spec(small=True)
    wts = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(4, 6, zc=spec.zc)
    good = O.decode(wts, z, guard_log2=8)
    bad = Recipe(wts, 8, True, skip=skip).decode(z).numpy()
    r = _rel(bad, good)
    print("slip %s: %.2e" % (skip, r))
    assert r > 1e-9


@pytest.mark.parametrize("skip", ["beta", "b1", "xn1", "xno"])
def test_a_slip_in_the_group_norm_decoder_is_caught(skip):
    """The GroupNorm decoder: its betas dropped, conv1's bias not added on
    the second norm's read, or an f16 site skipped, each moves the decode
    far past the oracle's 1e-12."""
    spec = synth.decoder_spec(small=True, norm="group")
    wts = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(4, 6, zc=spec.zc)
    good = O.decode(wts, z, guard_log2=8)
    bad = Recipe(wts, 8, True, skip=skip).decode(z).numpy()
    r = _rel(bad, good)
    print("GroupNorm decoder slip %s: %.2e" % (skip, r))
    assert r > 1e-9


def test_a_dropped_dupup_is_caught():
    """With the DupUp shortcut in every up stage, leaving it out of the
    transcription moves the decode far past the oracle's 1e-12."""
    spec = synth.decoder_spec(small=True, dupup=True)
    wts = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(4, 6, zc=spec.zc)
    good = O.decode(wts, z, guard_log2=8)
    bad = Recipe(wts, 8, True, skip="dupup").decode(z).numpy()
    assert _rel(bad, good) > 1e-3


@pytest.mark.parametrize("skip", ["xna", "q", "k", "vt", "p", "o", "bp2"])
def test_a_slip_in_the_attention_is_caught(skip):
    spec = synth.decoder_spec(small=True)
    wts = synth.decoder_weights(spec, seed_config=4)
    C = spec.attn_c
    x = synth.normal(4, 902, (C, 4, 6), 1.0, np.float64)
    good = O.attention(x.reshape(C, 24), wts["attn"]).reshape(C, 4, 6) - x
    bad = Recipe(wts, 8, True, skip=skip).attention(_t(x)).numpy() - x
    r = _rel(bad, good)
    print("attention slip %s: %.2e" % (skip, r))
    assert r > 1e-6
