"""Seeded synthetic inputs for the NHWC implicit-GEMM VAE-decoder path.

This module only draws random numbers. It holds none of the path's
arithmetic (no norm, no convolution, no layout packing, no channel padding),
so both the CPU oracle's tests and the HIP path's tests, benchmark and smoke
run can take their inputs from it without sharing any computation.

Every array comes from ``numpy.random.Generator(PCG64(seed))`` with
``seed = 1000 * config + tensor_index``. Normal draws are made in float64 and
then cast (float16 for weights, float32 for everything else). ``N(0, v)``
means variance ``v`` throughout, so ``N(0, 4)`` has standard deviation 2 and
a bias ``N(0, 0.02)`` has standard deviation about 0.141.

Layouts handed out:

* activations: NHWC float32 ``[H, W, C]`` (the path's layout);
* conv weights: ``[cout, cin, k, k]`` float16 (the usual OIHW order in which
  decoders publish their weights; each side packs or reads it on its own);
* biases and norm scales ``gamma``: float32 ``[C]``;
* decoder latents: NCHW float32 ``[16, h0, w0]`` (the decoder's input).
"""

from __future__ import annotations

import hashlib

import numpy as np

__all__ = [
    "rng",
    "normal",
    "uniform",
    "digest",
    "config1",
    "config2",
    "config3",
    "DecoderSpec",
    "decoder_spec",
    "decoder_weights",
    "decoder_latent",
]


def rng(config: int, index: int) -> np.random.Generator:
    """The generator for tensor ``index`` of ``config``."""
    return np.random.Generator(np.random.PCG64(1000 * int(config) + int(index)))


def normal(config, index, shape, var, dtype=np.float32):
    """``N(0, var)`` (variance ``var``) drawn in float64, cast to ``dtype``."""
    g = rng(config, index)
    return (g.standard_normal(shape) * np.sqrt(var)).astype(dtype)


def uniform(config, index, shape, lo, hi, dtype=np.float32):
    """``U(lo, hi)`` drawn in float64, cast to ``dtype``."""
    g = rng(config, index)
    return g.uniform(lo, hi, shape).astype(dtype)


def digest(a: np.ndarray) -> str:
    """SHA-256 of an array's bytes (logged beside results)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ---------------------------------------------------------------------------
# per-kernel configurations
# ---------------------------------------------------------------------------


def config1(h=64, w=64, c=128):
    """One resnet half-unit: RMS_norm + SiLU -> f16 -> 3x3 conv c -> c.

    x ~ N(0, 1), gamma ~ U(0.5, 1.5), W ~ N(0, 1/(9c)) f16, b ~ N(0, 0.02).
    """
    return {
        "x": normal(1, 0, (h, w, c), 1.0),
        "gamma": uniform(1, 1, (c,), 0.5, 1.5),
        "w": normal(1, 2, (c, c, 3, 3), 1.0 / (9 * c), np.float16),
        "b": normal(1, 3, (c,), 0.02),
    }


def config2(h=128, w=128, c=256, guard_log2=8):
    """Guarded cast -> nearest-2x conv c -> c, plus a 1x1 shortcut c -> c.

    x ~ N(0, 4); W_up ~ N(0, 1/(9c)); W_sc ~ N(0, 1/c); biases ~ N(0, 0.02).
    """
    return {
        "x": normal(2, 0, (h, w, c), 4.0),
        "w_up": normal(2, 1, (c, c, 3, 3), 1.0 / (9 * c), np.float16),
        "b_up": normal(2, 2, (c,), 0.02),
        "w_sc": normal(2, 3, (c, c, 1, 1), 1.0 / c, np.float16),
        "b_sc": normal(2, 4, (c,), 0.02),
        "guard_log2": guard_log2,
    }


_CFG3_INDEX = {128: 0, 288: 10, 144: 20}


def config3(c=128, h=512, w=512):
    """Large-tile conv: x ~ N(0, 1) (normalised by the path with gamma = 1),
    W ~ N(0, 1/(9c)) f16, b ~ N(0, 0.02). ``c`` is the real channel count
    (128, or 288 / 144 for the variants stored with padded channels)."""
    base = _CFG3_INDEX.get(c, 30)
    return {
        "x": normal(3, base + 0, (h, w, c), 1.0),
        "gamma": np.ones((c,), np.float32),
        "w": normal(3, base + 1, (c, c, 3, 3), 1.0 / (9 * c), np.float16),
        "b": normal(3, base + 2, (c,), 0.02),
    }


# ---------------------------------------------------------------------------
# the synthetic decoder
# ---------------------------------------------------------------------------


class DecoderSpec:
    """Shape of the synthetic decoder: latent channels, conv_in width, the
    channel count of each up stage, resnets per stage, output channels."""

    def __init__(self, zc=16, c_in=512, stages=(512, 256, 128), n_res=2, out_c=3, dupup=False, norm="rms",
                 groups=32, eps=1e-6):
        self.zc = zc
        self.c_in = c_in
        self.stages = tuple(stages)
        self.n_res = n_res
        self.out_c = out_c
        self.attn_c = c_in
        self.dupup = bool(dupup)  # every up stage adds the DupUp shortcut of its input (ft = 1)
        # every norm site: RMS_norm, or GroupNorm(groups, eps) with a beta
        # (a FLUX-class decoder)
        assert norm in ("rms", "group")
        self.norm = norm
        self.groups = int(groups)
        self.eps = float(eps)

    def as_dict(self):
        return {
            "zc": self.zc,
            "c_in": self.c_in,
            "stages": list(self.stages),
            "n_res": self.n_res,
            "out_c": self.out_c,
            "dupup": self.dupup,
            "norm": self.norm,
        }


def decoder_spec(small=False, dupup=False, norm="rms"):
    """The decoder of the full-decode configurations, or a narrow copy with
    the same structure for CPU-sized tests; dupup: the up stages also add
    the DupUp shortcut of their input (stage channel pairs (in, out) then
    take repeats 4 when in == out and 2 when in == 2 out); norm "group":
    GroupNorm(32, 1e-6) at every norm site instead of RMS_norm."""
    if small:
        return DecoderSpec(zc=4, c_in=128, stages=(128, 64, 64), n_res=2, out_c=3, dupup=dupup, norm=norm)
    return DecoderSpec(dupup=dupup, norm=norm)


def _conv(cfg, idx, cout, cin, k, gain=1.0):
    w = normal(cfg, idx, (cout, cin, k, k), 1.0 / (k * k * cin), np.float64)
    return {
        "w": (w * gain).astype(np.float16),
        "b": normal(cfg, idx + 1, (cout,), 0.02),
    }


def _gamma(cfg, idx, c):
    return uniform(cfg, idx, (c,), 0.5, 1.5)


def _resnet(cfg, idx, cin, cout, group_norm=False):
    r = {
        "g1": _gamma(cfg, idx, cin),
        "c1": _conv(cfg, idx + 1, cout, cin, 3),
        "g2": _gamma(cfg, idx + 3, cout),
        "c2": _conv(cfg, idx + 4, cout, cout, 3),
        "sc": None,
    }
    if cin != cout:
        r["sc"] = _conv(cfg, idx + 6, cout, cin, 1)
    if group_norm:
        r["beta1"] = normal(cfg, idx + 8, (cin,), 0.02)
        r["beta2"] = normal(cfg, idx + 9, (cout,), 0.02)
    return r


def decoder_weights(spec: DecoderSpec, seed_config=4, conv_in_gain=1.0):
    """Weights of the synthetic decoder.

    3x3 convs ~ N(0, 1/(9 cin)), 1x1 convs and attention projections
    ~ N(0, 1/cin), biases (and GroupNorm's betas) ~ N(0, 0.02), gammas
    ~ U(0.5, 1.5), every weight rounded to f16. ``conv_in_gain`` (a power of two) scales conv_in's
    weights; the full-decode configuration uses it to push the residual
    stream past the f16 range.
    """
    cfg = seed_config
    idx = 100
    d = {"spec": spec.as_dict()}
    gn = spec.norm == "group"
    d["norm"] = {"kind": "group", "groups": spec.groups, "eps": spec.eps} if gn else {"kind": "rms"}
    d["conv_in"] = _conv(cfg, idx, spec.c_in, spec.zc, 3, conv_in_gain)
    idx += 10
    d["mid"] = []
    for _ in range(2):
        d["mid"].append(_resnet(cfg, idx, spec.c_in, spec.c_in, gn))
        idx += 10
    c = spec.attn_c
    d["attn"] = {"gamma": _gamma(cfg, idx, c)}
    for j, name in enumerate(("q", "k", "v", "proj")):
        d["attn"][name] = _conv(cfg, idx + 1 + 2 * j, c, c, 1)
    if gn:
        d["attn"]["beta"] = normal(cfg, idx + 9, (c,), 0.02)
    idx += 10
    d["ups"] = []
    prev = spec.c_in
    for cs in spec.stages:
        st = {"res": []}
        for r in range(spec.n_res):
            st["res"].append(_resnet(cfg, idx, prev if r == 0 else cs, cs, gn))
            idx += 10
        st["up"] = _conv(cfg, idx, cs, cs, 3)
        st["dupup"] = {"ft": 1} if spec.dupup else None
        idx += 10
        d["ups"].append(st)
        prev = cs
    d["norm_out"] = _gamma(cfg, idx, prev)
    d["conv_out"] = _conv(cfg, idx + 1, spec.out_c, prev, 3)
    if gn:
        d["norm_out_beta"] = normal(cfg, idx + 3, (prev,), 0.02)
    return d


def decoder_latent(h0, w0, zc=16, config=4, scale=1.0):
    """The decoder's NCHW f32 latent ``[zc, h0, w0]`` ~ N(0, 1) * scale."""
    z = normal(config, 0, (zc, h0, w0), 1.0, np.float64) * scale
    return z.astype(np.float32)
