"""CPU oracle for the resident image-VAE decoder's conv path.

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it; the HIP library and its Python binding
never import it, and it imports nothing from them.

What it computes is the plain definition of each step, in float64, NCHW:

* the loops (convolution, upsample, RMS_norm, f16 rounding) are plain C in
  ``oracle.c``, built here with gcc;
* attention and the decoder's composition are numpy, with ``numpy.matmul``
  as the only library step (a matrix product);
* f16 rounding is applied exactly at the sites where the path stores f16:
  conv inputs after a norm or a cast, the latent, q, k, V^T and P in the
  attention and its output before the projection (page "cortiq-engine 0.8.3,
  src/gpu_wgpu/qi21_vae.rs": module doc and `attention`).

Sources (the pages are cited by title and item):

* qi21_vae.rs (cortiq-engine 0.8.3): module doc; RMSN_SRC; CAST_SRC;
  `guard`; `Rec::resnet`; `attention`; `run_blocks`; `output_rows`; `decode`.
* vae.rs (cortiq-engine 0.7.6): `Conv2d::apply`; `upsample2x`; `silu` (the
  SiLU inside ``rmsnorm``);
  `AttnBlock::apply`; `VaeDecoder::decode`; `GroupNorm::apply`; its unit
  tests.
* qi21_vae.rs, the bands section: which rows a band of the up path needs
  (exact dependency sets; pinned by the pages' walk-back test and by banded
  evaluation of a 1-D decoder).

Parity status: every function here is pinned by ``tests/test_oracle.py``
(library routines, closed forms, invariants, the pages' own worked values).
The synthetic decoder as a whole (``decode``, with ``resnet`` and
``attention``) has no value printed on the pages; its composition -- the
order of the steps, the bias sites, the f16 sites, the DupUp shortcut -- is
pinned by ``tests/test_oracle_composition.py`` against a second, independent
transcription of the pages' recipe in torch float64 built from library
routines only, together with planted slips that this comparison catches.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(force=False):
    """Compile ``oracle.c`` with gcc (IEEE semantics: no fast-math, no FMA
    contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            lib.orc_f16_round.restype = ctypes.c_double
            lib.orc_f16_round.argtypes = [ctypes.c_double]
            lib.orc_f16_round_n.argtypes = [_D, _D, ctypes.c_int64]
            lib.orc_conv2d.argtypes = [_D, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D,
                                       ctypes.c_int, ctypes.c_int, _D, _D]
            lib.orc_conv2d_up2.argtypes = [_D, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D,
                                           ctypes.c_int, _D, _D]
            lib.orc_upsample2x.argtypes = [_D, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D]
            lib.orc_conv2d_at.argtypes = [_D, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _I64,
                                          ctypes.c_int64, _D]
            lib.orc_rmsnorm.argtypes = [_D, ctypes.c_int, ctypes.c_int64, _D, _D, ctypes.c_int,
                                        ctypes.c_double, _D]
            _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


# ---------------------------------------------------------------------------
# elementwise
# ---------------------------------------------------------------------------


def f16_scalar(v: float) -> float:
    """binary16 round-to-nearest-even of one value (oracle.c)."""
    return _load().orc_f16_round(float(v))


def f16(a) -> np.ndarray:
    """binary16 round-to-nearest-even of every element, returned as float64."""
    a = _f64(a)
    out = np.empty_like(a)
    _load().orc_f16_round_n(_p(a), _p(out), a.size)
    return out


def guard_cast(x, guard_log2, bias=None):
    """The range-guarded f16 cast of the raw residual stream (qi21_vae.rs,
    `guard`, CAST_SRC): f16((x + b) * 2^-g). The consumer multiplies its f32
    result by 2^g."""
    v = _f64(x)
    if bias is not None:
        v = v + _bcast(bias, v)
    return f16(v * (2.0 ** -int(guard_log2)))


def _bcast(b, v):
    """A per-channel vector against an NCHW-like array [c, ...]."""
    b = _f64(b)
    return b.reshape((-1,) + (1,) * (v.ndim - 1))


# ---------------------------------------------------------------------------
# convolutions (NCHW)
# ---------------------------------------------------------------------------


def conv2d(x, w, b=None):
    """x [ci,h,w] (*) w [co,ci,k,k] (+ b [co]): stride 1, zero pad k/2
    (vae.rs, `Conv2d::apply`)."""
    x = _f64(x)
    w = _f64(w)
    ci, h, wd = x.shape
    co, ci2, k, k2 = w.shape
    assert ci == ci2 and k == k2 and k in (1, 3)
    y = np.empty((co, h, wd), np.float64)
    bb = None if b is None else _f64(b)
    _load().orc_conv2d(_p(x), ci, h, wd, _p(w), co, k, _p(bb), _p(y))
    return y


def upsample2x(x):
    """Nearest 2x: y[c][r][q] = x[c][r//2][q//2] (vae.rs, `upsample2x`)."""
    x = _f64(x)
    c, h, w = x.shape
    y = np.empty((c, 2 * h, 2 * w), np.float64)
    _load().orc_upsample2x(_p(x), c, h, w, _p(y))
    return y


def conv2d_up2(x, w, b=None):
    """3x3 conv of the nearest-2x upsampled x with the upsample folded into
    the gather (qi21_vae.rs module doc, `Rec::conv_s` with `up`)."""
    x = _f64(x)
    w = _f64(w)
    ci, h, wd = x.shape
    co, ci2, k, _ = w.shape
    assert ci == ci2 and k == 3
    y = np.empty((co, 2 * h, 2 * wd), np.float64)
    bb = None if b is None else _f64(b)
    _load().orc_conv2d_up2(_p(x), ci, h, wd, _p(w), co, _p(bb), _p(y))
    return y


def conv2d_at(x, w, pix, b=None, up2=False):
    """Conv outputs at chosen output pixels (flat row-major indices of the
    output grid) -> [npix, co]."""
    x = _f64(x)
    w = _f64(w)
    ci, h, wd = x.shape
    co, ci2, k, _ = w.shape
    assert ci == ci2
    pix = np.ascontiguousarray(pix, dtype=np.int64)
    y = np.empty((pix.size, co), np.float64)
    bb = None if b is None else _f64(b)
    _load().orc_conv2d_at(_p(x), ci, h, wd, _p(w), co, k, int(bool(up2)), _p(bb),
                          pix.ctypes.data_as(_I64), pix.size, _p(y))
    return y


# ---------------------------------------------------------------------------
# RMS_norm
# ---------------------------------------------------------------------------


def rmsnorm(x, gamma, bias=None, silu=False, eps=1e-12):
    """Per-pixel RMS_norm over the channels (qi21_vae.rs, RMSN_SRC):
    v = x + b; y = v * sqrt(C) / max(||v||_2, eps) * gamma; optional SiLU.
    x: [c, ...] channel-first; C = c (the real channel count)."""
    x = _f64(x)
    c = x.shape[0]
    p = x.size // c
    y = np.empty_like(x)
    g = _f64(gamma)
    assert g.size == c
    bb = None if bias is None else _f64(bias)
    _load().orc_rmsnorm(_p(x), c, p, _p(bb), _p(g), int(bool(silu)), float(eps), _p(y))
    return y


# ---------------------------------------------------------------------------
# GroupNorm
# ---------------------------------------------------------------------------


def group_norm(x, groups, gamma, beta, bias=None, silu=False, eps=1e-6):
    """GroupNorm over channel groups (vae.rs, `GroupNorm::apply`): the
    channels split into `groups` consecutive groups of c / groups; per group,
    over all of its channels and pixels, mean and population variance (the
    mean of (v - mean)^2), then y = (v - mean) / sqrt(var + eps) * gamma +
    beta. The device recipe of page "cortiq-engine 0.8.72,
    src/gpu_wgpu/s2v_vae.rs" (GN_PART_SRC, GN_APPLY_SRC, `gn`) adds a bias
    on read (v = x + b) and an optional SiLU. x: [c, ...] channel-first."""
    x = _f64(x)
    c = x.shape[0]
    assert c % groups == 0
    per = c // groups
    v = x.reshape(c, -1).copy()
    if bias is not None:
        v += _f64(bias)[:, None]
    g = _f64(gamma)
    bt = _f64(beta)
    y = np.empty_like(v)
    for k in range(groups):
        span = v[k * per:(k + 1) * per]
        n = span.size
        mean = span.sum() / n
        var = ((span - mean) ** 2).sum() / n
        inv = 1.0 / np.sqrt(var + eps)
        y[k * per:(k + 1) * per] = (span - mean) * inv * g[k * per:(k + 1) * per, None] + bt[k * per:(k + 1) * per, None]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y.reshape(x.shape)


def norm_site(x, gamma, beta=None, bias=None, silu=False, norm=None):
    """A norm site of the decoder: RMS_norm (norm None or kind "rms"), or,
    for a FLUX-class decoder (vae.rs, `VaeDecoder::decode`), GroupNorm with
    the site's beta (norm {"kind": "group", "groups", "eps"})."""
    if norm is None or norm.get("kind", "rms") == "rms":
        return rmsnorm(x, gamma, bias=bias, silu=silu)
    return group_norm(x, norm["groups"], gamma, beta, bias=bias, silu=silu, eps=norm["eps"])


# ---------------------------------------------------------------------------
# attention (single head over the pixels)
# ---------------------------------------------------------------------------


def softmax_rows(s):
    """Row softmax, max-subtracted (vae.rs, `AttnBlock::apply`)."""
    s = _f64(s)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def attention_core(q, k, vt, bv=None):
    """The attention's core as its plain definition (qi21_vae.rs,
    `attention`; vae.rs, `AttnBlock::apply`): S = q k^T / sqrt(C) with
    q, k [m, C] and V^T [C, m]; P = softmax over the keys (max-subtracted);
    O = P V (+ bv). float64 throughout, no rounding of P: the reference
    both the chunked and the single-pass kernels are measured against.
    Returns (O [m, C], P [m, m])."""
    q, k, vt = _f64(q), _f64(k), _f64(vt)
    C = q.shape[1]
    p = softmax_rows(np.matmul(q, k.T) / np.sqrt(C))
    o = np.matmul(p, vt.T)
    if bv is not None:
        o = o + _f64(bv)
    return o, p


def attention(x, a, q_chunk=None, emulate_f16=True, norm=None):
    """The mid attention on the stream x [C, m] (qi21_vae.rs, `attention`;
    vae.rs, `AttnBlock::apply`): xn = f16(RMS_norm(x; gamma_a)) (no SiLU);
    q = f16(Wq xn + bq); k = f16(Wk xn + bk); V^T = f16(Wv xn) with V's bias
    deferred past P.V; per block of query rows S = q k^T / sqrt(C),
    P = f16(softmax(S)), O = P V; then x + Wp f16(O + bv) + bp.
    Query rows are independent, so the row blocks change nothing. norm:
    the decoder's norm kind (see ``norm_site``)."""
    rnd = f16 if emulate_f16 else _f64
    x = _f64(x)
    C, m = x.shape
    xn = rnd(norm_site(x, a["gamma"], a.get("beta"), silu=False, norm=norm))

    def w2(name):
        return _f64(a[name]["w"]).reshape(C, C), _f64(a[name]["b"])

    wq, bq = w2("q")
    wk, bk = w2("k")
    wv, bv = w2("v")
    wp, bp = w2("proj")
    q = rnd(np.matmul(wq, xn).T + bq)  # [m, C]
    k = rnd(np.matmul(wk, xn).T + bk)  # [m, C]
    vt = rnd(np.matmul(wv, xn))  # [C, m]
    scale = 1.0 / np.sqrt(C)
    step = m if not q_chunk else int(q_chunk)
    o = np.empty((m, C), np.float64)
    for r0 in range(0, m, step):
        r1 = min(m, r0 + step)
        s = np.matmul(q[r0:r1], k.T) * scale
        p = rnd(softmax_rows(s))
        o[r0:r1] = np.matmul(p, vt.T)
    o16 = rnd(o + bv)
    h = np.matmul(wp, o16.T)  # [C, m]
    return x + h + bp[:, None]


# ---------------------------------------------------------------------------
# the synthetic decoder
# ---------------------------------------------------------------------------


class Trace:
    """What a decode reports besides its output: the largest |x| of the raw
    stream at every guarded cast, in order."""

    def __init__(self):
        self.guard_max = []
        self.stages = {}


def resnet(x, r, guard_log2, emulate_f16=True, trace=None, norm=None):
    """One resnet unit on the stream x [cin, h, w] (qi21_vae.rs,
    `Rec::resnet`): xn = f16(RMSn(x; g1) -> SiLU); h = conv1(xn);
    xn = f16(RMSn(h + b1; g2) -> SiLU); h = conv2(xn); with a 1x1 shortcut
    x = 2^g conv_sc(f16(x 2^-g)) + b_sc + h + b2, else x = x + h + b2.
    norm: the decoder's norm kind (see ``norm_site``)."""
    rnd = f16 if emulate_f16 else _f64
    xn = rnd(norm_site(x, r["g1"], r.get("beta1"), silu=True, norm=norm))
    h = conv2d(xn, r["c1"]["w"])
    xn = rnd(norm_site(h, r["g2"], r.get("beta2"), bias=r["c1"]["b"], silu=True, norm=norm))
    h = conv2d(xn, r["c2"]["w"])
    b2 = _bcast(r["c2"]["b"], h)
    if r.get("sc") is not None:
        gs = 2.0 ** int(guard_log2)
        if trace is not None:
            trace.guard_max.append(float(np.max(np.abs(x))))
        xg = guard_cast(x, guard_log2) if emulate_f16 else x / gs
        s = gs * conv2d(xg, r["sc"]["w"])
        return s + _bcast(r["sc"]["b"], s) + h + b2
    return x + h + b2


def dupup(src, cout, ft=1):
    """The DupUp shortcut of an up stage (qi21_vae.rs, DUPUP_SRC and
    `run_blocks`): src [cin, h, w] -> [cout, 2h, 2w]; output channel o at
    sub-pixel (sy, sx) of source pixel (y, x) is src channel
    (o factor + 4 (ft - 1) + 2 sy + sx) // repeats of that pixel, with
    factor = 4 ft and repeats = cout factor / cin (an integer)."""
    src = _f64(src)
    cin, h, w = src.shape
    factor = 4 * int(ft)
    assert ft >= 1 and (cout * factor) % cin == 0
    repeats = cout * factor // cin
    out = np.empty((cout, 2 * h, 2 * w), np.float64)
    o = np.arange(cout)
    for sy in (0, 1):
        for sx in (0, 1):
            j = (o * factor + 4 * (ft - 1) + 2 * sy + sx) // repeats
            out[:, sy::2, sx::2] = src[j]
    return out


def decode(wts, z, guard_log2=8, q_chunk=None, emulate_f16=True, trace=None):
    """The synthetic decoder (readings stated in the design notes):
    f16(latent) -> conv_in (+b) -> resnet -> attention -> resnet -> per up
    stage: resnets, then x = 2^g conv_up2(f16(x 2^-g)) + b (+ the DupUp
    shortcut of the stage's input, for stages that have one) -> f16(RMSn(x;
    norm_out) -> SiLU) -> conv_out (+b); with wts["norm"] of kind "group",
    GroupNorm (with the sites' betas) at every norm site instead. z: NCHW [zc, h0, w0]; returns
    [out_c, 2^s h0, 2^s w0] (qi21_vae.rs, `decode`, `run_blocks`,
    `output_rows`; vae.rs, `VaeDecoder::decode`)."""
    rnd = f16 if emulate_f16 else _f64
    g = int(guard_log2)
    gs = 2.0 ** g
    nk = wts.get("norm")
    x = conv2d(rnd(z), wts["conv_in"]["w"], wts["conv_in"]["b"])
    x = resnet(x, wts["mid"][0], g, emulate_f16, trace, nk)
    C, h, w = x.shape
    x = attention(x.reshape(C, h * w), wts["attn"], q_chunk, emulate_f16, nk).reshape(C, h, w)
    x = resnet(x, wts["mid"][1], g, emulate_f16, trace, nk)
    if trace is not None:
        trace.stages["mid"] = x.copy()
    for si, st in enumerate(wts["ups"]):
        x_in = x
        for r in st["res"]:
            x = resnet(x, r, g, emulate_f16, trace, nk)
        if trace is not None:
            trace.guard_max.append(float(np.max(np.abs(x))))
        xg = guard_cast(x, g) if emulate_f16 else x / gs
        x = gs * conv2d_up2(xg, st["up"]["w"])
        x = x + _bcast(st["up"]["b"], x)
        if st.get("dupup") is not None:
            x = x + dupup(x_in, x.shape[0], st["dupup"].get("ft", 1))
        if trace is not None:
            trace.stages["up%d" % si] = x.copy() if x.size <= (1 << 24) else None
    xn = rnd(norm_site(x, wts["norm_out"], wts.get("norm_out_beta"), silu=True, norm=nk))
    return conv2d(xn, wts["conv_out"]["w"], wts["conv_out"]["b"])


# ---------------------------------------------------------------------------
# bands (qi21_vae.rs, the bands section)
# ---------------------------------------------------------------------------


def plan_band(n_res, has_up, h0, band_from, keep):
    """The rows a band of the up path needs, as exact dependency sets.

    After the mid block every step only looks at nearby rows (qi21_vae.rs,
    the bands section), so a band of kept output rows needs only some rows
    of each level. The steps from block band_from's input to the frame are
    listed in order -- per block 2 n_res 3x3 convs, then, with has_up, the
    nearest-2x upsample and its 3x3 conv; conv_out last -- and the set of
    kept rows is carried back through them: a 3x3 conv on a level of h rows
    reads rows r - 1, r, r + 1 of its input where they exist (0 <= . < h;
    outside, the zero padding), an upsample reads row r // 2.

    Returns ((first, end) of the rows of block band_from's input the band
    needs, {block i: (first, end) of the rows block i hands to its
    upsample}). Every set is a contiguous range; the returned ranges are
    its first row and one past its last."""
    h = h0 << sum(1 for u in has_up[:band_from] if u)
    steps = []
    for i in range(band_from, len(n_res)):
        steps += [("conv", h, i)] * (2 * n_res[i])
        if has_up[i]:
            steps.append(("up", 0, i))
            h *= 2
            steps.append(("conv", h, i))
    steps.append(("conv", h, None))  # conv_out
    rows = set(range(keep[0], keep[1]))
    feed = {}
    for kind, height, block in reversed(steps):
        if kind == "conv":
            rows = {r + d for r in rows for d in (-1, 0, 1) if 0 <= r + d < height}
        else:
            rows = {r // 2 for r in rows}
            feed[block] = (min(rows), max(rows) + 1)
    return (min(rows), max(rows) + 1), feed


# ---------------------------------------------------------------------------
# metrics
# ---------------------------------------------------------------------------


def to_u8(v):
    """The decoder's RGB range [-1, 1] onto 0..255: clamp(floor((v + 1)
    127.5 + 0.5), 0, 255)."""
    v = _f64(v)
    return np.clip(np.floor((v + 1.0) * 127.5 + 0.5), 0, 255)


def psnr_u8(a, b):
    """10 log10(255^2 / MSE) over the u8 images of a and b (inf if equal)."""
    d = to_u8(a) - to_u8(b)
    mse = float(np.mean(d * d))
    if mse == 0.0:
        return float("inf")
    return 10.0 * np.log10(255.0 ** 2 / mse)
