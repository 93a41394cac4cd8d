"""ctypes binding of libigconv (include/ig_conv.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the library, and raises ``IgError`` on a nonzero
status. Tensors must already live on the GPU with the documented dtype and
layout; nothing here computes, converts or falls back to the CPU. If the
library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libigconv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libigconv.so is not built (%s); run `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python implicit_gemm_conv_nhwc_amd/build.py`" % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)

_c_int = ctypes.c_int
_c_float = ctypes.c_float
_vp = ctypes.c_void_p
_size_t = ctypes.c_size_t

IG_MAX_RES = 4
IG_MAX_UP = 8

STATUS = {0: "IG_OK", -1: "IG_EINVAL", -2: "IG_EUNSUPPORTED", -3: "IG_EWORKSPACE", -4: "IG_EHIP"}


class IgError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s: %s" % (STATUS.get(code, code), msg))
        self.code = code


def _sig(name, argtypes, restype=_c_int):
    f = getattr(lib, name)
    f.argtypes = argtypes
    f.restype = restype
    return f


lib.ig_last_error.restype = ctypes.c_char_p
lib.ig_last_error.argtypes = []
lib.ig_version.restype = _c_int

_pack = _sig("ig_pack_conv_weights", [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp])
_conv3 = _sig("conv3x3_nhwc", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_float, _vp, _vp])
_conv3u = _sig("conv3x3_up2_nhwc", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_float, _vp, _vp])
_convx = _sig("ig_conv_nhwc_ex", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_float,
                                  _c_int, _vp, _vp])
_gemm = _sig("gemm1x1", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _c_float, _vp, _c_int,
                         _c_int, _vp])
_gemm_acc = _sig("gemm1x1_acc", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _c_float, _vp,
                                 _c_int, _vp])
_rms = _sig("rmsnorm_silu_f16", [_vp, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_float, _vp, _vp])
_rms_cast = _sig("rmsnorm_silu_guard_cast_f16", [_vp, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_float, _vp,
                                                 _c_int, _vp, _vp])
_conv_g = _sig("ig_conv3x3_guard_out_nhwc", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_float, _c_int,
                                             _vp, _c_int, _c_int, _vp, _vp])
_cast = _sig("guard_cast", [_vp, _c_int, _c_int, _vp, _c_int, _vp, _vp])
_comb = _sig("ig_combine", [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp])
_smax = _sig("ig_softmax_rows_f16", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp])
_lat = _sig("ig_latent_to_nhwc_f16", [_vp, _c_int, _c_int, _c_int, _vp, _vp])
_out = _sig("ig_nhwc_to_nchw", [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp])
_zero = _sig("ig_zero_rows_f16", [_vp, _c_int, _c_int, _c_int, _vp])
_conv_norm = _sig("ig_conv3x3_norm_nhwc", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp,
                                          _c_float, _vp, _c_int, _c_float, _vp, _vp, _vp])
_gn_ws = lib.ig_groupnorm_workspace_bytes
_gn_ws.argtypes = [_c_int, _c_int, _c_int]
_gn_ws.restype = ctypes.c_size_t
_gn = _sig("groupnorm_silu_f16", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, _c_float, _vp,
                                  ctypes.c_size_t, _vp, _vp])
_gn_na = _sig("groupnorm_silu_f16_noalloc", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, _c_float,
                                           _vp, _vp])
_gn_pb = _sig("ig_conv_gn_partials_bytes", [_c_int, _c_int, _c_int, _c_int], ctypes.c_size_t)
_conv_gn = _sig("ig_conv3x3_gn_stats_nhwc", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_float, _c_int,
                                             _vp, _c_int, _c_int, _vp, ctypes.c_size_t, _vp])
_gn_part = _sig("groupnorm_silu_f16_from_partials", [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_float,
                                                     _vp, _c_int, _vp, ctypes.c_size_t, _vp, _vp])
_attn_ws = _sig("ig_attention_workspace_bytes", [_c_int, _c_int], ctypes.c_size_t)
_attn = _sig("attention_f16", [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, ctypes.c_size_t, _vp, _vp])
_conv_out = _sig("ig_conv3x3_out_nchw", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp])
_dupup = _sig("ig_dupup_add", [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _vp])


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc):
    if rc != 0:
        raise IgError(rc, lib.ig_last_error().decode())
    return rc


def last_error():
    return lib.ig_last_error().decode()


def version():
    v = lib.ig_version()
    return (v >> 16, v & 0xFFFF)


# ---------------------------------------------------------------------------
# entry points (names as in include/ig_conv.h)
# ---------------------------------------------------------------------------


def plane_shape(cout_p, cin_p, k):
    """Shape of a packed weight plane (include/ig_conv.h, weight packing):
    3x3 -> [cin_p/16][9][cout_p][16], 1x1 -> [cout_p][cin_p]."""
    return (cin_p // 16, 9, cout_p, 16) if k == 3 else (cout_p, cin_p)


def pack_conv_weights(w, cout, cin, k, cout_p, cin_p, plane, stream=None):
    """OIHW f16 w -> the zero-padded plane of plane_shape(cout_p, cin_p, k)."""
    return _check(_pack(_ptr(w), cout, cin, k, cout_p, cin_p, _ptr(plane), _stream(stream)))


def conv3x3_nhwc(x, H, W, cin_p, w, cout_p, bias, oscale, y, stream=None):
    return _check(_conv3(_ptr(x), H, W, cin_p, _ptr(w), cout_p, _ptr(bias), float(oscale), _ptr(y),
                         _stream(stream)))


def conv3x3_up2_nhwc(x, H, W, cin_p, w, cout_p, bias, oscale, y, stream=None):
    return _check(_conv3u(_ptr(x), H, W, cin_p, _ptr(w), cout_p, _ptr(bias), float(oscale), _ptr(y),
                          _stream(stream)))


def conv_nhwc_ex(x, H, W, cin_p, mode, w, cout_p, bias, oscale, accumulate, y, stream=None):
    return _check(_convx(_ptr(x), H, W, cin_p, mode, _ptr(w), cout_p, _ptr(bias), float(oscale),
                         int(accumulate), _ptr(y), _stream(stream)))


def gemm1x1(a, M, K, lda, b, N, ldb, bias, oscale, c, ldc, c_is_f16, stream=None):
    return _check(_gemm(_ptr(a), M, K, lda, _ptr(b), N, ldb, _ptr(bias), float(oscale), _ptr(c), ldc,
                        int(c_is_f16), _stream(stream)))


def gemm1x1_acc(a, M, K, lda, b, N, ldb, bias, oscale, c, ldc, stream=None):
    return _check(_gemm_acc(_ptr(a), M, K, lda, _ptr(b), N, ldb, _ptr(bias), float(oscale), _ptr(c),
                            ldc, _stream(stream)))


def rmsnorm_silu_f16(x, M, cp, c_real, bias, gamma, silu, eps, y, stream=None):
    return _check(_rms(_ptr(x), M, cp, c_real, _ptr(bias), _ptr(gamma), int(silu), float(eps), _ptr(y),
                       _stream(stream)))


def rmsnorm_silu_guard_cast_f16(x, M, cp, c_real, bias, gamma, silu, eps, y, guard_log2, yg, stream=None):
    return _check(_rms_cast(_ptr(x), M, cp, c_real, _ptr(bias), _ptr(gamma), silu, eps, _ptr(y), guard_log2,
                            _ptr(yg), _stream(stream)))


def conv3x3_guard_out_nhwc(x, H, W, cin_p, mode, w, cout_p, bias, oscale, accumulate, y, write_y, guard_log2, yg,
                           stream=None):
    return _check(_conv_g(_ptr(x), H, W, cin_p, mode, _ptr(w), cout_p, _ptr(bias), oscale, accumulate, _ptr(y),
                          write_y, guard_log2, _ptr(yg), _stream(stream)))


def guard_cast(x, M, C, bias, guard_log2, y, stream=None):
    return _check(_cast(_ptr(x), M, C, _ptr(bias), int(guard_log2), _ptr(y), _stream(stream)))


def combine(x, h, hb, s, sb, M, C, mode, stream=None):
    return _check(_comb(_ptr(x), _ptr(h), _ptr(hb), _ptr(s), _ptr(sb), M, C, mode, _stream(stream)))


def softmax_rows_f16(S, rows, lds, valid, ncols, P, ldp, stream=None):
    return _check(_smax(_ptr(S), rows, lds, valid, ncols, _ptr(P), ldp, _stream(stream)))


def latent_to_nhwc_f16(z, zc, M, cp, y, stream=None):
    return _check(_lat(_ptr(z), zc, M, cp, _ptr(y), _stream(stream)))


def nhwc_to_nchw(y, M, ld, nch, bias, out, stream=None):
    return _check(_out(_ptr(y), M, ld, nch, _ptr(bias), _ptr(out), _stream(stream)))


def conv3x3_norm_nhwc(x, H, W, cin_p, mode, w, cout_p, c_real, bias, oscale, gamma, silu, eps, y, yn,
                      stream=None):
    return _check(_conv_norm(_ptr(x), H, W, cin_p, mode, _ptr(w), cout_p, c_real, _ptr(bias), oscale,
                             _ptr(gamma), silu, eps, _ptr(y), _ptr(yn), _stream(stream)))


def groupnorm_workspace_bytes(M, cp, groups):
    return int(_gn_ws(M, cp, groups))


def groupnorm_silu_f16(x, M, cp, c_real, groups, bias, gamma, beta, silu, eps, ws, ws_bytes, y, stream=None):
    return _check(_gn(_ptr(x), M, cp, c_real, groups, _ptr(bias), _ptr(gamma), _ptr(beta), silu, eps, _ptr(ws),
                      ws_bytes, _ptr(y), _stream(stream)))


def groupnorm_silu_f16_noalloc(x, M, cp, c_real, groups, bias, gamma, beta, silu, eps, y, stream=None):
    return _check(_gn_na(_ptr(x), M, cp, c_real, groups, _ptr(bias), _ptr(gamma), _ptr(beta), silu, eps, _ptr(y),
                         _stream(stream)))


def conv_gn_partials_bytes(mode, H, W, groups):
    return int(_gn_pb(mode, H, W, groups))


def conv3x3_gn_stats_nhwc(x, H, W, cin_p, mode, w, cout_p, bias, oscale, accumulate, y, c_real, groups, part,
                          part_bytes, stream=None):
    return _check(_conv_gn(_ptr(x), H, W, cin_p, mode, _ptr(w), cout_p, _ptr(bias), float(oscale), int(accumulate),
                           _ptr(y), c_real, groups, _ptr(part), part_bytes, _stream(stream)))


def groupnorm_silu_f16_from_partials(x, M, cp, c_real, groups, gamma, beta, silu, eps, part, nchunk, ws, ws_bytes,
                                     y, stream=None):
    return _check(_gn_part(_ptr(x), M, cp, c_real, groups, _ptr(gamma), _ptr(beta), silu, eps, _ptr(part), nchunk,
                           _ptr(ws), ws_bytes, _ptr(y), _stream(stream)))


def conv3x3_out_nchw(x, H, W, cin_p, w, cout, cout_p, bias, out, stream=None):
    return _check(_conv_out(_ptr(x), H, W, cin_p, _ptr(w), cout, cout_p, _ptr(bias), _ptr(out),
                            _stream(stream)))


def zero_rows_f16(y, r0, r1, ld, stream=None):
    return _check(_zero(_ptr(y), r0, r1, ld, _stream(stream)))


def dupup_add(src, H, W, cin_p, x, cout, cout_p, factor, repeats, ft, stream=None):
    return _check(_dupup(_ptr(src), H, W, cin_p, _ptr(x), cout, cout_p, factor, repeats, ft,
                         _stream(stream)))


# ---------------------------------------------------------------------------
# the decoder descriptor (mirrors the structs of include/ig_conv.h)
# ---------------------------------------------------------------------------


class ConvW(ctypes.Structure):
    _fields_ = [("w", _vp), ("b", _vp), ("cin", _c_int), ("cout", _c_int), ("cin_p", _c_int),
                ("cout_p", _c_int), ("k", _c_int)]


class ResnetW(ctypes.Structure):
    _fields_ = [("g1", _vp), ("c1", ConvW), ("g2", _vp), ("c2", ConvW), ("has_sc", _c_int),
                ("sc", ConvW), ("beta1", _vp), ("beta2", _vp)]


class AttnW(ctypes.Structure):
    _fields_ = [("gamma", _vp), ("q", ConvW), ("k", ConvW), ("v", ConvW), ("proj", ConvW), ("beta", _vp)]


class UpW(ctypes.Structure):
    _fields_ = [("n_res", _c_int), ("res", ResnetW * IG_MAX_RES), ("has_up", _c_int), ("up", ConvW),
                ("dupup", _c_int), ("dupup_ft", _c_int)]


class DecoderDesc(ctypes.Structure):
    _fields_ = [("zc", _c_int), ("conv_in", ConvW), ("mid", ResnetW * 2), ("attn", AttnW),
                ("n_up", _c_int), ("ups", UpW * IG_MAX_UP), ("norm_out_gamma", _vp),
                ("norm_out_c", _c_int), ("conv_out", ConvW), ("norm_kind", _c_int), ("norm_groups", _c_int),
                ("norm_eps", _c_float), ("norm_out_beta", _vp)]

IG_NORM_RMS, IG_NORM_GROUP = 0, 1


_ws_bytes = _sig("ig_decoder_workspace_bytes", [ctypes.POINTER(DecoderDesc), _c_int, _c_int, _c_int],
                 _size_t)
_dec = _sig("decoder_forward", [ctypes.POINTER(DecoderDesc), _vp, _c_int, _c_int, _c_int, _c_int, _vp,
                                _size_t, _vp, _vp])


_bws_bytes = _sig("ig_decoder_bands_workspace_bytes", [ctypes.POINTER(DecoderDesc), _c_int, _c_int, _c_int, _c_int,
                                                       _c_int], ctypes.c_size_t)
_dec_bands = _sig("decoder_forward_bands", [ctypes.POINTER(DecoderDesc), _vp, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _vp, ctypes.c_size_t, _vp, _vp])
_band_plan = _sig("ig_band_plan", [_c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp])


def band_plan(n_res, has_up, h0, band_from, keep_lo, keep_hi):
    """Host-only band planner: ((lo, hi) of block band_from's input rows,
    [(lo, hi) fed to each block's upsample])."""
    n = len(n_res)
    a_res = (ctypes.c_int * max(n, 1))(*n_res)
    a_up = (ctypes.c_int * max(n, 1))(*[int(bool(u)) for u in has_up])
    inp = (ctypes.c_int * 2)()
    feed = (ctypes.c_int * max(2 * n, 1))()
    _check(_band_plan(n, ctypes.cast(a_res, _vp), ctypes.cast(a_up, _vp), h0, band_from, keep_lo, keep_hi,
                      ctypes.cast(inp, _vp), ctypes.cast(feed, _vp)))
    return (inp[0], inp[1]), [(feed[2 * i], feed[2 * i + 1]) for i in range(n)]


_clock_probe = _sig("ig_set_clock_probe", [_vp])


def set_clock_probe(buf):
    """Measurement hook (benchmarks): while ``buf`` (a device tensor of 4
    int64, or None to stop) is set, each launch of the register-weight 3x3
    conv writes [clock0, realtime0, clock1, realtime1] of its first wave."""
    return _check(_clock_probe(_ptr(buf)))


def decoder_bands_workspace_bytes(desc, h0, w0, q_chunk, band_rows, band_from):
    n = int(_bws_bytes(ctypes.byref(desc), h0, w0, q_chunk, band_rows, band_from))
    if n == 0:
        raise IgError(-1, last_error())
    return n


def decoder_forward_bands(desc, latent, h0, w0, guard_log2, q_chunk, band_rows, band_from, ws, ws_bytes, out,
                          stream=None):
    return _check(_dec_bands(ctypes.byref(desc), _ptr(latent), h0, w0, guard_log2, q_chunk, band_rows, band_from,
                             _ptr(ws), ws_bytes, _ptr(out), _stream(stream)))


def decoder_workspace_bytes(desc, h0, w0, q_chunk=0):
    n = _ws_bytes(ctypes.byref(desc), h0, w0, q_chunk)
    if n == 0:
        raise IgError(-1, last_error())
    return n


def decoder_forward(desc, latent, h0, w0, guard_log2, q_chunk, ws, ws_bytes, out, stream=None):
    return _check(_dec(ctypes.byref(desc), _ptr(latent), h0, w0, int(guard_log2), int(q_chunk),
                       _ptr(ws), ws_bytes, _ptr(out), _stream(stream)))


def attention_workspace_bytes(m, C):
    return int(_attn_ws(m, C))


def attention_f16(q, k, vt, m, ld, C, bv, ws, ws_bytes, out, stream=None):
    return _check(_attn(_ptr(q), _ptr(k), _ptr(vt), m, ld, C, _ptr(bv), _ptr(ws), ws_bytes, _ptr(out),
                        _stream(stream)))
