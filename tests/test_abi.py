"""The C ABI without a GPU: libigconv loads, exports every function that
include/ig_conv.h declares, its descriptor structs have the layout the C
compiler gives them, and invalid calls are rejected before anything is
enqueued (no kernel runs in these tests)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ig_conv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def ig():
    import implicit_gemm_conv_nhwc_amd as m

    return m


def test_header_declares_the_path(ig):
    names = _declared_functions()
    for want in ("conv3x3_nhwc", "conv3x3_up2_nhwc", "gemm1x1", "rmsnorm_silu_f16", "guard_cast",
                 "decoder_forward", "ig_decoder_workspace_bytes", "ig_last_error"):
        assert want in names


def test_every_declared_symbol_is_exported(ig):
    lib = ctypes.CDLL(ig._lib.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_descriptor_layout_matches_c(ig, tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "ig_conv.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(ig_conv_w), sizeof(ig_resnet_w), sizeof(ig_attn_w),
         sizeof(ig_up_w), sizeof(ig_decoder));
  printf("%zu %zu %zu %zu %zu %zu\n", offsetof(ig_decoder, attn), offsetof(ig_decoder, n_up),
         offsetof(ig_decoder, ups), offsetof(ig_decoder, norm_out_gamma),
         offsetof(ig_decoder, norm_out_c), offsetof(ig_decoder, conv_out));
  printf("%zu %zu %zu\n", offsetof(ig_resnet_w, has_sc), offsetof(ig_resnet_w, sc), offsetof(ig_up_w, up));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = subprocess.check_output([str(exe)]).decode().split()
    L = ig._lib
    want = [ctypes.sizeof(L.ConvW), ctypes.sizeof(L.ResnetW), ctypes.sizeof(L.AttnW), ctypes.sizeof(L.UpW),
            ctypes.sizeof(L.DecoderDesc),
            L.DecoderDesc.attn.offset, L.DecoderDesc.n_up.offset, L.DecoderDesc.ups.offset,
            L.DecoderDesc.norm_out_gamma.offset, L.DecoderDesc.norm_out_c.offset,
            L.DecoderDesc.conv_out.offset,
            L.ResnetW.has_sc.offset, L.ResnetW.sc.offset, L.UpW.up.offset]
    assert [int(v) for v in got] == want


def _rc(f, *args):
    return f(*args)


def test_validation_rejects_before_enqueueing(ig):
    lib = ig.lib
    f1 = ctypes.c_float(1.0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    # convolutions
    assert lib.conv3x3_nhwc(fake, 4, 4, 100, fake, 64, None, f1, fake, None) == -2
    assert lib.conv3x3_nhwc(fake, 4, 4, 64, fake, 96, None, f1, fake, None) == -2
    assert lib.conv3x3_nhwc(None, 4, 4, 64, fake, 64, None, f1, fake, None) == -1
    assert lib.conv3x3_nhwc(ctypes.c_void_p((1 << 20) + 8), 4, 4, 64, fake, 64, None, f1, fake, None) == -1
    assert lib.conv3x3_up2_nhwc(fake, -1, 4, 64, fake, 64, None, f1, fake, None) == -1
    assert lib.ig_conv_nhwc_ex(fake, 4, 4, 64, 5, fake, 64, None, f1, 0, fake, None) == -1
    # the 3x3 kernels address their f16 input with 32-bit byte offsets: an
    # input of 2^31 - 2^16 bytes or more is refused (a 1x1 GEMM of the same
    # size is not); channel counts above 8192 too
    assert lib.conv3x3_nhwc(fake, 2048, 8192, 64, fake, 64, None, f1, fake, None) == -2
    assert lib.conv3x3_up2_nhwc(fake, 2048, 8192, 64, fake, 64, None, f1, fake, None) == -2
    assert lib.conv3x3_nhwc(fake, 4, 4, 8256, fake, 64, None, f1, fake, None) == -2
    assert lib.conv3x3_nhwc(fake, 4, 4, 64, fake, 8256, None, f1, fake, None) == -2
    # empty inputs are valid and enqueue nothing
    assert lib.conv3x3_nhwc(None, 0, 4, 64, None, 64, None, f1, None, None) == 0
    # GEMM
    assert lib.gemm1x1(fake, 10, 48, 48, fake, 64, 48, None, f1, fake, 64, 0, None) == -2
    assert lib.gemm1x1(fake, 10, 64, 64, fake, 96, 64, None, f1, fake, 96, 0, None) == -2
    assert lib.gemm1x1(fake, 10, 64, 32, fake, 64, 64, None, f1, fake, 64, 0, None) == -1
    assert lib.gemm1x1(fake, 0, 64, 64, fake, 64, 64, None, f1, fake, 64, 0, None) == 0
    # norm, cast, softmax
    assert lib.rmsnorm_silu_f16(fake, 8, 100, 100, None, fake, 1, ctypes.c_float(1e-12), fake, None) == -2
    assert lib.rmsnorm_silu_f16(fake, 8, 128, 129, None, fake, 1, ctypes.c_float(1e-12), fake, None) == -1
    assert lib.rmsnorm_silu_f16(fake, 8, 128, 128, None, None, 1, ctypes.c_float(1e-12), fake, None) == -1
    assert lib.guard_cast(fake, 8, 64, None, 15, fake, None) == -1
    assert lib.guard_cast(fake, 8, 66, None, 8, fake, None) == -2
    assert lib.ig_softmax_rows_f16(fake, 4, 64, 65, 65, fake, 64, None) == -1
    assert "valid" in ig.last_error() or "softmax" in ig.last_error()
    assert lib.ig_dupup_add(fake, 2, 2, 64, fake, 64, 64, 4, 1, 1, None) == -1
    assert lib.ig_dupup_add(fake, 2, 2, 64, fake, 62, 66, 4, 4, 1, None) == -2  # cout_p % 4
    # attention: q, k and V^T are addressed with 32-bit byte offsets, so a
    # row stride whose ld * C * 2 reaches 0x7fff0000 bytes is refused (a
    # wrapped offset would silently read zeros)
    lib.attention_f16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2 + \
        [ctypes.c_size_t] + [ctypes.c_void_p] * 2
    big = 0x7fff0000 // (512 * 2)
    assert lib.attention_f16(fake, fake, fake, 1024, big + 8, 512, None, fake, 1 << 30, fake, None) == -1
    assert "ld" in ig.last_error()
    assert lib.attention_f16(fake, fake, fake, 1024, 1 << 22, 512, None, fake, 1 << 30, fake, None) == -1
    # head widths: 128, 256, 384 and 512 run in one pass; others are refused
    big256 = 0x7fff0000 // (256 * 2)
    assert lib.attention_f16(fake, fake, fake, 1024, big256 + 8, 256, None, fake, 1 << 30, fake, None) == -1
    for c in (64, 192, 320, 640, 1024):
        assert lib.attention_f16(fake, fake, fake, 64, 64, c, None, fake, 1 << 30, fake, None) == -2, c
        assert ig.attention_workspace_bytes(64, c) == 0
    for c in (128, 256, 384, 512):
        assert ig.attention_workspace_bytes(16384, c) > 0
        assert ig.attention_workspace_bytes(64, c) == 0 and ig.last_error() == ""
    # groupnorm without a workspace: the same checks as with one
    lib.groupnorm_silu_f16_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.groupnorm_silu_f16_noalloc(fake, 8, 1028, 1028, 4, None, fake, fake, 1, ctypes.c_float(1e-6), fake,
                                          None) == -2
    assert lib.groupnorm_silu_f16_noalloc(fake, 8, 128, 128, 3, None, fake, fake, 1, ctypes.c_float(1e-6), fake,
                                          None) == -2
    assert lib.groupnorm_silu_f16_noalloc(fake, 8, 128, 128, 32, None, None, fake, 1, ctypes.c_float(1e-6), fake,
                                          None) == -1
    # GroupNorm statistics from a conv's epilogue: 3x3 modes only, groups
    # of 4..64 channels dividing 64, a partials buffer of the stated size
    assert ig.conv_gn_partials_bytes(1, 64, 64, 32) == 2 * 4 * 32 * 12  # 16 x 32-pixel tiles
    assert ig.conv_gn_partials_bytes(2, 32, 32, 32) == 2 * 4 * 32 * 12
    assert ig.conv_gn_partials_bytes(1, 65, 33, 32) == 5 * 2 * 32 * 12  # ragged tiles count
    assert ig.conv_gn_partials_bytes(0, 64, 64, 32) == 0
    sz = ig.conv_gn_partials_bytes(1, 16, 32, 32)
    C = ctypes.c_size_t
    f = lib.ig_conv3x3_gn_stats_nhwc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(fake, 16, 32, 64, 0, fake, 128, None, 1.0, 0, fake, 128, 32, fake, C(sz), None) == -1  # not 3x3
    assert f(fake, 16, 32, 64, 1, fake, 320, None, 1.0, 0, fake, 288, 32, fake, C(1 << 20), None) == -2  # 9 per group
    assert f(fake, 16, 32, 64, 1, fake, 64, None, 1.0, 0, fake, 64, 32, fake, C(1 << 20), None) == -2  # 2 per group
    assert f(fake, 16, 32, 64, 1, fake, 128, None, 1.0, 0, fake, 128, 32, fake, C(sz - 4), None) == -3
    assert "partials" in ig.last_error()
    g = lib.groupnorm_silu_f16_from_partials
    g.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert g(fake, 8, 128, 128, 32, fake, fake, 1, 1e-6, fake, 0, fake, C(1536), fake, None) == -1
    assert g(fake, 8, 128, 128, 32, fake, fake, 1, 1e-6, fake, 4, fake, C(1535), fake, None) == -3
    assert g(fake, 8, 128, 128, 32, fake, fake, 1, 1e-6, fake, 4, ctypes.c_void_p((1 << 20) + 4), C(4096), fake,
             None) == -3
    assert g(fake, 8, 128, 128, 3, fake, fake, 1, 1e-6, fake, 4, fake, C(4096), fake, None) == -2


def test_decoder_descriptor_validation(ig):
    L = ig._lib
    d = L.DecoderDesc()
    assert L._ws_bytes(ctypes.byref(d), 4, 4, 0) == 0
    assert "zc" in ig.last_error()
    fake = 1 << 20

    def conv(cin, cout, k):
        c = L.ConvW()
        c.w, c.b = fake, fake
        c.cin, c.cout, c.cin_p, c.cout_p, c.k = cin, cout, (cin + 63) // 64 * 64, (cout + 63) // 64 * 64, k
        return c

    def res(cin, cout):
        r = L.ResnetW()
        r.g1 = r.g2 = fake
        r.c1, r.c2 = conv(cin, cout, 3), conv(cout, cout, 3)
        if cin != cout:
            r.has_sc, r.sc = 1, conv(cin, cout, 1)
        return r

    d.zc = 16
    d.conv_in = conv(16, 128, 3)
    d.mid[0] = res(128, 128)
    d.mid[1] = res(128, 128)
    d.attn.gamma = fake
    d.attn.q = d.attn.k = d.attn.v = d.attn.proj = conv(128, 128, 1)
    d.n_up = 1
    d.ups[0].n_res = 1
    d.ups[0].res[0] = res(128, 64)
    d.ups[0].has_up = 1
    d.ups[0].up = conv(64, 64, 3)
    d.norm_out_gamma = fake
    d.norm_out_c = 64
    d.conv_out = conv(64, 3, 3)
    n = L._ws_bytes(ctypes.byref(d), 8, 8, 0)
    assert n > 0, ig.last_error()
    # a frame whose conv inputs pass the 3x3 kernels' 2 GB offset range
    # (64 channels f16 at 4096 x 4096 = 2 GB) is refused in one pass...
    assert L._ws_bytes(ctypes.byref(d), 2048, 2048, 128) == 0
    assert "bands" in ig.last_error()
    # ...and planned in bands of 64 output rows
    assert ig.lib.ig_decoder_bands_workspace_bytes(ctypes.byref(d), 2048, 2048, 128, 64, 0) > 0, ig.last_error()
    # too small a workspace: rejected, nothing enqueued
    assert ig.lib.decoder_forward(ctypes.byref(d), fake, 8, 8, 8, 0, fake, n - 1, fake, None) == -3
    assert ig.lib.decoder_forward(ctypes.byref(d), fake, 8, 8, 15, 0, fake, n, fake, None) == -1
    # a width mismatch is caught
    d.conv_out = conv(128, 3, 3)
    assert L._ws_bytes(ctypes.byref(d), 8, 8, 0) == 0
    assert "conv_out" in ig.last_error()
