"""The allocation-free GroupNorm entry point (groupnorm_silu_f16_noalloc),
whose statistics live in a device array built into the library, against the
workspace entry point groupnorm_silu_f16 on the same inputs: the same
kernels on the same data, so the f16 outputs must be bit for bit equal.
Three calls in a row on one GPU share the array; the second is smaller than
the first and the third uses all of it (1024 partial chunks x 128 groups,
1024 channels), so stale statistics left by an earlier call would show."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, nan_f16, pad_last

import implicit_gemm_conv_nhwc_amd as ig

pytestmark = pytest.mark.gpu


def _inputs(M, c, cp, seed, with_bias):
    x = pad_last(synth.normal(21, seed, (M, c), 4.0), cp)
    gamma = pad_last(synth.uniform(21, seed + 1, (c,), 0.5, 1.5), cp)
    beta = pad_last(synth.normal(21, seed + 2, (c,), 0.1), cp)
    bias = pad_last(synth.normal(21, seed + 3, (c,), 0.02), cp) if with_bias else None
    return dev(x), dev(gamma), dev(beta), (dev(bias) if bias is not None else None)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_groupnorm_noalloc_matches_the_workspace_call(order):
    cases = [
        (512 * 512, 128, 128, 32, True, 1),   # 1024 partial chunks
        (7 * 9, 288, 320, 32, False, 1),      # smaller: few chunks, padded channels
        (300 * 300, 1024, 1024, 128, True, 0),  # the array's full size
    ]
    for i, (M, c, cp, groups, with_bias, silu) in enumerate(cases):
        x, gamma, beta, bias = _inputs(M, c, cp, 100 + 10 * i, with_bias)
        nbytes = ig.groupnorm_workspace_bytes(M, cp, groups)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ref = nan_f16((M, cp))
        ig.groupnorm_silu_f16(x, M, cp, c, groups, bias, gamma, beta, silu, 1e-6, ws, nbytes, ref)
        got = nan_f16((M, cp))
        ig.groupnorm_silu_f16_noalloc(x, M, cp, c, groups, bias, gamma, beta, silu, 1e-6, got)
        torch.cuda.synchronize()
        assert not torch.isnan(got.float()).any(), "case %d: output not fully written" % i
        same = torch.equal(got.view(torch.int16), ref.view(torch.int16))
        print("noalloc groupnorm case %d: M=%d cp=%d groups=%d, workspace %d bytes, equal %s" % (
            i, M, cp, groups, nbytes, same))
        assert same, "case %d differs from the workspace entry point" % i


def test_groupnorm_noalloc_rejects_what_the_workspace_call_rejects():
    y = nan_f16((4, 1028))
    z = torch.zeros(1028, device="cuda")
    with pytest.raises(ig.IgError) as e:
        ig.groupnorm_silu_f16_noalloc(torch.zeros((4, 1028), device="cuda"), 4, 1028, 1028, 4, None, z, z, 1, 1e-6, y)
    assert e.value.code == -2
    assert torch.isnan(y.float()).all(), "a rejected call must leave its output untouched"
