"""Helpers for the GPU parity tests: device uploads, layout conversions
between the path's NHWC and the oracle's NCHW, f16 ulp distances, and the
tolerance of the per-conv comparisons (max |d| <= 2e-3 * RMS of the
oracle's output)."""

import numpy as np
import torch

CONV_TOL = 2e-3  # per-conv bar: max |d| <= CONV_TOL * RMS(oracle output)
DEV = "cuda"


def cpad(c):
    return (int(c) + 63) // 64 * 64


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device=DEV, dtype=dtype) if dtype is not None else t.to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def pad_last(a, cp):
    """Zero-pad the last axis of a host array to cp (test input plumbing)."""
    out = np.zeros(a.shape[:-1] + (cp,), a.dtype)
    out[..., : a.shape[-1]] = a
    return out


def nhwc_to_chw(a, H, W):
    """[H*W, C] or [H, W, C] host array -> [C, H, W]."""
    return np.ascontiguousarray(a.reshape(H, W, -1).transpose(2, 0, 1))


def nan_f32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def nan_f16(shape):
    return torch.full(shape, float("nan"), dtype=torch.float16, device=DEV)


def packed(w16, stream=None):
    """Upload an OIHW f16 weight and pack it on the GPU."""
    import implicit_gemm_conv_nhwc_amd as ig

    cout, cin, k, _ = w16.shape
    src = dev(w16)
    plane = torch.empty(ig.plane_shape(cpad(cout), cpad(cin), k), dtype=torch.float16, device=DEV)
    ig.pack_conv_weights(src, cout, cin, k, cpad(cout), cpad(cin), plane, stream)
    return plane


def padded_vec(v, n):
    t = torch.zeros(n, dtype=torch.float32, device=DEV)
    t[: len(v)] = dev(np.asarray(v, np.float32))
    return t


def f16_ulps(a, b):
    """Distance in binary16 ulps between two f16 arrays (finite values)."""
    def key(x):
        i = np.asarray(x, np.float16).view(np.int16).astype(np.int32)
        return np.where(i < 0, -(i & 0x7FFF), i)

    return np.abs(key(a) - key(b))


def conv_err(got, ref):
    """(max |d|, RMS of ref, ratio) over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err, rms, (err / rms if rms > 0 else err)


def sample_pixels(H, W, n, seed):
    """Flat output-pixel indices: every border pixel of the first/last rows
    and columns plus n seeded interior picks."""
    g = np.random.default_rng(seed)
    border = set()
    for c in range(W):
        border.add(c)
        border.add((H - 1) * W + c)
    for r in range(H):
        border.add(r * W)
        border.add(r * W + W - 1)
    border = np.array(sorted(border), np.int64)
    if len(border) > n:
        border = g.choice(border, n, replace=False)
    inner = g.integers(0, H * W, n)
    return np.unique(np.concatenate([border, inner]))
