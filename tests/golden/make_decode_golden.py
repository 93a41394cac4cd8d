"""Write the stored oracle rows of the full-size synthetic decode.

The full-size decoder (1024^2 or 2048^2 output, latent N(0,1)*8, conv_in
weights scaled by 2^11 so that the residual stream passes the f16 range at
the guarded casts, guard shift 8) takes the CPU oracle minutes, too long for
a test. This script runs the oracle once and stores sampled output rows:

* ``u8``: the u8 image (the decoder's [-1, 1] range onto 0..255) of every
  ``stride``-th output row, ``[3][rows][W]``;
* ``f32``: the float values of every ``8 * stride``-th row, ``[3][rows][W]``;
* ``guard_max``: the largest |x| of the raw stream at every guarded cast;

together with the SHA-256 of the whole u8 frame and the digests of the
seeded weights and latent, so a reader can tell which inputs they belong to.
Only ``oracle`` and ``synth`` are used; no value comes from the GPU path.

    python tests/golden/make_decode_golden.py --size 1024
    python tests/golden/make_decode_golden.py --size 2048
    python tests/golden/make_decode_golden.py --size 1024 --norm group

``--norm group`` stores the GroupNorm (FLUX-class) decoder of the same
seeds: every norm site GroupNorm(32, 1e-6) with its beta.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

STRIDE = {1024: 16, 2048: 64}
GAIN_LOG2 = 11
LATENT_SCALE = 8.0
GUARD_LOG2 = 8


def _stem(size: int, norm: str = "rms") -> str:
    return "decode_%d%s_rows" % (size, "" if norm == "rms" else "_" + norm)


def golden_path(size: int, norm: str = "rms") -> str:
    return os.path.join(HERE, _stem(size, norm) + ".npz")


def inputs(size: int, norm: str = "rms"):
    """The seeded weights and latent of the full-size decode."""
    spec = synth.decoder_spec(norm=norm)
    w = synth.decoder_weights(spec, seed_config=4, conv_in_gain=2.0 ** GAIN_LOG2)
    h0 = size // 8
    z = synth.decoder_latent(h0, h0, zc=spec.zc, config=5, scale=LATENT_SCALE)
    return w, z


def weights_digest(w) -> str:
    h = hashlib.sha256()

    def add(v):
        if isinstance(v, np.ndarray):
            h.update(v.tobytes())
        elif isinstance(v, dict):
            for k in sorted(v):
                add(v[k])
        elif isinstance(v, (list, tuple)):
            for e in v:
                add(e)

    add({k: v for k, v in w.items() if k != "spec"})
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--size", type=int, choices=sorted(STRIDE), default=1024)
    ap.add_argument("--q-chunk", type=int, default=4096)
    ap.add_argument("--norm", choices=("rms", "group"), default="rms")
    a = ap.parse_args()
    O.build()
    w, z = inputs(a.size, a.norm)
    t0 = time.time()
    tr = O.Trace()
    out = O.decode(w, z, guard_log2=GUARD_LOG2, q_chunk=a.q_chunk, trace=tr)
    secs = time.time() - t0
    assert out.shape == (3, a.size, a.size), out.shape
    stride = STRIDE[a.size]
    rows = np.arange(0, a.size, stride)
    frows = np.arange(0, a.size, 8 * stride)
    u8 = O.to_u8(out).astype(np.uint8)
    np.savez_compressed(
        golden_path(a.size, a.norm),
        rows=rows.astype(np.int32),
        u8=np.ascontiguousarray(u8[:, rows, :]),
        frows=frows.astype(np.int32),
        f32=np.ascontiguousarray(out[:, frows, :].astype(np.float32)),
        guard_max=np.asarray(tr.guard_max, dtype=np.float64),
    )
    meta = {
        "size": a.size,
        "norm": a.norm,
        "latent": [16, a.size // 8, a.size // 8],
        "latent_scale": LATENT_SCALE,
        "conv_in_gain_log2": GAIN_LOG2,
        "guard_log2": GUARD_LOG2,
        "latent_digest": hashlib.sha256(z.tobytes()).hexdigest()[:16],
        "weights_digest": weights_digest(w),
        "frame_u8_sha256": hashlib.sha256(u8.tobytes()).hexdigest(),
        "out_mean": float(out.mean()),
        "out_std": float(out.std()),
        "clipped_fraction": float(np.mean(np.abs(out) > 1.0)),
        "guard_max": tr.guard_max,
        "oracle_seconds": round(secs, 1),
        "command": "python tests/golden/make_decode_golden.py --size %d%s" % (
            a.size, "" if a.norm == "rms" else " --norm " + a.norm),
    }
    with open(os.path.join(HERE, _stem(a.size, a.norm) + ".json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(json.dumps(meta, indent=1))


if __name__ == "__main__":
    main()
