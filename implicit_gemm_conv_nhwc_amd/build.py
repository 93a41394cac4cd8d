"""Build libigconv.so in-tree with hipcc for gfx950.

Each HIP source compiles to an object under ``_build/`` (in parallel), then
hipcc links the shared library next to this file. Every HIP compile uses
``-Xclang -target-feature -Xclang -packed-fp32-ops``: packed-f32 VALU
instructions stay out of the code (hipcc's host pass warns that it does not
know the feature; that is harmless).
"""

from __future__ import annotations

import concurrent.futures as cf
import importlib.util
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libigconv.so")
ARCH = os.environ.get("IG_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "igemm.hip", "gemm2.hip", "conv_halo.hip", "conv_ws.hip", "conv_out.hip", "attn_flash.hip", "groupnorm.hip", "elementwise.hip", "decoder.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# sources whose MFMAs are inline asm: their device assembly is scanned for
# accesses the compiler placed inside an MFMA's latency window
ASM_MFMA_SOURCES = ["conv_ws.hip", "attn_flash.hip"]


def _check_isa(src: str) -> list:
    out = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *CFLAGS, "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, r.stderr))
    spec = importlib.util.spec_from_file_location("_ig_isa_check", os.path.join(HERE, "isa_check.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(out) as f:
        text = f.read()
    return [(src,) + x for x in mod.scan(text) + mod.scan_m0(text) + mod.scan_vmem(text)]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libigconv.so; returns its path.

    Refuses to link when the device code of an asm-MFMA source reads an
    MFMA result (or overwrites its accumulator) too early, uses M0 beyond
    the patch loads, or touches the registers of a load still in flight."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(ASM_MFMA_SOURCES))) as ex:
        objs_f = [ex.submit(_compile, src) for src in SOURCES]
        isa_f = [ex.submit(_check_isa, src) for src in ASM_MFMA_SOURCES]
        objs = [f.result() for f in objs_f]
        findings = [x for f in isa_f for x in f.result()]
    if findings:
        raise RuntimeError("hazards in the device code (isa_check.py):\n" +
                           "\n".join("%s %s: %s -> %s" % f for f in findings[:20]))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
