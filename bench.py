#!/usr/bin/env python3
"""Benchmark of the resident decoder's conv path on one MI355X.

One step = one whole decode (decoder_forward) of the synthetic decoder at
1024x1024 output: latent [16, 128, 128] ~ N(0,1)*8, conv_in gain 2^11 (the
stream passes the f16 range), guard 2^-8, every tensor resident in HBM.
`value` is the decode's algorithmic TFLOP/s (real channels; 3x3 and 1x1
convs at 2*M*cin*cout*k^2, attention at 2*m^2*C per product plus its four
projections); `decode_s` is seconds per decode. `decode_graph`: the same
decode captured once into a HIP graph and replayed (every kernel still
runs; no host launch per kernel), with a check that a replay's frame equals
the eager decode's.

Also measured, in the same process and on the stream the kernels run on:
  * roofline: the dominant kernel, the 3x3 implicit-GEMM conv at
    512x512x128 -> 128 (77.31 GFLOP per launch), against the dense f16
    MFMA peak of 2.5 PFLOP/s; inputs and outputs rotate through a pool
    larger than the 256 MB Infinity Cache;
  * roofline_norm: RMS_norm + f16 store at 512x512x128 (201 MB moved per
    launch: f32 read + f16 write) against 8 TB/s HBM;
  * roofline_cast: the guarded f16 cast at 512x512x128 (same 201 MB);
  * roofline_groupnorm: GroupNorm(32) + SiLU at 512x512x128, algorithmic
    201 MB (its statistics pass reads the input once more);
  * roofline_groupnorm_gathered: the same GroupNorm when the producing conv
    gathered the statistics in its epilogue (one read of the input), and
    the gathering's cost to a 256x256x256 conv (without, with);
  * roofline_attention: the single-pass attention core at 16384 tokens x
    512 (the 1024^2 decode's mid block; 4 m^2 C = 550 GFLOP per launch:
    Q.K^T and P.V) against the f16 MFMA peak;
  * cpu_baseline: the CPU oracle decoding the 256x256 configuration (a
    bounded sample of the same decoder), in TFLOP/s.

`python bench.py --digest-trace <kernel_trace.csv>` turns a rocprofv3
kernel trace of this command into the per-kernel summary kept in profiles/.
"""

from __future__ import annotations

import argparse
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
WARM_SECONDS = 0.05  # untimed launches for this long before each roofline's timed region


def _warm(fn, seconds=WARM_SECONDS):
    """Launch fn(i) until `seconds` of GPU work have passed: measured, the
    clock keeps rising for tens of milliseconds after the GPU was idle
    (host-side setup), and the timed regions should see the steady state."""
    import time

    import torch

    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(10):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i
ROOF_KERNEL = "k_conv_ws<1, false, false, true, false>"  # the 3x3 conv instantiation for 512^2 x 128
CONV_SRC = os.path.join(ROOT, "implicit_gemm_conv_nhwc_amd", "csrc", "conv_ws.hip")
CHIP_CLOCK_GHZ = 2.4  # the clock the published peaks are quoted at
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv3x3_512x512x128_traffic.json")


def conv_source_hash():
    import hashlib

    with open(CONV_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the roofline conv from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != conv_source_hash():
        return None
    return t.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _batches(fn, reps, batch=10):
    """Time reps launches of fn(i) in batches of `batch`, each batch between
    two HIP events on the current stream: per-launch ms as (median, mean)
    over the batches."""
    import statistics

    import torch

    per = []
    i = 0
    for _ in range(max(1, reps // batch)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(batch):
            fn(i)
            i += 1
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / batch)
    return statistics.median(per), statistics.fmean(per)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------


def decode_flops(spec, h0, w0):
    """Algorithmic FLOP of one decode (real channel counts)."""
    f = 0.0
    M = h0 * w0
    f += 2.0 * M * spec.zc * spec.c_in * 9  # conv_in

    def resnet(cin, cout, M):
        v = 2.0 * M * cin * cout * 9 + 2.0 * M * cout * cout * 9
        if cin != cout:
            v += 2.0 * M * cin * cout
        return v

    c = spec.c_in
    f += 2 * resnet(c, c, M)
    C = spec.attn_c
    f += 4 * 2.0 * M * C * C + 2 * 2.0 * M * M * C  # q, k, v, proj; QK^T and P.V
    for cs in spec.stages:
        for r in range(spec.n_res):
            f += resnet(c if r == 0 else cs, cs, M)
        c = cs
        M *= 4
        f += 2.0 * M * c * c * 9  # the up conv at the doubled size
    f += 2.0 * M * c * spec.out_c * 9  # conv_out
    return f


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------


def bench_decode(steps, warmup, h0, q_chunk, graph=False, norm="rms"):
    import torch

    import implicit_gemm_conv_nhwc_amd as ig
    import synth

    spec = synth.decoder_spec(norm=norm)
    w = synth.decoder_weights(spec, seed_config=4, conv_in_gain=2.0 ** 11)
    z = synth.decoder_latent(h0, h0, zc=spec.zc, config=5, scale=8.0)
    dd = ig.DeviceDecoder(w)
    zd = torch.from_numpy(z).cuda()
    ws = dd.alloc_workspace(h0, h0, q_chunk)
    H = h0 << dd.n_up
    out = torch.empty((dd.out_c, H, H), dtype=torch.float32, device="cuda")
    log("decode %dx%d: workspace %.2f GB" % (H, H, ws[1] / 1e9))
    for _ in range(warmup):
        dd.forward(zd, h0, h0, guard_log2=8, q_chunk=q_chunk, ws=ws, out=out)
    torch.cuda.synchronize()
    import statistics

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for k in range(steps):
        dd.forward(zd, h0, h0, guard_log2=8, q_chunk=q_chunk, ws=ws, out=out)
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
    ev_ms = sum(per)
    finite = bool(torch.isfinite(out).all().item())
    flops = decode_flops(spec, h0, h0)
    res = {"wall_s": wall, "event_ms": ev_ms, "median_ms": statistics.median(per), "flops": flops,
           "finite": finite, "H": H, "spec": spec}
    if graph:
        # the same decode captured once into a HIP graph and replayed: every
        # kernel still runs, without a host launch per kernel
        ref = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dd.forward(zd, h0, h0, guard_log2=8, q_chunk=q_chunk, ws=ws, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dd.forward(zd, h0, h0, guard_log2=8, q_chunk=q_chunk, ws=ws, out=out)
        for _ in range(max(warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(out, ref))
        gevs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        gevs[0].record()
        for k in range(steps):
            g.replay()
            gevs[k + 1].record()
        torch.cuda.synchronize()
        gper = [gevs[k].elapsed_time(gevs[k + 1]) for k in range(steps)]
        res["graph"] = {"median_s": round(statistics.median(gper) / 1000.0, 6),
                        "mean_s": round(sum(gper) / steps / 1000.0, 6), "steps": steps,
                        "equals_eager": same and bool(torch.equal(out, ref))}
        del g
    del ws
    return res


def bench_conv_roofline(reps, H=512, W=512, C=128):
    """The 3x3 conv of the 512^2 x 128 -> 128 configuration, timed with HIP
    events on the launch stream, buffers rotated through > 1 GB."""
    import numpy as np
    import torch

    import implicit_gemm_conv_nhwc_amd as ig
    import synth

    d = synth.config3(C, H, W)
    M = H * W
    dev = torch.device("cuda")
    w16 = torch.from_numpy(d["w"]).to(dev)
    plane = torch.empty(ig.plane_shape(C, C, 3), dtype=torch.float16, device=dev)
    ig.pack_conv_weights(w16, C, C, 3, C, C, plane)
    bias = torch.from_numpy(d["b"]).to(dev)
    gamma = torch.from_numpy(d["gamma"]).to(dev)
    x32 = torch.from_numpy(d["x"].reshape(M, C)).to(dev)
    per_set = M * C * (2 + 4)
    nsets = max(2, int(np.ceil(1.2e9 / per_set)))
    xs = [torch.empty((M, C), dtype=torch.float16, device=dev) for _ in range(nsets)]
    ys = [torch.empty((M, C), dtype=torch.float32, device=dev) for _ in range(nsets)]
    for t in xs:
        ig.rmsnorm_silu_f16(x32, M, C, C, None, gamma, 0, 1e-12, t)
    # warm up to the steady clock (the host-side setup above leaves the GPU
    # idle for seconds)
    run = lambda i: ig.conv3x3_nhwc(xs[i % nsets], H, W, C, plane, C, bias, 1.0, ys[i % nsets])  # noqa: E731
    nwarm = _warm(run)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / reps
    med_ms, _ = _batches(run, reps)
    # the clock the conv runs at: its first wave's shader-clock and 100 MHz
    # real-time counters, over a few more launches (the last one's kept)
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    ig.set_clock_probe(clk)
    try:
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
    finally:
        ig.set_clock_probe(None)
    ck0, rt0, ck1, rt1 = [int(v) for v in clk.cpu()]
    ghz = (ck1 - ck0) / ((rt1 - rt0) / 1e8) / 1e9 if rt1 > rt0 else None
    flops = 2.0 * M * C * C * 9
    byts = M * C * 2 + C * 9 * C * 2 + M * C * 4
    ok = bool(torch.isfinite(ys[(reps - 1) % nsets]).all().item())
    return {"avg_ms": avg_ms, "median_ms": med_ms, "clock_ghz": ghz, "flops": flops, "bytes": byts,
            "launches": reps, "warm_launches": nwarm, "finite": ok, "sets": nsets}


def bench_norm_roofline(reps, H=512, W=512, C=128):
    import numpy as np
    import torch

    import implicit_gemm_conv_nhwc_amd as ig
    import synth

    d = synth.config3(C, H, W)
    M = H * W
    dev = torch.device("cuda")
    gamma = torch.from_numpy(d["gamma"]).to(dev)
    per_set = M * C * 6
    nsets = max(2, int(np.ceil(1.2e9 / per_set)))
    x0 = torch.from_numpy(d["x"].reshape(M, C)).to(dev)
    xs = [x0.clone() for _ in range(nsets)]
    ys = [torch.empty((M, C), dtype=torch.float16, device=dev) for _ in range(nsets)]
    run = lambda i: ig.rmsnorm_silu_f16(xs[i % nsets], M, C, C, None, gamma, 1, 1e-12, ys[i % nsets])  # noqa: E731
    _warm(run)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / reps
    med, _ = _batches(run, reps)
    return {"avg_ms": avg_ms, "median_ms": med, "bytes": M * C * 6, "sets": nsets}


def _pool_timed(fn, reps, per_set_bytes, make_set):
    """Time `fn(set)` over a rotating pool of input/output sets larger than
    the Infinity Cache; returns (avg ms, sets)."""
    import numpy as np
    import torch

    nsets = max(2, int(np.ceil(1.2e9 / per_set_bytes)))
    sets = [make_set() for _ in range(nsets)]
    _warm(lambda i: fn(sets[i % nsets]))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(sets[i % nsets])
    e1.record()
    torch.cuda.synchronize()
    med, _ = _batches(lambda i: fn(sets[i % nsets]), reps)
    return e0.elapsed_time(e1) / reps, nsets, med


def bench_cast_roofline(reps, H=512, W=512, C=128):
    """guard_cast f32 -> f16 (x 2^-8) at 512x512x128: 6 bytes per element."""
    import torch

    import implicit_gemm_conv_nhwc_amd as ig

    M = H * W
    dev = torch.device("cuda")
    x0 = torch.randn((M, C), device=dev) * 300.0
    ms, nsets, med = _pool_timed(lambda st: ig.guard_cast(st[0], M, C, None, 8, st[1]), reps, M * C * 6,
                                 lambda: (x0.clone(), torch.empty((M, C), dtype=torch.float16, device=dev)))
    return {"avg_ms": ms, "median_ms": med, "bytes": M * C * 6, "sets": nsets}


def bench_groupnorm_roofline(reps, H=512, W=512, C=128, groups=32):
    """GroupNorm(32) + SiLU -> f16 at 512x512x128. Algorithmic bytes: 6 per
    element (f32 read, f16 write); the kernels read the input twice (the
    statistics must be complete before any output)."""
    import torch

    import implicit_gemm_conv_nhwc_amd as ig

    M = H * W
    dev = torch.device("cuda")
    x0 = torch.randn((M, C), device=dev)
    gamma = torch.rand(C, device=dev) + 0.5
    beta = torch.randn(C, device=dev) * 0.1
    nbytes = ig.groupnorm_workspace_bytes(M, C, groups)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ms, nsets, med = _pool_timed(
        lambda st: ig.groupnorm_silu_f16(st[0], M, C, C, groups, None, gamma, beta, 1, 1e-6, ws, nbytes, st[1]),
        reps, M * C * 6, lambda: (x0.clone(), torch.empty((M, C), dtype=torch.float16, device=dev)))
    return {"avg_ms": ms, "median_ms": med, "bytes": M * C * 6, "sets": nsets}


def bench_groupnorm_fused(reps, H=512, W=512, C=128, groups=32):
    """GroupNorm(32) + SiLU at 512x512x128 when the producing 3x3 conv has
    gathered the group statistics in its epilogue: the final merge and one
    read of the stream (201 MB algorithmic, 6 bytes per element). Also the
    cost of the gathering to the conv: 256x256x256 -> 256 with and without
    it (both the general-width conv kernel)."""
    import torch

    import implicit_gemm_conv_nhwc_amd as ig

    M = H * W
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    gamma = torch.rand(C, device=dev, generator=g) + 0.5
    beta = torch.randn(C, device=dev, generator=g) * 0.1

    def conv_setup(h, w, c):
        x16 = torch.randn((h * w, c), device=dev, generator=g).half()
        wt = (torch.randn((c, c, 3, 3), device=dev, generator=g) / (3.0 * c ** 0.5)).half()
        plane = torch.empty(ig.plane_shape(c, c, 3), dtype=torch.float16, device=dev)
        ig.pack_conv_weights(wt, c, c, 3, c, c, plane)
        nb = ig.conv_gn_partials_bytes(1, h, w, groups)
        return x16, plane, nb, torch.empty(nb // 4, dtype=torch.float32, device=dev)

    x16, plane, nbytes, part = conv_setup(H, W, C)
    y32 = torch.empty((M, C), dtype=torch.float32, device=dev)
    ig.conv3x3_gn_stats_nhwc(x16, H, W, C, 1, plane, C, None, 1.0, 0, y32, C, groups, part, nbytes)
    nchunk = nbytes // (12 * groups)
    tab = torch.empty(3 * C, dtype=torch.float32, device=dev)
    ms, nsets, med = _pool_timed(
        lambda st: ig.groupnorm_silu_f16_from_partials(st[0], M, C, C, groups, gamma, beta, 1, 1e-6, part, nchunk,
                                                       tab, tab.numel() * 4, st[1]),
        reps, M * C * 6, lambda: (y32.clone(), torch.empty((M, C), dtype=torch.float16, device=dev)))
    # the gathering's cost: the same conv with and without it, interleaved
    h2, c2 = 256, 256
    x2, plane2, nb2, part2 = conv_setup(h2, h2, c2)
    ys = [torch.empty((h2 * h2, c2), dtype=torch.float32, device=dev) for _ in range(6)]
    plain = lambda i: ig.conv_nhwc_ex(x2, h2, h2, c2, 1, plane2, c2, None, 1.0, 0, ys[i % 6])  # noqa: E731
    gath = lambda i: ig.conv3x3_gn_stats_nhwc(x2, h2, h2, c2, 1, plane2, c2, None, 1.0, 0, ys[i % 6], c2,  # noqa: E731
                                              groups, part2, nb2)
    _warm(plain)
    pm, gm = [], []
    for _ in range(3):
        pm.append(_batches(plain, reps)[0])
        gm.append(_batches(gath, reps)[0])
    import statistics

    return {"avg_ms": ms, "median_ms": med, "bytes": M * C * 6, "sets": nsets,
            "conv_plain_us": statistics.median(pm) * 1000, "conv_gather_us": statistics.median(gm) * 1000}


def bench_attention_roofline(reps, m=16384, C=512):
    """attention_f16 (single pass) at m tokens x C: 4 m^2 C FLOP per launch."""
    import torch

    import implicit_gemm_conv_nhwc_amd as ig

    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    q = torch.randn((m, C), device=dev, generator=g).half()
    k = torch.randn((m, C), device=dev, generator=g).half()
    vt = torch.randn((C, m), device=dev, generator=g).half()
    bv = torch.zeros(C, device=dev)
    nb = ig.attention_workspace_bytes(m, C)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((m, C), dtype=torch.float16, device=dev)
    run = lambda i: ig.attention_f16(q, k, vt, m, m, C, bv, ws, nb, out)  # noqa: E731
    _warm(run)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    med, _ = _batches(run, reps, batch=1)
    return {"avg_ms": e0.elapsed_time(e1) / reps, "median_ms": med, "flops": 4.0 * m * m * C}


def bench_cfg2(reps):
    """Config 2 at 128x128x256: the guarded input's nearest-2x 3x3 up conv
    256 -> 256 (M = 65536 outputs, K = 2304: 77.3 GFLOP) and its 1x1
    shortcut 256 -> 256 (2.15 GFLOP), outputs rotated past the cache."""
    import numpy as np
    import torch

    import implicit_gemm_conv_nhwc_amd as ig
    import synth

    d = synth.config2()
    H, W, C = d["x"].shape
    M = H * W
    dev = torch.device("cuda")
    gs = float(2 ** d["guard_log2"])
    xg = torch.empty((M, C), dtype=torch.float16, device=dev)
    ig.guard_cast(torch.from_numpy(d["x"].reshape(M, C)).to(dev), M, C, None, d["guard_log2"], xg)
    p_up = torch.empty(ig.plane_shape(C, C, 3), dtype=torch.float16, device=dev)
    ig.pack_conv_weights(torch.from_numpy(d["w_up"]).to(dev), C, C, 3, C, C, p_up)
    p_sc = torch.empty(ig.plane_shape(C, C, 1), dtype=torch.float16, device=dev)
    ig.pack_conv_weights(torch.from_numpy(d["w_sc"]).to(dev), C, C, 1, C, C, p_sc)
    b_up = torch.from_numpy(d["b_up"]).to(dev)
    b_sc = torch.from_numpy(d["b_sc"]).to(dev)
    n_up = max(2, int(np.ceil(1.2e9 / (4 * M * C * 4))))
    ups = [torch.empty((4 * M, C), dtype=torch.float32, device=dev) for _ in range(n_up)]
    run_up = lambda i: ig.conv3x3_up2_nhwc(xg, H, W, C, p_up, C, b_up, gs, ups[i % n_up])  # noqa: E731
    _warm(run_up)
    up_med, up_avg = _batches(run_up, reps)
    n_sc = max(2, int(np.ceil(1.2e9 / (M * C * 4))))
    scs = [torch.empty((M, C), dtype=torch.float32, device=dev) for _ in range(n_sc)]
    run_sc = lambda i: ig.gemm1x1(xg, M, C, C, p_sc, C, C, b_sc, gs, scs[i % n_sc], C, 0)  # noqa: E731
    _warm(run_sc)
    sc_med, sc_avg = _batches(run_sc, reps)
    out = {}
    for name, med, avg, fl in (("up_conv_3x3_128x128x256_to_256x256x256", up_med, up_avg, 2.0 * 4 * M * C * C * 9),
                               ("shortcut_1x1_128x128x256", sc_med, sc_avg, 2.0 * M * C * C)):
        out[name] = {"median_us": round(med * 1000, 3), "mean_us": round(avg * 1000, 3), "gflop": round(fl / 1e9, 3),
                     "tflops": round(fl / (med / 1000.0) / 1e12, 2),
                     "frac_of_peak": round(fl / (med / 1000.0) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
    return out


def bench_cfg3_padded(reps, c, H=512, W=512):
    """Config 3's padded variant: c real channels stored in cp (288 in 320,
    144 in 192), the 3x3 conv at 512x512; algorithmic FLOP counts the real
    channels, executed FLOP the padded ones."""
    import numpy as np
    import torch

    import implicit_gemm_conv_nhwc_amd as ig
    import synth

    cp = {288: 320, 144: 192}[c]
    d = synth.config3(c, H, W)
    M = H * W
    dev = torch.device("cuda")
    gamma = torch.zeros(cp, device=dev)
    gamma[:c] = torch.from_numpy(d["gamma"]).to(dev)
    bias = torch.zeros(cp, device=dev)
    bias[:c] = torch.from_numpy(d["b"]).to(dev)
    x32 = torch.zeros((M, cp), device=dev)
    x32[:, :c] = torch.from_numpy(d["x"].reshape(M, c)).to(dev)
    plane = torch.empty(ig.plane_shape(cp, cp, 3), dtype=torch.float16, device=dev)
    ig.pack_conv_weights(torch.from_numpy(d["w"]).to(dev), c, c, 3, cp, cp, plane)
    nsets = max(2, int(np.ceil(1.2e9 / (M * cp * 6))))
    xs = [torch.empty((M, cp), dtype=torch.float16, device=dev) for _ in range(nsets)]
    ys = [torch.empty((M, cp), dtype=torch.float32, device=dev) for _ in range(nsets)]
    for t in xs:
        ig.rmsnorm_silu_f16(x32, M, cp, c, None, gamma, 0, 1e-12, t)
    run = lambda i: ig.conv3x3_nhwc(xs[i % nsets], H, W, cp, plane, cp, bias, 1.0, ys[i % nsets])  # noqa: E731
    _warm(run)
    med, avg = _batches(run, reps)
    alg = 2.0 * M * c * c * 9
    exe = 2.0 * M * cp * cp * 9
    return {"median_us": round(med * 1000, 3), "mean_us": round(avg * 1000, 3),
            "algorithmic_gflop": round(alg / 1e9, 2), "executed_gflop": round(exe / 1e9, 2),
            "algorithmic_tflops": round(alg / (med / 1000.0) / 1e12, 2),
            "executed_tflops": round(exe / (med / 1000.0) / 1e12, 2),
            "executed_frac_of_peak": round(exe / (med / 1000.0) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


def cpu_conv(H=512, W=512, C=128):
    """The oracle's 3x3 conv (float64 direct loop, OpenMP) at config 3's
    512x512x128 -> 128 on the host: seconds for one conv."""
    import numpy as np

    import oracle as O
    import synth

    d = synth.config3(C, H, W)
    x = np.ascontiguousarray(d["x"].transpose(2, 0, 1), dtype=np.float64)
    O.conv2d(x[:, :8, :8], d["w"], d["b"])  # build + load the library
    t0 = time.perf_counter()
    O.conv2d(x, d["w"], d["b"])
    t = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    fl = 2.0 * H * W * C * C * 9
    return {"seconds": round(t, 3), "gflops": round(fl / t / 1e9, 2), "cores": threads, "kind": "oracle",
            "sample": "one oracle conv2d (f64) at 512x512x128 -> 128, the roofline conv's configuration"}


def cpu_baseline(min_seconds=10.0):
    """The oracle (as it is) decoding the 256x256 configuration on the host."""
    import oracle as O
    import synth

    spec = synth.decoder_spec()
    w = synth.decoder_weights(spec, seed_config=4)
    z = synth.decoder_latent(32, 32, zc=spec.zc, config=4)
    O.decode(w, z, guard_log2=8, q_chunk=256)  # build + warm the library
    n, t = 0, 0.0
    while t < min_seconds or n == 0:
        t0 = time.perf_counter()
        O.decode(w, z, guard_log2=8, q_chunk=256)
        t += time.perf_counter() - t0
        n += 1
    flops = decode_flops(spec, 32, 32) * n
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d oracle decode(s) of the 256x256 configuration (latent 32x32x16, same "
                      "decoder, f64 direct loops), %.1f s" % (n, t)}


# ---------------------------------------------------------------------------
# rocprofv3 trace digest
# ---------------------------------------------------------------------------


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size (torch elementwise kernel), for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print("copy calibration: %d launches, %d bytes read and %d written per launch" % (reps, nbytes, nbytes))


def _is_roof(name):
    """The roofline conv's kernel, by its demangled or mangled name."""
    return ROOF_KERNEL.replace(" ", "") in name.replace(" ", "") or "k_conv_wsILi1ELb0ELb0ELb1ELb0E" in name


def digest_pmc(conv_csv, copy_csv, counter, roof_launches, nbytes=1 << 30):
    """Average of `counter` over the roofline conv launches, scaled by the
    counter's reading for the plain copy (bytes moved / counter value)."""
    import csv

    def rows(path):
        return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]

    conv = [float(r["Counter_Value"]) for r in sorted(rows(conv_csv), key=lambda r: int(r["Start_Timestamp"]))
            if _is_roof(r["Kernel_Name"])][-roof_launches:]
    cp = [float(r["Counter_Value"]) for r in rows(copy_csv) if "mul" in r["Kernel_Name"].lower()
          or "elementwise" in r["Kernel_Name"].lower()]
    scale = nbytes / (sum(cp) / len(cp))
    avg = sum(conv) / len(conv)
    print("%s: conv %.1f (n=%d), copy %.1f per %d bytes -> scale %.4f bytes/unit -> %.1f MB per launch" % (
        counter, avg, len(conv), sum(cp) / len(cp), nbytes, scale, avg * scale / 1e6))
    return avg * scale


def digest_pmc_stream(fetch_csv, write_csv, copyf_csv, copyw_csv, roof_launches, nbytes=1 << 30):
    """HBM bytes per launch of the RMS_norm and guarded-cast rooflines (the
    last `roof_launches` dispatches of each), scaled like the conv's."""
    import csv

    def scale(copy_csv, counter):
        cp = [float(r["Counter_Value"]) for r in csv.DictReader(open(copy_csv)) if r["Counter_Name"] == counter
              and ("mul" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower())]
        return nbytes / (sum(cp) / len(cp))

    def avg(path, counter, match):
        v = [float(r["Counter_Value"]) for r in sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
             if r["Counter_Name"] == counter and match(r["Kernel_Name"])][-roof_launches:]
        return sum(v) / len(v) if v else float("nan")

    fs, ws = scale(copyf_csv, "FETCH_SIZE"), scale(copyw_csv, "WRITE_SIZE")
    for title, match, algo in (("rmsnorm 512^2x128 (k_rmsnorm<2>)", lambda n: "k_rmsnorm" in n and "ILi2E" in n, 262144 * 128 * 6),
                               ("guard_cast 512^2x128 (k_guard_cast)", lambda n: "k_guard_cast" in n, 262144 * 128 * 6)):
        f = avg(fetch_csv, "FETCH_SIZE", match) * fs
        w = avg(write_csv, "WRITE_SIZE", match) * ws
        print("%s: read %.1f MB, written %.1f MB, total %.1f MB per launch (algorithmic %.1f MB)" % (
            title, f / 1e6, w / 1e6, (f + w) / 1e6, algo / 1e6))


def digest_counters(path, roof_launches, n_xcd=8, n_simd=1024):
    """Averages of every counter over the conv roofline's last
    `roof_launches` dispatches and the attention roofline's last 10, and
    what they imply: the clock (GRBM_GUI_ACTIVE counts per XCD) and the MFMA
    pipes' busy share (SQ_VALU_MFMA_BUSY_CYCLES summed over the 1024 SIMDs)."""
    import csv

    rows = list(csv.DictReader(open(path)))
    kernels = [("conv3x3 512^2x128 (%s)" % ROOF_KERNEL, _is_roof, roof_launches, None, None),
               # the single-pass kernel at 16384 tokens (128 queries per
               # workgroup, key ranges split over 256 workgroups): the
               # roofline's grid; the 256^2 and 2048^2 decodes after it
               # run other grids
               ("attention 16384 x 512 (k_flash)", lambda n: "k_flash<" in n or "k_flashILi" in n, 10, "65536", None)]
    # the 1024^2 decode's convs: every dispatch before the roofline region
    # (the decodes run first), the last 10 of each conv kernel and grid
    t_roof = min([int(r["Start_Timestamp"]) for r in rows if _is_roof(r["Kernel_Name"])] or [1 << 62])
    conv = lambda n: "k_conv_ws" in n or "k_conv_halo" in n  # noqa: E731
    seen = sorted({(r["Kernel_Name"], r["Grid_Size"]) for r in rows
                   if conv(r["Kernel_Name"]) and int(r["Start_Timestamp"]) < t_roof})
    for name, g in seen:
        m = re.search(r"k_conv_\w+<[^>]*>", name)
        short = m.group(0) if m else name[:60]
        kernels.append(("1024^2 decode: %s, grid %s" % (short, g), (lambda nm: lambda n: n == nm)(name), 10, g, t_roof))
    res = {}
    for title, match, last, grid, before in kernels:
        by = {}
        for r in rows:
            if match(r["Kernel_Name"]) and (grid is None or r["Grid_Size"] == grid) and \
                    (before is None or int(r["Start_Timestamp"]) < before):
                by.setdefault(r["Counter_Name"], []).append((int(r["Start_Timestamp"]), float(r["Counter_Value"]),
                                                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        if not by:
            continue
        print("%s:" % title)
        out = {}
        dur_ns = 1.0
        for name, v in sorted(by.items()):
            v = sorted(v)[-last:]
            out[name] = sum(x[1] for x in v) / len(v)
            dur_ns = sum(x[2] for x in v) / len(v)
            print("  %-28s %16.1f   (n=%d, dispatch %.1f us)" % (name, out[name], len(v), dur_ns / 1e3))
        if "GRBM_GUI_ACTIVE" in out:
            cyc = out["GRBM_GUI_ACTIVE"] / n_xcd
            print("  clock: %.0f cycles per XCD over %.1f us = %.2f GHz" % (cyc, dur_ns / 1e3, cyc / dur_ns))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in out:
                busy = out["SQ_VALU_MFMA_BUSY_CYCLES"] / n_simd
                print("  MFMA busy: %.0f cycles per SIMD = %.1f%% of the dispatch" % (busy, 100 * busy / cyc))
        res[title] = out
    return res


def digest_trace(path, roof_launches):
    """Per-kernel totals of a rocprofv3 kernel trace, plus the average of the
    roofline region's launches of the dominant kernel (its last
    `roof_launches` dispatches: that region runs after the decodes)."""
    import csv

    rows = list(csv.DictReader(open(path)))
    stats = {}
    seq = []
    for r in rows:
        name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        s = stats.setdefault(name, [0, 0.0])
        s[0] += 1
        s[1] += t
        seq.append((int(r["Start_Timestamp"]), name, t, r.get("Grid_Size", r.get("Grid_Size_X", ""))))
    seq.sort()
    tot = sum(v[1] for v in stats.values())
    print("kernel | calls | total us | avg us | share")
    for name, (n, t) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        short = name if len(name) < 90 else name[:87] + "..."
        print("%s | %d | %.1f | %.2f | %.1f%%" % (short, n, t, t / n, 100 * t / tot))
    roof = [x for x in seq if _is_roof(x[1])]
    last = roof[-roof_launches:]
    t_roof = roof[0][0] if roof else 1 << 62
    if last:
        avg = sum(x[2] for x in last) / len(last)
        print("roofline region: last %d dispatches of %s (grid %s): avg %.2f us" % (
            len(last), ROOF_KERNEL, last[-1][3], avg))
    # the roofline's timed launches in order: roof_launches for the average,
    # roof_launches in batches of 10 for the median, then 5 with the clock
    # probe set (bench_conv_roofline)
    n_probe = 5
    if len(roof) >= 2 * roof_launches + n_probe:
        a = roof[-(2 * roof_launches + n_probe):-(roof_launches + n_probe)]
        b = roof[-(roof_launches + n_probe):-n_probe]
        print("  the bench's average launches: avg %.2f us; its median batches: avg %.2f us, median %.2f us" % (
            sum(x[2] for x in a) / len(a), sum(x[2] for x in b) / len(b), sorted(x[2] for x in b)[len(b) // 2]))
    # the last 1024^2 decode alone (the decodes before the roofline region):
    # from its latent cast (k_latent) to its output conv (k_conv_out), by
    # kernel and grid
    starts = [i for i, x in enumerate(seq) if "k_latent" in x[1] and x[0] < t_roof]
    if starts:
        dec = seq[starts[-1]:]
        ends = [i for i, x in enumerate(dec) if "k_conv_out" in x[1]]
        dec = dec[:ends[0] + 1] if ends else dec
        per = {}
        for _, name, t, grid in dec:
            short = name if len(name) < 70 else name[:67] + "..."
            e = per.setdefault((short, grid), [0, 0.0])
            e[0] += 1
            e[1] += t
        busy = sum(v[1] for v in per.values())
        print("\nlast 1024^2 decode: %d dispatches, %.1f us of kernel time" % (len(dec), busy))
        print("kernel | grid (threads) | calls | total us | share")
        for (name, grid), (n, t) in sorted(per.items(), key=lambda kv: -kv[1][1]):
            print("%s | %s | %d | %.1f | %.1f%%" % (name, grid, n, t, 100 * t / busy))


# ---------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--latent", type=int, default=128, help="latent side (output = 8x)")
    ap.add_argument("--q-chunk", type=int, default=0)
    ap.add_argument("--roof-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--digest-trace", default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--digest-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"))
    ap.add_argument("--digest-counters", default=None, metavar="COUNTER_CSV")
    args = ap.parse_args()

    if args.digest_counters:
        digest_counters(args.digest_counters, args.roof_reps)
        return 0

    if args.digest_trace:
        digest_trace(args.digest_trace, args.roof_reps)
        return 0
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.digest_pmc:
        f = digest_pmc(args.digest_pmc[0], args.digest_pmc[2], "FETCH_SIZE", args.roof_reps)
        w = digest_pmc(args.digest_pmc[1], args.digest_pmc[3], "WRITE_SIZE", args.roof_reps)
        digest_pmc_stream(*args.digest_pmc, args.roof_reps)
        print(json.dumps({"source_sha256_16": conv_source_hash(), "fetch_bytes_per_launch": round(f),
                          "write_bytes_per_launch": round(w), "bytes_per_launch": round(f + w)}))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decoder runs on a single MI355X "
              "(--gpus %d requested); sharding across GPUs is not implemented." % args.gpus,
              file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("device:", torch.cuda.get_device_name(0))

    dec = bench_decode(args.steps, args.warmup, args.latent, args.q_chunk, graph=True)
    ms = dec["wall_s"] * 1000.0 / args.steps
    ev_ms = dec["event_ms"] / args.steps
    tflops = dec["flops"] / (ms / 1000.0) / 1e12
    log("decode %d^2: %.3f ms/step (events %.3f), %.1f TFLOP/s, finite=%s" % (
        dec["H"], ms, ev_ms, tflops, dec["finite"]))
    log("decode %d^2 replayed from a HIP graph: median %.3f ms (equals eager: %s)" % (
        dec["H"], dec["graph"]["median_s"] * 1000.0, dec["graph"]["equals_eager"]))

    conv = bench_conv_roofline(args.roof_reps)
    conv_tf = conv["flops"] / (conv["avg_ms"] / 1000.0) / 1e12
    log("conv3x3 512^2x128: %.2f us, %.1f TFLOP/s (%.1f%% of MFMA peak)" % (
        conv["avg_ms"] * 1000, conv_tf, 100 * conv_tf / MFMA_F16_PEAK_TFLOPS))
    norm = bench_norm_roofline(args.roof_reps)
    norm_gbs = norm["bytes"] / (norm["avg_ms"] / 1000.0) / 1e9
    log("rmsnorm 512^2x128: %.2f us, %.0f GB/s (%.1f%% of HBM)" % (
        norm["avg_ms"] * 1000, norm_gbs, 100 * norm_gbs / HBM_PEAK_GBS))

    cast = bench_cast_roofline(args.roof_reps)
    cast_gbs = cast["bytes"] / (cast["avg_ms"] / 1000.0) / 1e9
    log("guard_cast 512^2x128: %.2f us, %.0f GB/s (%.1f%% of HBM)" % (
        cast["avg_ms"] * 1000, cast_gbs, 100 * cast_gbs / HBM_PEAK_GBS))
    gn = bench_groupnorm_roofline(args.roof_reps)
    gn_gbs = gn["bytes"] / (gn["avg_ms"] / 1000.0) / 1e9
    log("groupnorm 512^2x128 (32 groups): %.2f us, %.0f GB/s algorithmic (%.1f%% of HBM)" % (
        gn["avg_ms"] * 1000, gn_gbs, 100 * gn_gbs / HBM_PEAK_GBS))
    gnf = bench_groupnorm_fused(args.roof_reps)
    gnf_gbs = gnf["bytes"] / (gnf["avg_ms"] / 1000.0) / 1e9
    log("groupnorm 512^2x128 from conv-gathered statistics: %.2f us, %.0f GB/s (%.1f%% of HBM); the gathering "
        "in a 256^2x256 conv: %.2f -> %.2f us" % (gnf["avg_ms"] * 1000, gnf_gbs, 100 * gnf_gbs / HBM_PEAK_GBS,
                                                 gnf["conv_plain_us"], gnf["conv_gather_us"]))
    att = bench_attention_roofline(max(5, args.roof_reps // 5))
    att_tf = att["flops"] / (att["avg_ms"] / 1000.0) / 1e12
    log("attention 16384 x 512: %.1f us, %.1f TFLOP/s (%.1f%% of MFMA peak)" % (
        att["avg_ms"] * 1000, att_tf, 100 * att_tf / MFMA_F16_PEAK_TFLOPS))

    # the other configurations' figures
    decodes = {}
    for lat, st, wu, nm in ((32, 10, 3, "rms"), (256, 3, 1, "rms"), (128, 10, 3, "group")):
        dx = bench_decode(st, wu, lat, args.q_chunk, norm=nm)
        decodes["%dx%d%s" % (dx["H"], dx["H"], "" if nm == "rms" else "_groupnorm")] = {
            "median_s": round(dx["median_ms"] / 1000.0, 6), "mean_s": round(dx["event_ms"] / st / 1000.0, 6),
            "steps": st, "tflop": round(dx["flops"] / 1e12, 4),
            "tflops": round(dx["flops"] / (dx["median_ms"] / 1000.0) / 1e12, 2), "output_finite": dx["finite"]}
        log("decode %d^2 (%s): median %.3f ms" % (dx["H"], nm, dx["median_ms"]))
    cfg2 = bench_cfg2(args.roof_reps)
    log("config 2:", json.dumps(cfg2))
    cfg3p = {}
    for c in (288, 144):
        r = bench_cfg3_padded(args.roof_reps, c)
        cfg3p["%d_in_%d" % (c, {288: 320, 144: 192}[c])] = r
        log("config 3, %d channels padded: %s" % (c, json.dumps(r)))

    cpu = cpu_c = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
        log("cpu baseline: %.4f TFLOP/s on %d threads (%s)" % (cpu["value"], cpu["cores"], cpu["sample"]))
        cpu_c = cpu_conv()
        log("cpu conv: %.2f s (%.1f GFLOP/s) on %d threads" % (cpu_c["seconds"], cpu_c["gflops"], cpu_c["cores"]))

    spec = dec["spec"]
    res = {
        "metric": "3x3 conv TFLOP/s (f16->f32, % MFMA peak) + full decode s at 1024^2",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": "synthetic VAE decoder, %dx%d output, whole frame resident in HBM" % (dec["H"], dec["H"]),
            "latent": [spec.zc, args.latent, args.latent],
            "channels": [spec.c_in] + list(spec.stages),
            "resnets_per_stage": spec.n_res,
            "attention_tokens": args.latent * args.latent,
            "guard_log2": 8,
            "q_chunk": args.q_chunk or "default",
        },
        "decode_s": round(ms / 1000.0, 6),
        "decode_s_median": round(dec["median_ms"] / 1000.0, 6),
        "decode_graph": dec["graph"],
        "decode_tflop": round(dec["flops"] / 1e12, 4),
        "output_finite": dec["finite"],
        "roofline": {
            "kernel": "conv3x3_nhwc %s, 512x512x128->128" % ROOF_KERNEL,
            "bound": "mfma",
            "achieved": round(conv_tf, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(conv_tf / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "avg_launch_us": round(conv["avg_ms"] * 1000, 3),
            "median_launch_us": round(conv["median_ms"] * 1000, 3),
            "algorithmic_bytes": conv["bytes"],
            # the fraction of the peak at the clock the conv ran at (its first
            # wave's shader-clock over 100 MHz real-time counters)
            "clock_ghz": round(conv["clock_ghz"], 3) if conv["clock_ghz"] else None,
            "frac_at_clock": round(conv_tf / (MFMA_F16_PEAK_TFLOPS * conv["clock_ghz"] / CHIP_CLOCK_GHZ), 4)
            if conv["clock_ghz"] else None,
        },
        "roofline_norm": {
            "kernel": "rmsnorm_silu_f16 512x512x128",
            "bound": "hbm",
            "achieved": round(norm_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(norm_gbs / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(norm["avg_ms"] * 1000, 3),
            "median_launch_us": round(norm["median_ms"] * 1000, 3),
        },
        "roofline_cast": {
            "kernel": "guard_cast 512x512x128 (g=8)",
            "bound": "hbm",
            "achieved": round(cast_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(cast_gbs / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(cast["avg_ms"] * 1000, 3),
            "median_launch_us": round(cast["median_ms"] * 1000, 3),
        },
        "roofline_groupnorm": {
            "kernel": "groupnorm_silu_f16 512x512x128, 32 groups (stats + finalize + apply)",
            "bound": "hbm",
            "achieved": round(gn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gn_gbs / HBM_PEAK_GBS, 4),
            "avg_us": round(gn["avg_ms"] * 1000, 3),
            "median_us": round(gn["median_ms"] * 1000, 3),
        },
        "roofline_groupnorm_gathered": {
            "kernel": "groupnorm_silu_f16_from_partials 512x512x128, 32 groups (statistics gathered by the "
                      "producing conv; finalize + apply)",
            "bound": "hbm",
            "achieved": round(gnf_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gnf_gbs / HBM_PEAK_GBS, 4),
            "avg_us": round(gnf["avg_ms"] * 1000, 3),
            "median_us": round(gnf["median_ms"] * 1000, 3),
            "gathering_in_conv_256x256x256_us": [round(gnf["conv_plain_us"], 3), round(gnf["conv_gather_us"], 3)],
        },
        "roofline_attention": {
            "kernel": "attention_f16 single pass (k_flash + k_flash_merge), 16384 tokens x 512",
            "bound": "mfma",
            "achieved": round(att_tf, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tf / MFMA_F16_PEAK_TFLOPS, 4),
            "avg_us": round(att["avg_ms"] * 1000, 3),
            "median_us": round(att["median_ms"] * 1000, 3),
            "algorithmic_flop": att["flops"],
        },
        "decodes": decodes,
        "config2": cfg2,
        "config3_padded": cfg3p,
        "cpu_baseline": cpu,
        "cpu_conv": cpu_c,
        "context": "pages: 0.49-0.61 s per 1024^2 decode on an RTX PRO 4000 Blackwell "
                   "(Qwen-Image-2.1 VAE, real weights; other model and machine)",
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
