"""Device-resident decoder weights and the descriptor decoder_forward reads.

Uploading is plumbing: host arrays are copied to the GPU as they are
(OIHW f16 weights, f32 biases and gammas); the (tap, channel) weight plane
is produced on the GPU by ``ig_pack_conv_weights``; biases and gammas are
placed into zero-filled buffers of the padded width (channels padded to
multiples of 64, page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs",
`cpad` and `gamma`). The caller owns every buffer; this object keeps them
alive as long as the descriptor is used (the pages' per-model weight cache,
`VSTATE`, becomes plain ownership).
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def cpad(c: int) -> int:
    """Channels padded to the next multiple of 64."""
    return (int(c) + 63) // 64 * 64


class DeviceDecoder:
    def __init__(self, weights: dict, device="cuda", stream=None):
        self.device = torch.device(device)
        self.stream = stream
        self._keep = []
        w = weights
        spec = w["spec"]
        d = L.DecoderDesc()
        d.zc = int(spec["zc"])
        d.conv_in = self._conv(w["conv_in"])
        for i in range(2):
            d.mid[i] = self._resnet(w["mid"][i])
        a = w["attn"]
        d.attn.gamma = self._vec(a["gamma"], cpad(len(a["gamma"])))
        d.attn.q = self._conv(a["q"])
        d.attn.k = self._conv(a["k"])
        d.attn.v = self._conv(a["v"])
        d.attn.proj = self._conv(a["proj"])
        # the norm: RMS_norm, or GroupNorm with a beta at every site
        nk = w.get("norm") or {"kind": "rms"}
        self.group_norm = nk["kind"] == "group"
        if self.group_norm:
            d.norm_kind = L.IG_NORM_GROUP
            d.norm_groups = int(nk["groups"])
            d.norm_eps = float(nk["eps"])
            d.attn.beta = self._vec(a["beta"], cpad(len(a["beta"])))
        elif nk["kind"] != "rms":
            raise ValueError("norm kind %r" % nk["kind"])
        if len(w["ups"]) > L.IG_MAX_UP:
            raise ValueError("too many up stages")
        d.n_up = len(w["ups"])
        for s, st in enumerate(w["ups"]):
            if len(st["res"]) > L.IG_MAX_RES:
                raise ValueError("too many resnets in a stage")
            d.ups[s].n_res = len(st["res"])
            for r, rw in enumerate(st["res"]):
                d.ups[s].res[r] = self._resnet(rw)
            if st.get("up") is not None:
                d.ups[s].has_up = 1
                d.ups[s].up = self._conv(st["up"])
                if st.get("dupup") is not None:
                    d.ups[s].dupup = 1
                    d.ups[s].dupup_ft = int(st["dupup"].get("ft", 1))
        d.norm_out_gamma = self._vec(w["norm_out"], cpad(len(w["norm_out"])))
        d.norm_out_c = len(w["norm_out"])
        if self.group_norm:
            d.norm_out_beta = self._vec(w["norm_out_beta"], cpad(len(w["norm_out_beta"])))
        d.conv_out = self._conv(w["conv_out"])
        self.desc = d
        self.out_c = int(np.asarray(w["conv_out"]["b"]).shape[0])
        self.n_up = sum(1 for st in w["ups"] if st.get("up") is not None)
        torch.cuda.synchronize(self.device)

    # -- uploads -----------------------------------------------------------
    def _dev(self, arr, dtype):
        t = torch.from_numpy(np.ascontiguousarray(arr)).to(device=self.device, dtype=dtype)
        self._keep.append(t)
        return t

    def _vec(self, v, n):
        v = np.asarray(v, np.float32)
        t = torch.zeros(n, dtype=torch.float32, device=self.device)
        t[: v.shape[0]] = torch.from_numpy(v).to(self.device)
        self._keep.append(t)
        return t.data_ptr()

    def _conv(self, c):
        wt = np.asarray(c["w"])
        assert wt.dtype == np.float16
        cout, cin, k, _ = wt.shape
        cout_p, cin_p = cpad(cout), cpad(cin)
        src = self._dev(wt, torch.float16)
        plane = torch.empty(L.plane_shape(cout_p, cin_p, k), dtype=torch.float16, device=self.device)
        self._keep.append(plane)
        L.pack_conv_weights(src, cout, cin, k, cout_p, cin_p, plane, self.stream)
        cw = L.ConvW()
        cw.w = plane.data_ptr()
        cw.b = self._vec(c["b"], cout_p) if c.get("b") is not None else None
        cw.cin, cw.cout, cw.cin_p, cw.cout_p, cw.k = cin, cout, cin_p, cout_p, k
        return cw

    def _resnet(self, r):
        rw = L.ResnetW()
        rw.g1 = self._vec(r["g1"], cpad(len(r["g1"])))
        rw.c1 = self._conv(r["c1"])
        rw.g2 = self._vec(r["g2"], cpad(len(r["g2"])))
        rw.c2 = self._conv(r["c2"])
        if r.get("sc") is not None:
            rw.has_sc = 1
            rw.sc = self._conv(r["sc"])
        if r.get("beta1") is not None:
            rw.beta1 = self._vec(r["beta1"], cpad(len(r["beta1"])))
            rw.beta2 = self._vec(r["beta2"], cpad(len(r["beta2"])))
        return rw

    # -- running -------------------------------------------------------------
    def workspace_bytes(self, h0, w0, q_chunk=0):
        return L.decoder_workspace_bytes(self.desc, h0, w0, q_chunk)

    def alloc_workspace(self, h0, w0, q_chunk=0):
        n = self.workspace_bytes(h0, w0, q_chunk)
        return torch.empty(n, dtype=torch.uint8, device=self.device), n

    def forward(self, latent, h0, w0, guard_log2=8, q_chunk=0, ws=None, out=None, stream=None):
        """latent: device f32 [zc, h0, w0] (NCHW); returns device f32
        [out_c, H, W]."""
        if ws is None:
            ws, nbytes = self.alloc_workspace(h0, w0, q_chunk)
        else:
            ws, nbytes = ws
        H, W = h0 << self.n_up, w0 << self.n_up
        if out is None:
            out = torch.empty((self.out_c, H, W), dtype=torch.float32, device=self.device)
        L.decoder_forward(self.desc, latent, h0, w0, guard_log2, q_chunk, ws, nbytes, out,
                          stream if stream is not None else self.stream)
        return out

    def forward_bands(self, latent, h0, w0, band_rows, band_from, guard_log2=8, q_chunk=0, out=None,
                      stream=None):
        """The banded decode: up blocks band_from.. in bands of band_rows
        kept output rows (the same output as forward)."""
        n = L.decoder_bands_workspace_bytes(self.desc, h0, w0, q_chunk, band_rows, band_from)
        ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        H, W = h0 << self.n_up, w0 << self.n_up
        if out is None:
            out = torch.empty((self.out_c, H, W), dtype=torch.float32, device=self.device)
        L.decoder_forward_bands(self.desc, latent, h0, w0, guard_log2, q_chunk, band_rows, band_from, ws, n, out,
                                stream if stream is not None else self.stream)
        return out
