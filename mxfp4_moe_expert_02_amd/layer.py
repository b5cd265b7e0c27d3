"""A device-resident MoE expert layer built from a seeded synthetic workload.

Weights are drawn as float32 by ``workloads`` (host, thread pool), copied to
the GPU one expert at a time and encoded to MXFP4 there by the library's own
``moe_mxfp4_quantize``.  The result holds exactly the tensors the C ABI
takes, laid out as include/moe_mxfp4.h describes.  ``build_shared`` does
the same for the optional MXFP8 shared expert (``moe_mxfp8_quantize``,
``moe_mxfp8_prepack``).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from workloads import (Config, iter_weights_fp32, make_logits, make_shared_weight_fp32,
                       make_x_bf16)

from . import _lib


@dataclasses.dataclass
class DeviceLayer:
    cfg: Config
    x: "torch.Tensor"        # [T, H] bfloat16
    logits: "torch.Tensor"   # [T, E] float32
    wgu: "torch.Tensor"      # [E, 2I, H/2] uint8
    sgu: "torch.Tensor"      # [E, 2I, H/32] uint8
    wdn: "torch.Tensor"      # [E, H, I/2] uint8
    sdn: "torch.Tensor"      # [E, H, I/32] uint8
    out: "torch.Tensor"      # [T, H] bfloat16
    # the same weights in the MFMA tile layout (moe_mxfp4_prepack), or None
    wgu_t: "torch.Tensor" = None
    sgu_t: "torch.Tensor" = None
    wdn_t: "torch.Tensor" = None
    sdn_t: "torch.Tensor" = None

    @property
    def scales(self):
        return (self.sgu, self.sdn)

    @property
    def tile_scales(self):
        return (self.sgu_t, self.sdn_t)

    def weights(self, layout: int):
        """(W_gate_up, W_down, scales) in the given layout."""
        if layout == _lib.MOE_LAYOUT_TILES:
            return self.wgu_t, self.wdn_t, self.tile_scales
        return self.wgu, self.wdn, self.scales

    def expert_bytes(self) -> int:
        """Packed + scale bytes of one expert (both matrices)."""
        c = self.cfg
        return 2 * c.I * c.H // 2 + 2 * c.I * c.H // 32 + c.H * c.I // 2 + c.H * c.I // 32


def build_layer(cfg: Config, device: str = "cuda", workers: int | None = None,
                x_bf16: np.ndarray | None = None, logits: np.ndarray | None = None,
                tiles: bool = True, weights_from: DeviceLayer | None = None) -> DeviceLayer:
    """``weights_from``: a layer built from the same weight draws (same seed
    and E, H, I) whose device weights are shared instead of rebuilt."""
    import torch
    dev = torch.device(device)
    T, E, H, I = cfg.T, cfg.E, cfg.H, cfg.I
    xb = make_x_bf16(cfg) if x_bf16 is None else x_bf16
    lg = make_logits(cfg) if logits is None else logits
    x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    lt = torch.from_numpy(np.ascontiguousarray(lg, np.float32)).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if weights_from is not None:
        d = weights_from.cfg
        if (d.seed, d.E, d.H, d.I) != (cfg.seed, E, H, I):
            raise ValueError(f"{d.name} and {cfg.name} do not share weight draws")
        src = weights_from
        return DeviceLayer(cfg, x, lt, src.wgu, src.sgu, src.wdn, src.sdn, out,
                           src.wgu_t, src.sgu_t, src.wdn_t, src.sdn_t)
    wgu = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    sgu = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    wdn = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    sdn = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    for which, wp, sp in (("gate_up", wgu, sgu), ("down", wdn, sdn)):
        staging = None
        for e, w in iter_weights_fp32(cfg, which, workers=workers):
            if staging is None:
                staging = torch.empty(w.shape, dtype=torch.float32, device=dev)
            staging.copy_(torch.from_numpy(w))
            _lib.moe_mxfp4_quantize(staging, wp[e], sp[e])
        del staging
    layer = DeviceLayer(cfg, x, lt, wgu, sgu, wdn, sdn, out)
    if tiles:
        layer.wgu_t, layer.sgu_t = torch.empty_like(wgu), torch.empty_like(sgu)
        layer.wdn_t, layer.sdn_t = torch.empty_like(wdn), torch.empty_like(sdn)
        _lib.moe_mxfp4_prepack(wgu, sgu, layer.wgu_t, layer.sgu_t, gate_up_pairs=True)
        _lib.moe_mxfp4_prepack(wdn, sdn, layer.wdn_t, layer.sdn_t, gate_up_pairs=False)
    torch.cuda.synchronize(dev)
    return layer


@dataclasses.dataclass
class SharedExpert:
    """The MXFP8 shared expert: row-major codes and scales, and the tile
    layout the layer reads."""
    gu: "torch.Tensor"       # [2I, H] uint8 E4M3 codes
    gus: "torch.Tensor"      # [2I, H/32] uint8 E8M0
    dn: "torch.Tensor"       # [H, I]
    dns: "torch.Tensor"      # [H, I/32]
    gu_t: "torch.Tensor"
    gus_t: "torch.Tensor"
    dn_t: "torch.Tensor"
    dns_t: "torch.Tensor"

    @property
    def tiles(self):
        """The four tensors of the ``shared`` argument of forward_ex."""
        return (self.gu_t, self.gus_t, self.dn_t, self.dns_t)

    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.gu, self.gus, self.dn, self.dns))


def build_shared(cfg: Config, device: str = "cuda", fp32: dict | None = None) -> SharedExpert:
    """The shared expert of ``cfg`` encoded on the device.  ``fp32``: optional
    {"gate_up": [2I, H], "down": [H, I]} float32 matrices to encode instead
    of the seeded draws."""
    import torch
    dev = torch.device(device)
    mats = []
    for which in ("gate_up", "down"):
        w = make_shared_weight_fp32(cfg, which) if fp32 is None else fp32[which]
        rows, cols = w.shape
        wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(dev)
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        _lib.moe_mxfp8_quantize(wd, codes, scales)
        tiles, tscales = torch.empty_like(codes), torch.empty_like(scales)
        _lib.moe_mxfp8_prepack(codes.view(1, rows, cols), scales.view(1, rows, cols // 32),
                               tiles, tscales, gate_up_pairs=which == "gate_up")
        mats.append((codes, scales, tiles, tscales))
    (gu, gus, gu_t, gus_t), (dn, dns, dn_t, dns_t) = mats
    torch.cuda.synchronize(dev)
    return SharedExpert(gu, gus, dn, dns, gu_t, gus_t, dn_t, dns_t)
