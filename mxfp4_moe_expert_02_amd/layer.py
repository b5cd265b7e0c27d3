"""A device-resident MoE expert layer built from a seeded synthetic workload.

Weights are drawn as float32 by ``workloads`` (host, thread pool), copied to
the GPU one expert at a time and encoded to MXFP4 there by the library's own
``moe_mxfp4_quantize``.  The result holds exactly the tensors the C ABI
takes, laid out as include/moe_mxfp4.h describes.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from workloads import Config, iter_weights_fp32, make_logits, make_x_bf16

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
