"""Shared helpers of the GPU parity tests (oracle side built on the CPU)."""
from __future__ import annotations

import sys

import numpy as np

from workloads import Config, make_shared_weight_fp32, make_weight_fp32


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


_layers = {}


def get_layer(cfg: Config, logits=None):
    """Device layer of a workload, built once per process.  Layers whose
    weights come from the same draws (same seed and shapes) share them."""
    from mxfp4_moe_expert_02_amd.layer import build_layer
    key = (cfg, None if logits is None else logits.tobytes())
    if key not in _layers:
        donor = next((l for (c, _), l in _layers.items()
                      if (c.seed, c.E, c.H, c.I) == (cfg.seed, cfg.E, cfg.H, cfg.I)), None)
        say(f"building layer {cfg.name} seed {cfg.seed}"
            + (f" (weights of {donor.cfg.name})" if donor is not None else ""))
        _layers[key] = build_layer(cfg, logits=logits, weights_from=donor)
    return _layers[key]


_shared = {}


def get_shared(cfg: Config):
    """Device MXFP8 shared expert of a workload (built once per process)."""
    from mxfp4_moe_expert_02_amd.layer import build_shared
    key = (cfg.seed, cfg.H, cfg.I)
    if key not in _shared:
        say(f"building shared expert of {cfg.name}")
        _shared[key] = build_shared(cfg)
    return _shared[key]


def oracle_shared(oracle, cfg: Config):
    """Oracle-encoded MXFP8 shared expert from the same float32 draws."""
    gc, gs = oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "gate_up").astype(np.float64))
    dc, ds = oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "down").astype(np.float64))
    return (gc, gs, dc, ds)


def run(M, layer, path=0, debug=False, act=0, launch=0, init=True, router=None, shared=None):
    """One forward through the C ABI on every token of the layer; returns
    the requested debug outputs (routing; with MXFP8 also the codes of x)
    as numpy arrays.  out is NaN-filled first, so every element it holds
    afterwards was written by this call.  launch: MOE_LAUNCH_* (the fused
    launch also returns its wait-error flag as "wait_error"); init=False
    keeps the current workspace (and whatever an earlier call left in it).
    router: a [E, H] bf16 device router weight -- the layer then computes its
    own logits (returned as "logits") and is given no router_logits.
    shared: the four tile tensors of an MXFP8 shared expert, or None."""
    import torch
    c = layer.cfg
    if init:
        M.moe_mxfp4_init(c.T, c.E, c.H, c.I, c.k)
    dbg = {}
    if debug:
        S = c.T * c.k
        dbg = dict(ids=torch.empty((c.T, c.k), dtype=torch.int32, device="cuda"),
                   weights=torch.empty((c.T, c.k), dtype=torch.float32, device="cuda"),
                   counts=torch.empty(c.E, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(c.E + 1, dtype=torch.int32, device="cuda"),
                   sorted=torch.empty(S, dtype=torch.int32, device="cuda"))
        if act == M.MOE_ACT_MXFP8:
            dbg["x_codes"] = torch.empty((c.T, c.H), dtype=torch.uint8, device="cuda")
            dbg["x_scales"] = torch.empty((c.T, c.H // 32), dtype=torch.uint8, device="cuda")
            dbg["h_codes"] = torch.empty((S, c.I), dtype=torch.uint8, device="cuda")
            dbg["h_scales"] = torch.empty((S, c.I // 32), dtype=torch.uint8, device="cuda")
    if launch == M.MOE_LAUNCH_FUSED:
        dbg["wait_error"] = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    extra = {}
    if router is not None:
        dbg["logits_out"] = torch.full((c.T, c.E), float("nan"), dtype=torch.float32, device="cuda")
        extra["router_weight"] = router
    layer.out.fill_(float("nan"))
    torch.cuda.synchronize()
    say(f"forward {c.name} T={c.T} E={c.E} H={c.H} I={c.I} k={c.k} path={path} act={act} "
        f"launch={launch} shared={shared is not None}")
    mfma = path == M.MOE_PATH_MFMA or act == M.MOE_ACT_MXFP8
    layout = M.MOE_LAYOUT_TILES if mfma else M.MOE_LAYOUT_ROWS
    wgu, wdn, scales = layer.weights(layout)
    M.moe_mxfp4_forward_ex(layer.x, None if router is not None else layer.logits, c.k, wgu, wdn,
                           scales, layer.out, gemm_path=path, weight_layout=layout,
                           act_format=act, launch=launch, shared=shared, **dbg, **extra)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dbg.items()}


def oracle_experts(oracle, cfg: Config, experts) -> dict:
    """Oracle-encoded weights of the given experts, from the same float32
    draws the device layer was built from."""
    out = {}
    for e in sorted(set(int(v) for v in experts)):
        gp, gs = oracle.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e))
        dp, ds = oracle.quantize_mxfp4(make_weight_fp32(cfg, "down", e))
        out[e] = (gp, gs, dp, ds)
    return out


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def parity_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / rms(ref): the acceptance quantity (bar: <= 2e-2)."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.abs(gpu - ref).max() / rms)


def check_mxfp8_h(oracle, cfg: Config, x_bf16, experts, route, dbg, rel: float = 1e-4):
    """The encoding decision of h on the MXFP8 path, taken from fp32 values on
    the GPU and fp64 ones in the oracle, may differ where a value sits on a
    decision boundary.  Checks that every difference is such a case -- a block
    scale that differs only where the block's largest |h| is within `rel` of a
    power of two, an element code that differs only where the GPU's code is a
    nearest one up to rel * (block max) -- and returns the oracle's output
    finished from the GPU's own h codes (fp64, [T, H])."""
    from oracle import brute
    rows = brute.hidden_mxfp8_rows(x_bf16, cfg.k, cfg.I, experts, route["ids"], route["sorted"])
    codes, scales = oracle.quantize_mxfp8(rows)
    hq, hs = dbg["h_codes"], dbg["h_scales"]
    S, I = rows.shape
    blocks = np.abs(rows).reshape(S, I // 32, 32).max(axis=2)
    bad_scale = hs != scales
    for p, b in zip(*np.nonzero(bad_scale)):
        a = blocks[p, b]
        assert abs(int(hs[p, b]) - int(scales[p, b])) == 1, (p, b)
        assert a > 0 and abs(a / 2.0 ** np.round(np.log2(a)) - 1.0) <= rel, (p, b, a)
    gpu_v = brute.mxfp8_dequant(hq, hs)
    ora_v = brute.mxfp8_dequant(codes, scales)
    same_scale = np.repeat(~bad_scale, 32, axis=1)
    diff = (hq != codes) & same_scale
    slack = 2 * rel * np.repeat(blocks, 32, axis=1)
    d_gpu = np.abs(rows - gpu_v)
    d_ora = np.abs(rows - ora_v)
    assert np.all(d_gpu[diff] <= d_ora[diff] + slack[diff])
    say(f"h codes: {int(diff.sum())} of {diff.size} differ at a boundary, "
        f"{int(bad_scale.sum())} block scales")
    return brute.down_from_h(hq, hs, cfg.k, experts, route["ids"], route["w"], route["pos"])
