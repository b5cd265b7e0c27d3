"""Shared helpers of the GPU parity tests (oracle side built on the CPU)."""
from __future__ import annotations

import sys

import numpy as np

from workloads import Config, make_weight_fp32


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


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
