"""GPU: the expert layer in one persistent launch (MOE_LAUNCH_FUSED).

The fused kernel runs the same gate_up and down units as the split launch,
with the same accumulation order, so its output must equal the split
launch's bit for bit; it is also checked against the CPU oracle on sampled
tokens, with a routing that changes between two calls on one workspace
(the down units must read the h rows this call wrote, never older ones), and
its bounded waits must never give up (wait_error stays 0).
"""
import numpy as np
import pytest

from tests.gpu_common import (bf16_tensor_to_f64, get_layer, oracle_experts, parity_ratio, run,
                              say)
from workloads import Config, get_config, make_logits, make_x_bf16

pytestmark = pytest.mark.gpu

TOL = 2e-2
MFMA = 2


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


def _hot_cfg():
    return Config("hot", "hot_t37_e8_h384_i256_k3", 37, 8, 384, 256, 3, "normal", "bf16", 11)


def _wide_cfg():
    return Config("wide", "wide_t100_e4_h256_i256_k2", 100, 4, 256, 256, 2, "normal", "bf16", 17)


def _layer(key):
    """Workloads by name: the configs, a one-hot expert, wide ragged items."""
    if key == "hot":
        cfg = _hot_cfg()
        logits = make_logits(cfg)
        logits[:, 3] += 100.0
        return cfg, get_layer(cfg, logits=logits)
    if key == "wide":
        cfg = _wide_cfg()
        logits = make_logits(cfg)
        logits[:, 1] += 100.0
        return cfg, get_layer(cfg, logits=logits)
    if key.startswith("edge"):
        T, k = (int(v) for v in key[4:].split("_"))
        cfg = Config("edge", f"edge_t{T}_e8_h256_i128_k{k}", T, 8, 256, 128, k, "normal", "bf16",
                     21 + T)
        return cfg, get_layer(cfg)
    cfg = get_config(key)
    return cfg, get_layer(cfg)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "hot", "wide", "edge1_1", "edge1_8",
                                 "edge2_5"])
def test_fused_matches_split_bit_exact(M, key):
    import torch
    cfg, layer = _layer(key)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SPLIT)
    split = layer.out.clone()
    dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED)
    assert int(dbg["wait_error"][0]) == 0
    assert torch.equal(split.view(torch.int16), layer.out.view(torch.int16)), cfg.name


@pytest.mark.parametrize("key,tokens", [("c2", list(range(9))), ("c4", [0, 143, 287])])
def test_fused_parity(M, oracle_lib, key, tokens):
    cfg, layer = _layer(key)
    dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED)
    assert int(dbg["wait_error"][0]) == 0
    lg = make_logits(cfg)
    ids = oracle_lib.route(lg, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg, cfg.k, cfg.H, cfg.I, ex, tokens=tokens)
    full = bf16_tensor_to_f64(layer.out)
    assert np.isfinite(full).all()
    ratio = parity_ratio(full[tokens], ref)
    say(f"fused parity {cfg.name} tokens={tokens} max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_fused_new_routing_on_same_workspace(M, oracle_lib, key):
    """Two calls on one workspace with different routings: the second call's
    items (and h rows) differ from the first's; its output must match the
    oracle for its own routing and the split launch bit for bit."""
    import torch
    cfg = get_config(key)
    base = get_layer(cfg)
    lg2 = make_logits(cfg)[::-1].copy()  # the same logit rows, tokens reversed
    lg2 = np.roll(lg2, 5, axis=1)       # and experts rotated: another routing
    other = get_layer(cfg, logits=lg2)
    run(M, base, path=MFMA, launch=M.MOE_LAUNCH_FUSED)
    dbg = run(M, other, path=MFMA, launch=M.MOE_LAUNCH_FUSED, init=False)
    assert int(dbg["wait_error"][0]) == 0
    fused = other.out.clone()
    run(M, other, path=MFMA, launch=M.MOE_LAUNCH_SPLIT, init=False)
    assert torch.equal(fused.view(torch.int16), other.out.view(torch.int16))
    tokens = [0, cfg.T // 2, cfg.T - 1]
    ids = oracle_lib.route(lg2, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg2, cfg.k, cfg.H, cfg.I, ex, tokens=tokens)
    ratio = parity_ratio(bf16_tensor_to_f64(fused)[tokens], ref)
    say(f"fused parity {cfg.name} (second routing) tokens={tokens} max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


def test_fused_deterministic(M):
    import torch
    cfg, layer = _layer("c4")
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED)
    a = layer.out.clone()
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED, init=False)
    assert torch.equal(a.view(torch.int16), layer.out.view(torch.int16))
