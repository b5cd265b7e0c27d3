"""GPU: the router linear layer ahead of the routing (router_weight option).

The layer computes logits = x . W_router^T (bf16 products, fp32 sums) and
routes on them.  Checked: the logits against the fp64 oracle within the
rigorous bound of an fp32 summation (|d| <= H * 2^-24 * sum|x w|); the
routing bit-exact against the oracle's top-k on the same fp32 logits (the
decision taken in the same precision on both sides); the output
bit-identical to the layer given those logits directly, and within the
parity bar against the oracle; determinism (the split-K partials are
added in a fixed order).  Shapes cover the split-K kernel (few tiles) and
the single-pass one (many tiles), ragged tiles, and the self-routed,
routed, wide and MXFP8 paths.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_common import (bf16_tensor_to_f64, get_layer, oracle_experts, parity_ratio, run,
                              say)
from workloads import Config, get_config, make_router_weight_bf16, make_x_bf16

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


def _router(cfg):
    import torch
    w = make_router_weight_bf16(cfg)
    return w, torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda")


def _cfg(key):
    shapes = {  # T, E, H, I, k, act
        "ragged": (7, 13, 256, 128, 3, "bf16"),       # partial expert and token tiles
        "single": (512, 128, 256, 128, 2, "bf16"),    # 256 tiles: one pass, no split
        "mx8": (300, 16, 256, 128, 2, "mxfp8"),       # MXFP8 activations
    }
    if key in ("c1", "c2", "c3", "c4"):
        return get_config(key)
    T, E, H, I, k, act = shapes[key]
    return Config("router", f"router_{key}_t{T}_e{E}_h{H}_i{I}_k{k}", T, E, H, I, k, "normal", act,
                  70 + T + E)


KEYS = ["c1", "c2", "c3", "ragged", "single", "mx8"]


@pytest.mark.parametrize("key", KEYS)
def test_router_logits_routing_and_output(M, oracle_lib, key):
    import torch
    cfg = _cfg(key)
    layer = get_layer(cfg)
    w_np, w_dev = _router(cfg)
    act = M.MOE_ACT_MXFP8 if cfg.act == "mxfp8" else M.MOE_ACT_BF16
    path = 0 if act == M.MOE_ACT_MXFP8 else MFMA
    dbg = run(M, layer, path=path, act=act, debug=True, router=w_dev)
    lg = dbg["logits_out"]
    assert np.isfinite(lg).all()
    # 1. the logits: within the fp32 summation bound of the exact fp64 value
    x_np = make_x_bf16(cfg)
    ref = oracle.router_logits(x_np, w_np)
    bound = cfg.H * 2.0 ** -24 * oracle.router_logits_abs(x_np, w_np)
    err = np.abs(lg.astype(np.float64) - ref)
    say(f"router logits {cfg.name}: max|d| = {err.max():.3e}, max|d|/bound = {(err / bound).max():.3e}")
    assert np.all(err <= bound)
    # 2. the routing: bit-exact against the oracle on the same fp32 logits
    r = oracle_lib.route(lg, cfg.k)
    np.testing.assert_array_equal(dbg["ids"], r["ids"])
    np.testing.assert_array_equal(dbg["counts"], r["counts"])
    np.testing.assert_array_equal(dbg["offsets"], r["offsets"])
    np.testing.assert_array_equal(dbg["sorted"], r["sorted"])
    out_router = layer.out.clone()
    # 3. the same layer given those logits directly: the same bits
    given = get_layer(cfg, logits=lg)
    run(M, given, path=path, act=act, init=False)
    assert torch.equal(out_router.view(torch.int16), given.out.view(torch.int16))
    # 4. the output against the oracle on sampled tokens
    tokens = sorted({0, cfg.T // 2, cfg.T - 1})
    ex = oracle_experts(oracle_lib, cfg, r["ids"][tokens].ravel())
    want = oracle_lib.forward(x_np, lg, cfg.k, cfg.H, cfg.I, ex, tokens=tokens,
                              act_mxfp8=cfg.act == "mxfp8")
    ratio = parity_ratio(bf16_tensor_to_f64(out_router)[tokens], want)
    say(f"router parity {cfg.name} tokens={tokens} max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


@pytest.mark.parametrize("key", ["c2", "ragged"])
def test_router_deterministic(M, key):
    """Two calls (split-K partials summed by whichever split finishes last)
    give the same logits and output bits."""
    import torch
    cfg = _cfg(key)
    layer = get_layer(cfg)
    _, w_dev = _router(cfg)
    a = run(M, layer, path=MFMA, router=w_dev)["logits_out"]
    out_a = layer.out.clone()
    b = run(M, layer, path=MFMA, router=w_dev, init=False)["logits_out"]
    np.testing.assert_array_equal(a.view(np.int32), b.view(np.int32))
    assert torch.equal(out_a.view(torch.int16), layer.out.view(torch.int16))


def test_router_with_fused_launch(M, oracle_lib):
    import torch
    cfg = _cfg("c2")
    layer = get_layer(cfg)
    _, w_dev = _router(cfg)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SPLIT, router=w_dev)
    split = layer.out.clone()
    dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED, router=w_dev, init=False)
    assert int(dbg["wait_error"][0]) == 0
    assert torch.equal(split.view(torch.int16), layer.out.view(torch.int16))


def test_router_weight_validation(M):
    """A misaligned router weight is rejected before anything runs; with a
    router weight, router_logits may be NULL."""
    import torch
    cfg = _cfg("ragged")
    layer = get_layer(cfg)
    _, w_dev = _router(cfg)
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    wgu, wdn, scales = layer.weights(M.MOE_LAYOUT_TILES)
    flat = torch.empty(w_dev.numel() + 8, dtype=torch.bfloat16, device="cuda")
    bad = flat[1:1 + w_dev.numel()].view(cfg.E, cfg.H)  # 2-byte offset: misaligned
    rc = M.moe_mxfp4_forward_ex(layer.x, None, cfg.k, wgu, wdn, scales, layer.out,
                                weight_layout=M.MOE_LAYOUT_TILES, router_weight=bad, check=False)
    assert rc == M.MOE_E_ALIGN
    rc = M.moe_mxfp4_forward_ex(layer.x, None, cfg.k, wgu, wdn, scales, layer.out,
                                weight_layout=M.MOE_LAYOUT_TILES, check=False, validate=False)
    assert rc == M.MOE_E_NULL
    torch.cuda.synchronize()
