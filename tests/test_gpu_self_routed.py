"""GPU: the self-routed layer (MOE_LAUNCH_SELF_ROUTED, no sorting pass).

The GEMM workgroups find their experts' tokens themselves: small layers
rank each expert in every GEMM workgroup, large ones (E*(I/32 + H/128) >=
2048 workgroups: c2, t16e200k5, t4e1000k3 here) in a pre-pass that writes
per-expert slot lists.  h and y are indexed by slot; the arithmetic and its
order are those of the routed split launch, and the combine weights come
from the same rank-count code, so the output must equal the routed
launch's bit for bit.  Cases span the eligible range (1..16 tokens, T*E up
to 4096, E not a multiple of 4 or 64, k = 1 .. E), a hot expert that gets a
full 16-token tile, logits with many exact ties (the index tie-break
decides), two routings in a row on one workspace (no row of the first call
may leak into the second), and the oracle on sampled tokens.
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


def _cfg(T, E, H, I, k, seed):
    return Config("self", f"self_t{T}_e{E}_h{H}_i{I}_k{k}", T, E, H, I, k, "normal", "bf16", seed)


def _layer(key):
    """Eligible layers by name (the workloads, shape edges, a hot expert, ties)."""
    if key in ("c1", "c2"):
        cfg = get_config(key)
        return cfg, get_layer(cfg)
    if key == "hot16":  # every token picks expert 3 first: one full 16-token tile
        cfg = _cfg(16, 8, 256, 128, 1, 41)
        lg = make_logits(cfg)
        lg[:, 3] += 100.0
        return cfg, get_layer(cfg, logits=lg)
    if key == "ties":  # logits in {-2, ..., 2}: most ranks decided by the index
        cfg = _cfg(9, 64, 256, 128, 8, 43)
        lg = np.round(make_logits(cfg)).astype(np.float32)
        return cfg, get_layer(cfg, logits=lg)
    shapes = {
        "t1e8k1": (1, 8, 256, 128, 1),
        "t16e32k4": (16, 32, 256, 128, 4),     # the most tokens
        "t16e256k8": (16, 256, 256, 128, 8),   # T*E at its limit (4096)
        "t4e1000k3": (4, 1000, 128, 128, 3),   # E not a multiple of 4; 16 compare passes
        "t16e200k5": (16, 200, 512, 256, 5),   # slot lists, 16 tokens, ragged E
        "t7e13k3": (7, 13, 256, 128, 3),
        "t5e4k4": (5, 4, 256, 128, 4),         # k = E: every expert takes every token
        "t7e1k1": (7, 1, 256, 128, 1),         # one expert
    }
    T, E, H, I, k = shapes[key]
    cfg = _cfg(T, E, H, I, k, 50 + T + E + k)
    return cfg, get_layer(cfg)


KEYS = ["c1", "c2", "hot16", "ties", "t1e8k1", "t16e32k4", "t16e256k8", "t4e1000k3", "t16e200k5",
        "t7e13k3", "t5e4k4", "t7e1k1"]


@pytest.mark.parametrize("key", KEYS)
def test_self_routed_matches_split_bit_exact(M, key):
    import torch
    cfg, layer = _layer(key)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SPLIT)
    split = layer.out.clone()
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    assert torch.isfinite(layer.out.float()).all()
    assert torch.equal(split.view(torch.int16), layer.out.view(torch.int16)), cfg.name


def test_auto_takes_self_routed_and_keeps_routing_outputs(M, oracle_lib):
    """AUTO on the one-sequence verify layer runs self-routed; asking for the
    routing outputs adds the routing pass, whose ids and counts are the
    oracle's, and changes no output bit."""
    import torch
    cfg, layer = _layer("c2")
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    plain = layer.out.clone()
    dbg = run(M, layer, path=MFMA, debug=True)
    assert torch.equal(plain.view(torch.int16), layer.out.view(torch.int16))
    r = oracle_lib.route(make_logits(cfg), cfg.k)
    np.testing.assert_array_equal(dbg["ids"], r["ids"])
    np.testing.assert_array_equal(dbg["counts"], r["counts"])


@pytest.mark.parametrize("key,tokens", [("c2", [0, 4, 8]), ("t16e256k8", [0, 7, 15]),
                                        ("t4e1000k3", [0, 3]), ("t16e200k5", [0, 9, 15])])
def test_self_routed_parity(M, oracle_lib, key, tokens):
    cfg, layer = _layer(key)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    lg = make_logits(cfg)
    ids = oracle_lib.route(lg, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg, cfg.k, cfg.H, cfg.I, ex, tokens=tokens)
    full = bf16_tensor_to_f64(layer.out)
    assert np.isfinite(full).all()
    ratio = parity_ratio(full[tokens], ref)
    say(f"self-routed parity {cfg.name} tokens={tokens} max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


def test_self_routed_new_routing_on_same_workspace(M, oracle_lib):
    """A second routing on the same workspace: every slot row is rewritten,
    so the output is that routing's (split launch and oracle)."""
    import torch
    cfg = get_config("c2")
    base = get_layer(cfg)
    lg2 = np.roll(make_logits(cfg)[::-1].copy(), 7, axis=1)
    other = get_layer(cfg, logits=lg2)
    run(M, base, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    run(M, other, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED, init=False)
    mine = other.out.clone()
    run(M, other, path=MFMA, launch=M.MOE_LAUNCH_SPLIT, init=False)
    assert torch.equal(mine.view(torch.int16), other.out.view(torch.int16))
    tokens = [0, 4, 8]
    ids = oracle_lib.route(lg2, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg2, cfg.k, cfg.H, cfg.I, ex, tokens=tokens)
    assert parity_ratio(bf16_tensor_to_f64(mine)[tokens], ref) <= TOL


@pytest.mark.parametrize("shape", [(17, 8, 256, 128, 2), (16, 8, 256, 128, 4)])
def test_self_routed_rejects_ineligible(M, shape):
    """17 tokens (more than one column tile), and 16 tokens averaging 8 per
    expert (wide items): MOE_E_OPTION, nothing launched."""
    T, E, H, I, k = shape
    cfg = _cfg(T, E, H, I, k, 60)
    layer = get_layer(cfg)
    with pytest.raises(M.MoeError) as ei:
        run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    assert ei.value.status == M.MOE_E_OPTION


def test_rejected_call_enqueues_nothing(M):
    """A self-routed call on an ineligible layer is rejected before anything
    reaches the stream: the stage event it was given keeps the time it was
    recorded at before the call (recording it again would move it past a
    later reference event), and the router linear layer it asked for does
    not run."""
    import time

    import torch
    cfg = _cfg(17, 8, 256, 128, 2, 60)
    layer = get_layer(cfg)
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    ev = torch.cuda.Event(enable_timing=True)
    ev.record()
    torch.cuda.synchronize()
    time.sleep(0.01)
    ref = torch.cuda.Event(enable_timing=True)
    ref.record()
    torch.cuda.synchronize()
    router = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
    wgu, wdn, scales = layer.weights(M.MOE_LAYOUT_TILES)
    rc = M.moe_mxfp4_forward_ex(layer.x, None, cfg.k, wgu, wdn, scales, layer.out,
                                weight_layout=M.MOE_LAYOUT_TILES, launch=M.MOE_LAUNCH_SELF_ROUTED,
                                events=[ev], router_weight=router, check=False)
    torch.cuda.synchronize()
    assert rc == M.MOE_E_OPTION
    assert ref.elapsed_time(ev) < 0  # ev still holds its earlier time


@pytest.mark.parametrize("key", KEYS)
def test_self_routed_single_launch_bit_exact(M, key):
    """The whole self-routed layer in one launch (MOE_LAUNCH_FUSED on an
    eligible layer: routing weights, slot lists, gate_up, down and the
    combine as units of one persistent kernel) gives the bits of the
    self-routed launches, and none of its bounded waits gives up."""
    import torch
    cfg, layer = _layer(key)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    ref = layer.out.clone()
    dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED)
    assert int(dbg["wait_error"][0]) == 0
    assert torch.equal(ref.view(torch.int16), layer.out.view(torch.int16))


@pytest.mark.parametrize("key", ["ties", "t16e256k8", "t16e200k5"])
def test_single_launch_repeats_track_inputs(M, key):
    """Back-to-back single launches with x changed in place between them each
    give the self-routed bits of their own x.  The layers have I < 1024, where
    unpadded rows of h's scales would share cache lines across experts; such
    sharing once let a down unit read another expert's scale row before its
    gate_up units had written it (one token's 128 output columns wrong, now
    and then)."""
    import dataclasses

    import torch
    cfg, shared_layer = _layer(key)
    # a private copy of the cached layer: its own x (changed in place) and out
    layer = dataclasses.replace(shared_layer, x=shared_layer.x.clone(), out=shared_layer.out.clone())
    gen = torch.Generator().manual_seed(7)
    for rep in range(4):
        x = torch.randn(layer.x.shape, generator=gen).to(torch.bfloat16)
        layer.x.copy_(x.to(layer.x.device))
        run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED, init=rep == 0)
        ref = layer.out.clone()
        dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED, init=False)
        assert int(dbg["wait_error"][0]) == 0
        assert torch.equal(ref.view(torch.int16), layer.out.view(torch.int16)), rep


def test_single_launch_after_other_paths(M):
    """The single launch resets its own counters: after a VALU call and a
    routed call on the same workspace (which leave their own counts behind)
    it still gives the self-routed bits, twice in a row."""
    import torch
    cfg = get_config("c2")
    layer = get_layer(cfg)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SELF_ROUTED)
    ref = layer.out.clone()
    run(M, layer, path=1, init=False)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SPLIT, init=False)
    for _ in range(2):
        dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_FUSED, init=False)
        assert int(dbg["wait_error"][0]) == 0
        assert torch.equal(ref.view(torch.int16), layer.out.view(torch.int16))
