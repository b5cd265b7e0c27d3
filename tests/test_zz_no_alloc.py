"""GPU: the allocation-free entry point (moe_mxfp4_forward_noalloc) gives the
bits of the workspace entry point (moe_mxfp4_forward_ex, self-routed, the
same kernels in the same order) on consecutive calls that share its fixed
device array: the 9-token verify layer (slot-list pre-pass), then a smaller
input of 4 of its tokens, then a small layer that ranks its experts in the
GEMM workgroups; and it rejects a layer past its limits."""
import numpy as np
import pytest

from tests.gpu_common import bf16_tensor_to_f64, get_layer, oracle_experts, parity_ratio, say
from workloads import get_config, make_logits, make_x_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


def _both(M, layer, T):
    """out of the workspace entry point and of the allocation-free one on the
    first T tokens of the layer"""
    import torch
    c = layer.cfg
    x, lg = layer.x[:T].contiguous(), layer.logits[:T].contiguous()
    wgu, wdn, scales = layer.weights(M.MOE_LAYOUT_TILES)
    ref = torch.full((T, c.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = torch.full((T, c.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_mxfp4_init(c.T, c.E, c.H, c.I, c.k)
    say(f"workspace entry point {c.name} T={T}")
    M.moe_mxfp4_forward_ex(x, lg, c.k, wgu, wdn, scales, ref, weight_layout=M.MOE_LAYOUT_TILES,
                           launch=M.MOE_LAUNCH_SELF_ROUTED)
    torch.cuda.synchronize()
    say(f"allocation-free entry point {c.name} T={T}")
    M.moe_mxfp4_forward_noalloc(x, lg, c.k, wgu, wdn, scales, got, c.E, c.H, c.I)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_point(M, oracle_lib):
    import torch
    for key, T in (("c2", 9), ("c2", 4), ("c1", 9)):
        cfg = get_config(key)
        layer = get_layer(cfg)
        ref, got = _both(M, layer, T)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), (key, T)
        if key == "c2" and T == 4:  # and within the bar of the oracle
            lg = make_logits(cfg)[:T]
            ids = oracle_lib.route(lg, cfg.k)["ids"]
            ex = oracle_experts(oracle_lib, cfg, ids.ravel())
            o = oracle_lib.forward(make_x_bf16(cfg)[:T], lg, cfg.k, cfg.H, cfg.I, ex)
            ratio = parity_ratio(bf16_tensor_to_f64(got), o)
            say(f"noalloc {cfg.name} T={T}: max|d|/rms = {ratio:.3e}")
            assert ratio <= 2e-2


def test_noalloc_rejects_past_its_limits(M):
    import torch
    cfg = get_config("c1")
    layer = get_layer(cfg)
    wgu, wdn, scales = layer.weights(M.MOE_LAYOUT_TILES)
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    rc = M.moe_mxfp4_forward_noalloc(layer.x, layer.logits, 9, wgu, wdn, scales, out, cfg.E, cfg.H,
                                     cfg.I, check=False)  # top_k 9 > 8
    assert rc in (M.MOE_E_LIMIT, M.MOE_E_TOPK)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()  # nothing was enqueued
