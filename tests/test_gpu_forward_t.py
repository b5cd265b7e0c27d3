"""GPU: the descriptor entry point (moe_mxfp4_forward_t) runs the layer
forward_ex runs, bit for bit, on both weight layouts, and rejects a layer
whose sizes differ from the workspace's before enqueueing anything."""
import pytest

from tests.gpu_common import get_layer, run
from workloads import get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


@pytest.mark.parametrize("key", ["c1", "c2"])
@pytest.mark.parametrize("layout", ["rows", "tiles"])
def test_forward_t_matches_forward_ex(M, key, layout):
    import torch
    cfg = get_config(key)
    layer = get_layer(cfg)
    lay = M.MOE_LAYOUT_TILES if layout == "tiles" else M.MOE_LAYOUT_ROWS
    run(M, layer, path=0, layout=lay)  # forward_ex, AUTO path, the same layout
    ref = layer.out.clone()
    wgu, wdn, scales = layer.weights(lay)
    layer.out.fill_(float("nan"))
    M.moe_mxfp4_forward_t(layer.x, layer.logits, cfg.k, wgu, wdn, scales, layer.out, weight_layout=lay)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), layer.out.view(torch.int16))


def test_forward_t_rejects_sizes_other_than_the_workspace(M):
    import torch
    cfg = get_config("c1")
    layer = get_layer(cfg)
    M.moe_mxfp4_init(cfg.T, cfg.E + 1, cfg.H, cfg.I, cfg.k)  # one more expert than the layer has
    layer.out.fill_(float("nan"))
    rc = M.moe_mxfp4_forward_t(layer.x, layer.logits, cfg.k, layer.wgu, layer.wdn, layer.scales,
                               layer.out, check=False)
    torch.cuda.synchronize()
    assert rc == M.MOE_E_SHAPE
    assert torch.isnan(layer.out.float()).all()
    x16 = layer.x.view(torch.int16)  # a wrong element type
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    rc = M.moe_mxfp4_forward_t(x16, layer.logits, cfg.k, layer.wgu, layer.wdn, layer.scales,
                               layer.out, check=False)
    assert rc == M.MOE_E_DTYPE
