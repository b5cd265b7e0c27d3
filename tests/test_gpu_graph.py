"""GPU: the layer captured in a HIP graph (torch.cuda.CUDAGraph over the
caller's stream) and replayed.  The forward calls allocate nothing and
enqueue no memset, so a captured layer must give the eager bits on every
replay -- also after the program's own eager work between replays, and
after x changes in place (nothing of the capture-time inputs is baked in).
Covered: self-routed, split, single-launch, wide, MXFP8, VALU GEMV, and a
shared expert."""
import numpy as np
import pytest

from tests.gpu_common import get_layer, get_shared, say
from workloads import Config, get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


def _small(T, E, act="bf16", seed=None):
    return Config("graph", f"graph_t{T}_e{E}_h256_i128_k2_{act}", T, E, 256, 128, 2, "normal", act,
                  seed if seed is not None else 60 + T)


CASES = {  # name: (config, path, act, launch, shared)
    "self": ("c1", 2, 0, 0, False),
    "split": ("c1", 2, 0, 1, False),
    "fused": ("c1", 2, 0, 2, False),
    "wide": (("t", 40, 4), 2, 0, 0, False),
    "mx8": (("t", 33, 8, "mxfp8"), 0, 1, 0, False),
    "gemv": ("c1", 1, 0, 0, False),
    "self_shared": ("c1", 2, 0, 0, True),
    "split_shared": (("t", 70, 64), 2, 0, 0, True),
}


def _cfg(spec):
    if isinstance(spec, str):
        return get_config(spec)
    return _small(spec[1], spec[2], spec[3] if len(spec) > 3 else "bf16")


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_give_the_eager_bits(M, name):
    import torch
    spec, path, act, launch, shared = CASES[name]
    cfg = _cfg(spec)
    layer = get_layer(cfg)
    sh = get_shared(cfg).tiles if shared else None
    layout = M.MOE_LAYOUT_TILES if (path == M.MOE_PATH_MFMA or act) else M.MOE_LAYOUT_ROWS
    wgu, wdn, scales = layer.weights(layout)
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    x0 = layer.x.clone()
    x1 = (layer.x.float() * -0.5).to(torch.bfloat16)  # other inputs, same shape

    def fwd():
        M.moe_mxfp4_forward_ex(layer.x, layer.logits, cfg.k, wgu, wdn, scales, layer.out,
                               gemm_path=path, weight_layout=layout, act_format=act, launch=launch,
                               shared=sh)

    def eager(x):
        layer.x.copy_(x)
        layer.out.fill_(float("nan"))
        fwd()
        torch.cuda.synchronize()
        return layer.out.clone()

    try:
        say(f"graph {name}: eager references")
        ref0, ref1 = eager(x0), eager(x1)
        assert not torch.equal(ref0.view(torch.int16), ref1.view(torch.int16))
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fwd()  # warm the capture stream
        torch.cuda.synchronize()
        say(f"graph {name}: capture")
        with torch.cuda.graph(g, stream=s):
            fwd()
        torch.cuda.synchronize()
        for rep, (x, ref) in enumerate(((x0, ref0), (x1, ref1), (x0, ref0), (x1, ref1))):
            layer.x.copy_(x)
            layer.out.fill_(float("nan"))
            torch.cuda.synchronize()
            say(f"graph {name}: replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)), (name, rep)
            # the program's own eager work between replays (another call of the layer)
            eager(x1 if rep % 2 == 0 else x0)
    finally:  # the layer is shared with other tests: restore its x
        layer.x.copy_(x0)
        torch.cuda.synchronize()
