"""GPU: the layer at the limits the ABI accepts -- 1024 experts, top-32
(kMaxTopK), the largest self-routed layer with top-32, and top-32 on the
VALU, matrix-core and MXFP8 paths -- bit-exact routing and the output of
every token within the bar against the oracle."""
import numpy as np
import pytest

from tests.gpu_common import (bf16_tensor_to_f64, get_layer, oracle_experts, parity_ratio, run,
                              say)
from workloads import Config, make_logits, make_x_bf16

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


CASES = {  # name: (T, E, k, act, path, launch)
    "e1024_k32_split": (40, 1024, 32, "bf16", 2, 1),      # grid route, 1024 experts, top-32
    "e1024_k32_gemv": (24, 1024, 32, "bf16", 1, 0),
    "e256_k32_self": (16, 256, 32, "bf16", 2, 3),         # T*E = 4096: the largest self-routed layer
    "e64_k32_wide": (200, 64, 32, "bf16", 2, 0),          # 100 tokens per expert: wide items
    "e1024_k32_mx8": (150, 1024, 32, "mxfp8", 0, 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_at_the_limits(M, oracle_lib, name):
    T, E, k, act_s, path, launch = CASES[name]
    cfg = Config("limits", f"limits_{name}_t{T}_e{E}_h128_i128_k{k}", T, E, 128, 128, k, "normal",
                 act_s, 500 + T + E)
    act = M.MOE_ACT_MXFP8 if act_s == "mxfp8" else M.MOE_ACT_BF16
    layer = get_layer(cfg)
    dbg = run(M, layer, path=path, act=act, launch=launch, debug=True)
    lg = make_logits(cfg)
    r = oracle_lib.route(lg, k)
    np.testing.assert_array_equal(dbg["ids"], r["ids"])
    np.testing.assert_array_equal(dbg["counts"], r["counts"])
    if launch != M.MOE_LAUNCH_SELF_ROUTED:
        np.testing.assert_array_equal(dbg["sorted"], r["sorted"])
    ex = oracle_experts(oracle_lib, cfg, r["ids"].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg, k, cfg.H, cfg.I, ex, act_mxfp8=bool(act))
    got = bf16_tensor_to_f64(layer.out)
    assert np.isfinite(got).all()
    ratio = parity_ratio(got, ref)
    say(f"limits {name}: max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL
