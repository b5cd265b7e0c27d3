"""GPU: the expert GEMMs as one launch of one workgroup per unit
(MOE_LAUNCH_QUEUE; AUTO's choice for wide layers without a shared expert).

The queue kernels run the split launch's gate_up and down units with the
same accumulation order, so their output must equal the split launch's bit
for bit, on narrow (16-token items) and wide (64-token items) layers alike;
a second call with another routing on the same workspace must read the h
rows it wrote itself; the bounded waits must never give up (wait_error
stays 0); AUTO must give the same bits on wide layers.  Parity against the
CPU oracle on every touched expert and item of the full-size layers runs in
test_gpu_parity.py (through AUTO, which takes this launch there).
"""
import numpy as np
import pytest

from tests.gpu_common import bf16_tensor_to_f64, get_layer, oracle_experts, parity_ratio, run, say
from tests.test_gpu_fused import _layer
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


def _queue_layer(key):
    """The fused tests' workloads, plus a narrow layer (T*k < 4E: 16-token
    items) whose one hot expert has three items."""
    if key == "narrowhot":
        cfg = Config("narrowhot", "narrowhot_t40_e16_h256_i128_k1", 40, 16, 256, 128, 1, "normal",
                     "bf16", 31)
        logits = make_logits(cfg)
        logits[:, 2] += 100.0
        return cfg, get_layer(cfg, logits=logits)
    return _layer(key)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "hot", "wide", "narrowhot", "edge1_1",
                                 "edge1_8", "edge2_5"])
def test_queue_matches_split_bit_exact(M, key):
    import torch
    cfg, layer = _queue_layer(key)
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_SPLIT)
    split = layer.out.clone()
    dbg = run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_QUEUE)
    assert int(dbg["wait_error"][0]) == 0
    assert torch.equal(split.view(torch.int16), layer.out.view(torch.int16)), cfg.name


@pytest.mark.parametrize("key", ["c3", "c4", "wide", "hot"])
def test_auto_takes_queue_on_wide_layers(M, key):
    """AUTO on a wide layer gives the queue launch's bits (and the split
    launch's)."""
    import torch
    cfg, layer = _queue_layer(key)
    assert cfg.T * cfg.k >= 4 * cfg.E
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_QUEUE)
    queue = layer.out.clone()
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_AUTO, init=False)
    assert torch.equal(queue.view(torch.int16), layer.out.view(torch.int16)), cfg.name


@pytest.mark.parametrize("key", ["c2", "c3"])
def test_queue_new_routing_on_same_workspace(M, oracle_lib, key):
    """Two calls on one workspace with different routings: the second call's
    items (and h rows) differ from the first's; its output must match the
    oracle for its own routing and the split launch bit for bit."""
    import torch
    cfg = get_config(key)
    base = get_layer(cfg)
    lg2 = make_logits(cfg)[::-1].copy()  # the same logit rows, tokens reversed
    lg2 = np.roll(lg2, 5, axis=1)       # and experts rotated: another routing
    other = get_layer(cfg, logits=lg2)
    run(M, base, path=MFMA, launch=M.MOE_LAUNCH_QUEUE)
    dbg = run(M, other, path=MFMA, launch=M.MOE_LAUNCH_QUEUE, init=False)
    assert int(dbg["wait_error"][0]) == 0
    queue = other.out.clone()
    run(M, other, path=MFMA, launch=M.MOE_LAUNCH_SPLIT, init=False)
    assert torch.equal(queue.view(torch.int16), other.out.view(torch.int16))
    tokens = [0, cfg.T // 2, cfg.T - 1]
    ids = oracle_lib.route(lg2, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg2, cfg.k, cfg.H, cfg.I, ex, tokens=tokens)
    ratio = parity_ratio(bf16_tensor_to_f64(queue)[tokens], ref)
    say(f"queue parity {cfg.name} (second routing) tokens={tokens} max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


def test_queue_deterministic(M):
    import torch
    cfg, layer = _queue_layer("c4")
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_QUEUE)
    a = layer.out.clone()
    run(M, layer, path=MFMA, launch=M.MOE_LAUNCH_QUEUE, init=False)
    assert torch.equal(a.view(torch.int16), layer.out.view(torch.int16))
