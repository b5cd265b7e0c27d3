"""CPU: the oracle's router linear layer (logits = x . W_router^T in fp64),
pinned against a brute-force exactly-rounded loop, torch's bfloat16 decode,
a unit-vector closed form and exact sign / power-of-two identities."""
import math

import numpy as np
import pytest

import oracle
from workloads import Config, make_router_weight_bf16, make_x_bf16


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _cfg(T=3, E=5, H=128, seed=7):
    return Config("r", f"router_t{T}_e{E}_h{H}", T, E, H, 128, 1, "normal", "bf16", seed)


def test_bf16_decode_matches_torch_for_every_pattern():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_router_logits_brute_force_loop():
    """Every logit against math.fsum of the exact products (an exactly
    rounded sum): the fp64 matmul may only differ by its own rounding."""
    cfg = _cfg()
    x, w = make_x_bf16(cfg), make_router_weight_bf16(cfg)
    got = oracle.router_logits(x, w)
    xv = oracle.bf16_bits_to_f64(x)
    wv = oracle.bf16_bits_to_f64(w)
    for t in range(cfg.T):
        for e in range(cfg.E):
            prods = [float(xv[t, h]) * float(wv[e, h]) for h in range(cfg.H)]
            exact = math.fsum(prods)
            scale = math.fsum(abs(p) for p in prods)
            assert abs(got[t, e] - exact) <= cfg.H * 2.0 ** -52 * scale


def test_router_logits_unit_vectors_select_columns():
    """W[e] = unit vector at column p(e) (1.0 is exact in bf16): logit[t, e]
    = x[t, p(e)] exactly; a transposed operand or wrong axis fails this."""
    cfg = _cfg(T=4, E=6, H=128)
    x = make_x_bf16(cfg)
    perm = np.random.default_rng(3).permutation(cfg.H)[:cfg.E]
    w = np.zeros((cfg.E, cfg.H), np.float32)
    w[np.arange(cfg.E), perm] = 1.0
    got = oracle.router_logits(x, _bf16_bits(w))
    np.testing.assert_array_equal(got, oracle.bf16_bits_to_f64(x)[:, perm])


def test_router_logits_sign_and_power_of_two_identities():
    cfg = _cfg(T=5, E=7, H=256)
    x, w = make_x_bf16(cfg), make_router_weight_bf16(cfg)
    base = oracle.router_logits(x, w)
    neg_x = (x ^ np.uint16(0x8000)).astype(np.uint16)  # flip the sign bit
    np.testing.assert_array_equal(oracle.router_logits(neg_x, w), -base)
    w2 = _bf16_bits(oracle.bf16_bits_to_f64(w).astype(np.float32) * 2.0)  # exact in bf16
    np.testing.assert_array_equal(oracle.router_logits(x, w2), 2.0 * base)


def test_router_weight_recipe_gives_unit_scale_logits():
    """The recipe W ~ N(0, 1/sqrt(H)) makes logits about N(0, 1), like the
    workloads' logits (checked on a larger draw)."""
    cfg = _cfg(T=64, E=64, H=2048, seed=11)
    lg = oracle.router_logits(make_x_bf16(cfg), make_router_weight_bf16(cfg))
    assert abs(lg.mean()) < 0.1 and 0.85 < lg.std() < 1.15


@pytest.mark.parametrize("H", [128, 512])
def test_router_abs_bound_dominates(H):
    cfg = _cfg(T=3, E=4, H=H)
    x, w = make_x_bf16(cfg), make_router_weight_bf16(cfg)
    assert np.all(oracle.router_logits_abs(x, w) >= np.abs(oracle.router_logits(x, w)))
