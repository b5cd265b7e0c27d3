"""Pins for the oracle's expert FFN and combine: closed forms, exact scale
identities, and agreement with the independent brute-force restatement."""
import numpy as np
import pytest

from workloads import bf16_bits_to_f32, get_config, make_logits, make_weight_fp32, make_x_bf16


def _x_bf16(T, H, seed, scale=1.0):
    import torch
    x = (np.random.default_rng(seed).standard_normal((T, H)) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _identity_experts(oracle_lib, H, I, up_scale=1.0, down_scale=1.0):
    gu = np.zeros((2 * I, H), np.float32)
    gu[np.arange(I), np.arange(I)] = 1.0
    gu[I + np.arange(I), np.arange(I)] = up_scale
    dn = np.zeros((H, I), np.float32)
    dn[np.arange(I), np.arange(I)] = down_scale
    return (*oracle_lib.quantize_mxfp4(gu), *oracle_lib.quantize_mxfp4(dn))


def _sig(v):
    return 1.0 / (1.0 + np.exp(-v))


def test_closed_form_identity_expert(oracle_lib):
    """E = 1, k = 1, gate = up = identity on the first I columns, down =
    identity rows: out_n = x_n^2 * sigmoid(x_n) for n < I, 0 beyond."""
    T, H, I = 9, 256, 128
    x = _x_bf16(T, H, 0)
    logits = np.zeros((T, 1), np.float32)
    ex = _identity_experts(oracle_lib, H, I)
    assert (ex[1][np.arange(I), np.arange(I) // 32] == 127 - 2).all()  # 1.0 -> code 4 at 2^-2
    out = oracle_lib.forward(x, logits, 1, H, I, {0: ex})
    xf = bf16_bits_to_f32(x).astype(np.float64)
    want = np.zeros((T, H))
    want[:, :I] = xf[:, :I] ** 2 * _sig(xf[:, :I])
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-300)


def test_closed_form_pins_gate_up_order(oracle_lib):
    """gate = I, up = 2I gives 2 x^2 sigmoid(x); the swapped reading would give
    2 x^2 sigmoid(2x), which differs."""
    T, H, I = 5, 256, 128
    x = _x_bf16(T, H, 1, scale=2.0)
    logits = np.zeros((T, 1), np.float32)
    out = oracle_lib.forward(x, logits, 1, H, I, {0: _identity_experts(oracle_lib, H, I, 2.0)})
    xf = bf16_bits_to_f32(x).astype(np.float64)[:, :I]
    right = 2 * xf ** 2 * _sig(xf)
    swapped = 2 * xf ** 2 * _sig(2 * xf)
    np.testing.assert_allclose(out[:, :I], right, rtol=1e-14)
    assert np.abs(out[:, :I] - swapped).max() > 1e-3


def _rand_experts(oracle_lib, E, H, I, seed):
    rng = np.random.default_rng(seed)
    ex = {}
    for e in range(E):
        gu = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
        dn = (rng.standard_normal((H, I)) * 0.02).astype(np.float32)
        ex[e] = (*oracle_lib.quantize_mxfp4(gu), *oracle_lib.quantize_mxfp4(dn))
    return ex


def test_down_scale_bump_doubles_expert_contribution(oracle_lib):
    """+1 on every E8M0 code of one expert's down matrix doubles exactly that
    expert's term of the weighted sum (k = 1, so per token)."""
    T, E, H, I = 12, 2, 64, 64
    x = _x_bf16(T, H, 2)
    logits = np.random.default_rng(3).standard_normal((T, E)).astype(np.float32)
    ex = _rand_experts(oracle_lib, E, H, I, 4)
    base = oracle_lib.forward(x, logits, 1, H, I, ex)
    gp, gs, dp, ds = ex[0]
    bumped = dict(ex)
    bumped[0] = (gp, gs, dp, (ds + 1).astype(np.uint8))
    out = oracle_lib.forward(x, logits, 1, H, I, bumped)
    to0 = np.argmax(logits, 1) == 0
    assert to0.any() and (~to0).any()
    assert np.array_equal(out[to0], 2 * base[to0])
    assert np.array_equal(out[~to0], base[~to0])


def test_single_block_scale_is_local(oracle_lib):
    """+1 on one down-matrix block (e, n, kb) changes output column n of the
    tokens routed to e and nothing else."""
    T, E, H, I, k = 10, 3, 64, 96, 2
    x = _x_bf16(T, H, 5)
    logits = np.random.default_rng(6).standard_normal((T, E)).astype(np.float32)
    ex = _rand_experts(oracle_lib, E, H, I, 7)
    base = oracle_lib.forward(x, logits, k, H, I, ex)
    gp, gs, dp, ds = ex[1]
    ds2 = ds.copy()
    ds2[17, 2] += 1
    mod = dict(ex)
    mod[1] = (gp, gs, dp, ds2)
    out = oracle_lib.forward(x, logits, k, H, I, mod)
    routed = (oracle_lib.route(logits, k)["ids"] == 1).any(1)
    diff = out != base
    assert diff[:, 17][routed].all()
    diff[:, 17] = False
    assert not diff.any()


def test_unrouted_expert_weights_are_not_read(oracle_lib):
    """NaN scales (E8M0 0xFF) on every expert no token picks leave the output
    unchanged; a routed expert with NaN scales makes it NaN."""
    T, E, H, I, k = 6, 6, 64, 64, 2
    x = _x_bf16(T, H, 8)
    logits = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32)
    logits[:, 4:] -= 100.0   # experts 4 and 5 are never chosen
    ex = _rand_experts(oracle_lib, E, H, I, 10)
    base = oracle_lib.forward(x, logits, k, H, I, ex)
    pois = dict(ex)
    for e in (4, 5):
        gp, gs, dp, ds = ex[e]
        pois[e] = (gp, np.full_like(gs, 255), dp, np.full_like(ds, 255))
    assert np.array_equal(oracle_lib.forward(x, logits, k, H, I, pois), base)
    gp, gs, dp, ds = ex[0]
    pois[0] = (gp, np.full_like(gs, 255), dp, ds)
    out = oracle_lib.forward(x, logits, k, H, I, pois)
    to0 = (oracle_lib.route(logits, k)["ids"] == 0).any(1)
    assert np.isnan(out[to0]).all() and not np.isnan(out[~to0]).any()


def test_missing_routed_expert_raises(oracle_lib):
    T, E, H, I = 3, 2, 32, 32
    x = _x_bf16(T, H, 11)
    logits = np.zeros((T, E), np.float32)
    with pytest.raises(KeyError):
        oracle_lib.forward(x, logits, 1, H, I, {})


def test_tiny_workload_matches_brute_force(oracle_lib):
    from oracle import brute
    cfg = get_config("c1")
    x = make_x_bf16(cfg)
    logits = make_logits(cfg)
    ex = {e: (*oracle_lib.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e)),
              *oracle_lib.quantize_mxfp4(make_weight_fp32(cfg, "down", e)))
          for e in range(cfg.E)}
    out = oracle_lib.forward(x, logits, cfg.k, cfg.H, cfg.I, ex)
    ref = brute.forward(x, logits, cfg.k, cfg.H, cfg.I, ex)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.abs(out - ref).max() <= 1e-12 * scale
    # a token subset gives the same rows
    sub = oracle_lib.forward(x, logits, cfg.k, cfg.H, cfg.I, ex, tokens=[4, 0])
    assert np.array_equal(sub, out[[4, 0]])


def test_tiny_mxfp8_activations_match_brute_force(oracle_lib):
    from oracle import brute
    T, E, H, I, k = 7, 4, 128, 64, 2
    x = _x_bf16(T, H, 12)
    logits = np.random.default_rng(13).standard_normal((T, E)).astype(np.float32)
    ex = _rand_experts(oracle_lib, E, H, I, 14)
    out = oracle_lib.forward(x, logits, k, H, I, ex, act_mxfp8=True)
    ref = brute.forward(x, logits, k, H, I, ex, act_mxfp8=True)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.abs(out - ref).max() <= 1e-12 * scale
    plain = oracle_lib.forward(x, logits, k, H, I, ex)
    assert np.abs(plain - out).max() > 1e-6 * scale  # the MXFP8 step is really applied
