"""Pins for the oracle's MXFP8 shared expert (one SiLU-gated FFN of the
routed experts' shape, every token, weight 1, added to the routed sum):
an MXFP8 copy of an MXFP4 expert gives the pinned MXFP4 result exactly,
a closed form with E4M3 values that E2M1 cannot hold, exact scale
identities, the gate/up order, and the independent brute-force
restatement on tiny layers (bf16 and MXFP8 activations)."""
import numpy as np
import pytest

from workloads import (bf16_bits_to_f32, get_config, make_logits, make_shared_weight_fp32,
                       make_weight_fp32, make_x_bf16)


def _x_bf16(T, H, seed, scale=1.0):
    import torch
    x = (np.random.default_rng(seed).standard_normal((T, H)) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _sig(v):
    return 1.0 / (1.0 + np.exp(-v))


def _zero_expert(H, I):
    """An MXFP4 expert whose every element is +0 (code 0, scale 2^0)."""
    return (np.zeros((2 * I, H // 2), np.uint8), np.full((2 * I, H // 32), 127, np.uint8),
            np.zeros((H, I // 2), np.uint8), np.full((H, I // 32), 127, np.uint8))


def _rand_shared(oracle_lib, H, I, seed):
    rng = np.random.default_rng(seed)
    gu = rng.standard_normal((2 * I, H)) * 0.02
    dn = rng.standard_normal((H, I)) * 0.02
    return (*oracle_lib.quantize_mxfp8(gu), *oracle_lib.quantize_mxfp8(dn))


def _e2m1_to_e4m3_codes(oracle_lib):
    """E2M1 code -> the E4M3 code of the same value, found by search over the
    E4M3 table (every E2M1 value is an E4M3 value)."""
    e4 = {oracle_lib.e4m3_value(c): c for c in range(256) if c not in (0x7F, 0xFF, 0x80)}
    table = np.zeros(16, np.uint8)
    for c in range(16):
        v = oracle_lib.e2m1_value(c)
        table[c] = 0x80 if (c == 8) else e4[v]
    return table


def _unpack(packed):
    return np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], -1)


def test_mxfp8_copy_of_an_mxfp4_expert_gives_the_same_output(oracle_lib):
    """Layer A: one routed MXFP4 expert (k = 1, weight 1), no shared expert.
    Layer B: the routed expert all zeros, the shared expert its MXFP8 copy
    (same values, same scales).  Same products in the same order: the
    outputs are equal to the last bit."""
    T, H, I = 6, 128, 64
    x = _x_bf16(T, H, 20)
    logits = np.zeros((T, 1), np.float32)
    rng = np.random.default_rng(21)
    gp, gs = oracle_lib.quantize_mxfp4((rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32))
    dp, ds = oracle_lib.quantize_mxfp4((rng.standard_normal((H, I)) * 0.02).astype(np.float32))
    a = oracle_lib.forward(x, logits, 1, H, I, {0: (gp, gs, dp, ds)})
    tab = _e2m1_to_e4m3_codes(oracle_lib)
    shared = (tab[_unpack(gp)], gs, tab[_unpack(dp)], ds)
    for c in range(16):
        assert oracle_lib.e4m3_value(int(tab[c])) == oracle_lib.e2m1_value(c)
    b = oracle_lib.forward(x, logits, 1, H, I, {0: _zero_expert(H, I)}, shared=shared)
    assert np.abs(a).max() > 0
    np.testing.assert_array_equal(a, b)


def test_closed_form_with_e4m3_only_values(oracle_lib):
    """gate = 1.125 * I, up = 0.875 * I (three mantissa bits: not E2M1
    values), down = 2^-3 * 1.25 * I on the first I columns; the routed
    expert is zero.  out_n = 1.25/8 * silu(1.125 x_n) * 0.875 x_n for n < I,
    0 beyond.  A swapped gate/up reading gives silu(0.875 x) * 1.125 x."""
    T, H, I = 5, 256, 128
    x = _x_bf16(T, H, 22, scale=2.0)
    n = np.arange(I)
    gu = np.zeros((2 * I, H))
    gu[n, n] = 1.125
    gu[I + n, n] = 0.875
    dn = np.zeros((H, I))
    dn[n, n] = 1.25 / 8
    gc, gs = oracle_lib.quantize_mxfp8(gu)
    dc, ds = oracle_lib.quantize_mxfp8(dn)
    assert oracle_lib.e4m3_value(int(gc[0, 0])) * 2.0 ** (int(gs[0, 0]) - 127) == 1.125
    out = oracle_lib.forward(x, np.zeros((T, 1), np.float32), 1, H, I, {0: _zero_expert(H, I)},
                             shared=(gc, gs, dc, ds))
    xf = bf16_bits_to_f32(x).astype(np.float64)[:, :I]
    g, u = 1.125 * xf, 0.875 * xf
    want = 1.25 / 8 * g * _sig(g) * u
    np.testing.assert_allclose(out[:, :I], want, rtol=1e-14, atol=1e-300)
    assert not out[:, I:].any()
    swapped = 1.25 / 8 * (0.875 * xf) * _sig(0.875 * xf) * (1.125 * xf)
    assert np.abs(out[:, :I] - swapped).max() > 1e-3


def test_shared_term_is_added_to_the_routed_sum(oracle_lib):
    """out(routed + shared) = out(routed) + out(shared alone) for every
    token (fp64; the two terms are summed once more)."""
    T, E, H, I, k = 8, 4, 64, 64, 2
    x = _x_bf16(T, H, 23)
    logits = np.random.default_rng(24).standard_normal((T, E)).astype(np.float32)
    rng = np.random.default_rng(25)
    ex = {e: (*oracle_lib.quantize_mxfp4((rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)),
              *oracle_lib.quantize_mxfp4((rng.standard_normal((H, I)) * 0.02).astype(np.float32)))
          for e in range(E)}
    sh = _rand_shared(oracle_lib, H, I, 26)
    both = oracle_lib.forward(x, logits, k, H, I, ex, shared=sh)
    routed = oracle_lib.forward(x, logits, k, H, I, ex)
    alone = oracle_lib.forward(x, logits, k, H, I, {e: _zero_expert(H, I) for e in range(E)},
                               shared=sh)
    scale = np.abs(both).max()
    assert np.abs(both - (routed + alone)).max() <= 1e-15 * scale
    assert np.abs(alone).max() > 0.1 * np.abs(routed).max()


def test_shared_down_scale_bump_doubles_its_term(oracle_lib):
    T, H, I = 7, 64, 96
    x = _x_bf16(T, H, 27)
    zero = {0: _zero_expert(H, I)}
    lg = np.zeros((T, 1), np.float32)
    gc, gs, dc, ds = _rand_shared(oracle_lib, H, I, 28)
    base = oracle_lib.forward(x, lg, 1, H, I, zero, shared=(gc, gs, dc, ds))
    out = oracle_lib.forward(x, lg, 1, H, I, zero, shared=(gc, gs, dc, (ds + 1).astype(np.uint8)))
    np.testing.assert_array_equal(out, 2 * base)
    # one block of one gate row: only that row's h changes (all columns of y may)
    gs2 = gs.copy()
    gs2[5, 1] += 1
    one = oracle_lib.forward(x, lg, 1, H, I, zero, shared=(gc, gs2, dc, ds))
    assert not np.array_equal(one, base)


def test_shared_nan_scale_poisons_every_token(oracle_lib):
    """The shared expert is applied to every token: a NaN scale in it
    reaches all outputs."""
    T, H, I = 4, 64, 64
    x = _x_bf16(T, H, 29)
    gc, gs, dc, ds = _rand_shared(oracle_lib, H, I, 30)
    ds = ds.copy()
    ds[:, 0] = 255
    out = oracle_lib.forward(x, np.zeros((T, 1), np.float32), 1, H, I, {0: _zero_expert(H, I)},
                             shared=(gc, gs, dc, ds))
    assert np.isnan(out).all()


@pytest.mark.parametrize("act_mxfp8", [False, True])
def test_tiny_layer_with_shared_expert_matches_brute_force(oracle_lib, act_mxfp8):
    from oracle import brute
    cfg = get_config("c1")
    x = make_x_bf16(cfg)
    logits = make_logits(cfg)
    ex = {e: (*oracle_lib.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e)),
              *oracle_lib.quantize_mxfp4(make_weight_fp32(cfg, "down", e)))
          for e in range(cfg.E)}
    sh = (*oracle_lib.quantize_mxfp8(make_shared_weight_fp32(cfg, "gate_up").astype(np.float64)),
          *oracle_lib.quantize_mxfp8(make_shared_weight_fp32(cfg, "down").astype(np.float64)))
    out = oracle_lib.forward(x, logits, cfg.k, cfg.H, cfg.I, ex, act_mxfp8=act_mxfp8, shared=sh)
    ref = brute.forward(x, logits, cfg.k, cfg.H, cfg.I, ex, act_mxfp8=act_mxfp8, shared=sh)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.abs(out - ref).max() <= 1e-12 * scale
    plain = oracle_lib.forward(x, logits, cfg.k, cfg.H, cfg.I, ex, act_mxfp8=act_mxfp8)
    assert np.abs(out - plain).max() > 0.1 * scale  # the shared term is really there


def test_partial_shared_expert_is_rejected(oracle_lib):
    T, H, I = 2, 32, 32
    x = _x_bf16(T, H, 31)
    gc, gs, dc, ds = _rand_shared(oracle_lib, H, I, 32)
    import ctypes
    L = oracle_lib.lib()
    arrays = (ctypes.c_void_p * 1)()
    out = np.zeros((T, H))
    toks = np.arange(T, dtype=np.int32)
    lg = np.zeros((T, 1), np.float32)
    rc = L.oracle_forward_ex(x.ctypes.data, lg.ctypes.data, T, 1, H, I, 1,
                             ctypes.addressof(arrays), ctypes.addressof(arrays),
                             ctypes.addressof(arrays), ctypes.addressof(arrays),
                             gc.ctypes.data, None, dc.ctypes.data, ds.ctypes.data, 0,
                             toks.ctypes.data, T, out.ctypes.data)
    assert rc == -2
