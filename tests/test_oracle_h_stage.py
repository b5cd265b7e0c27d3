"""CPU: the MXFP8 path split at h (oracle/brute.py), pinned to the whole layer.

hidden_mxfp8_rows gives h per expert-sorted row before its encoding, and
down_from_h finishes the layer from given MXFP8 codes of h.  Fed the MXFP8
encoding of its own rows, the pair must reproduce the C oracle's whole MXFP8
layer (an independent implementation) to rounding; a wrong row order, slot
mapping or weight makes it fail.  A one-step change of one h code must move
exactly the one token whose slot uses that row.
"""
import numpy as np

import oracle
from oracle import brute
from workloads import Config, make_logits, make_weight_fp32, make_x_bf16


def _layer(seed=321, T=11, E=6, k=3, H=128, I=128):
    cfg = Config("hstage", f"hstage_t{T}_e{E}", T, E, H, I, k, "normal", "mxfp8", seed)
    lg = make_logits(cfg)
    r = oracle.route(lg, k)
    ex = {}
    for e in sorted(set(int(v) for v in r["ids"].ravel())):
        gp, gs = oracle.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e))
        dp, ds = oracle.quantize_mxfp4(make_weight_fp32(cfg, "down", e))
        ex[e] = (gp, gs, dp, ds)
    return cfg, lg, r, ex


def test_h_stage_reproduces_the_whole_layer(oracle_lib):
    cfg, lg, r, ex = _layer()
    x = make_x_bf16(cfg)
    rows = brute.hidden_mxfp8_rows(x, cfg.k, cfg.I, ex, r["ids"], r["sorted"])
    codes, scales = oracle.quantize_mxfp8(rows)
    out = brute.down_from_h(codes, scales, cfg.k, ex, r["ids"], r["w"], r["pos"])
    ref = oracle.forward(x, lg, cfg.k, cfg.H, cfg.I, ex, act_mxfp8=True)
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


def test_one_h_code_moves_only_its_token(oracle_lib):
    cfg, lg, r, ex = _layer(seed=322)
    x = make_x_bf16(cfg)
    rows = brute.hidden_mxfp8_rows(x, cfg.k, cfg.I, ex, r["ids"], r["sorted"])
    codes, scales = oracle.quantize_mxfp8(rows)
    base = brute.down_from_h(codes, scales, cfg.k, ex, r["ids"], r["w"], r["pos"])
    p = 7
    c2 = codes.copy()
    i = int(np.argmax(np.abs(rows[p])))
    c2[p, i] ^= 1  # the neighbouring E4M3 code
    moved = brute.down_from_h(c2, scales, cfg.k, ex, r["ids"], r["w"], r["pos"])
    t = int(r["sorted"][p]) // cfg.k
    changed = np.flatnonzero(np.abs(moved - base).max(axis=1) > 0)
    assert changed.tolist() == [t]
