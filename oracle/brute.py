"""Independent brute-force restatement of the layer -- TEST INFRASTRUCTURE ONLY.

A second, separately written fp64 implementation used to cross-check
``oracle.c`` on tiny shapes.  It deliberately takes other routes to the same
definitions:

* E2M1 decode is a literal value table; E4M3 decode uses torch's
  ``float8_e4m3fn`` dtype (a library implementation of the OCP FN format).
* Encoding rounds v / X to a multiple of the element quantum of its binade
  with ``numpy.rint`` (round half to even), where ``oracle.c`` searches the
  code table for the nearest value.
* Routing is a Python ``sorted`` per token; the FFN is a dense fp64 matmul
  over fully decoded weights, one token and one slot at a time.

Only meant for small inputs (pure-Python loops over tokens and slots).
"""
from __future__ import annotations

import math
from typing import Mapping, Sequence

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    return np.where(codes == 255, np.nan, np.ldexp(1.0, codes - 127))


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] codes, even k in the low nibble."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=1)


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = e2m1_decode(unpack_nibbles(packed))
    return vals * np.repeat(e8m0_decode(scales), 32, axis=1)


def _round_to_format(q: np.ndarray, mbits: int, emin: int, maxval: float) -> np.ndarray:
    """Round |q| to a binary format with ``mbits`` mantissa bits whose smallest
    normal exponent is ``emin`` (subnormals below), ties to even, saturating."""
    a = np.abs(q)
    _, ex = np.frexp(a)              # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, emin)     # binade exponent (floored at emin)
    quantum = np.ldexp(1.0, e - mbits)
    r = np.rint(a / quantum) * quantum
    r = np.minimum(r, maxval)
    return np.copysign(r, q)


def _mx_encode_values(v: np.ndarray, emax: int, mbits: int, emin: int,
                      maxval: float) -> tuple[np.ndarray, np.ndarray]:
    """Block-32 MX rule on rows of v; returns (dequantised values, scale codes)."""
    rows, cols = v.shape
    blocks = v.reshape(rows, cols // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    se = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    se[nz] = ex - 1 - emax
    se = np.clip(se, -127, 127)
    q = np.ldexp(blocks, -se[..., None])
    r = _round_to_format(q, mbits, emin, maxval)
    deq = np.ldexp(r, se[..., None]).reshape(rows, cols)
    return deq, (se + 127).astype(np.uint8)


def mxfp4_encode_values(w: np.ndarray):
    return _mx_encode_values(np.asarray(w, np.float64), emax=2, mbits=1, emin=0, maxval=6.0)


def mxfp8_encode_values(v: np.ndarray):
    return _mx_encode_values(np.asarray(v, np.float64), emax=8, mbits=3, emin=-6, maxval=448.0)


def route(logits: np.ndarray, k: int):
    T, E = logits.shape
    ids = np.zeros((T, k), np.int64)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        ids[t] = order
        ls = np.array([float(logits[t, e]) for e in order])
        p = np.exp(ls - ls.max())
        w[t] = p / p.sum()
    return ids, w


def _ffn(wgu: np.ndarray, wdn: np.ndarray, xt: np.ndarray, I: int, act_mxfp8: bool) -> np.ndarray:
    g = wgu[:I] @ xt
    u = wgu[I:] @ xt
    h = np.array([gi / (1.0 + math.exp(-gi)) for gi in g]) * u
    if act_mxfp8:
        h = mxfp8_encode_values(h[None, :])[0][0]
    return wdn @ h


def forward(x_bf16: np.ndarray, logits: np.ndarray, k: int, H: int, I: int,
            experts: Mapping[int, Sequence[np.ndarray]], act_mxfp8: bool = False,
            shared: Sequence[np.ndarray] | None = None) -> np.ndarray:
    xf = (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    T = xf.shape[0]
    ids, w = route(logits, k)
    dense = {}
    for e, (gp, gs, dp, ds) in experts.items():
        dense[e] = (mxfp4_dequant(gp, gs), mxfp4_dequant(dp, ds))
    sh = None
    if shared is not None:
        sgc, sgs, sdc, sds = shared
        sh = (mxfp8_dequant(sgc, sgs), mxfp8_dequant(sdc, sds))
    out = np.zeros((T, H))
    for t in range(T):
        xt = xf[t:t + 1]
        if act_mxfp8:
            xt, _ = mxfp8_encode_values(xt)
        for j in range(k):
            wgu, wdn = dense[int(ids[t, j])]
            out[t] += w[t, j] * _ffn(wgu, wdn, xt[0], I, act_mxfp8)
        if sh is not None:
            out[t] += _ffn(sh[0], sh[1], xt[0], I, act_mxfp8)
    return out


def _silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    return np.array([gi / (1.0 + math.exp(-gi)) for gi in g]) * u


def hidden_mxfp8_rows(x_bf16: np.ndarray, k: int, I: int,
                      experts: Mapping[int, Sequence[np.ndarray]], ids: np.ndarray,
                      sorted_slots: np.ndarray) -> np.ndarray:
    """h of the MXFP8 path before its own MXFP8 encoding, in fp64, one row per
    position p of the expert-sorted order: slot s = sorted_slots[p] = t*k + j
    gives SiLU(Wg x_t) * (Wu x_t) of expert ids[t, j], x_t being the MXFP8
    encoding of token t.  The encoding decision of h is then taken from these
    values (by a caller)."""
    xf = (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gate_up = {}
    rows = np.zeros((len(sorted_slots), I))
    for p, s in enumerate(sorted_slots):
        t, j = divmod(int(s), k)
        e = int(ids[t, j])
        if e not in gate_up:
            gp, gs = experts[e][0], experts[e][1]
            gate_up[e] = mxfp4_dequant(gp, gs)
        xt = mxfp8_encode_values(xf[t:t + 1])[0][0]
        w = gate_up[e]
        rows[p] = _silu_mul(w[:I] @ xt, w[I:] @ xt)
    return rows


def down_from_h(h_codes: np.ndarray, h_scales: np.ndarray, k: int,
                experts: Mapping[int, Sequence[np.ndarray]], ids: np.ndarray, w: np.ndarray,
                pos: np.ndarray, tokens: Sequence[int] | None = None) -> np.ndarray:
    """The rest of the layer on a given MXFP8 h (rows in expert-sorted order,
    pos[t*k + j] = the row of slot t*k + j): out[t] = sum_j w[t, j] *
    Wdown[ids[t, j]] @ dequant(h row pos[t*k + j]), in fp64, slots in order,
    for the given tokens (default all; rows of the result in that order).
    Each expert's down matrix is decoded once, its slots taken together."""
    tokens = list(range(ids.shape[0])) if tokens is None else [int(t) for t in tokens]
    by_expert = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append((i, t, j))
    terms = {}
    for e, slots in by_expert.items():
        down = mxfp4_dequant(experts[e][2], experts[e][3])
        for i, t, j in slots:
            p = int(pos[t * k + j])
            hrow = mxfp8_dequant(h_codes[p:p + 1], h_scales[p:p + 1])[0]
            terms[(i, j)] = w[t, j] * (down @ hrow)
        del down
    out = np.zeros((len(tokens), next(iter(terms.values())).shape[0]))
    for i in range(len(tokens)):
        for j in range(k):
            out[i] += terms[(i, j)]
    return out
