"""CPU oracle for the MXFP4 MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library: ``oracle.c`` is compiled by gcc on its own and loaded with ctypes,
and ``brute.py`` is an independent numpy re-statement used to cross-check it.

Parity status per function (what pins it is in ``tests/test_oracle_*.py``):
  e2m1/e4m3/e8m0 decode ....... pinned (code tables, torch float8_e4m3fn)
  quantize_mxfp4/mxfp8 ........ pinned (round trip, midpoints, saturation,
                                  brute-force nearest search, torch RNE)
  route ....................... pinned (brute-force sort, softmax identity)
  forward ..................... pinned (closed forms, scale identities,
                                  brute.py on tiny shapes)
  router_logits ............... pinned (brute-force loop, unit-vector
                                  closed form, exact power-of-two scaling)
  forward(shared=...) ......... pinned (brute.py on tiny shapes, an MXFP8
                                  copy of an MXFP4 expert gives the same
                                  result, closed forms, scale identities)
  brute.hidden_mxfp8_rows /
  brute.down_from_h ........... pinned (together they reproduce the C
                                  oracle's whole MXFP8 layer; one h code
                                  moves only its own token)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Mapping, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB may name another build of oracle.c (the sanitizer build of the
# CPU tests)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """oracle.c with AddressSanitizer and UBSan (a UB report fatal), at
    `out`; loaded with gcc's libasan preloaded."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", _SRC, "-o", out,
                    "-lm"], check=True)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [i32]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [i32]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [i32]
        L.oracle_quantize_mxfp4.restype = i32
        L.oracle_quantize_mxfp4.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_quantize_mxfp8.restype = i32
        L.oracle_quantize_mxfp8.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_forward.restype = i32
        L.oracle_forward.argtypes = [vp, vp, i64, i64, i64, i64, i32,
                                     vp, vp, vp, vp, i32, vp, i64, vp]
        L.oracle_forward_ex.restype = i32
        L.oracle_forward_ex.argtypes = [vp, vp, i64, i64, i64, i64, i32,
                                        vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i64, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e8m0_value(code: int) -> float:
    return lib().oracle_e8m0_value(int(code))


def quantize_mxfp4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 [rows, cols] -> (packed uint8 [rows, cols/2], scales uint8 [rows, cols/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = lib().oracle_quantize_mxfp4(_p(w), rows, cols, _p(packed), _p(scales))
    if rc:
        raise ValueError(f"oracle_quantize_mxfp4 failed ({rc})")
    return packed, scales


def quantize_mxfp8(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp64 [rows, cols] -> (E4M3 codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows, cols = v.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = lib().oracle_quantize_mxfp8(_p(v), rows, cols, _p(codes), _p(scales))
    if rc:
        raise ValueError(f"oracle_quantize_mxfp8 failed ({rc})")
    return codes, scales


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> their exact values (a bf16 is the top half of
    an IEEE binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to quiet NaNs
        return b.view(np.float32).astype(np.float64)


def router_logits(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """Router logits [T, E] in fp64: logits[t, e] = sum_h x[t, h] * W[e, h]
    over the exact bf16 values (the router linear layer upstream of top-k,
    kept at the activations' precision).  Products of two bf16 are exact in
    fp64; only the sum rounds."""
    x = bf16_bits_to_f64(x_bf16)
    w = bf16_bits_to_f64(w_bf16)
    assert x.ndim == 2 and w.ndim == 2 and x.shape[1] == w.shape[1]
    return x @ w.T


def router_logits_abs(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """sum_h |x[t, h] * W[e, h]| -- the scale of the rounding error of any
    summation order of the router products (for error bounds)."""
    return np.abs(bf16_bits_to_f64(x_bf16)) @ np.abs(bf16_bits_to_f64(w_bf16)).T


def route(logits: np.ndarray, k: int) -> dict:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    rc = lib().oracle_route(_p(logits), T, E, k, _p(ids), _p(w), _p(counts), _p(offsets),
                            _p(sorted_), _p(pos))
    if rc:
        raise ValueError(f"oracle_route failed ({rc})")
    return {"ids": ids, "w": w, "counts": counts, "offsets": offsets,
            "sorted": sorted_, "pos": pos}


def forward(x_bf16: np.ndarray, logits: np.ndarray, k: int, H: int, I: int,
            experts: Mapping[int, Sequence[np.ndarray]], tokens: Sequence[int] | None = None,
            act_mxfp8: bool = False, shared: Sequence[np.ndarray] | None = None) -> np.ndarray:
    """Layer output (fp64) for ``tokens`` (default: all).

    ``experts[e] = (gu_packed [2I,H/2], gu_scales [2I,H/32], dn_packed [H,I/2],
    dn_scales [H,I/32])`` for every expert the listed tokens are routed to.
    ``shared = (gu_codes [2I,H], gu_scales [2I,H/32], dn_codes [H,I],
    dn_scales [H,I/32])``: the MXFP8 shared expert added with weight 1.
    """
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert x_bf16.shape == (T, H)
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    ptr_t = ctypes.c_void_p * E
    keep = []
    arrays = [ptr_t(), ptr_t(), ptr_t(), ptr_t()]
    for e, mats in experts.items():
        for i, m in enumerate(mats):
            m = np.ascontiguousarray(m, dtype=np.uint8)
            keep.append(m)
            arrays[i][e] = m.ctypes.data
    sh = [None] * 4
    if shared is not None:
        shapes = [(2 * I, H), (2 * I, H // 32), (H, I), (H, I // 32)]
        for i, m in enumerate(shared):
            m = np.ascontiguousarray(m, dtype=np.uint8)
            assert m.shape == shapes[i], (m.shape, shapes[i])
            keep.append(m)
            sh[i] = m.ctypes.data
    out = np.zeros((len(toks), H), np.float64)
    rc = lib().oracle_forward_ex(_p(x_bf16), _p(logits), T, E, H, I, k,
                                 ctypes.addressof(arrays[0]), ctypes.addressof(arrays[1]),
                                 ctypes.addressof(arrays[2]), ctypes.addressof(arrays[3]),
                                 sh[0], sh[1], sh[2], sh[3],
                                 1 if act_mxfp8 else 0, _p(toks), len(toks), _p(out))
    if rc == -2:
        raise KeyError("oracle_forward: a routed expert's weights were not given")
    if rc:
        raise ValueError(f"oracle_forward failed ({rc})")
    return out
