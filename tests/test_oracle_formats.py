"""Pins for the oracle's MX element/scale decoding and block encoding.

Each check compares the oracle with something other than itself: the format
tables in tests/golden (OCP MX / OFP8 specifications), torch's float8_e4m3fn
dtype, an exhaustive nearest-value search, or the independent quantum-rounding
restatement in oracle/brute.py.
"""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split()
        out.append((int(a, 0), float(b)) if not name.endswith("rounding.txt") else (float(a), float(b)))
    return out


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e2m1_all_16_codes_match_table(oracle_lib):
    table = _read_pairs("e2m1_values.txt")
    assert len(table) == 16
    for code, val in table:
        assert _same(oracle_lib.e2m1_value(code), val), code


def test_e4m3_landmarks(oracle_lib):
    for code, val in _read_pairs("e4m3_values.txt"):
        assert _same(oracle_lib.e4m3_value(code), val), hex(code)


def test_e4m3_all_256_codes_match_torch(oracle_lib):
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle_lib.e4m3_value(c), float(ref[c])), hex(c)


def test_e8m0_values(oracle_lib):
    assert oracle_lib.e8m0_value(127) == 1.0
    assert oracle_lib.e8m0_value(128) == 2.0
    assert oracle_lib.e8m0_value(126) == 0.5
    assert oracle_lib.e8m0_value(0) == 2.0 ** -127
    assert oracle_lib.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle_lib.e8m0_value(255))
    for u in range(255):  # each code is exactly twice the previous one
        if u:
            assert oracle_lib.e8m0_value(u) == 2 * oracle_lib.e8m0_value(u - 1)


def _decode4(packed, scales):
    from oracle import brute
    return brute.mxfp4_dequant(packed, scales)


def test_mxfp4_rounding_table(oracle_lib):
    """Values placed in a block whose amax fixes the scale at 2^0: a block with
    one element 4.0 has floor(log2 4) - 2 = 0, so the other elements are coded
    as themselves."""
    for v, expect in _read_pairs("e2m1_rounding.txt"):
        if abs(v) >= 8:
            continue
        w = np.zeros((1, 32), np.float32)
        w[0, 0] = 4.0
        w[0, 1] = v
        if abs(v) >= 4:  # keep the scale at 2^0: amax must stay in [4, 8)
            w[0, 0] = 0.0
        packed, scales = oracle_lib.quantize_mxfp4(w)
        assert scales[0, 0] == 127
        got = oracle_lib.e2m1_value(int(packed[0, 0] >> 4)) * 1.0
        assert _same(got, expect), (v, got, expect)


def test_mxfp4_round_trip_every_code_and_scale(oracle_lib):
    """encode(decode(c) * 2^s) == c for every code and a sweep of scales, with
    a 6.0 (code 7) in the block so that the block scale is exactly 2^s."""
    rng = np.random.default_rng(0)
    for s in [-127 + 2, -60, -7, 0, 5, 60, 125]:
        codes = rng.integers(0, 16, size=(64, 32))
        codes[:, 0] = 7
        vals = np.array([[oracle_lib.e2m1_value(int(c)) for c in row] for row in codes])
        w = (vals * 2.0 ** s).astype(np.float32)
        packed, scales = oracle_lib.quantize_mxfp4(w)
        assert (scales == s + 127).all(), s
        got = np.stack([packed & 15, packed >> 4], -1).reshape(64, 32)
        # -0 (code 8) and +0 (code 0) encode the same value; compare values and signs
        want = codes.copy()
        assert (got == want).all(), s


def test_mxfp4_scale_rule_amax_range(oracle_lib):
    """amax / X lies in [4, 8) for every non-zero block (X = 2^(floor(log2 amax) - 2))."""
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    w[3, :32] = 2.0 ** -5              # exact power of two
    w[4, :32] = np.nextafter(np.float32(2.0 ** -5), np.float32(0))  # just below one
    _, scales = oracle_lib.quantize_mxfp4(w)
    amax = np.abs(w.reshape(256, 8, 32)).max(-1).astype(np.float64)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    r = amax / X
    assert ((r >= 4) & (r < 8)).all()
    assert scales[3, 0] == 127 - 5 - 2
    assert scales[4, 0] == 127 - 6 - 2


def test_mxfp4_brute_force_nearest(oracle_lib):
    """Each element is the nearest of the 16 scaled E2M1 values (exhaustive
    search), ties to the even code, saturating."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    packed, scales = oracle_lib.quantize_mxfp4(w)
    deq = _decode4(packed, scales)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    q = np.abs(w.astype(np.float64)) / X
    dist = np.abs(q[..., None] - mags)
    best = dist.min(-1)
    # every candidate at the minimum distance; choose even index if tie
    cand = dist == best[..., None]
    idx = np.where(cand.sum(-1) > 1, np.argmax(cand & (np.arange(8) % 2 == 0), -1), np.argmax(cand, -1))
    expect = np.copysign(mags[idx], w) * X
    assert np.array_equal(deq, expect)


def test_mxfp4_matches_brute_restatement(oracle_lib):
    from oracle import brute
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                      # all-zero block -> scale code 0
    w[1, :32] = 1e-42                    # subnormal fp32 inputs
    w[2, :32] = 3.0e38                   # near fp32 max
    packed, scales = oracle_lib.quantize_mxfp4(w)
    deq_b, sc_b = brute.mxfp4_encode_values(w)
    assert np.array_equal(scales, sc_b)
    assert np.array_equal(_decode4(packed, scales), deq_b)
    assert scales[0, 0] == 0


def test_mxfp4_packed_size_invariant(oracle_lib):
    """4 bits per parameter plus one byte per 32 (bjdmk.com.cn page, co-design
    section: MXFP4 stores each parameter in 4 bits): N*K/2 + N*K/32 bytes,
    0.53125x the bytes of an FP8 matrix."""
    w = np.zeros((96, 320), np.float32)
    packed, scales = oracle_lib.quantize_mxfp4(w)
    assert packed.nbytes + scales.nbytes == 96 * 320 // 2 + 96 * 320 // 32
    assert (packed.nbytes + scales.nbytes) / (96 * 320) == 0.53125


def test_mxfp8_matches_torch_rne_and_brute(oracle_lib):
    """Elements: torch's float32 -> float8_e4m3fn conversion (round to nearest
    even) of v / X, where no element exceeds 448; scale X = 2^(floor(log2 amax) - 8)."""
    import torch
    from oracle import brute
    rng = np.random.default_rng(4)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, size=(64, 1)))
    v[5, 32:64] = 0.0
    codes, scales = oracle_lib.quantize_mxfp8(v)
    amax = np.abs(v.reshape(64, 8, 32)).max(-1)
    nz = amax > 0
    r = amax[nz] / np.ldexp(1.0, scales[nz].astype(np.int64) - 127)
    assert ((r >= 256) & (r < 512)).all()
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    q = v / X
    fits = np.abs(q) <= 448
    tq = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = codes.copy()
    # compare where no saturation is involved; +0/-0 compare by value
    dec_t = brute.e4m3_decode(tq)
    dec_o = brute.e4m3_decode(ours)
    assert np.array_equal(dec_t[fits], dec_o[fits])
    # saturation: anything above 448 after scaling becomes 448
    assert np.all(np.abs(dec_o[~fits]) == 448.0)
    deq_b, sc_b = brute.mxfp8_encode_values(v)
    assert np.array_equal(scales, sc_b)
    assert np.array_equal(dec_o * X, deq_b)


def test_mxfp8_midpoint_ties_even(oracle_lib):
    # scale fixed at 2^0 by a 256.0 element; 1.0625 lies halfway between
    # 1.0 (0x38, even) and 1.125 (0x39) -> 1.0; 1.1875 between 1.125 and 1.25 -> 1.25 (0x3a)
    v = np.zeros((1, 32))
    v[0, 0] = 256.0
    v[0, 1] = 1.0625
    v[0, 2] = 1.1875
    v[0, 3] = -1.0625
    v[0, 4] = 464.0 / 2  # 232: halfway between 224 (0x76) and 240 (0x77) -> 224
    codes, scales = oracle_lib.quantize_mxfp8(v)
    assert scales[0, 0] == 127
    assert codes[0, 1] == 0x38 and codes[0, 2] == 0x3A and codes[0, 3] == 0xB8
    assert codes[0, 4] == 0x76


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
@pytest.mark.parametrize("where", [0, 3, 17, 31])
def test_non_finite_element_anywhere_makes_the_block_nan(oracle_lib, bad, where):
    """A block holding a NaN or an infinity at any position encodes as scale
    0xFF with element codes 0, whatever finite values follow it; the other
    blocks of the row are encoded as if it were not there."""
    rng = np.random.default_rng(where)
    row = rng.standard_normal(96)
    alone = row.copy()
    row[32 + where] = bad
    p4, s4 = oracle_lib.quantize_mxfp4(row[None, :].astype(np.float32))
    a4, t4 = oracle_lib.quantize_mxfp4(alone[None, :].astype(np.float32))
    assert s4[0, 1] == 255 and not p4[0, 16:32].any()
    assert s4[0, 0] == t4[0, 0] and s4[0, 2] == t4[0, 2]
    assert np.array_equal(p4[0, :16], a4[0, :16]) and np.array_equal(p4[0, 32:], a4[0, 32:])
    c8, s8 = oracle_lib.quantize_mxfp8(row[None, :])
    b8, t8 = oracle_lib.quantize_mxfp8(alone[None, :])
    assert s8[0, 1] == 255 and not c8[0, 32:64].any()
    assert s8[0, 0] == t8[0, 0] and s8[0, 2] == t8[0, 2]
    assert np.array_equal(c8[0, :32], b8[0, :32]) and np.array_equal(c8[0, 64:], b8[0, 64:])
