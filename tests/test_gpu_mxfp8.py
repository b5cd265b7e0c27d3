"""GPU parity of the prefill path (MXFP8 activations, scaled FP4 x FP8
matrix cores) against the CPU oracle run with the same MXFP8 rule.

* the MXFP8 encoding of x (E4M3 codes and E8M0 scales) bit-exact: both
  sides start from the same bf16 values and the encoding is exact
  arithmetic on them
* routing bit-exact (the prefill path groups up to 128 tokens per work item)
* layer output: h is encoded from fp32 on the GPU and from fp64 in the
  oracle, so a code of h may differ where the value sits within fp32 error
  of a rounding boundary: the decision is taken in the kernel's precision.
  Every code of h of the compared tokens is checked to be such a case
  (check_mxfp8_h) and max |out - ref| <= 2e-2 * rms(ref) against the oracle
  finished from the GPU's own h codes; against the plain fp64 oracle too,
  except the layers listed in MXFP8_PLAIN_OVER (twice the bar).
  Full-size layers compare a set of tokens that puts one compared token in
  every prefill item (or 16-token tile) of every touched expert.
"""
import numpy as np
import pytest

from tests.gpu_common import (bf16_tensor_to_f64, check_mxfp8_h, covering_tokens, get_layer,
                              oracle_experts, parity_detail, parity_ratio, parity_ratio_past_rounding,
                              run, say)
from workloads import Config, get_config, make_logits, make_x_bf16

pytestmark = pytest.mark.gpu

TOL = 2e-2
MX8 = 1  # MOE_ACT_MXFP8
# Layers whose output, against the plain fp64 oracle, lands over the bar
# while every code of h is a correct rounding of its value within the fp32
# error bound (check_mxfp8_h) and the output is within the bar against the
# oracle finished from those codes: an E4M3 code that flips on a rounding
# boundary moves h by up to 1/8 of its value.  They are held to twice the
# bar against the plain oracle.
MXFP8_PLAIN_OVER = {"batched_verify_t72_e128_h7168_i2048_k8", "prefill_t4096_e128_h7168_i2048_k8"}
# Layers where the rounding of out to bf16 alone exceeds the bar: an output
# element far above the rms (batched-verify shape: 7.0 x rms, where half a
# bf16 step is 2.38e-2 of rms and the GPU's value is the correctly rounded
# reference).  There the error past that rounding must be within the bar.
OUT_ROUNDING_OVER = {"batched_verify_t72_e128_h7168_i2048_k8"}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    return torch


@pytest.fixture(scope="module")
def M():
    import mxfp4_moe_expert_02_amd as M
    assert M.MOE_ACT_MXFP8 == MX8
    return M


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 values that are exact in bf16 -> their bf16 bit patterns."""
    v = np.ascontiguousarray(v, np.float32)
    bits = v.view(np.uint32)
    assert not (bits & 0xFFFF).any(), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _x_codes_ref(oracle_lib, x_bits: np.ndarray):
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return oracle_lib.quantize_mxfp8(x)


def _parity(M, oracle_lib, cfg, layer, tokens, logits=None, x_bits=None):
    dbg = run(M, layer, act=MX8, debug=True)
    lg = make_logits(cfg) if logits is None else logits
    xb = make_x_bf16(cfg) if x_bits is None else x_bits
    route = oracle_lib.route(lg, cfg.k)
    assert np.array_equal(dbg["ids"], route["ids"])
    assert np.array_equal(dbg["sorted"], route["sorted"])
    assert np.array_equal(dbg["offsets"], route["offsets"])
    full = bf16_tensor_to_f64(layer.out)
    assert np.isfinite(full).all()  # every (token, column) was written
    ex = oracle_experts(oracle_lib, cfg, route["ids"][tokens].ravel())
    ref = oracle_lib.forward(xb, lg, cfg.k, cfg.H, cfg.I, ex, tokens=tokens, act_mxfp8=True)
    plain = parity_ratio(full[tokens], ref)
    # h's encoding decision checked code by code, then the oracle finished
    # from the GPU's own h codes
    sref = check_mxfp8_h(oracle_lib, cfg, xb, ex, route, dbg, tokens)
    staged = parity_ratio(full[tokens], sref)
    say(f"mxfp8 parity {cfg.name} {len(tokens)} tokens max|d|/rms = {plain:.3e} (plain), "
        f"{staged:.3e} (from the GPU's h codes); {parity_detail(full[tokens], sref)}")
    if cfg.name in OUT_ROUNDING_OVER:
        past = parity_ratio_past_rounding(full[tokens], sref)
        say(f"mxfp8 parity {cfg.name}: past the rounding of out {past:.3e}")
        assert past <= TOL and staged <= 2 * TOL
    else:
        assert staged <= TOL
    assert plain <= (2 * TOL if cfg.name in MXFP8_PLAIN_OVER else TOL)
    return dbg


def test_x_encoding_edge_blocks_bit_exact(torch_dev, M, oracle_lib):
    """Blocks that exercise every branch of the E4M3 block encoding: ties to
    the even code, saturation at 448, the subnormal range, scale clamping,
    signed zeros, an all-zero block and a non-finite block."""
    from mxfp4_moe_expert_02_amd.layer import build_layer
    base = Config("mx8e", "mxfp8_edges_t6_e8_h256_i128_k2", 6, 8, 256, 128, 2, "normal",
                  "mxfp8", 41)
    rng = np.random.default_rng(3)
    blk = rng.standard_normal((base.T, base.H // 32, 32)).astype(np.float32)
    # amax 256 -> scale 2^0, so the elements are quantised as given
    blk[0, 0] = [256.0, 1.0625, 1.1875, -1.0625, 3.0e-3, 2.0 ** -10, 3 * 2.0 ** -10, 300.0,
                 -304.0, 0.0, -0.0, 2.0 ** -7, 2.0 ** -9, 7.5, 0.5, 0.625] + [1.0] * 16
    blk[0, 1] = 0.0                                  # all-zero block: scale code 0
    blk[0, 2] = -0.0
    blk[0, 3, :] = 448.0 * 2.0 ** -3
    blk[0, 3, 5] = 500.0 * 2.0 ** -3                 # saturates
    blk[1, 0, :] = 2.0 ** -133                       # bf16 subnormal: scale clamps at 2^-127
    blk[1, 1, :] = np.linspace(-3e38, 3e38, 32).astype(np.float32)
    blk[1, 2, :] = np.float32(3.3895314e38)          # largest bf16
    blk[2, 0, 7] = np.inf                            # non-finite block: scale 0xFF
    blk[2, 1, 3] = np.nan
    blk[3, :, :] = rng.integers(-16, 17, size=(base.H // 32, 32)) * 2.0 ** -4
    xv = blk.reshape(base.T, base.H).astype(np.float32)
    xv = (xv.view(np.uint32) & 0xFFFF0000).view(np.float32)   # make every value bf16-exact
    bits = _bf16_bits(xv)
    layer = build_layer(base, x_bf16=bits, weights_from=get_layer(base))
    dbg = run(M, layer, act=MX8, debug=True)
    codes, scales = _x_codes_ref(oracle_lib, bits)
    assert np.array_equal(dbg["x_scales"], scales)
    assert np.array_equal(dbg["x_codes"], codes)


def test_x_encoding_prefill_rows_bit_exact(torch_dev, M, oracle_lib):
    cfg = get_config("c5")
    dbg = run(M, get_layer(cfg), act=MX8, debug=True)
    xb = make_x_bf16(cfg)
    for rows in (slice(0, 128), slice(cfg.T - 128, cfg.T)):
        codes, scales = _x_codes_ref(oracle_lib, xb[rows])
        assert np.array_equal(dbg["x_codes"][rows], codes)
        assert np.array_equal(dbg["x_scales"][rows], scales)


def test_mxfp8_forward_tiny_all_tokens(torch_dev, M, oracle_lib):
    cfg = get_config("c1")
    _parity(M, oracle_lib, cfg, get_layer(cfg), list(range(cfg.T)))


@pytest.mark.parametrize("T,k", [(1, 1), (1, 8), (2, 5)])
def test_mxfp8_forward_small_edges(torch_dev, M, oracle_lib, T, k):
    cfg = Config("edge", f"edge_t{T}_e8_h256_i128_k{k}", T, 8, 256, 128, k, "normal", "bf16", 21 + T)
    _parity(M, oracle_lib, cfg, get_layer(cfg), list(range(T)))


def test_mxfp8_forward_one_hot_expert_ragged_items(torch_dev, M, oracle_lib):
    """300 tokens all pick expert 3 first: its items hold 112, 96 and 92
    tokens (7, 6 and 6 tiles, the last one ragged); the other experts get
    ragged smaller items."""
    cfg = Config("hot8", "hot_t300_e8_h384_i256_k3", 300, 8, 384, 256, 3, "normal", "mxfp8", 13)
    logits = make_logits(cfg)
    logits[:, 3] += 100.0
    layer = get_layer(cfg, logits=logits)
    _parity(M, oracle_lib, cfg, layer, list(range(0, cfg.T, 7)) + [cfg.T - 1], logits=logits)


def _covering(oracle_lib, cfg, unit_rows=16, item_tok=None):
    tokens, runs = covering_tokens(oracle_lib.route(make_logits(cfg), cfg.k), cfg.k, unit_rows, item_tok)
    what = f"items of up to {item_tok} tokens" if item_tok else f"runs of {unit_rows} rows"
    say(f"{cfg.name}: {len(tokens)} tokens cover {runs} {what} of the touched experts")
    return tokens


def test_mxfp8_forward_batched_shape_every_tile(torch_dev, M, oracle_lib):
    """72 tokens over 128 experts at the full hidden sizes (mostly 1-10
    token items) with MXFP8 activations."""
    cfg = get_config("c3")
    _parity(M, oracle_lib, cfg, get_layer(cfg), _covering(oracle_lib, cfg, 16))


def test_mxfp8_forward_prefill_every_item(torch_dev, M, oracle_lib):
    """The prefill chunk: one compared token in each of its items (up to 128
    tokens of one expert each)."""
    cfg = get_config("c5")
    _parity(M, oracle_lib, cfg, get_layer(cfg), _covering(oracle_lib, cfg, item_tok=128))


def test_mxfp8_forward_deterministic(torch_dev, M):
    cfg = get_config("c5")
    layer = get_layer(cfg)
    run(M, layer, act=MX8)
    a = layer.out.clone()
    run(M, layer, act=MX8)
    assert torch_dev.equal(a.view(torch_dev.int16), layer.out.view(torch_dev.int16))


def test_mxfp8_untouched_experts_are_not_read(torch_dev, M):
    import torch
    cfg = Config("pois8", "poison_t70_e16_h256_i128_k2", 70, 16, 256, 128, 2, "normal", "mxfp8", 31)
    logits = make_logits(cfg)
    logits[:, 10:] -= 100.0
    layer = get_layer(cfg, logits=logits)
    run(M, layer, act=MX8)
    base = layer.out.clone()
    saved = [s.clone() for s in (layer.sgu_t, layer.sdn_t)]
    layer.sgu_t[10:] = 255
    layer.sdn_t[10:] = 255
    run(M, layer, act=MX8)
    assert torch.isfinite(layer.out.float()).all()
    assert torch.equal(base.view(torch.int16), layer.out.view(torch.int16))
    for s, v in zip((layer.sgu_t, layer.sdn_t), saved):
        s.copy_(v)


def test_mxfp8_needs_tile_layout(torch_dev, M):
    cfg = get_config("c1")
    layer = get_layer(cfg)
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    rc = M.moe_mxfp4_forward_ex(layer.x, layer.logits, cfg.k, layer.wgu, layer.wdn, layer.scales,
                                layer.out, act_format=MX8, weight_layout=M.MOE_LAYOUT_ROWS,
                                check=False)
    assert rc == M.MOE_E_OPTION
