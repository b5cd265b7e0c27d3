"""GPU: the MXFP8 shared expert beside the MXFP4 routed experts.

Checked through the C ABI: the MXFP8 weight encoder bit-exact against the
oracle's (special blocks included); the MXFP8 tile layout bit-exact
against a host re-layout; a layer whose shared expert is an MXFP8 copy of
an MXFP4 expert gives the same output bits as the layer routing every
token to that expert (same bf16 operands, same MFMA order); the layer with
a shared expert against the fp64 oracle on every path and launch (VALU
GEMV, self-routed, split, single-launch, wide, MXFP8 prefill) and on ragged
token counts; determinism; and a plain call after a shared one on the
same workspace.
"""
import numpy as np
import pytest

from tests.gpu_common import (bf16_tensor_to_f64, get_layer, get_shared, oracle_experts,
                              oracle_shared, parity_ratio, run, say)
from workloads import Config, get_config, make_logits, make_x_bf16

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


def _encode_fp8(M, w):
    import torch
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    codes = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((w.shape[0], w.shape[1] // 32), dtype=torch.uint8, device="cuda")
    M.moe_mxfp8_quantize(wd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_mxfp8_weight_encoder_bit_exact(M, oracle_lib):
    rng = np.random.default_rng(40)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[0] = 0.0                                   # amax 0: scale code 0
    w[1, 5] = np.nan                             # non-finite blocks: scale 0xFF, codes 0
    w[1, 40] = np.inf
    w[2, :32] = rng.standard_normal(32).astype(np.float32) * np.float32(3e38)  # top of the range
    w[3, :32] = np.float32(1e-42) * np.arange(32, dtype=np.float32)  # fp32 subnormals
    # exact midpoints between neighbouring E4M3 values (block amax 1.0: scale 2^-8)
    mids = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 0.5 + 1 / 32, 2.0 ** -7 * 3 / 16], np.float32)
    w[4, :32] = np.resize(np.concatenate([mids, -mids]), 32)
    w[4, 0] = 1.0
    w[5, :32] = np.float32(500.0)                 # saturates at 448 * scale
    w[5, 1] = np.float32(-1e5)
    codes, scales = _encode_fp8(M, w)
    want_c, want_s = oracle_lib.quantize_mxfp8(w.astype(np.float64))
    np.testing.assert_array_equal(scales, want_s)
    np.testing.assert_array_equal(codes, want_c)
    assert scales[0, 0] == 0 and scales[1, 0] == 255 and scales[1, 1] == 255


def _host_relayout(codes, scales, pairs):
    """The MXFP8 tile layout written out with plain indexing."""
    N, rows, cols = codes.shape
    quads, chunks = rows // 64, cols // 128
    tiles = np.zeros(codes.size, np.uint8)
    tsc = np.zeros(scales.size, np.uint8)
    half_rows = rows // 2
    for mat in range(N):
        for q in range(quads):
            for rg in range(4):
                for r in range(16):
                    row = (((0 if rg < 2 else half_rows) + 32 * q + 16 * (rg & 1) + r) if pairs
                           else 64 * q + 16 * rg + r)
                    for c in range(chunks):
                        for g in range(4):
                            lane = r + 16 * g
                            base = ((mat * quads + q) * chunks + c) * 8192 + rg * 2048 + lane * 16
                            blk = codes[mat, row, c * 128 + 32 * g: c * 128 + 32 * g + 32]
                            tiles[base:base + 16] = blk[:16]
                            tiles[base + 1024:base + 1040] = blk[16:]
                            tsc[((mat * quads + q) * chunks + c) * 256 + lane * 4 + rg] = \
                                scales[mat, row, c * 4 + g]
    return tiles, tsc


@pytest.mark.parametrize("pairs", [False, True])
def test_mxfp8_prepack_layout(M, pairs):
    import torch
    rng = np.random.default_rng(41 + pairs)
    codes = rng.integers(0, 256, (2, 128, 256), dtype=np.uint8)
    scales = rng.integers(0, 256, (2, 128, 8), dtype=np.uint8)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    td, tsd = torch.empty_like(cd), torch.empty_like(sd)
    M.moe_mxfp8_prepack(cd, sd, td, tsd, gate_up_pairs=pairs)
    torch.cuda.synchronize()
    want_t, want_s = _host_relayout(codes, scales, pairs)
    np.testing.assert_array_equal(td.cpu().numpy().ravel(), want_t)
    np.testing.assert_array_equal(tsd.cpu().numpy().ravel(), want_s)


def _e2m1_to_e4m3(oracle_lib):
    e4 = {oracle_lib.e4m3_value(c): c for c in range(127)}
    tab = np.array([e4[oracle_lib.e2m1_value(c)] for c in range(8)], np.uint8)
    return np.concatenate([tab, tab | 0x80])


@pytest.mark.parametrize("launch", ["auto", "split"])
def test_mxfp8_copy_of_an_mxfp4_expert_gives_the_same_bits(M, oracle_lib, launch):
    """Layer A: 4 experts, every token routed to expert 0 (k = 1, weight 1).
    Layer B: the routed experts zero, the shared expert the MXFP8 copy of
    expert 0.  Same weight values and the same h terms in the same MFMA
    order (the routed items are single 16-token tiles, as the shared
    expert's blocks): the same output bits."""
    import torch
    T, E, H, I = 9, 4, 256, 128
    rng = np.random.default_rng(43)
    dev = "cuda"
    mats = {}
    for which, shape in (("gate_up", (2 * I, H)), ("down", (H, I))):
        w = torch.from_numpy((rng.standard_normal(shape) * 0.02).astype(np.float32)).to(dev)
        p = torch.empty((shape[0], shape[1] // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((shape[0], shape[1] // 32), dtype=torch.uint8, device=dev)
        M.moe_mxfp4_quantize(w, p, s)
        mats[which] = (p, s)
    torch.cuda.synchronize()
    tab = torch.from_numpy(_e2m1_to_e4m3(oracle_lib)).to(dev).long()

    def routed(expert0):
        out = []
        for which in ("gate_up", "down"):
            p, s = mats[which]
            pk = torch.zeros((E,) + tuple(p.shape), dtype=torch.uint8, device=dev)
            sc = torch.full((E,) + tuple(s.shape), 127, dtype=torch.uint8, device=dev)
            if expert0:
                pk[0], sc[0] = p, s
            tp, ts = torch.empty_like(pk), torch.empty_like(sc)
            M.moe_mxfp4_prepack(pk, sc, tp, ts, gate_up_pairs=which == "gate_up")
            out.append((tp, ts))
        return out

    def fp8_copy():
        out = []
        for which in ("gate_up", "down"):
            p, s = mats[which]
            nib = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1).long()
            codes = tab[nib].to(torch.uint8).contiguous()
            tc, ts = torch.empty_like(codes), torch.empty_like(s)
            M.moe_mxfp8_prepack(codes.view(1, *codes.shape), s.view(1, *s.shape), tc, ts,
                                gate_up_pairs=which == "gate_up")
            out += [tc, ts]
        return tuple(out)

    x = torch.from_numpy(make_x_bf16(Config("s", "s", T, E, H, I, 1, "normal", "bf16", 44))
                         .view(np.int16)).view(torch.bfloat16).to(dev)
    lg = torch.zeros((T, E), dtype=torch.float32, device=dev)
    lg[:, 1:] = -1.0  # expert 0 for every token
    lmode = M.MOE_LAUNCH_SPLIT if launch == "split" else M.MOE_LAUNCH_AUTO
    M.moe_mxfp4_init(T, E, H, I, 1)
    outs = []
    for expert0, shared in ((True, None), (False, fp8_copy())):
        (gu, gus), (dn, dns) = routed(expert0)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
        say(f"shared copy test launch={launch} shared={shared is not None}")
        M.moe_mxfp4_forward_ex(x, lg, 1, gu, dn, (gus, dns), out, gemm_path=M.MOE_PATH_MFMA,
                               weight_layout=M.MOE_LAYOUT_TILES, launch=lmode, shared=shared)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[0].float()).all() and outs[0].float().abs().max() > 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def _small(T, seed, E=8, H=256, I=128, k=2, act="bf16"):
    return Config("shared", f"shared_t{T}_e{E}_h{H}_i{I}_k{k}_{act}", T, E, H, I, k, "normal", act,
                  seed)


CASES = {  # name: (config, path, act, launch, sampled tokens or None = all)
    "c1_gemv": ("c1", 1, 0, 0, None),
    "c1_self": ("c1", 2, 0, 0, None),
    "c1_split": ("c1", 2, 0, 1, None),
    "c1_fused": ("c1", 2, 0, 2, None),
    "c1_mx8": ("c1", 0, 1, 0, None),
    "t1_self": (("t", 1), 2, 0, 0, None),
    "t17_split": (("t", 17), 2, 0, 0, None),
    "t40_wide": (("t", 40, 4), 2, 0, 0, None),
    "t33_mx8": (("t", 33), 0, 1, 0, None),
    "t50_gemv": (("t", 50), 1, 0, 0, None),
    "t70_wide": (("t", 70, 4), 2, 0, 0, None),      # 64-token shared tiles, a ragged one
    "t100_mx8": (("t", 100), 0, 1, 0, None),
    "t130_split": (("t", 130, 64), 2, 0, 0, None),   # shared blocks inside the split kernels
    "t80_gemv": (("t", 80), 1, 0, 0, None),          # own launches, 64-token tiles
    "t70_fused": (("t", 70, 64), 2, 0, 2, None),
    "c2_self": ("c2", 2, 0, 0, [0, 4, 8]),
    "c3_split": ("c3", 2, 0, 0, [0, 35, 71]),
    "c4_wide": ("c4", 2, 0, 0, [0, 143, 287]),
    "c5_mx8": ("c5", 0, 1, 0, [0, 2047, 4095]),
}


def _cfg(spec, act):
    if isinstance(spec, str):
        return get_config(spec)
    T = spec[1]
    E = spec[2] if len(spec) > 2 else 8
    return _small(T, 50 + T, E=E, k=min(2, E), act="mxfp8" if act else "bf16")


@pytest.mark.parametrize("name", list(CASES))
def test_layer_with_shared_expert_vs_oracle(M, oracle_lib, name):
    spec, path, act, launch, tokens = CASES[name]
    cfg = _cfg(spec, act)
    layer = get_layer(cfg)
    sh = get_shared(cfg)
    dbg = run(M, layer, path=path, act=act, launch=launch, shared=sh.tiles)
    if launch == M.MOE_LAUNCH_FUSED:
        assert int(dbg["wait_error"][0]) == 0
    full = bf16_tensor_to_f64(layer.out)
    assert np.isfinite(full).all()
    toks = list(range(cfg.T)) if tokens is None else tokens
    lg = make_logits(cfg)
    ids = oracle_lib.route(lg, cfg.k)["ids"]
    ex = oracle_experts(oracle_lib, cfg, ids[toks].ravel())
    osh = oracle_shared(oracle_lib, cfg)
    # the device encoder gave the oracle's bytes (checked bit-exact above)
    np.testing.assert_array_equal(sh.gus.cpu().numpy(), osh[1])
    ref = oracle_lib.forward(make_x_bf16(cfg), lg, cfg.k, cfg.H, cfg.I, ex, tokens=toks,
                             act_mxfp8=bool(act), shared=osh)
    ratio = parity_ratio(full[toks], ref)
    plain = oracle_lib.forward(make_x_bf16(cfg), lg, cfg.k, cfg.H, cfg.I, ex, tokens=toks,
                               act_mxfp8=bool(act))
    without = parity_ratio(full[toks], plain)
    say(f"shared parity {name}: max|d|/rms = {ratio:.3e} (against the layer without it: "
        f"{without:.3e})")
    assert ratio <= TOL
    assert without > 10 * TOL  # the shared term is really in the output


def test_shared_deterministic_and_plain_after_shared(M):
    import torch
    cfg = get_config("c2")
    layer = get_layer(cfg)
    sh = get_shared(cfg)
    run(M, layer, path=2, shared=sh.tiles)
    a = layer.out.clone()
    run(M, layer, path=2, shared=sh.tiles, init=False)
    assert torch.equal(a.view(torch.int16), layer.out.view(torch.int16))
    run(M, layer, path=2, init=False)  # no shared expert: nothing of it left in the output
    plain = layer.out.clone()
    run(M, layer, path=2)
    assert torch.equal(plain.view(torch.int16), layer.out.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), plain.view(torch.int16))


@pytest.mark.parametrize("key", ["c2", "mx8"])
def test_shared_expert_with_router_weight(M, oracle_lib, key):
    """Both options together: the layer computes its logits from a bf16
    router weight and adds the shared expert.  The routing is checked on
    the GPU's fp32 logits (the decision in the same precision on both
    sides), the output against the oracle on those logits."""
    import torch
    from workloads import make_router_weight_bf16
    cfg = get_config("c2") if key == "c2" else _small(40, 77, E=8, act="mxfp8")
    act = M.MOE_ACT_MXFP8 if cfg.act == "mxfp8" else M.MOE_ACT_BF16
    layer = get_layer(cfg)
    sh = get_shared(cfg)
    w = make_router_weight_bf16(cfg)
    w_dev = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda")
    dbg = run(M, layer, path=0 if act else 2, act=act, debug=True, router=w_dev, shared=sh.tiles)
    lg = dbg["logits_out"]
    r = oracle_lib.route(lg, cfg.k)
    np.testing.assert_array_equal(dbg["ids"], r["ids"])
    tokens = sorted({0, cfg.T // 2, cfg.T - 1})
    ex = oracle_experts(oracle_lib, cfg, r["ids"][tokens].ravel())
    ref = oracle_lib.forward(make_x_bf16(cfg), lg, cfg.k, cfg.H, cfg.I, ex, tokens=tokens,
                             act_mxfp8=bool(act), shared=oracle_shared(oracle_lib, cfg))
    ratio = parity_ratio(bf16_tensor_to_f64(layer.out)[tokens], ref)
    say(f"shared + router parity {cfg.name}: max|d|/rms = {ratio:.3e}")
    assert ratio <= TOL


@pytest.mark.parametrize("path", [2, 0])
def test_shared_nan_scales_reach_every_token(M, path):
    """A NaN block scale (E8M0 0xFF) throughout the shared expert's down
    matrix makes every output NaN (the shared expert is applied to every
    token); the same layer without it stays finite."""
    import torch
    act = M.MOE_ACT_MXFP8 if path == 0 else M.MOE_ACT_BF16
    cfg = _small(20, 91, act="mxfp8" if act else "bf16")
    layer = get_layer(cfg)
    sh = get_shared(cfg)
    bad = (sh.gu_t, sh.gus_t, sh.dn_t, torch.full_like(sh.dns_t, 255))
    run(M, layer, path=path, act=act)
    assert torch.isfinite(layer.out.float()).all()
    run(M, layer, path=path, act=act, shared=bad, init=False)
    assert torch.isnan(layer.out.float()).all()
