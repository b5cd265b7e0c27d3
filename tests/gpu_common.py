"""Shared helpers of the GPU parity tests (oracle side built on the CPU)."""
from __future__ import annotations

import sys

import numpy as np

from workloads import Config, make_shared_weight_fp32, make_weight_fp32


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


_layers = {}


def get_layer(cfg: Config, logits=None):
    """Device layer of a workload, built once per process.  Layers whose
    weights come from the same draws (same seed and shapes) share them."""
    from mxfp4_moe_expert_02_amd.layer import build_layer
    key = (cfg, None if logits is None else logits.tobytes())
    if key not in _layers:
        donor = next((l for (c, _), l in _layers.items()
                      if (c.seed, c.E, c.H, c.I) == (cfg.seed, cfg.E, cfg.H, cfg.I)), None)
        say(f"building layer {cfg.name} seed {cfg.seed}"
            + (f" (weights of {donor.cfg.name})" if donor is not None else ""))
        _layers[key] = build_layer(cfg, logits=logits, weights_from=donor)
    return _layers[key]


_shared = {}


def get_shared(cfg: Config):
    """Device MXFP8 shared expert of a workload (built once per process)."""
    from mxfp4_moe_expert_02_amd.layer import build_shared
    key = (cfg.seed, cfg.H, cfg.I)
    if key not in _shared:
        say(f"building shared expert of {cfg.name}")
        _shared[key] = build_shared(cfg)
    return _shared[key]


def oracle_shared(oracle, cfg: Config):
    """Oracle-encoded MXFP8 shared expert from the same float32 draws."""
    gc, gs = oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "gate_up").astype(np.float64))
    dc, ds = oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "down").astype(np.float64))
    return (gc, gs, dc, ds)


def run(M, layer, path=0, debug=False, act=0, launch=0, init=True, router=None, shared=None,
        layout=None):
    """One forward through the C ABI on every token of the layer; returns
    the requested debug outputs (routing; with MXFP8 also the codes of x)
    as numpy arrays.  out is NaN-filled first, so every element it holds
    afterwards was written by this call.  launch: MOE_LAUNCH_* (the fused
    and queue launches also return their wait-error flag as "wait_error"); init=False
    keeps the current workspace (and whatever an earlier call left in it).
    router: a [E, H] bf16 device router weight -- the layer then computes its
    own logits (returned as "logits") and is given no router_logits.
    shared: the four tile tensors of an MXFP8 shared expert, or None.
    layout: MOE_LAYOUT_* of the weights (default: the tile layout when the
    matrix cores are asked for explicitly or MXFP8 runs, else row-major)."""
    import torch
    c = layer.cfg
    if init:
        M.moe_mxfp4_init(c.T, c.E, c.H, c.I, c.k)
    dbg = {}
    if debug:
        S = c.T * c.k
        dbg = dict(ids=torch.empty((c.T, c.k), dtype=torch.int32, device="cuda"),
                   weights=torch.empty((c.T, c.k), dtype=torch.float32, device="cuda"),
                   counts=torch.empty(c.E, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(c.E + 1, dtype=torch.int32, device="cuda"),
                   sorted=torch.empty(S, dtype=torch.int32, device="cuda"))
        if act == M.MOE_ACT_MXFP8:
            dbg["x_codes"] = torch.empty((c.T, c.H), dtype=torch.uint8, device="cuda")
            dbg["x_scales"] = torch.empty((c.T, c.H // 32), dtype=torch.uint8, device="cuda")
            dbg["h_codes"] = torch.empty((S, c.I), dtype=torch.uint8, device="cuda")
            dbg["h_scales"] = torch.empty((S, c.I // 32), dtype=torch.uint8, device="cuda")
    if launch in (M.MOE_LAUNCH_FUSED, M.MOE_LAUNCH_QUEUE):
        dbg["wait_error"] = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    extra = {}
    if router is not None:
        dbg["logits_out"] = torch.full((c.T, c.E), float("nan"), dtype=torch.float32, device="cuda")
        extra["router_weight"] = router
    layer.out.fill_(float("nan"))
    torch.cuda.synchronize()
    if layout is None:  # the tile layout on an explicit matrix-core request, else row-major
        mfma = path == M.MOE_PATH_MFMA or act == M.MOE_ACT_MXFP8
        layout = M.MOE_LAYOUT_TILES if mfma else M.MOE_LAYOUT_ROWS
    say(f"forward {c.name} T={c.T} E={c.E} H={c.H} I={c.I} k={c.k} path={path} layout={layout} act={act} "
        f"launch={launch} shared={shared is not None}")
    wgu, wdn, scales = layer.weights(layout)
    M.moe_mxfp4_forward_ex(layer.x, None if router is not None else layer.logits, c.k, wgu, wdn,
                           scales, layer.out, gemm_path=path, weight_layout=layout,
                           act_format=act, launch=launch, shared=shared, **dbg, **extra)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dbg.items()}


def oracle_experts(oracle, cfg: Config, experts) -> dict:
    """Oracle-encoded weights of the given experts, from the same float32
    draws the device layer was built from (experts in parallel threads:
    numpy's generators and the C encoder release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(e):
        gp, gs = oracle.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e))
        dp, ds = oracle.quantize_mxfp4(make_weight_fp32(cfg, "down", e))
        return e, (gp, gs, dp, ds)

    todo = sorted(set(int(v) for v in experts))
    with ThreadPoolExecutor(min(8, max(1, len(todo)))) as ex:
        return dict(ex.map(one, todo))


def covering_tokens(route: dict, k: int, unit_rows: int = 16, item_tok: int | None = None) -> tuple[list, int]:
    """Tokens whose outputs, compared with the oracle, exercise every unit
    of work of the layer, each unit holding at least one chosen token.  The
    units are the expert-sorted rows of each touched expert cut into runs
    of `unit_rows` (the 16-token column tiles of the matrix-core items), or,
    with `item_tok`, the items of the route's work list: an expert's c rows
    in ceil(c / item_tok) items of equal numbers of 16-token tiles (+-1),
    the larger ones first.  Greedy set cover (the token covering the most
    uncovered units first, ties to the lower token).  Returns (tokens in
    ascending order, number of units)."""
    sorted_slots, offsets = route["sorted"], route["offsets"]
    runs = []
    for e in range(len(offsets) - 1):
        o0, o1 = int(offsets[e]), int(offsets[e + 1])
        if item_tok is None:
            bounds = [(r0, min(r0 + unit_rows, o1)) for r0 in range(o0, o1, unit_rows)]
        else:
            c = o1 - o0
            groups, tiles = -(-c // item_tok), -(-c // 16)
            per, extra = (tiles // groups, tiles % groups) if c else (0, 0)
            bounds = []
            for q in range(groups):
                t0 = q * per + min(q, extra)
                nt = per + (1 if q < extra else 0)
                bounds.append((o0 + 16 * t0, min(o0 + 16 * (t0 + nt), o1)))
        for r0, r1 in bounds:
            runs.append({int(s) // k for s in sorted_slots[r0:r1]})
    by_token = {}
    for i, toks in enumerate(runs):
        for t in toks:
            by_token.setdefault(t, set()).add(i)
    left, chosen = set(range(len(runs))), []
    while left:
        t = min(by_token, key=lambda t: (-len(by_token[t] & left), t))
        chosen.append(t)
        left -= by_token[t]
    return sorted(chosen), len(runs)


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def parity_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / rms(ref): the acceptance quantity (bar: <= 2e-2)."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.abs(gpu - ref).max() / rms)


def parity_ratio_past_rounding(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of (|gpu - ref| - half a bf16 step of ref) / rms(ref):
    the error beyond the rounding of the exact result to the bf16 output,
    which alone costs up to half a step (2^-9 relative) per element."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    return float(np.maximum(np.abs(gpu - ref) - half, 0.0).max() / rms)


def parity_detail(gpu: np.ndarray, ref: np.ndarray) -> str:
    """Where the largest difference sits: row, column, both values, the
    reference's rms, and the bf16 half-step at that value (the rounding of
    out alone can cost that much)."""
    d = np.abs(gpu - ref)
    r, c = np.unravel_index(int(np.argmax(d)), d.shape)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half = float(np.ldexp(1.0, np.frexp(abs(ref[r, c]))[1] - 9))
    return (f"max at row {r} col {c}: gpu {gpu[r, c]:.6g} ref {ref[r, c]:.6g} rms {rms:.4g} "
            f"(|ref|/rms {abs(ref[r, c]) / rms:.1f}, bf16 half-step {half:.3g})")


def _h_rows_and_bound(x_bf16, k: int, I: int, experts, ids, sorted_slots, rows_wanted):
    """fp64 h of the MXFP8 path before its own encoding (as
    brute.hidden_mxfp8_rows) for positions `rows_wanted` of the expert-sorted
    order, and, per element, a bound on how far an fp32 evaluation of it may
    land: the fp32 sums g and u over H products err by at most
    H * 2^-24 * sum |x w| (the standard bound for recursive summation,
    whatever the order), which moves SiLU(g) * u by at most
    |u| * max|SiLU'| * dg + |SiLU(g)| * du (max |SiLU'| < 1.1), and the fp32
    SiLU and product add a few ulps plus the rounding of the exponential's
    argument (relative |g| * 2^-24).  One expert's weights decoded at a
    time."""
    from oracle import brute
    xf = (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    H = xf.shape[1]
    u32 = 2.0 ** -24
    rows = np.zeros((len(rows_wanted), I))
    eta = np.zeros((len(rows_wanted), I))
    by_expert = {}
    for i, p in enumerate(rows_wanted):
        t, j = divmod(int(sorted_slots[p]), k)
        by_expert.setdefault(int(ids[t, j]), []).append((i, t))
    for e, todo in by_expert.items():
        w = brute.mxfp4_dequant(experts[e][0], experts[e][1])
        wa = np.abs(w)
        for i, t in todo:
            xt = brute.mxfp8_encode_values(xf[t:t + 1])[0][0]
            g, u = w[:I] @ xt, w[I:] @ xt
            sg, su = wa[:I] @ np.abs(xt), wa[I:] @ np.abs(xt)
            sig = 1.0 / (1.0 + np.exp(-g))
            rows[i] = g * sig * u
            eta[i] = (H * u32 * (1.1 * np.abs(u) * sg + np.abs(g * sig) * su)
                      + (8 + 2 * np.abs(g)) * u32 * np.abs(rows[i]))
        del w, wa
    return rows, eta


def check_mxfp8_h(oracle, cfg: Config, x_bf16, experts, route, dbg, tokens=None):
    """The encoding decision of h on the MXFP8 path is taken on fp32 values
    on the GPU and on fp64 ones in the oracle, so it may differ where a
    value sits within fp32 error of a decision boundary; the decision is
    then taken in the kernel's precision on both sides.  Checks, on the h
    rows of the given tokens (default all), that every difference is such a
    case:
    * a block scale differs by one, only where the block's largest |h| is
      within its fp32 error bound of a power of two;
    * every GPU code, at the GPU's block scale X, is the E4M3 rounding (ties
      to even, saturating) of some value within v +- eta / X, v = h / X the
      fp64 value and eta its fp32 error bound (_h_rows_and_bound): one of
      the at most two adjacent codes rounding can give there.  Blocks whose
      scale differs are re-encoded at the GPU's scale and checked the same
      way.
    Returns the oracle's output for those tokens finished from the GPU's own
    h codes (fp64, [len(tokens), H])."""
    from oracle import brute
    T, k = route["ids"].shape
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    want = sorted({int(route["pos"][t * k + j]) for t in tokens for j in range(k)})
    rows, eta = _h_rows_and_bound(x_bf16, k, cfg.I, experts, route["ids"], route["sorted"], want)
    codes, scales = oracle.quantize_mxfp8(rows)
    hq, hs = dbg["h_codes"][want], dbg["h_scales"][want]
    S, I = rows.shape
    amax = np.abs(rows).reshape(S, I // 32, 32).max(axis=2)
    eta_b = eta.reshape(S, I // 32, 32).max(axis=2)
    bad_scale = hs != scales
    for p, b in zip(*np.nonzero(bad_scale)):
        a = amax[p, b]
        assert abs(int(hs[p, b]) - int(scales[p, b])) == 1, (p, b)
        pw = 2.0 ** np.round(np.log2(a))
        assert a > 0 and abs(a - pw) <= eta_b[p, b], (p, b, a, eta_b[p, b])
    X = np.repeat(np.ldexp(1.0, hs.astype(np.int64) - 127), 32, axis=1)
    v, d = rows / X, eta / X
    lo = brute._round_to_format(v - d, 3, -6, 448.0)
    hi = brute._round_to_format(v + d, 3, -6, 448.0)
    gv = brute.e4m3_decode(hq)
    ok = (gv >= lo) & (gv <= hi)
    assert ok.all(), (f"{int((~ok).sum())} h codes are no rounding of a value within the fp32 "
                      f"error bound", np.argwhere(~ok)[:5])
    diff = (hq != codes) & ~np.repeat(bad_scale, 32, axis=1)
    say(f"h codes: {int(diff.sum())} of {diff.size} differ within the fp32 error bound, "
        f"{int(bad_scale.sum())} block scales")
    full_q = np.zeros_like(dbg["h_codes"])
    full_s = np.zeros_like(dbg["h_scales"])
    full_q[want], full_s[want] = hq, hs
    return brute.down_from_h(full_q, full_s, k, experts, route["ids"], route["w"], route["pos"],
                             tokens=tokens)
