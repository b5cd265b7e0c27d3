#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

Workload (default): the 9-token speculative-decode verify step (8 drafts + 1)
on one GPU's expert share: 64 experts, hidden 6144, intermediate 2048, top-8,
synthetic seeded inputs (x ~ N(0,1) bf16, router logits ~ N(0,1), expert
weights ~ N(0,0.02) encoded to MXFP4 on the GPU).

One step = one full layer (route -> gate_up + SiLU*up -> down -> combine) on
inputs already resident in HBM; layers of at most 16 tokens run self-routed
(the GEMM workgroups rank their own experts: no routing kernel).  The steps
rotate through --weight-sets separately allocated copies of the expert
weights (default 3), so a step never finds the previous step's weights in
L2 or the 256 MiB Infinity Cache, as in a decode that reads each layer's
own weights once.  Prints ONE JSON line:
  value  = touched-expert weight bytes (packed E2M1 + E8M0) / mean layer time, GB/s
  step_us = median / p10 / p90 of single steps (events between steps)
  cold   = steps after a 1 GiB cache-allocating read that evicts L2 and the
           Infinity Cache (then a stream sync, so no write-back lands in the
           step), per stage, median over 30
  roofline = the dominant kernel (gate_up: 2/3 of the bytes) against the
             8 TB/s HBM peak, timed live with HIP events the library records
             between its kernels
  cpu_baseline = the fp64 CPU oracle on the host cores, same workload (every
                 token up to 32 tokens; above that an evenly spaced sample
                 of 32 tokens, the time scaled to the whole layer)

--config c5 runs the prefill chunk (4096 tokens) with MXFP8 activations on
the scaled FP4 x FP8 matrix cores; its roofline is the gate_up kernel's
TFLOP/s against the dense FP8 matrix-core peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0   # dense MFMA with an FP8 operand (the FP4 x FP8 instruction's rate)
FP4_PEAK_TFLOPS = 10100.0  # dense MFMA, FP4 x FP4
CPU_SAMPLE_TOKENS = 32
METRIC = "MoE layer µs + achieved HBM GB/s (% peak) at 9-token verify step, 1 GPU"
STAGES = ["route", "gate_up", "down_combine"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="c2",
                   help="workload key c1..c5 (default: c2, 9-token verify; c5: MXFP8 prefill)")
    p.add_argument("--path", type=int, default=0,
                   help="1: VALU GEMV over row-major weights; 2 (default): bf16 MFMA over "
                        "the tile layout (weights prepacked once before timing)")
    p.add_argument("--launch", choices=["auto", "split", "self", "fused", "queue"], default="auto",
                   help="bf16 MFMA path: auto (the library's choice: self-routed for at most "
                        "16 tokens, queue for layers whose experts average 4 or more tokens), "
                        "split (routing kernel, then the GEMMs), self (no routing "
                        "kernel: each GEMM workgroup ranks its own expert), fused (one "
                        "persistent launch: the whole layer for at most 16 tokens), queue "
                        "(both GEMMs in one launch of one workgroup per dequeued unit)")
    p.add_argument("--router", action="store_true",
                   help="compute the router logits in the layer from a bf16 router weight [E, H] "
                        "(x . W_router^T on the matrix cores) instead of taking them as input")
    p.add_argument("--shared", action="store_true",
                   help="add an MXFP8 shared expert (gate_up [2I,H], down [H,I]) applied to every "
                        "token; its bytes count in the touched bytes")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true")
    p.add_argument("--no-probe", action="store_true", help="skip the HBM streaming-read probe")
    p.add_argument("--graph", action="store_true",
                   help="also time the layer replayed from a captured HIP graph")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="also run one probe copy of this many bytes (counter calibration)")
    p.add_argument("--seed", type=int, default=None,
                   help="base seed of the synthetic inputs (default: the workload's own); the "
                        "profiled HBM traffic applies to the default seed only")
    p.add_argument("--weight-sets", type=int, default=3,
                   help="separately allocated copies of the expert weights; step i uses copy "
                        "i mod N (1: every step rereads the same weights)")
    return p.parse_args()


def build_info() -> dict:
    """What produced the numbers: git commit (if the tree has .git), the
    kernel sources' sha256, ROCm and HIP runtime versions."""
    import subprocess
    sha = None
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    rocm = None
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(f):
            rocm = open(f).read().strip()
            break
    built = None  # the commit the in-tree library was built from (build.py)
    info = os.path.join(ROOT, "mxfp4_moe_expert_02_amd", "_build_info.json")
    if os.path.exists(info):
        try:
            built = json.load(open(info))
        except (OSError, ValueError):
            built = None
    import torch
    return {"git_sha": sha, "library_built_from": built, "kernel_sources_sha256": sources_sha256(),
            "rocm_version": rocm, "hip_runtime": torch.version.hip, "torch": torch.__version__}


def touched_bytes(counts: np.ndarray, H: int, I: int) -> tuple[int, int]:
    """Algorithmic bytes: packed E2M1 + E8M0 of every expert with >= 1 token,
    split (gate_up, down)."""
    n = int((counts > 0).sum())
    gu = n * (2 * I * H // 2 + 2 * I * H // 32)
    dn = n * (H * I // 2 + H * I // 32)
    return gu, dn


CSRC = os.path.join(ROOT, "mxfp4_moe_expert_02_amd", "csrc")


def sources_sha256() -> str:
    """sha256 over every HIP source and header of the library: a traffic
    figure taken with other kernel code does not apply."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from profiles/traffic.txt
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated by a copy of known size),
    or None if none was taken with the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    digest = sources_sha256()
    for line in open(path):
        parts = line.split()
        if len(parts) == 4 and not line.startswith("#"):
            w, k, sha, nbytes = parts
            if w == workload and k == kernel and sha == digest:
                return int(nbytes)
    return None


def probe_bandwidth(M, torch, nbytes: int = 4 << 30, reps: int = 20) -> float:
    """Achievable HBM read bandwidth: a plain 128-bit streaming read of
    ``nbytes`` (far above the 256 MiB Infinity Cache), GB/s."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(M.moe_probe_sink_words(), dtype=torch.int32, device="cuda")
    for _ in range(3):
        M.moe_probe_stream_read(buf, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        M.moe_probe_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    return gbs


def cpu_baseline(cfg, gbytes_total: float, shared: bool = False) -> dict:
    """The oracle as it stands, on the host cores: the whole layer when it
    has at most CPU_SAMPLE_TOKENS tokens, else that many evenly spaced
    tokens with the time scaled by T / sample (the oracle's cost is per
    token and per routed expert)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from workloads import make_logits, make_weight_fp32, make_x_bf16

    lg = make_logits(cfg)
    x = make_x_bf16(cfg)
    ids = oracle.route(lg, cfg.k)["ids"]
    n = min(cfg.T, CPU_SAMPLE_TOKENS)
    tokens = np.unique(np.linspace(0, cfg.T - 1, n).round().astype(np.int32))
    experts = sorted(set(int(e) for e in ids[tokens].ravel()))

    def prep(e):
        gp, gs = oracle.quantize_mxfp4(make_weight_fp32(cfg, "gate_up", e))
        dp, ds = oracle.quantize_mxfp4(make_weight_fp32(cfg, "down", e))
        return e, (gp, gs, dp, ds)

    with ThreadPoolExecutor(4) as ex:
        weights = dict(ex.map(prep, experts))
    sh = None
    if shared:
        from workloads import make_shared_weight_fp32
        sh = (*oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "gate_up").astype(np.float64)),
              *oracle.quantize_mxfp8(make_shared_weight_fp32(cfg, "down").astype(np.float64)))
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.forward(x, lg, cfg.k, cfg.H, cfg.I, weights, tokens=tokens,
                   act_mxfp8=cfg.act == "mxfp8", shared=sh)
    dt = (time.perf_counter() - t0) * cfg.T / len(tokens)
    what = (f"whole layer: all {cfg.T} tokens" if len(tokens) == cfg.T else
            f"{len(tokens)} of {cfg.T} tokens evenly spaced, time scaled by {cfg.T}/{len(tokens)}")
    return {"value": round(gbytes_total / dt, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "us_per_layer": round(dt * 1e6, 1),
            "sample": f"{what} x top-{cfg.k} ({len(experts)} experts in the sample), fp64, "
                      f"OpenMP threads={cores}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}); "
              "its multi-GPU expert-parallel form is a design, not code.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_moe_expert_02_amd as M
    from mxfp4_moe_expert_02_amd.layer import build_layer
    from workloads import get_config

    cfg = get_config(args.config) if args.seed is None else get_config(args.config, seed=args.seed)
    mx8 = cfg.act == "mxfp8"
    act = M.MOE_ACT_MXFP8 if mx8 else M.MOE_ACT_BF16
    if mx8 and args.path == M.MOE_PATH_GEMV:
        print("bench.py: MXFP8 activations run on the matrix cores only (--path 0 or 2)",
              file=sys.stderr)
        sys.exit(2)
    lib_path = os.path.abspath(M.lib()._name)
    print(f"[bench] library {lib_path}", file=sys.stderr, flush=True)
    print(f"[bench] building {cfg.name}", file=sys.stderr, flush=True)
    layer = build_layer(cfg)
    M.moe_mxfp4_init(cfg.T, cfg.E, cfg.H, cfg.I, cfg.k)
    stream = torch.cuda.current_stream()

    path = args.path or M.MOE_PATH_MFMA
    layout = M.MOE_LAYOUT_TILES if path == M.MOE_PATH_MFMA else M.MOE_LAYOUT_ROWS
    wgu, wdn, scales = layer.weights(layout)
    # the weight sets the steps rotate through: the layer's own, then copies
    nsets = max(1, args.weight_sets)
    wsets = [(wgu, wdn, scales)] + [(wgu.clone(), wdn.clone(), tuple(t.clone() for t in scales))
                                    for _ in range(nsets - 1)]
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")

    launch = {"auto": M.MOE_LAUNCH_AUTO, "split": M.MOE_LAUNCH_SPLIT,
              "self": M.MOE_LAUNCH_SELF_ROUTED, "fused": M.MOE_LAUNCH_FUSED,
              "queue": M.MOE_LAUNCH_QUEUE}[args.launch]
    wide = cfg.T * cfg.k >= 4 * cfg.E  # the library's wide items (experts average >= 4 tokens)
    self_ok = (path == M.MOE_PATH_MFMA and not mx8 and cfg.T * cfg.k < 8 * cfg.E and cfg.T <= 16
               and cfg.T * cfg.E <= 4096)
    self_routed = self_ok and launch in (M.MOE_LAUNCH_AUTO, M.MOE_LAUNCH_SELF_ROUTED)
    # one launch for the whole layer (the single-launch kernel's time is the
    # "gate_up" stage, and it moves every touched byte)
    fused = path == M.MOE_PATH_MFMA and not mx8 and launch == M.MOE_LAUNCH_FUSED
    # both routed GEMMs in one launch of one workgroup per unit (AUTO's choice
    # for wide layers without a shared expert; its time is the "gate_up"
    # stage, and it moves every touched byte)
    queue = (path == M.MOE_PATH_MFMA and not mx8 and not self_routed and
             (launch == M.MOE_LAUNCH_QUEUE or (launch == M.MOE_LAUNCH_AUTO and wide and not args.shared)))

    router = None
    if args.router:
        from workloads import make_router_weight_bf16
        router = torch.from_numpy(make_router_weight_bf16(cfg).view(np.int16)).view(
            torch.bfloat16).to("cuda")

    shared = None
    if args.shared:
        from mxfp4_moe_expert_02_amd.layer import build_shared
        shared = build_shared(cfg)

    def step(i=0, events=None):
        w_gu, w_dn, w_sc = wsets[i % nsets]
        M.moe_mxfp4_forward_ex(layer.x, None if router is not None else layer.logits, cfg.k, w_gu,
                               w_dn, w_sc, layer.out, gemm_path=path, weight_layout=layout,
                               events=events, act_format=act, launch=launch, router_weight=router,
                               shared=None if shared is None else shared.tiles)

    M.moe_mxfp4_forward_ex(layer.x, None if router is not None else layer.logits, cfg.k, wgu, wdn,
                           scales, layer.out, gemm_path=path, weight_layout=layout, counts=counts,
                           act_format=act, router_weight=router,
                           shared=None if shared is None else shared.tiles)
    torch.cuda.synchronize()
    counts_np = counts.cpu().numpy()
    gu_bytes, dn_bytes = touched_bytes(counts_np, cfg.H, cfg.I)
    if shared is not None:  # MXFP8: one byte per weight plus one scale byte per 32
        gu_bytes += 2 * cfg.I * cfg.H + 2 * cfg.I * cfg.H // 32
        dn_bytes += cfg.H * cfg.I + cfg.H * cfg.I // 32
    total_bytes = gu_bytes + dn_bytes

    print(f"[bench] warmup {args.warmup}, {nsets} weight set(s)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back layers, bracketed by synchronisation
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr,
          flush=True)

    # the distribution of single steps: the same K steps with an event between
    # consecutive steps
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    sev[0].record(stream)
    for i in range(args.steps):
        step(i)
        sev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)])

    graph_ms = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(stream)
        with torch.cuda.stream(s_cap):
            step()  # warm the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s_cap):
                step()  # one weight set: the graph holds its pointers
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps

    # per-kernel times: the same K steps again with the library recording HIP
    # events on `stream` at its kernel boundaries
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events=ev[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, s in enumerate(STAGES)}
    dn_ms = stage_ms["down_combine"]

    # cold steps: a 1 GiB cache-allocating read evicts L2 and the 256 MiB
    # Infinity Cache without leaving dirty lines, and the stream is synced
    # before the step, whose stages are timed by the library's events; for
    # comparison, the earlier method: a 512 MiB write enqueued just before
    # the step
    cold = None
    if not args.no_cold:
        evict = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        sink = torch.empty(M.moe_probe_sink_words(), dtype=torch.int32, device="cuda")
        reps = min(args.steps, 30)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
               for _ in range(reps)]
        for r in range(reps):
            M.moe_probe_read_cached(evict, sink)
            torch.cuda.synchronize()
            step(r, events=cev[r])
            torch.cuda.synchronize()
        del evict, sink
        cold_ms = np.array([cev[r][0].elapsed_time(cev[r][-1]) for r in range(reps)])
        cold_stage = {s: float(np.median([cev[r][j].elapsed_time(cev[r][j + 1]) for r in range(reps)]))
                      for j, s in enumerate(STAGES)}
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        wf = []
        for r in range(reps):
            flush.fill_(r & 0xff)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(r)
            e1.record(stream)
            torch.cuda.synchronize()
            wf.append(e0.elapsed_time(e1))
        del flush
        cold = {"method": "1 GiB read with cache-allocating loads, stream sync, then one step "
                          "(stage events included)", "reps": reps,
                "us_per_layer": round(float(np.median(cold_ms)) * 1e3, 2),
                "p10_us": round(float(np.percentile(cold_ms, 10)) * 1e3, 2),
                "p90_us": round(float(np.percentile(cold_ms, 90)) * 1e3, 2),
                "GBps": round(total_bytes / (float(np.median(cold_ms)) * 1e-3) / 1e9, 2),
                "stage_us": {k: round(v * 1e3, 2) for k, v in cold_stage.items()},
                "write_flush_us_per_layer": round(float(np.median(wf)) * 1e3, 2)}

    probe_gbs = None if args.no_probe else probe_bandwidth(M, torch)
    # calibrated HBM bytes of the roofline kernel, taken on the plain layer
    # only: none apply with the router or shared-expert options
    traffic = None
    # the gate_up kernel the library runs for this layer (the wide bf16
    # kernels when the experts average >= 4 tokens each; the self-routed one
    # for at most 16 tokens unless the split launch is asked for)
    kname = ("mx8_gate_up_kernel" if mx8 else
             ("self_fused_kernel" if self_ok else "wide_fused_kernel" if wide else "mfma_fused_kernel")
             if fused else
             ("wide_queue_kernel" if wide else "mfma_queue_kernel") if queue else
             "self_gate_up_kernel" if self_routed else
             ("wide_gate_up_kernel" if wide else "mfma_gate_up_kernel") if path == M.MOE_PATH_MFMA
             else "gemv_gate_up_kernel")
    if shared is None and router is None and args.seed is None:
        traffic = measured_traffic(cfg.name, kname)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        M.moe_probe_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst
    us = ms_per_step * 1e3
    gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    gu_ms = stage_ms["gate_up"]
    kbytes = total_bytes if fused or queue else gu_bytes  # one launch moves every byte
    gu_gbs = kbytes / (gu_ms * 1e-3) / 1e9
    S = cfg.T * cfg.k
    S_all = S + (cfg.T if shared is not None else 0)  # rows through the FFN
    gu_flops = 2.0 * S_all * 2 * cfg.I * cfg.H
    dn_flops = 2.0 * S_all * cfg.H * cfg.I
    if mx8:
        gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma",
                "kernel": kname + " (fused gate+up MXFP4 x MXFP8 scaled-MFMA GEMM + SiLU*up)",
                "achieved": round(gu_tf, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tf / FP8_PEAK_TFLOPS, 4),
                "frac_of_fp4_peak": round(gu_tf / FP4_PEAK_TFLOPS, 4),
                "traffic": traffic,
                "algorithmic_flops_per_launch": gu_flops,
                "algorithmic_bytes_per_launch": int(gu_bytes)}
    else:
        roof = {"bound": "hbm",
                "kernel": kname + (" (the whole layer in one launch)" if fused else
                                   " (gate_up + SiLU*up and down, one workgroup per unit)" if queue
                                   else " (fused gate+up MXFP4 GEMM + SiLU*up)"),
                "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "frac_of_probe": round(gu_gbs / probe_gbs, 4) if probe_gbs else None,
                "algorithmic_bytes_per_launch": int(kbytes)}
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_layer": round(us, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "hbm_probe_GBps": round(probe_gbs, 1) if probe_gbs else None,
        "pct_of_probe": round(100 * gbs / probe_gbs, 2) if probe_gbs else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4xmxfp8->f32" if mx8 else "mxfp4xbf16->f32",
        "data": "synthetic",
        "config": dict(cfg.describe(), touched_experts=int((counts_np > 0).sum()),
                       max_tokens_per_expert=int(counts_np.max()),
                       touched_weight_bytes=int(total_bytes),
                       gemm_path="mfma" if path == M.MOE_PATH_MFMA else "gemv",
                       launch=("single_launch" if fused else "queue" if queue else
                               "self_routed" if self_routed else "split"),
                       router="computed in the layer from W_router [E,H] bf16" if router is not None
                       else "logits given",
                       weight_layout="tiles" if layout == M.MOE_LAYOUT_TILES else "rows",
                       shared_expert="MXFP8 gate_up [2I,H] + down [H,I], every token"
                       if shared is not None else "none",
                       activations="mxfp8" if mx8 else "bf16"),
        "tflops": {"layer": round((gu_flops + dn_flops) / (ms_per_step * 1e-3) / 1e12, 2),
                   "gate_up": round(gu_flops / (gu_ms * 1e-3) / 1e12, 2),
                   "down_combine": round(dn_flops / (dn_ms * 1e-3) / 1e12, 2)},
        "library": lib_path,
        "build": build_info(),
        "weight_sets": nsets,
        "step_us": {"median": round(float(np.median(step_ms)) * 1e3, 2),
                    "p10": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                    "p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2)},
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        # with the GEMMs in one launch its stage ("gate_up") moves every byte
        "stage_GBps": ({"gate_up_and_down": round(total_bytes / (stage_ms["gate_up"] * 1e-3) / 1e9, 1)}
                       if fused or queue else
                       {"gate_up": round(gu_bytes / (stage_ms["gate_up"] * 1e-3) / 1e9, 1),
                        "down_combine": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1)}),
        "roofline": roof,
    }
    if graph_ms is not None:
        result["graph_us_per_layer"] = round(graph_ms * 1e3, 2)
    if cold is not None:
        result["cold"] = cold
        result["cold_us_per_layer"] = cold["us_per_layer"]
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, total_bytes / 1e9, shared=shared is not None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
