"""Seeded synthetic workloads for the MXFP4 MoE expert layer.

The pages describe a trillion-parameter MoE whose expert weights are stored in
MXFP4 and which is decoded with block speculative decoding of 8 draft tokens
(bjdmk.com.cn news page, section on the co-design: FP4 experts, block size 8).
They publish no trained weights that are usable here and no per-layer inputs,
so every input below is synthetic, seeded, and shaped like one MoE layer of
such a model at a verify step (8 drafts + 1) or a prefill chunk.

Recipe (all draws from numpy's PCG64 ``default_rng`` seeded by a
``SeedSequence([seed, stream, index])``):

* x: N(0, 1) float32, rounded to bfloat16 (round-to-nearest-even, by torch).
* router logits: N(0, 1) float32; the batched-verify workload adds one N(0, 0.5)
  bias per expert; the skewed workload uses a Gumbel-top-k construction whose
  expert popularity follows Zipf(s = 1.1) (see ``make_logits``).
* expert weights: N(0, 0.02) float32, one independent stream per
  (expert, matrix).  gate_up is [2I, H] (rows 0..I-1 gate, I..2I-1 up),
  down is [H, I].  Quantisation to MXFP4 is *not* done here: each side
  (the HIP library and the oracle) encodes these float32 values itself.
* shared expert weights (optional): the same shapes and distribution from
  streams of their own; each side encodes them to MXFP8 itself.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Iterator, Sequence

import numpy as np

# stream tags inside a SeedSequence
_S_X, _S_LOGITS, _S_BIAS, _S_ZIPF_RANK, _S_GATE_UP, _S_DOWN = 1, 2, 3, 4, 10, 11
_S_ROUTER = 12
_S_SHARED_GATE_UP, _S_SHARED_DOWN = 13, 14

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Config:
    key: str          # short key, c1..c5
    name: str         # workload name
    T: int            # tokens
    E: int            # resident experts
    H: int            # hidden size
    I: int            # expert intermediate size
    k: int            # top-k
    logits: str       # "normal" | "normal_bias" | "zipf"
    act: str          # "bf16" | "mxfp8"  (activation format fed to the GEMMs)
    seed: int         # base seed

    @property
    def assignments(self) -> int:
        return self.T * self.k

    def describe(self) -> dict:
        return {"workload": self.name, "tokens": self.T, "experts": self.E,
                "hidden": self.H, "intermediate": self.I, "top_k": self.k,
                "router": self.logits, "activations": self.act, "seed": self.seed}


CONFIGS = {
    # tiny layer the oracle finishes in well under a second
    "c1": Config("c1", "tiny_moe_t9_e8_h256_i128_k2", 9, 8, 256, 128, 2, "normal", "bf16", 1001),
    # one sequence verify step: 8 drafts + 1
    "c2": Config("c2", "verify_t9_e64_h6144_i2048_k8", 9, 64, 6144, 2048, 8, "normal", "bf16", 1002),
    # 8 sequences x 9 tokens, per-expert router bias makes the load uneven
    "c3": Config("c3", "batched_verify_t72_e128_h7168_i2048_k8", 72, 128, 7168, 2048, 8,
                 "normal_bias", "bf16", 1003),
    # 32 sequences x 9 tokens, Zipf(1.1) expert popularity.  The seed is the
    # first one from 1004 up whose routing leaves at least one expert empty and
    # gives at least one expert more than 60 tokens (checked by a CPU test).
    "c4": Config("c4", "zipf_verify_t288_e128_h7168_i2048_k8", 288, 128, 7168, 2048, 8,
                 "zipf", "bf16", 1005),
    # prefill chunk, activations quantised to MXFP8 on the fly
    "c5": Config("c5", "prefill_t4096_e128_h7168_i2048_k8", 4096, 128, 7168, 2048, 8,
                 "normal", "mxfp8", 1005),
}


def get_config(key: str, **overrides) -> Config:
    cfg = CONFIGS[key]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, index]))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 values (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_x_bf16(cfg: Config, seed: int | None = None) -> np.ndarray:
    """x [T, H] as bfloat16 bit patterns (uint16), from N(0, 1)."""
    import torch  # conversion only; torch rounds float32 -> bfloat16 to nearest even
    seed = cfg.seed if seed is None else seed
    x = _rng(seed, _S_X).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_logits(cfg: Config, seed: int | None = None) -> np.ndarray:
    """Router logits [T, E] float32.

    * ``normal``: iid N(0, 1).
    * ``normal_bias``: iid N(0, 1) plus one N(0, 0.5) bias per expert, added
      here by the harness (the layer only ever sees logits).
    * ``zipf``: logit[t, e] = -s * log(rank_e) + Gumbel(0, 1), s = 1.1, with
      rank a seeded permutation of 1..E.  Taking the k largest of these is
      sampling k experts without replacement with probability proportional
      to rank^-s (the Gumbel-top-k identity), so expert popularity is Zipf.
    """
    seed = cfg.seed if seed is None else seed
    shape = (cfg.T, cfg.E)
    if cfg.logits == "normal":
        return _rng(seed, _S_LOGITS).standard_normal(shape, dtype=np.float32)
    if cfg.logits == "normal_bias":
        z = _rng(seed, _S_LOGITS).standard_normal(shape, dtype=np.float32)
        bias = (_rng(seed, _S_BIAS).standard_normal(cfg.E, dtype=np.float32)
                * np.float32(0.5))
        return (z + bias[None, :]).astype(np.float32)
    if cfg.logits == "zipf":
        rank = _rng(seed, _S_ZIPF_RANK).permutation(cfg.E).astype(np.float64) + 1.0
        g = _rng(seed, _S_LOGITS).gumbel(size=shape)
        return (-1.1 * np.log(rank)[None, :] + g).astype(np.float32)
    raise ValueError(f"unknown logits recipe {cfg.logits!r}")


def make_router_weight_bf16(cfg: Config, seed: int | None = None) -> np.ndarray:
    """Router weight [E, H] as bfloat16 bit patterns (uint16), from
    N(0, 1/sqrt(H)): with x ~ N(0, 1) the logits x . w_e are then about
    N(0, 1), the configs' logit distribution."""
    import torch  # conversion only; torch rounds float32 -> bfloat16 to nearest even
    seed = cfg.seed if seed is None else seed
    w = _rng(seed, _S_ROUTER).standard_normal((cfg.E, cfg.H), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(cfg.H))
    return torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def weight_shape(cfg: Config, which: str) -> tuple[int, int]:
    if which == "gate_up":
        return (2 * cfg.I, cfg.H)
    if which == "down":
        return (cfg.H, cfg.I)
    raise ValueError(which)


def make_weight_fp32(cfg: Config, which: str, expert: int,
                     seed: int | None = None) -> np.ndarray:
    """One expert's float32 weight matrix, N(0, 0.02), before any encoding."""
    seed = cfg.seed if seed is None else seed
    stream = _S_GATE_UP if which == "gate_up" else _S_DOWN
    w = _rng(seed, stream, expert).standard_normal(weight_shape(cfg, which), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def make_shared_weight_fp32(cfg: Config, which: str, seed: int | None = None) -> np.ndarray:
    """The shared expert's float32 matrix (gate_up [2I, H] or down [H, I]),
    N(0, 0.02), before any encoding."""
    seed = cfg.seed if seed is None else seed
    stream = _S_SHARED_GATE_UP if which == "gate_up" else _S_SHARED_DOWN
    w = _rng(seed, stream).standard_normal(weight_shape(cfg, which), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_weights_fp32(cfg: Config, which: str, experts: Sequence[int] | None = None,
                      seed: int | None = None, workers: int | None = None,
                      ) -> Iterator[tuple[int, np.ndarray]]:
    """Yield (expert, float32 matrix) in expert order, generated on a thread pool.

    numpy releases the GIL while filling arrays, so the pool scales with
    cores.  At most ``2 * workers`` matrices are alive at once.
    """
    experts = list(range(cfg.E)) if experts is None else list(experts)
    workers = workers or default_workers()
    with ThreadPoolExecutor(workers) as ex:
        pending = []
        it: Iterable[int] = iter(experts)
        for e in it:
            pending.append((e, ex.submit(make_weight_fp32, cfg, which, e, seed)))
            if len(pending) >= 2 * workers:
                e0, f0 = pending.pop(0)
                yield e0, f0.result()
        for e0, f0 in pending:
            yield e0, f0.result()
