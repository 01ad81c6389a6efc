"""Seeded synthetic inputs for the sparse MoE layer (896 routed experts, top-16).

This module is the only code shared by the HIP path's callers (tests, bench)
and the CPU oracle's callers. It draws random tensors and nothing else: no
routing, no softmax, no expert arithmetic lives here.

Workloads (the shapes and distributions the MoE pages describe):

* ``tiny_f32``        T=64, d=128, E=16, k=4, f=64, fp32 (parity case)
* ``full_router``     T=4096, d=2048, E=896, k=16, f=256, bf16, all experts local
* ``ep64_rank``       T=16384, d=4096, E=896, k=16, f=1024, bf16, local experts 0..13
                      (896 experts over an expert-parallel group of 64 ranks leaves
                      14 per rank: "Trillion-Parameter MoE Model Training Adaptation:
                      Full-Stack Optimization Practices", §4.1)
* ``skewed_capacity`` T=8192, d=2048, E=896, k=16, f=256, bf16, Zipf(1.2) logit bias,
                      capacity factor 1.25 -> 183 rows per expert
                      ("Day-Level Adaptation and LoRA Fine-Tuning of Ultra-Large-Scale
                      Sparse MoE Models", §3.2 sets expert_capacity=1.25)
* ``lora_step``       ``ep64_rank`` plus rank-16 LoRA (alpha=32) on the up and down
                      projections and an upstream gradient dY ("Adapting Trillion-
                      Parameter MoE Models for LoRA Fine-Tuning: A Full-Stack
                      Engineering Guide", §3 gives r=16, alpha=32)

Distributions: x ~ N(0,1); router, gate and up weights ~ N(0, 1/d); down weights
~ N(0, 1/f); LoRA A ~ N(0, 1/d) (d = hidden size, for both adapters); LoRA B = 0
(``lora_b="zero"``) or ~ N(0, 1e-3) (variance; ``lora_b="normal"``); dY ~ N(0,1).
bf16 workloads are drawn in float32 and rounded to bfloat16 (round to nearest
even); the tiny workload stays float32.

Latent-space router variant (``latent_dc`` > 0): tokens are projected to d_c
dimensions before routing; w_latent [d_c, d] ~ N(0, 1/d) and the router
weight becomes [E, d_c] ~ N(0, 1/d_c).

Seeding: ``SeedSequence(seed).spawn(12)`` gives one child per tensor in the fixed
order [x, w_router, w_gate, w_up, w_down, bias_perm, a_up, b_up, a_down, b_down, dy,
w_latent] (the first eleven are the children ``spawn(11)`` gives).
Each child is split further into independent per-chunk streams (one per expert for
expert tensors, one per 1024 rows for token tensors), so the result does not depend
on how many threads draw it.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

_TENSOR_ORDER = ("x", "w_router", "w_gate", "w_up", "w_down", "bias_perm",
                 "a_up", "b_up", "a_down", "b_down", "dy", "w_latent")
_ROWS_PER_CHUNK = 1024


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    d: int                 # hidden size
    E: int                 # routed experts (router width)
    k: int                 # experts per token
    f: int                 # expert FFN width
    e_lo: int = 0          # first local expert
    e_hi: int = -1         # one past the last local expert (-1 -> E)
    capacity: int = 0      # rows kept per expert, 0 = unlimited
    dtype: str = "bf16"    # "bf16" or "f32"
    zipf_s: float = 0.0    # Zipf exponent of the per-expert logit bias, 0 = no bias
    lora_r: int = 0        # LoRA rank, 0 = no adapters
    lora_alpha: float = 0.0
    lora_b: str = "normal"  # "zero" or "normal"
    aux_coef: float = 0.0  # load-balance loss coefficient (0 = not requested)
    latent_dc: int = 0     # latent routing width, 0 = the router reads x directly
    remap: bool = False    # overflowing assignments remapped to the next-ranked experts

    @property
    def local_hi(self) -> int:
        return self.E if self.e_hi < 0 else self.e_hi

    @property
    def L(self) -> int:
        return self.local_hi - self.e_lo

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", T=64, d=128, E=16, k=4, f=64, dtype="f32"),
    "full_router": Workload("full_router", T=4096, d=2048, E=896, k=16, f=256),
    "ep64_rank": Workload("ep64_rank", T=16384, d=4096, E=896, k=16, f=1024,
                          e_lo=0, e_hi=14),
    # capacity = ceil(1.25 * 8192 * 16 / 896) = ceil(182.857...) = 183
    "skewed_capacity": Workload("skewed_capacity", T=8192, d=2048, E=896, k=16, f=256,
                                capacity=183, zipf_s=1.2),
    "lora_step": Workload("lora_step", T=16384, d=4096, E=896, k=16, f=1024,
                          e_lo=0, e_hi=14, lora_r=16, lora_alpha=32.0,
                          lora_b="normal", aux_coef=0.01),
    # the skewed workload with overflow remapped instead of dropped
    "skewed_remap": Workload("skewed_remap", T=8192, d=2048, E=896, k=16, f=256,
                             capacity=183, zipf_s=1.2, remap=True),
    # the full-router workload routed from a d/8-dimensional projection
    "latent_router": Workload("latent_router", T=4096, d=2048, E=896, k=16, f=256,
                              latent_dc=256),
}


def _children(seed: int) -> Dict[str, np.random.SeedSequence]:
    kids = np.random.SeedSequence(seed).spawn(len(_TENSOR_ORDER))
    return dict(zip(_TENSOR_ORDER, kids))


def _normal(ss: np.random.SeedSequence, shape, std: float, chunk_rows: int,
            pool: ThreadPoolExecutor) -> np.ndarray:
    """float32 N(0, std^2) of ``shape``, drawn in independent chunks along axis 0."""
    out = np.empty(shape, dtype=np.float32)
    n0 = shape[0]
    nchunks = max(1, -(-n0 // chunk_rows))
    streams = ss.spawn(nchunks)

    def fill(c: int) -> None:
        lo, hi = c * chunk_rows, min(n0, (c + 1) * chunk_rows)
        g = np.random.Generator(np.random.PCG64(streams[c]))
        blk = out[lo:hi]
        g.standard_normal(out=blk, dtype=np.float32)
        blk *= np.float32(std)

    list(pool.map(fill, range(nchunks)))
    return out


def _to_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def generate(w: Workload, seed: int = 0, threads: Optional[int] = None,
             with_lora: bool = True, with_dy: bool = True) -> Dict[str, torch.Tensor]:
    """Draw every input of workload ``w`` as CPU tensors.

    Keys: x [T,d], w_router [E,d] ([E,d_c] with latent routing, plus
    w_latent [d_c,d]), bias [E] (fp32, only when zipf_s > 0),
    w_gate [L,f,d], w_up [L,f,d], w_down [L,d,f], for LoRA workloads
    a_up [L,r,d], b_up [L,f,r], a_down [L,r,f], b_down [L,d,r], and with
    with_dy the upstream gradient dy [T,d] of the backward.
    Expert tensors hold only the local experts e_lo..local_hi-1.
    """
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    ss = _children(seed)
    L, d, f, E, T = w.L, w.d, w.f, w.E, w.T
    out: Dict[str, torch.Tensor] = {}
    with ThreadPoolExecutor(max_workers=threads) as pool:
        out["x"] = _to_tensor(_normal(ss["x"], (T, d), 1.0, _ROWS_PER_CHUNK, pool), w.dtype)
        dr = w.latent_dc if w.latent_dc > 0 else d  # the router's input width
        out["w_router"] = _to_tensor(
            _normal(ss["w_router"], (E, dr), 1.0 / math.sqrt(dr), _ROWS_PER_CHUNK, pool), w.dtype)
        if w.latent_dc > 0:
            out["w_latent"] = _to_tensor(
                _normal(ss["w_latent"], (w.latent_dc, d), 1.0 / math.sqrt(d), _ROWS_PER_CHUNK, pool), w.dtype)
        out["w_gate"] = _to_tensor(_normal(ss["w_gate"], (L, f, d), 1.0 / math.sqrt(d), 1, pool), w.dtype)
        out["w_up"] = _to_tensor(_normal(ss["w_up"], (L, f, d), 1.0 / math.sqrt(d), 1, pool), w.dtype)
        out["w_down"] = _to_tensor(_normal(ss["w_down"], (L, d, f), 1.0 / math.sqrt(f), 1, pool), w.dtype)
        if w.zipf_s > 0:
            # Zipf(s) popularity over a seeded ranking of the experts, as a logit
            # bias: expert with rank r (1 = most popular) gets -s*ln(r).
            perm = np.random.Generator(np.random.PCG64(ss["bias_perm"])).permutation(E)
            rank = np.empty(E, dtype=np.float64)
            rank[perm] = np.arange(1, E + 1, dtype=np.float64)
            out["bias"] = torch.from_numpy((-w.zipf_s * np.log(rank)).astype(np.float32))
        if w.lora_r > 0 and with_lora:
            r = w.lora_r
            sa = 1.0 / math.sqrt(d)
            sb = math.sqrt(1e-3)
            out["a_up"] = _to_tensor(_normal(ss["a_up"], (L, r, d), sa, 1, pool), w.dtype)
            out["a_down"] = _to_tensor(_normal(ss["a_down"], (L, r, f), sa, 1, pool), w.dtype)
            if w.lora_b == "zero":
                out["b_up"] = _to_tensor(np.zeros((L, f, r), np.float32), w.dtype)
                out["b_down"] = _to_tensor(np.zeros((L, d, r), np.float32), w.dtype)
            else:
                out["b_up"] = _to_tensor(_normal(ss["b_up"], (L, f, r), sb, 1, pool), w.dtype)
                out["b_down"] = _to_tensor(_normal(ss["b_down"], (L, d, r), sb, 1, pool), w.dtype)
        if with_dy:
            out["dy"] = _to_tensor(_normal(ss["dy"], (T, d), 1.0, _ROWS_PER_CHUNK, pool), w.dtype)
    return out


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact float64 copy of a CPU tensor (bf16 and fp32 widen without rounding)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
