"""Buffers and the four-call forward of the MoE layer on top of the binding.

This module only allocates device tensors (through torch) and calls the C
entry points in order: route -> dispatch -> expert GEMM -> combine. It holds
no arithmetic of its own.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B
from .workloads import Workload


def shape_of(w: Workload) -> B.MoeShape:
    return B.make_shape(w.T, w.d, w.E, w.k, w.f, w.e_lo, w.local_hi, w.capacity,
                        B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32)


@dataclass
class Buffers:
    shape: B.MoeShape
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    logits: Optional[torch.Tensor]
    prob_sum: Optional[torch.Tensor]
    counts: torch.Tensor
    offsets: torch.Tensor
    slot: torch.Tensor
    row_src: torch.Tensor
    row_gate: torch.Tensor
    x_perm: Optional[torch.Tensor]   # None: the expert GEMM gathers x through row_src
    y_perm: torch.Tensor
    act_save: Optional[torch.Tensor]
    y: torch.Tensor
    dropped: torch.Tensor
    aux: torch.Tensor
    ws: torch.Tensor


def alloc(shape: B.MoeShape, lora_r: int = 0, logits: bool = False, prob: bool = False,
          act_save: bool = False, x_perm: bool = False, device: str = "cuda") -> Buffers:
    T, d, E, k, f = shape.T, shape.d, shape.E, shape.k, shape.f
    L = shape.e_hi - shape.e_lo
    rmax = B.moe_max_rows(shape)
    if rmax < 0:
        raise ValueError("invalid shape")
    dt = torch.bfloat16 if shape.dtype == B.MOE_BF16 else torch.float32
    kw = {"device": device}
    ws_bytes = B.moe_workspace_bytes(shape, lora_r)
    return Buffers(
        shape=shape,
        topk_idx=torch.empty((T, k), dtype=torch.int32, **kw),
        topk_gate=torch.empty((T, k), dtype=torch.float32, **kw),
        logits=torch.empty((T, E), dtype=torch.float32, **kw) if logits else None,
        prob_sum=torch.empty((E,), dtype=torch.float32, **kw) if prob else None,
        counts=torch.empty((E,), dtype=torch.int32, **kw),
        offsets=torch.empty((L + 1,), dtype=torch.int32, **kw),
        slot=torch.empty((T, k), dtype=torch.int32, **kw),
        row_src=torch.empty((max(rmax, 1),), dtype=torch.int32, **kw),
        row_gate=torch.empty((max(rmax, 1),), dtype=torch.float32, **kw),
        x_perm=torch.empty((max(rmax, 1), d), dtype=dt, **kw) if x_perm else None,
        y_perm=torch.empty((max(rmax, 1), d), dtype=dt, **kw),
        act_save=torch.empty((max(rmax, 1), 3 * f), dtype=dt, **kw) if act_save else None,
        y=torch.empty((T, d), dtype=dt, **kw),
        dropped=torch.zeros((1,), dtype=torch.int32, **kw),
        aux=torch.zeros((2,), dtype=torch.float32, **kw),
        ws=torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, **kw),
    )


def x_rows(b: Buffers, x):
    """(rows, row index) the expert GEMM reads: the gathered copy, or x itself
    through row_src."""
    return (b.x_perm, None) if b.x_perm is not None else (x, b.row_src)


def pack_weights(shape: B.MoeShape, w_gate, w_up, w_down, stream=None):
    """Packed copies (gate/up, down) of frozen expert weights (bitwise equal values)."""
    L, f, d = w_gate.shape
    gu = torch.empty((L, 2 * f, d), dtype=w_gate.dtype, device=w_gate.device)
    dn = torch.empty_like(w_down)
    B.moe_pack_expert_weights(shape, w_gate, w_up, w_down, gu, dn, stream)
    return gu, dn


@dataclass
class Variant:
    """Routing variants of the forward: remapping (alt [T,k] int32 and
    moved [1] int32 buffers) or a latent router (w_latent [d_c,d] and the
    z [T,d_c] buffer)."""
    alt: Optional[torch.Tensor] = None
    moved: Optional[torch.Tensor] = None
    w_latent: Optional[torch.Tensor] = None
    z: Optional[torch.Tensor] = None


def variant_buffers(w: Workload, dev, device: str = "cuda") -> Optional[Variant]:
    if w.remap:
        return Variant(alt=torch.empty((w.T, w.k), dtype=torch.int32, device=device),
                       moved=torch.zeros((1,), dtype=torch.int32, device=device))
    if w.latent_dc > 0:
        return Variant(w_latent=dev["w_latent"],
                       z=torch.empty((w.T, w.latent_dc), dtype=dev["x"].dtype, device=device))
    return None


def forward(b: Buffers, x, w_router, bias, w_gate, w_up, w_down, lora=None, stream=None,
            packed=None, variant: Optional[Variant] = None, fused_route: bool = True) -> None:
    """route -> dispatch -> expert GEMM -> combine; results stay in ``b``.
    packed: (gu_packed, down_packed) from pack_weights, used instead of the
    row-major expert weights. variant: remapped dispatch or latent routing.
    fused_route: the plain routing and dispatch as one call
    (moe_route_dispatch) instead of moe_route + moe_dispatch."""
    s = b.shape
    v = variant or Variant()
    if fused_route and v.w_latent is None and v.alt is None:
        B.moe_route_dispatch(s, x, w_router, bias, b.topk_idx, b.topk_gate, b.logits, b.prob_sum, b.counts,
                             b.offsets, b.slot, b.row_src, b.row_gate, b.x_perm, b.dropped, b.ws, stream)
    else:
        if v.w_latent is not None:
            B.moe_route_latent(s, v.z.shape[1], x, v.w_latent, w_router, bias, v.z, b.topk_idx, b.topk_gate,
                               b.logits, b.prob_sum, b.ws, stream)
        elif v.alt is not None:
            B.moe_route_alt(s, x, w_router, bias, b.topk_idx, b.topk_gate, v.alt, b.logits, b.prob_sum, b.ws,
                            stream)
        else:
            B.moe_route(s, x, w_router, bias, b.topk_idx, b.topk_gate, b.logits, b.prob_sum, b.ws, stream)
        if v.alt is not None:
            B.moe_dispatch_remap(s, b.topk_idx, b.topk_gate, v.alt, x, b.counts, b.offsets, b.slot, b.row_src,
                                 b.row_gate, b.x_perm, v.moved, b.dropped, b.ws, stream)
        else:
            B.moe_dispatch(s, b.topk_idx, b.topk_gate, x, b.counts, b.offsets, b.slot, b.row_src,
                           b.row_gate, b.x_perm, b.dropped, b.ws, stream)
    xr, src = x_rows(b, x)
    if packed is not None:
        B.moe_expert_gemm_packed(s, xr, src, b.offsets, packed[0], packed[1], lora, b.act_save,
                                 b.y_perm, b.ws, stream)
    else:
        B.moe_expert_gemm(s, xr, src, b.offsets, w_gate, w_up, w_down, lora, b.act_save, b.y_perm,
                          b.ws, stream)
    B.moe_combine(s, b.y_perm, b.slot, b.topk_gate, b.y, stream)


def capture(fn):
    """Record the kernels fn() enqueues (through the C entry points, on
    torch's current stream) into one HIP graph and return it; replay() then
    re-runs exactly those launches with the same pointers and sizes. The
    library enqueues no memset or allocation inside its entry points, so the
    whole forward is capturable."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    return g
