"""ctypes binding of libmoe_mi355x.so, one Python function per C entry point.

Argument marshalling only: each function checks that the tensors it is given
are contiguous, on the GPU and of the expected dtype, then passes their device
pointers and torch's current HIP stream to the C function of the same name.
Every computation runs in the library's HIP kernels; if the library is not
built, loading fails with an error instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

KERNELS = ["router_gemm", "topk", "prob_reduce", "hist", "scan", "scatter", "capacity",
           "gather", "tiles", "gate_up", "down", "combine", "aux", "lora_proj", "lora_dh",
           "lora_grad", "gate_bwd", "expert_dgu", "expert_dx", "unpermute", "router_bwd"]

EXPORTED = ["moe_workspace_bytes", "moe_max_rows", "moe_last_error", "moe_route", "moe_route_alt",
            "moe_route_latent", "moe_dispatch_remap", "moe_route_dispatch",
            "moe_dispatch", "moe_dispatch_noalloc", "moe_expert_gemm", "moe_pack_expert_weights", "moe_expert_gemm_packed",
            "moe_combine", "moe_aux_loss", "moe_lora_bwd", "moe_lora_bwd_packed", "moe_gate_bwd", "moe_expert_bwd",
            "moe_router_bwd", "moe_pack_backward_weights", "moe_expert_bwd_packed", "moe_pack_router_bwd",
            "moe_router_bwd_packed", "moe_router_bwd_unpermute_packed", "moe_timing_enable",
            "moe_timing_read"]


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "E", "k", "f", "e_lo", "e_hi", "capacity", "dtype")]


class MoeLora(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("alpha", ctypes.c_float), ("a_up", ctypes.c_void_p),
                ("b_up", ctypes.c_void_p), ("a_down", ctypes.c_void_p), ("b_down", ctypes.c_void_p),
                ("z_save", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mixture_experts_top_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    shp, lor = ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLora)
    L.moe_workspace_bytes.argtypes, L.moe_workspace_bytes.restype = [shp, i32], sz
    L.moe_max_rows.argtypes, L.moe_max_rows.restype = [shp], i64
    L.moe_last_error.argtypes, L.moe_last_error.restype = [], ctypes.c_char_p
    L.moe_route.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_route_dispatch.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_alt.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_latent.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_remap.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_gemm.argtypes = [shp, vp, vp, vp, vp, vp, vp, lor, vp, vp, vp, sz, vp]
    L.moe_pack_expert_weights.argtypes = [shp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_gemm_packed.argtypes = [shp, vp, vp, vp, vp, vp, lor, vp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [shp, vp, vp, vp, vp, vp]
    L.moe_aux_loss.argtypes = [shp, vp, vp, f32, vp, vp]
    L.moe_lora_bwd.argtypes = [shp, lor, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_lora_bwd_packed.argtypes = [shp, lor, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_gate_bwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp]
    L.moe_expert_bwd.argtypes = [shp, lor, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_router_bwd.argtypes = [shp, vp, vp, vp, vp, sz, vp]
    L.moe_pack_backward_weights.argtypes = [shp, vp, vp, vp, vp, vp, vp]
    L.moe_pack_router_bwd.argtypes = [shp, vp, vp, vp]
    L.moe_router_bwd_packed.argtypes = [shp, vp, vp, vp, vp, sz, vp]
    L.moe_router_bwd_unpermute_packed.argtypes = [shp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_bwd_packed.argtypes = [shp, lor, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_timing_enable.argtypes = [i32]
    L.moe_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for fn in ("moe_route", "moe_dispatch", "moe_expert_gemm", "moe_pack_expert_weights",
               "moe_expert_gemm_packed", "moe_combine", "moe_aux_loss", "moe_lora_bwd", "moe_lora_bwd_packed",
               "moe_gate_bwd", "moe_expert_bwd", "moe_router_bwd", "moe_pack_backward_weights",
               "moe_expert_bwd_packed", "moe_pack_router_bwd", "moe_router_bwd_packed",
               "moe_router_bwd_unpermute_packed", "moe_timing_enable", "moe_timing_read"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def make_shape(T, d, E, k, f, e_lo=0, e_hi=None, capacity=0, dtype=MOE_BF16) -> MoeShape:
    return MoeShape(T, d, E, k, f, e_lo, E if e_hi is None else e_hi, capacity, dtype)


def make_lora(r: int, alpha: float, a_up, b_up, a_down, b_down, z_save=None) -> MoeLora:
    """z_save: optional [2, Rmax, r] float32 buffer for the row projections kept
    from the forward to the backward."""
    for t in (a_up, b_up, a_down, b_down):
        _dev(t, torch.bfloat16)
    return MoeLora(r, alpha, a_up.data_ptr(), b_up.data_ptr(), a_down.data_ptr(), b_down.data_ptr(),
                   _dev(z_save, torch.float32))


def _dev(t: Optional[torch.Tensor], dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _fdt(shape: MoeShape):
    return torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def moe_workspace_bytes(shape: MoeShape, lora_r: int = 0) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape), lora_r))


def moe_max_rows(shape: MoeShape) -> int:
    return int(lib().moe_max_rows(ctypes.byref(shape)))


def moe_route(shape, x, w_router, bias, topk_idx, topk_gate, logits, prob_sum, ws, stream=None):
    dt = _fdt(shape)
    _check(lib().moe_route(ctypes.byref(shape), _dev(x, dt), _dev(w_router, dt),
                           _dev(bias, torch.float32), _dev(topk_idx, torch.int32),
                           _dev(topk_gate, torch.float32), _dev(logits, torch.float32),
                           _dev(prob_sum, torch.float32), _dev(ws, torch.uint8), ws.numel(),
                           _stream(stream)))


def moe_dispatch(shape, topk_idx, topk_gate, x, counts, offsets, slot, row_src, row_gate, x_perm,
                 dropped, ws, stream=None):
    dt, i32 = _fdt(shape), torch.int32
    _check(lib().moe_dispatch(ctypes.byref(shape), _dev(topk_idx, i32), _dev(topk_gate, torch.float32),
                              _dev(x, dt), _dev(counts, i32), _dev(offsets, i32), _dev(slot, i32),
                              _dev(row_src, i32), _dev(row_gate, torch.float32), _dev(x_perm, dt),
                              _dev(dropped, i32), _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_route_dispatch(shape, x, w_router, bias, topk_idx, topk_gate, logits, prob_sum, counts, offsets, slot,
                       row_src, row_gate, x_perm, dropped, ws, stream=None):
    """moe_route then moe_dispatch in one call (fewer kernels, same results)."""
    dt, i32, f32 = _fdt(shape), torch.int32, torch.float32
    _check(lib().moe_route_dispatch(ctypes.byref(shape), _dev(x, dt), _dev(w_router, dt), _dev(bias, f32),
                                    _dev(topk_idx, i32), _dev(topk_gate, f32), _dev(logits, f32),
                                    _dev(prob_sum, f32), _dev(counts, i32), _dev(offsets, i32), _dev(slot, i32),
                                    _dev(row_src, i32), _dev(row_gate, f32), _dev(x_perm, dt), _dev(dropped, i32),
                                    _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_route_alt(shape, x, w_router, bias, topk_idx, topk_gate, alt_idx, logits, prob_sum, ws, stream=None):
    """moe_route plus alt_idx [T, k]: the experts ranked k .. 2k-1."""
    dt = _fdt(shape)
    _check(lib().moe_route_alt(ctypes.byref(shape), _dev(x, dt), _dev(w_router, dt), _dev(bias, torch.float32),
                               _dev(topk_idx, torch.int32), _dev(topk_gate, torch.float32),
                               _dev(alt_idx, torch.int32), _dev(logits, torch.float32),
                               _dev(prob_sum, torch.float32), _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_route_latent(shape, d_c, x, w_latent, w_router, bias, z, topk_idx, topk_gate, logits, prob_sum, ws,
                     stream=None):
    """Routing from z = x w_latent^T ([T, d_c], written to z)."""
    dt = _fdt(shape)
    _check(lib().moe_route_latent(ctypes.byref(shape), int(d_c), _dev(x, dt), _dev(w_latent, dt),
                                  _dev(w_router, dt), _dev(bias, torch.float32), _dev(z, dt),
                                  _dev(topk_idx, torch.int32), _dev(topk_gate, torch.float32),
                                  _dev(logits, torch.float32), _dev(prob_sum, torch.float32),
                                  _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_dispatch_remap(shape, topk_idx, topk_gate, alt_idx, x, counts, offsets, slot, row_src, row_gate,
                       x_perm, moved, dropped, ws, stream=None):
    """Dispatch with overflowing assignments moved to the alternates."""
    dt, i32 = _fdt(shape), torch.int32
    _check(lib().moe_dispatch_remap(ctypes.byref(shape), _dev(topk_idx, i32), _dev(topk_gate, torch.float32),
                                    _dev(alt_idx, i32), _dev(x, dt), _dev(counts, i32), _dev(offsets, i32),
                                    _dev(slot, i32), _dev(row_src, i32), _dev(row_gate, torch.float32),
                                    _dev(x_perm, dt), _dev(moved, i32), _dev(dropped, i32),
                                    _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_dispatch_noalloc(shape, topk_idx, topk_gate, x, counts, offsets, slot, row_src, row_gate, x_perm,
                         dropped, stream=None):
    """moe_dispatch on the library's own scratch (no workspace argument)."""
    dt, i32 = _fdt(shape), torch.int32
    _check(lib().moe_dispatch_noalloc(ctypes.byref(shape), _dev(topk_idx, i32), _dev(topk_gate, torch.float32),
                                      _dev(x, dt), _dev(counts, i32), _dev(offsets, i32), _dev(slot, i32),
                                      _dev(row_src, i32), _dev(row_gate, torch.float32), _dev(x_perm, dt),
                                      _dev(dropped, i32), _stream(stream)))


def moe_expert_gemm(shape, x, row_src, offsets, w_gate, w_up, w_down, lora, act_save, y_perm, ws,
                    stream=None):
    """x: tokens [T, d] read through row_src, or x_perm [Rmax, d] with row_src=None."""
    dt = _fdt(shape)
    _check(lib().moe_expert_gemm(ctypes.byref(shape), _dev(x, dt), _dev(row_src, torch.int32),
                                 _dev(offsets, torch.int32), _dev(w_gate, dt), _dev(w_up, dt),
                                 _dev(w_down, dt), ctypes.byref(lora) if lora is not None else None,
                                 _dev(act_save, dt), _dev(y_perm, dt), _dev(ws, torch.uint8),
                                 ws.numel(), _stream(stream)))


def moe_pack_expert_weights(shape, w_gate, w_up, w_down, gu_packed, down_packed, stream=None):
    bf = torch.bfloat16
    _check(lib().moe_pack_expert_weights(ctypes.byref(shape), _dev(w_gate, bf), _dev(w_up, bf),
                                         _dev(w_down, bf), _dev(gu_packed, bf), _dev(down_packed, bf),
                                         _stream(stream)))


def moe_expert_gemm_packed(shape, x, row_src, offsets, gu_packed, down_packed, lora, act_save, y_perm,
                           ws, stream=None):
    bf = torch.bfloat16
    _check(lib().moe_expert_gemm_packed(ctypes.byref(shape), _dev(x, bf), _dev(row_src, torch.int32),
                                        _dev(offsets, torch.int32), _dev(gu_packed, bf),
                                        _dev(down_packed, bf),
                                        ctypes.byref(lora) if lora is not None else None,
                                        _dev(act_save, bf), _dev(y_perm, bf), _dev(ws, torch.uint8),
                                        ws.numel(), _stream(stream)))


def moe_combine(shape, y_perm, slot, topk_gate, y, stream=None):
    dt = _fdt(shape)
    _check(lib().moe_combine(ctypes.byref(shape), _dev(y_perm, dt), _dev(slot, torch.int32),
                             _dev(topk_gate, torch.float32), _dev(y, dt), _stream(stream)))


def moe_aux_loss(shape, counts, prob_sum, coef, out, stream=None):
    _check(lib().moe_aux_loss(ctypes.byref(shape), _dev(counts, torch.int32),
                              _dev(prob_sum, torch.float32), float(coef), _dev(out, torch.float32),
                              _stream(stream)))


def moe_lora_bwd_packed(shape, lora, dy, offsets, row_src, row_gate, x, x_src, act_save, dgu_packed, da_up,
                        db_up, da_down, db_down, ws, stream=None):
    """moe_lora_bwd with W_d^T packed by moe_pack_backward_weights (dgu_packed)."""
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check(lib().moe_lora_bwd_packed(ctypes.byref(shape), ctypes.byref(lora), _dev(dy, bf), _dev(offsets, i32),
                                     _dev(row_src, i32), _dev(row_gate, f32), _dev(x, bf), _dev(x_src, i32),
                                     _dev(act_save, bf), _dev(dgu_packed, bf), _dev(da_up, f32),
                                     _dev(db_up, f32), _dev(da_down, f32), _dev(db_down, f32),
                                     _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_lora_bwd(shape, lora, dy, offsets, row_src, row_gate, x, x_src, act_save, w_down, da_up,
                 db_up, da_down, db_down, ws, stream=None):
    """x, x_src: as for moe_expert_gemm (tokens + row_src, or x_perm + None)."""
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check(lib().moe_lora_bwd(ctypes.byref(shape), ctypes.byref(lora), _dev(dy, bf), _dev(offsets, i32),
                              _dev(row_src, i32), _dev(row_gate, f32), _dev(x, bf), _dev(x_src, i32),
                              _dev(act_save, bf), _dev(w_down, bf), _dev(da_up, f32),
                              _dev(db_up, f32), _dev(da_down, f32), _dev(db_down, f32),
                              _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_gate_bwd(shape, dy, y_perm, slot, topk_idx, topk_gate, logits, counts, aux_coef, dgate, dlogits,
                 stream=None):
    dt = _fdt(shape)
    f32, i32 = torch.float32, torch.int32
    _check(lib().moe_gate_bwd(ctypes.byref(shape), _dev(dy, dt), _dev(y_perm, dt), _dev(slot, i32),
                              _dev(topk_idx, i32), _dev(topk_gate, f32), _dev(logits, f32), _dev(counts, i32),
                              ctypes.c_float(aux_coef), _dev(dgate, f32), _dev(dlogits, f32), _stream(stream)))


def moe_expert_bwd(shape, lora, dy, offsets, row_src, row_gate, slot, act_save, w_gate, w_up, w_down, dgu,
                   dx_rows, dx, ws, stream=None):
    dt = _fdt(shape)
    f32, i32 = torch.float32, torch.int32
    _check(lib().moe_expert_bwd(ctypes.byref(shape), ctypes.byref(lora) if lora is not None else None,
                                _dev(dy, dt), _dev(offsets, i32), _dev(row_src, i32), _dev(row_gate, f32),
                                _dev(slot, i32), _dev(act_save, dt), _dev(w_gate, dt), _dev(w_up, dt),
                                _dev(w_down, dt), _dev(dgu, dt), _dev(dx_rows, f32), _dev(dx, f32),
                                _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_pack_backward_weights(shape, w_gate, w_up, w_down, dgu_packed, dx_packed, stream=None):
    bf = torch.bfloat16
    _check(lib().moe_pack_backward_weights(ctypes.byref(shape), _dev(w_gate, bf), _dev(w_up, bf), _dev(w_down, bf),
                                           _dev(dgu_packed, bf), _dev(dx_packed, bf), _stream(stream)))


def moe_expert_bwd_packed(shape, lora, dy, offsets, row_src, row_gate, slot, act_save, dgu_packed, dx_packed,
                          dgu, dx_rows, dx, ws, stream=None):
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check(lib().moe_expert_bwd_packed(ctypes.byref(shape), ctypes.byref(lora) if lora is not None else None,
                                       _dev(dy, bf), _dev(offsets, i32), _dev(row_src, i32), _dev(row_gate, f32),
                                       _dev(slot, i32), _dev(act_save, bf), _dev(dgu_packed, bf),
                                       _dev(dx_packed, bf), _dev(dgu, bf), _dev(dx_rows, f32), _dev(dx, f32),
                                       _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_pack_router_bwd(shape, w_router, wr_packed, stream=None):
    bf = torch.bfloat16
    _check(lib().moe_pack_router_bwd(ctypes.byref(shape), _dev(w_router, bf), _dev(wr_packed, bf), _stream(stream)))


def moe_router_bwd_packed(shape, dlogits, wr_packed, dx, ws, stream=None):
    _check(lib().moe_router_bwd_packed(ctypes.byref(shape), _dev(dlogits, torch.float32),
                                       _dev(wr_packed, torch.bfloat16), _dev(dx, torch.float32),
                                       _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_router_bwd_unpermute_packed(shape, dlogits, wr_packed, dx_rows, slot, dx, ws, stream=None):
    _check(lib().moe_router_bwd_unpermute_packed(ctypes.byref(shape), _dev(dlogits, torch.float32),
                                                 _dev(wr_packed, torch.bfloat16), _dev(dx_rows, torch.float32),
                                                 _dev(slot, torch.int32), _dev(dx, torch.float32),
                                                 _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_router_bwd(shape, dlogits, w_router, dx, ws, stream=None):
    dt = _fdt(shape)
    _check(lib().moe_router_bwd(ctypes.byref(shape), _dev(dlogits, torch.float32), _dev(w_router, dt),
                                _dev(dx, torch.float32), _dev(ws, torch.uint8), ws.numel(), _stream(stream)))


def moe_timing_enable(on=True) -> None:
    """on: False (off), True (every kernel kind) or an iterable of kind names."""
    if on is True:
        mask = -1
    elif not on:
        mask = 0
    else:
        mask = 0
        for name in on:
            mask |= 1 << KERNELS.index(name)
    _check(lib().moe_timing_enable(mask))


def moe_timing_read(kernel: str):
    """(total milliseconds, launches) of one kernel kind since the last enable."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().moe_timing_read(KERNELS.index(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
