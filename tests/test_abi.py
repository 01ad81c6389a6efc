"""The C ABI on the CPU: the library loads, exports what include/moe.h declares,
and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_top_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def shape(**kw):
    base = dict(T=64, d=128, E=16, k=4, f=64, e_lo=0, e_hi=16, capacity=0, dtype=B.MOE_F32)
    base.update(kw)
    return B.MoeShape(*[base[n] for n, _ in B.MoeShape._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), B.MOE_ERR_INVALID_ARG), (dict(k=17), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG), (dict(e_lo=5, e_hi=5), B.MOE_ERR_INVALID_ARG),
    (dict(e_hi=17), B.MOE_ERR_INVALID_ARG), (dict(dtype=7), B.MOE_ERR_INVALID_ARG),
    (dict(d=0), B.MOE_ERR_INVALID_ARG),
    (dict(E=1025, e_hi=1025), B.MOE_ERR_UNSUPPORTED), (dict(E=64, e_hi=64, k=33), B.MOE_ERR_UNSUPPORTED),
    (dict(dtype=B.MOE_BF16, d=96), B.MOE_ERR_UNSUPPORTED),
    (dict(dtype=B.MOE_BF16, d=128, f=96), B.MOE_ERR_UNSUPPORTED),
])
def test_bad_shapes_are_rejected_on_the_host(kw, status):
    lib = B.lib()
    s = shape(**kw)
    st = lib.moe_route(ctypes.byref(s), None, None, None, None, None, None, None, None, 0, None)
    assert st == status
    assert lib.moe_last_error()
    assert lib.moe_workspace_bytes(ctypes.byref(s), 0) == 0
    assert lib.moe_max_rows(ctypes.byref(s)) == -1


def test_null_pointers_and_small_workspace_are_rejected():
    lib = B.lib()
    s = shape()
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, None, None, None, None, 0,
                         None) == B.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in lib.moe_last_error()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(s), fake, fake, None, fake, fake, None, None, fake, 16,
                         None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_combine(ctypes.byref(s), fake, None, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    lo = B.MoeLora(16, 32.0, None, None, None, None)
    assert lib.moe_expert_gemm(ctypes.byref(s), fake, None, fake, fake, fake, fake, ctypes.byref(lo),
                               None, fake, fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    lo = B.MoeLora(16, 32.0, fake, fake, fake, fake)
    assert lib.moe_expert_gemm(ctypes.byref(s), fake, None, fake, fake, fake, fake, ctypes.byref(lo),
                               None, fake, fake, 1 << 30, None) == B.MOE_ERR_UNSUPPORTED  # fp32 LoRA
    assert lib.moe_timing_read(99, None, None) == B.MOE_ERR_INVALID_ARG


def test_max_rows_and_workspace_sizes():
    full = B.make_shape(4096, 2048, 896, 16, 256)
    assert B.moe_max_rows(full) == 4096 * 16
    ep = B.make_shape(16384, 4096, 896, 16, 1024, 0, 14)
    assert B.moe_max_rows(ep) == 16384 * 14
    cap = B.make_shape(8192, 2048, 896, 16, 256, capacity=183)
    assert B.moe_max_rows(cap) == min(8192 * 16, 896 * 183)
    assert B.moe_max_rows(B.make_shape(8192, 2048, 896, 16, 256, capacity=100)) == 896 * 100
    for s in (full, ep, cap):
        ws0, ws16 = B.moe_workspace_bytes(s, 0), B.moe_workspace_bytes(s, 16)
        assert 0 < ws0 < ws16
        assert ws0 % 256 == 0
    # the logits scratch alone is T*E fp32
    assert B.moe_workspace_bytes(full, 0) > 4096 * 896 * 4


def test_backward_entry_points_validate_on_the_host():
    lib = B.lib()
    s = shape()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    # gate backward: dlogits is required; logits only with counts and a coefficient
    assert lib.moe_gate_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, None, None, ctypes.c_float(0.0),
                            None, None, None) == B.MOE_ERR_INVALID_ARG
    assert b"dlogits is NULL" in lib.moe_last_error()
    assert lib.moe_gate_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, None, fake, ctypes.c_float(0.01),
                            None, fake, None) == B.MOE_ERR_INVALID_ARG
    assert b"logits is NULL" in lib.moe_last_error()
    # expert backward: scratch and output buffers, then the workspace size
    args = [fake] * 13
    args[9] = None  # dgu
    assert lib.moe_expert_bwd(ctypes.byref(s), None, *args, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert b"dgu is NULL" in lib.moe_last_error()
    args = [fake] * 13
    assert lib.moe_expert_bwd(ctypes.byref(s), None, *args, 16, None) == B.MOE_ERR_WORKSPACE
    # packed paths: bf16 with d, f % 128 == 0 (and E % 64 == 0 for the router)
    bf = shape(dtype=B.MOE_BF16, d=128, f=64)
    assert lib.moe_pack_backward_weights(ctypes.byref(bf), fake, fake, fake, fake, fake,
                                         None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_router_bwd(ctypes.byref(bf), fake, fake, None) == B.MOE_ERR_UNSUPPORTED  # E = 16
    bf2 = shape(dtype=B.MOE_BF16, d=128, f=128)
    assert lib.moe_pack_backward_weights(ctypes.byref(bf2), fake, fake, fake, None, None,
                                         None) == B.MOE_ERR_INVALID_ARG                      # no output
    assert lib.moe_router_bwd(ctypes.byref(s), None, fake, fake, fake, 1 << 30,
                              None) == B.MOE_ERR_INVALID_ARG


def test_lora_backward_packed_validates_on_the_host():
    lib = B.lib()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    lora = B.MoeLora(16, 32.0, 0x100000, 0x100000, 0x100000, 0x100000)
    bf = shape(dtype=B.MOE_BF16, d=128, f=128)
    args = [fake] * 13
    args[7] = None  # dgu_packed
    assert lib.moe_lora_bwd_packed(ctypes.byref(bf), ctypes.byref(lora), *args, 1 << 30,
                                   None) == B.MOE_ERR_INVALID_ARG
    assert b"dgu_packed is NULL" in lib.moe_last_error()
    # the packed transposes need d, f % 128 == 0 and bf16
    for bad in (shape(dtype=B.MOE_BF16, d=128, f=64), shape(dtype=B.MOE_F32, d=128, f=128)):
        assert lib.moe_lora_bwd_packed(ctypes.byref(bad), ctypes.byref(lora), *([fake] * 13), 1 << 30,
                                       None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_lora_bwd_packed(ctypes.byref(bf), ctypes.byref(lora), *([fake] * 13), 16,
                                   None) == B.MOE_ERR_WORKSPACE


def test_router_backward_with_unpermute_validates_on_the_host():
    lib = B.lib()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    ok = shape(dtype=B.MOE_BF16, d=128, f=128, E=64, e_hi=64)
    # the product runs on the packed transpose: bf16, d % 128 == 0, E % 64 == 0
    for bad in (shape(dtype=B.MOE_BF16, d=128, f=128),                      # E = 16
                shape(dtype=B.MOE_F32, d=128, f=128, E=64, e_hi=64),
                shape(dtype=B.MOE_BF16, d=192, f=128, E=64, e_hi=64)):
        assert lib.moe_router_bwd_unpermute_packed(ctypes.byref(bad), *([fake] * 5), fake, 1 << 30,
                                                   None) == B.MOE_ERR_UNSUPPORTED
    for i, name in enumerate(["dlogits", "wr_packed", "dx_rows", "slot", "dx"]):
        args = [fake] * 5
        args[i] = None
        assert lib.moe_router_bwd_unpermute_packed(ctypes.byref(ok), *args, fake, 1 << 30,
                                                   None) == B.MOE_ERR_INVALID_ARG, name
        assert f"{name} is NULL".encode() in lib.moe_last_error()
    assert lib.moe_router_bwd_unpermute_packed(ctypes.byref(ok), *([fake] * 5), fake, 16,
                                               None) == B.MOE_ERR_WORKSPACE


def test_expert_backward_packed_accepts_null_dx_and_slot():
    """dx NULL skips the per-token sum (done by the combined router call), so
    slot may be NULL with it: validation passes the pointer checks and stops
    at the too-small workspace; slot NULL with dx set is still an error."""
    lib = B.lib()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    bf = shape(dtype=B.MOE_BF16, d=128, f=128)
    # dy, offsets, row_src, row_gate, slot, act_save, dgu_packed, dx_packed, dgu, dx_rows, dx, ws
    args = [fake] * 12
    args[4] = None   # slot
    args[10] = None  # dx
    assert lib.moe_expert_bwd_packed(ctypes.byref(bf), None, *args, 16, None) == B.MOE_ERR_WORKSPACE
    args[10] = fake
    assert lib.moe_expert_bwd_packed(ctypes.byref(bf), None, *args, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert b"slot is NULL" in lib.moe_last_error()


def test_dispatch_noalloc_rejects_shapes_beyond_its_scratch():
    """The no-allocation dispatch checks the scratch a shape needs against the
    library's fixed array on the host, before any device call."""
    lib = B.lib()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    # 2^20 tokens over 1024 experts: 2 * 32768 * 1024 * 4 B = 256 MiB of tile histograms
    s = shape(T=1 << 20, E=1024, e_hi=1024, k=2, dtype=B.MOE_BF16, d=128, f=64)
    st = lib.moe_dispatch_noalloc(ctypes.byref(s), fake, fake, None, fake, fake, fake, fake, fake, None,
                                  None, None)
    assert st == B.MOE_ERR_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
    assert lib.moe_dispatch_noalloc(ctypes.byref(shape()), None, fake, None, fake, fake, fake, fake, fake,
                                    None, None, None) == B.MOE_ERR_INVALID_ARG


def test_remap_and_latent_routing_argument_checks():
    """Host-side validation of the remapping and latent-routing entry points."""
    lib = B.lib()
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    s = shape(dtype=B.MOE_BF16, d=128, f=64, capacity=0)
    assert lib.moe_dispatch_remap(ctypes.byref(s), fake, fake, fake, None, fake, fake, fake, fake, fake, None,
                                  None, None, fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG   # no capacity
    assert b"capacity" in lib.moe_last_error()
    s = shape(dtype=B.MOE_BF16, d=128, f=64, capacity=20, E=16, e_hi=16, k=9)            # 2k > E
    assert lib.moe_dispatch_remap(ctypes.byref(s), fake, fake, fake, None, fake, fake, fake, fake, fake, None,
                                  None, None, fake, 1 << 30, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_alt(ctypes.byref(s), fake, fake, None, fake, fake, fake, None, None, fake, 1 << 30,
                             None) == B.MOE_ERR_UNSUPPORTED
    s = shape(dtype=B.MOE_BF16, d=128, f=64)
    assert lib.moe_route_alt(ctypes.byref(s), fake, fake, None, fake, fake, None, None, None, fake, 1 << 30,
                             None) == B.MOE_ERR_INVALID_ARG                                  # alt_idx NULL
    assert lib.moe_route_latent(ctypes.byref(s), 96, fake, fake, fake, None, fake, fake, fake, None, None, fake,
                                1 << 30, None) == B.MOE_ERR_UNSUPPORTED                      # d_c % 64
    s32 = shape()
    assert lib.moe_route_latent(ctypes.byref(s32), 64, fake, fake, fake, None, fake, fake, fake, None, None, fake,
                                1 << 30, None) == B.MOE_ERR_UNSUPPORTED                      # fp32
    assert lib.moe_route_latent(ctypes.byref(s), 64, fake, None, fake, None, fake, fake, fake, None, None, fake,
                                1 << 30, None) == B.MOE_ERR_INVALID_ARG                      # w_latent NULL
