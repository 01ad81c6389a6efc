"""moe_dispatch_noalloc (the dispatch on the library's own scratch array)
against moe_dispatch with a caller workspace: bitwise equal outputs on two
calls in a row, the second with a smaller input, so the second call runs on
what the first left in the shared scratch. Both go through the C ABI; the
workspace path is itself checked against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import check_dispatch, check_route, say, upload
from sparse_mixture_experts_top_amd import binding as B
from sparse_mixture_experts_top_amd import layer
from sparse_mixture_experts_top_amd.workloads import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu

OUTS = ("counts", "offsets", "slot", "dropped")
ROWS = ("row_src", "row_gate", "x_perm")


def routed(w, seed):
    inp = generate(w, seed=seed)
    dev = upload(inp)
    s = layer.shape_of(w)
    buf = layer.alloc(s, logits=True, x_perm=True)
    B.moe_route(s, dev["x"], dev["w_router"], dev.get("bias"), buf.topk_idx, buf.topk_gate, buf.logits, None,
                buf.ws)
    torch.cuda.synchronize()
    return inp, dev, s, buf


def dispatch_both(w, seed):
    """The layer's dispatch with a workspace and without one, on the same
    routing; returns the two buffer sets after checking the first against
    the oracle."""
    say(f"[no-alloc dispatch {w.name}] T={w.T} E={w.E} k={w.k} L={w.L} cap={w.capacity}")
    inp, dev, s, ref = routed(w, seed)
    B.moe_dispatch(s, ref.topk_idx, ref.topk_gate, dev["x"], ref.counts, ref.offsets, ref.slot, ref.row_src,
                   ref.row_gate, ref.x_perm, ref.dropped, ref.ws)
    got = layer.alloc(s, x_perm=True)
    for t in (got.counts, got.offsets, got.slot, got.row_src, got.dropped):
        t.fill_(-7)
    got.row_gate.fill_(float("nan"))
    got.x_perm.fill_(float("nan"))
    B.moe_dispatch_noalloc(s, ref.topk_idx, ref.topk_gate, dev["x"], got.counts, got.offsets, got.slot,
                           got.row_src, got.row_gate, got.x_perm, got.dropped)
    torch.cuda.synchronize()
    lg, idx, gate = check_route(w, inp, ref, sample_tokens=np.arange(min(w.T, 64)))
    _, R = check_dispatch(w, dev, ref, idx, gate)
    for n in OUTS:
        assert torch.equal(getattr(got, n), getattr(ref, n)), n
    for n in ROWS:
        a, b = getattr(got, n)[:R], getattr(ref, n)[:R]
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), n
    say(f"  no-alloc dispatch bitwise equal to the workspace path (R = {R})")
    return R


def test_two_calls_in_a_row_second_smaller():
    # full size with capacity (candidate keys in the scratch), then a small
    # ragged shape with a local range and no capacity
    r1 = dispatch_both(WORKLOADS["skewed_capacity"], seed=0)
    r2 = dispatch_both(Workload("na_small", T=300, d=256, E=40, k=6, f=128, e_lo=5, e_hi=31), seed=1)
    assert r2 < r1


def test_full_size_then_capacity_then_tiny():
    # the largest scratch of the workloads (16384 tokens), then two smaller
    dispatch_both(WORKLOADS["ep64_rank"], seed=0)
    dispatch_both(Workload("na_cap", T=700, d=128, E=32, k=4, f=64, capacity=30, zipf_s=1.2), seed=2)
    dispatch_both(WORKLOADS["tiny_f32"], seed=3)
