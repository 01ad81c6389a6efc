"""Guard bands: no entry point writes outside the buffers it is given.

Every output (and the workspace) is a view into a larger allocation whose
bytes before and after the view hold a canary pattern; buffers sized by the
row bound also keep the canary in their rows past R (the interface promises
that only the R dispatched rows are written). The forward with LoRA and
saved activations, the adapter backward (plain and packed) and the full
backward (plain and packed) run through the C ABI, then every canary byte
is checked."""
import numpy as np
import pytest
import torch

from gpu_util import lora_of, say, upload
from sparse_mixture_experts_top_amd import binding as B
from sparse_mixture_experts_top_amd import layer
from sparse_mixture_experts_top_amd.workloads import Workload, generate

pytestmark = pytest.mark.gpu

CANARY = 0xA5
GUARD = 4096  # bytes on each side


class Guarded:
    """Views into canary-filled allocations, with a record of what each view
    may write (the whole view, or its first rows only)."""

    def __init__(self):
        self.items = []

    def make(self, name, shape, dtype, rows_written=None):
        el = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        nbytes = max(n * el, 1)
        raw = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        view = raw[GUARD:GUARD + n * el].view(dtype).view(*shape) if n else \
            raw[GUARD:GUARD].view(dtype).view(*shape)
        self.items.append((name, raw, nbytes, shape, el, rows_written))
        return view

    def check(self, R):
        torch.cuda.synchronize()
        for name, raw, nbytes, shape, el, rows_written in self.items:
            host = raw.cpu().numpy()
            assert (host[:GUARD] == CANARY).all(), f"{name}: written before the buffer"
            assert (host[GUARD + nbytes:] == CANARY).all(), f"{name}: written past the buffer"
            if rows_written is not None and len(shape) >= 1 and shape[0] > 0:
                row_bytes = nbytes // shape[0]
                tail = host[GUARD + R * row_bytes:GUARD + nbytes]
                assert (tail == CANARY).all(), f"{name}: rows past R = {R} written"
        say(f"  guards intact on {len(self.items)} buffers (R = {R})")


CASES = {
    # ragged tiles, a local range and LoRA at r = 16 (the extra K step)
    "lora_local": Workload("g_lora_local", T=300, d=256, E=16, k=4, f=128, e_lo=2, e_hi=13, lora_r=16,
                           lora_alpha=32.0, lora_b="normal", aux_coef=0.01),
    # capacity drops with Zipf skew; rank 8 (the fp32 adapter epilogue)
    "capacity_r8": Workload("g_capacity_r8", T=700, d=128, E=32, k=4, f=128, capacity=30, zipf_s=1.2,
                            lora_r=8, lora_alpha=16.0, lora_b="normal", aux_coef=0.01),
    # fp32, rows of an odd number of elements
    "f32_odd": Workload("g_f32_odd", T=131, d=45, E=9, k=2, f=19, capacity=40, zipf_s=1.0, dtype="f32"),
    # ~150 rows per expert: two 128-row tiles each, LoRA at r = 16
    "mid_lora": Workload("g_mid_lora", T=600, d=128, E=16, k=4, f=128, e_lo=1, e_hi=14, lora_r=16,
                         lora_alpha=32.0, lora_b="normal", aux_coef=0.01),
    # about 500 rows per expert: 320-row tiles (two per expert), LoRA at r = 16
    "tall_lora": Workload("g_tall_lora", T=2048, d=128, E=8, k=2, f=128, e_lo=1, e_hi=7, lora_r=16,
                          lora_alpha=32.0, lora_b="normal", aux_coef=0.01),
}


@pytest.mark.parametrize("name,packed", [("lora_local", False), ("lora_local", True),
                                         ("capacity_r8", True), ("f32_odd", False), ("tall_lora", True),
                                         ("mid_lora", True)])
def test_no_write_outside_buffers(name, packed):
    w = CASES[name]
    say(f"[guard {name} packed={packed}] T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} dtype={w.dtype}")
    inp = generate(w, seed=9)
    dev = upload(inp)
    s = layer.shape_of(w)
    T, d, E, k, f, L = w.T, w.d, w.E, w.k, w.f, w.L
    rmax = B.moe_max_rows(s)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    i32, f32 = torch.int32, torch.float32
    g = Guarded()
    ws_bytes = B.moe_workspace_bytes(s, w.lora_r)
    buf = layer.Buffers(
        shape=s,
        topk_idx=g.make("topk_idx", (T, k), i32), topk_gate=g.make("topk_gate", (T, k), f32),
        logits=g.make("logits", (T, E), f32), prob_sum=g.make("prob_sum", (E,), f32),
        counts=g.make("counts", (E,), i32), offsets=g.make("offsets", (L + 1,), i32),
        slot=g.make("slot", (T, k), i32),
        row_src=g.make("row_src", (rmax,), i32, rows_written=True),
        row_gate=g.make("row_gate", (rmax,), f32, rows_written=True),
        x_perm=g.make("x_perm", (rmax, d), dt, rows_written=True),
        y_perm=g.make("y_perm", (rmax, d), dt, rows_written=True),
        act_save=g.make("act_save", (rmax, 3 * f), dt, rows_written=True),
        y=g.make("y", (T, d), dt), dropped=g.make("dropped", (1,), i32), aux=g.make("aux", (2,), f32),
        ws=g.make("ws", (ws_bytes,), torch.uint8))
    lora = lora_of(w, dev)
    pk = layer.pack_weights(s, dev["w_gate"], dev["w_up"], dev["w_down"]) if packed else None
    layer.forward(buf, dev["x"], dev["w_router"], dev.get("bias"), dev["w_gate"], dev["w_up"],
                  dev["w_down"], lora, packed=pk)
    B.moe_aux_loss(s, buf.counts, buf.prob_sum, 0.01, buf.aux)
    torch.cuda.synchronize()
    R = int(buf.offsets[-1].item())
    assert 0 < R <= rmax
    if lora is not None:
        r = w.lora_r
        grads = [g.make(n, sh, f32) for n, sh in (("da_up", (L, r, d)), ("db_up", (L, f, r)),
                                                   ("da_down", (L, r, f)), ("db_down", (L, d, r)))]
        B.moe_lora_bwd(s, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, dev["x"], buf.row_src,
                       buf.act_save, dev["w_down"], *grads, buf.ws)
        if packed:
            dgu_p = torch.empty((L, f, d), dtype=torch.bfloat16, device="cuda")
            B.moe_pack_backward_weights(s, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
            grads_p = [g.make(n + "_p", sh, f32) for n, sh in (("da_up", (L, r, d)), ("db_up", (L, f, r)),
                                                               ("da_down", (L, r, f)), ("db_down", (L, d, r)))]
            B.moe_lora_bwd_packed(s, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.x_perm,
                                  None, buf.act_save, dgu_p, *grads_p, buf.ws)
    dgate = g.make("dgate", (T, k), f32)
    dlogits = g.make("dlogits", (T, E), f32)
    dgu = g.make("dgu", (rmax, 2 * f), dt, rows_written=True)
    dx_rows = g.make("dx_rows", (rmax, d), f32, rows_written=True)
    dx = g.make("dx", (T, d), f32)
    B.moe_gate_bwd(s, dev["dy"], buf.y_perm, buf.slot, buf.topk_idx, buf.topk_gate, buf.logits, buf.counts,
                   0.01, dgate, dlogits)
    if packed:
        dgu_p = torch.empty((L, f, d), dtype=torch.bfloat16, device="cuda")
        dx_p = torch.empty((L, d, 2 * f), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_backward_weights(s, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, dx_p)
        wr_p = torch.empty((d, E), dtype=torch.bfloat16, device="cuda")
        B.moe_expert_bwd_packed(s, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, None, buf.act_save,
                                dgu_p, dx_p, dgu, dx_rows, None, buf.ws)
        if E % 64 == 0:
            B.moe_pack_router_bwd(s, dev["w_router"], wr_p)
            B.moe_router_bwd_unpermute_packed(s, dlogits, wr_p, dx_rows, buf.slot, dx, buf.ws)
    else:
        B.moe_expert_bwd(s, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.slot, buf.act_save,
                         dev["w_gate"], dev["w_up"], dev["w_down"], dgu, dx_rows, dx, buf.ws)
        B.moe_router_bwd(s, dlogits, dev["w_router"], dx, buf.ws)
    g.check(R)
