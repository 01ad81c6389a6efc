"""GPU parity of the full backward (moe_gate_bwd, moe_expert_bwd,
moe_router_bwd) against the oracle, each stage fed the GPU's own upstream
outputs; small shapes over several tiles with ragged tails and the edge cases,
then sampled rows at full size. All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, check_act_save, host, lora_of, run_forward, say, upload
from sparse_mixture_experts_top_amd import binding as B
from sparse_mixture_experts_top_amd import layer
from sparse_mixture_experts_top_amd.workloads import WORKLOADS, Workload, generate, to_f64

pytestmark = pytest.mark.gpu

W = Workload
AUX = 0.01
CASES = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "ragged_bf16": W("ragged_bf16", T=300, d=256, E=40, k=6, f=128),
    "local_bf16": W("local_bf16", T=520, d=192, E=24, k=5, f=192, e_lo=3, e_hi=17),
    "capacity_bf16": W("capacity_bf16", T=700, d=128, E=32, k=4, f=64, capacity=30, zipf_s=1.2),
    "capacity_f32": W("capacity_f32", T=200, d=48, E=12, k=3, f=20, e_lo=2, e_hi=10,
                      capacity=25, zipf_s=1.0, dtype="f32"),
    "k1_bf16": W("k1_bf16", T=257, d=128, E=16, k=1, f=128),
    # fp32 rows that are not a multiple of 8 (d = 44) or of 4 elements (d = 45):
    # the element-wise paths of the gate gradient and of the row sums
    "d44_f32": W("d44_f32", T=150, d=44, E=10, k=3, f=24, e_lo=1, e_hi=9, dtype="f32"),
    "d45_f32": W("d45_f32", T=131, d=45, E=9, k=2, f=19, capacity=40, zipf_s=1.0, dtype="f32"),
    # E % 64 == 0: the router part runs on the matrix cores; two K steps of 64
    "router128_bf16": W("router128_bf16", T=333, d=320, E=128, k=4, f=64),
    # packable for every backward product (d, f % 128 == 0, E % 64 == 0)
    "router128p_bf16": W("router128p_bf16", T=333, d=256, E=128, k=4, f=128),
    # the same with a local expert range: most slots are remote (-1)
    "router128p_local_bf16": W("router128p_local_bf16", T=333, d=256, E=128, k=4, f=128, e_lo=40, e_hi=52),
    "lora_bf16": W("lora_bf16", T=256, d=128, E=12, k=4, f=128, e_lo=2, e_hi=9, lora_r=16,
                   lora_alpha=32.0, lora_b="normal"),
    # ~300 rows per expert: the layout with two compute waves per SIMD (three
    # row tiles per expert, the last one ragged), a local range and LoRA
    "wide_bf16": W("wide_bf16", T=1200, d=256, E=16, k=4, f=128, e_lo=2, e_hi=13, lora_r=16,
                   lora_alpha=32.0, lora_b="normal"),
}


def _lora64(w, inp):
    if w.lora_r <= 0:
        return None
    return {"scale": w.lora_alpha / w.lora_r, **{n: to_f64(inp[n]) for n in ("a_up", "b_up", "a_down", "b_down")}}


def dot_bound(a, b):
    """Rounding bound of an fp32-accumulated dot product of exactly given
    values: gamma_n sum |a_i b_i| (n terms, unit roundoff 2^-24)."""
    n = a.shape[-1]
    g = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    return g * np.sum(np.abs(a * b), axis=-1)


def pack_backward(w, dev):
    dgu_p = torch.empty((w.L, w.f, w.d), dtype=torch.bfloat16, device="cuda")
    dx_p = torch.empty((w.L, w.d, 2 * w.f), dtype=torch.bfloat16, device="cuda")
    B.moe_pack_backward_weights(layer.shape_of(w), dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, dx_p)
    return dgu_p, dx_p


def run_backward(w, dev, buf, packed=False):
    s = buf.shape
    T, d, E, k, f = w.T, w.d, w.E, w.k, w.f
    rmax = max(B.moe_max_rows(s), 1)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {
        "dgate": torch.full((T, k), float("nan"), device="cuda"),
        "dlogits": torch.full((T, E), float("nan"), device="cuda"),
        "dgu": torch.empty((rmax, 2 * f), dtype=dt, device="cuda"),
        "dx_rows": torch.empty((rmax, d), device="cuda"),
        "dx": torch.full((T, d), float("nan"), device="cuda"),
    }
    B.moe_gate_bwd(s, dev["dy"], buf.y_perm, buf.slot, buf.topk_idx, buf.topk_gate, buf.logits, buf.counts,
                   AUX, out["dgate"], out["dlogits"])
    if packed:
        dgu_p, dx_p = pack_backward(w, dev)
        B.moe_expert_bwd_packed(s, lora_of(w, dev), dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.slot,
                                buf.act_save, dgu_p, dx_p, out["dgu"], out["dx_rows"], out["dx"], buf.ws)
    else:
        B.moe_expert_bwd(s, lora_of(w, dev), dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.slot,
                         buf.act_save, dev["w_gate"], dev["w_up"], dev["w_down"], out["dgu"], out["dx_rows"],
                         out["dx"], buf.ws)
    torch.cuda.synchronize()
    out["dx_experts"] = out["dx"].clone()
    out["dx_router"] = torch.zeros((T, d), device="cuda")
    if packed and E % 64 == 0 and d % 128 == 0:
        wr_p = torch.empty((d, E), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_router_bwd(s, dev["w_router"], wr_p)
        B.moe_router_bwd_packed(s, out["dlogits"], wr_p, out["dx_router"], buf.ws)
        B.moe_router_bwd_packed(s, out["dlogits"], wr_p, out["dx"], buf.ws)  # accumulates
        # the fused pass: expert rows without their unpermute, then one pass
        # that sums them per token and adds the router product
        dgu2, rows2 = torch.empty_like(out["dgu"]), torch.full_like(out["dx_rows"], float("nan"))
        B.moe_expert_bwd_packed(s, lora_of(w, dev), dev["dy"], buf.offsets, buf.row_src, buf.row_gate, None,
                                buf.act_save, dgu_p, dx_p, dgu2, rows2, None, buf.ws)
        out["dx_fused"] = torch.full((T, d), float("nan"), device="cuda")
        B.moe_router_bwd_unpermute_packed(s, out["dlogits"], wr_p, rows2, buf.slot, out["dx_fused"], buf.ws)
    else:
        B.moe_router_bwd(s, out["dlogits"], dev["w_router"], out["dx_router"], buf.ws)
        B.moe_router_bwd(s, out["dlogits"], dev["w_router"], out["dx"], buf.ws)  # accumulates
    torch.cuda.synchronize()
    # same products, so the accumulated result is exactly one fp32 addition
    assert torch.equal(out["dx"], out["dx_experts"] + out["dx_router"])
    if "dx_fused" in out:   # same sums in the same order: bitwise equal
        assert torch.equal(out["dx_fused"], out["dx"])
    return out


PACKABLE = [n for n, w in CASES.items() if w.dtype == "bf16" and w.d % 128 == 0 and w.f % 128 == 0]


@pytest.mark.parametrize("name,packed", [(n, False) for n in sorted(CASES)] + [(n, True) for n in PACKABLE])
def test_backward_stagewise(name, packed):
    check_backward(CASES[name], packed)


def check_backward(w, packed, seed=3):
    """The forward, then every backward stage against the oracle fed the GPU's
    own upstream results."""
    say(f"[backward {w.name}] T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} local=[{w.e_lo},{w.local_hi}) "
        f"cap={w.capacity} lora={w.lora_r} dtype={w.dtype} packed={packed}")
    inp = generate(w, seed=seed)
    dev = upload(inp)
    buf = run_forward(w, dev, prob=True, act_save=True, x_perm=False)
    g = run_backward(w, dev, buf, packed=packed)
    T = w.T
    R = int(host(buf.offsets)[-1])
    # the saved G | H | U rows the backward reads
    lo = _lora64(w, inp)
    check_act_save(w, inp, buf, np.arange(R), lora=None if lo is None else {"scale": lo["scale"]})
    dy = to_f64(inp["dy"])
    slot = host(buf.slot).astype(np.int64)
    gate = buf.topk_gate.cpu().numpy().astype(np.float64)
    idx = host(buf.topk_idx).astype(np.int64)
    o_rows = host(buf.y_perm[:R]) if R else np.zeros((0, w.d))
    logits = buf.logits.cpu().numpy().astype(np.float64)
    counts = host(buf.counts)
    # gate gradients: exact dot products of the GPU's own rows
    dg_ref = oracle.gate_backward(dy, o_rows, slot, gate, T)
    dg = host(g["dgate"])
    bound = np.zeros_like(dg_ref)
    for t in range(T):
        for j in range(w.k):
            if slot[t, j] >= 0:
                bound[t, j] = dot_bound(dy[t], o_rows[slot[t, j]])
    err = np.abs(dg - dg_ref)
    say(f"  dgate: max_abs={err.max():.3e} max(err/bound)={(err / np.maximum(bound, 1e-30)).max():.3f}")
    assert (err <= 2 * bound + 1e-30).all()
    assert (dg[slot < 0] == 0).all()
    # logit gradients from the GPU's dg (fp32 softmax-Jacobian and aux terms)
    dl_ref = oracle.logits_backward(dg, idx, gate, logits, counts, AUX, w.k)
    dl = host(g["dlogits"])
    scale = max(1.0, float(np.abs(dl_ref).max()))
    e = np.abs(dl - dl_ref).max()
    say(f"  dlogits: max_abs={e:.3e} |ref|inf={np.abs(dl_ref).max():.3e}")
    assert e <= 1e-5 * scale
    assert np.abs(dl.sum(axis=1)).max() <= 1e-5 * scale * w.k   # softmax shift invariance
    # dx through the experts, oracle recomputing G and U from the rows in fp64
    x_perm = to_f64(inp["x"])[host(buf.row_src[:R]).astype(np.int64)] if R else np.zeros((0, w.d))
    dx_ref, _, _ = oracle.experts_backward(dy, host(buf.offsets), host(buf.row_src[:R]).astype(np.int64),
                                           buf.row_gate[:R].cpu().numpy().astype(np.float64), slot, x_perm,
                                           to_f64(inp["w_gate"]), to_f64(inp["w_up"]), to_f64(inp["w_down"]),
                                           T, lora=_lora64(w, inp))
    # dx through the experts sums products of bf16-stored inputs (G, U in
    # act_save, dG | dU in the scratch rows): their relative rounding stays in
    # the sum whatever its order, so with bf16 the max-abs bound scales with
    # max(1, |dx|inf)
    assert_close(host(g["dx_experts"]), dx_ref, w.dtype, "dx (experts)", scale_atol=w.dtype == "bf16")
    none = (slot < 0).all(axis=1)
    assert (host(g["dx_experts"])[none] == 0).all()
    # router part on the GPU's dlogits
    dxr_ref = oracle.router_backward(dl, to_f64(inp["w_router"]))
    assert_close(host(g["dx_router"]), dxr_ref, w.dtype, "dx (router)")


def test_backward_empty_and_no_local():
    for w in (W("empty_b", T=0, d=128, E=16, k=4, f=64),
              W("nolocal_b", T=90, d=64, E=16, k=4, f=64, e_lo=12, e_hi=16, zipf_s=0.0)):
        say(f"[backward {w.name}]")
        inp = generate(w, seed=1)
        dev = upload(inp)
        buf = run_forward(w, dev, prob=True, act_save=True, x_perm=False)
        g = run_backward(w, dev, buf)
        if w.T == 0:
            continue
        slot = host(buf.slot)
        dx = host(g["dx_experts"])
        assert (dx[(slot < 0).all(axis=1)] == 0).all()
        assert np.isfinite(host(g["dlogits"])).all() and np.isfinite(host(g["dx"])).all()


def test_router_backward_with_row_sums_and_no_local_rows():
    """No token picks a local expert (large bias on experts 0..3, local range
    40..48): the combined call must store exactly the router product, never
    reading the expert rows (filled with NaN here); T = 0 is a no-op."""
    for w in (W("nolocal_rb", T=90, d=128, E=64, k=4, f=128, e_lo=40, e_hi=48),
              W("empty_rb", T=0, d=128, E=64, k=4, f=128)):
        say(f"[router backward + row sums {w.name}]")
        inp = generate(w, seed=2)
        inp["bias"] = torch.tensor([50.0] * 4 + [0.0] * 60)
        dev = upload(inp)
        buf = run_forward(w, dev, prob=True, act_save=True, x_perm=False)
        s = buf.shape
        assert int(buf.offsets[-1].item()) == 0
        g = torch.Generator().manual_seed(7)
        dlogits = torch.randn((w.T, w.E), generator=g).to("cuda")
        wr_p = torch.empty((w.d, w.E), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_router_bwd(s, dev["w_router"], wr_p)
        ref = torch.zeros((w.T, w.d), device="cuda")
        B.moe_router_bwd_packed(s, dlogits, wr_p, ref, buf.ws)
        rows = torch.full((max(B.moe_max_rows(s), 1), w.d), float("nan"), device="cuda")
        dx = torch.full((w.T, w.d), float("nan"), device="cuda")
        B.moe_router_bwd_unpermute_packed(s, dlogits, wr_p, rows, buf.slot, dx, buf.ws)
        torch.cuda.synchronize()
        assert torch.equal(dx, ref)


@pytest.mark.parametrize("name", ["full_router", "ep64_rank", "skewed_capacity"])
def test_backward_full_size_sampled(name):
    """Full size, in the launch configuration of the benchmark's backward
    pass (packed transposed weights); the oracle checks sampled tokens (their gate and logit gradients,
    their dx summed from their rows, and the router part)."""
    w = WORKLOADS[name]
    say(f"[backward full {name}]")
    inp = generate(w, seed=0)
    dev = upload(inp)
    buf = run_forward(w, dev, prob=True, act_save=True, x_perm=False, packed=True)
    g = run_backward(w, dev, buf, packed=True)
    rng = np.random.default_rng(5)
    slot_all = host(buf.slot).astype(np.int64)
    local = np.nonzero((slot_all >= 0).any(axis=1))[0]
    toks = np.unique(np.concatenate([rng.choice(w.T, 6, replace=False), rng.choice(local, 6, replace=False),
                                     [0, w.T - 1]]))
    counts = host(buf.counts)
    offsets = host(buf.offsets)
    ts = torch.as_tensor(toks, device="cuda")
    dy = to_f64(inp["dy"][toks])
    slot = slot_all[toks]
    gate = buf.topk_gate[ts].cpu().numpy().astype(np.float64)
    idx = host(buf.topk_idx[ts]).astype(np.int64)
    logits = buf.logits[ts].cpu().numpy().astype(np.float64)
    rows = np.unique(slot[slot >= 0])
    o = {int(r): v for r, v in zip(rows, host(buf.y_perm[torch.as_tensor(rows, device="cuda")]))}
    dg_ref = np.zeros((len(toks), w.k))
    bound = np.zeros_like(dg_ref)
    for a in range(len(toks)):
        for j in range(w.k):
            if slot[a, j] >= 0:
                dg_ref[a, j] = float(np.dot(dy[a], o[int(slot[a, j])]))
                bound[a, j] = dot_bound(dy[a], o[int(slot[a, j])])
    dg = host(g["dgate"][ts])
    # each gate gradient is an fp32 dot product of d terms (|dgate| reaches
    # ~85 at d = 2048): held to the same rounding bound as the small cases
    err = np.abs(dg - dg_ref)
    rel = float(np.linalg.norm(dg - dg_ref) / max(np.linalg.norm(dg_ref), 1e-30))
    say(f"  dgate (sampled): max_abs={err.max():.3e} max(err/bound)={(err / np.maximum(bound, 1e-30)).max():.3f} "
        f"rel_frob={rel:.3e}")
    assert (err <= 2 * bound + 1e-30).all()
    assert rel <= 1e-5  # the fp32 relative Frobenius bound
    assert (dg[slot < 0] == 0).all()
    dl_ref = oracle.logits_backward(dg, idx, gate, logits, counts, AUX, w.k, T_total=w.T)
    dl = host(g["dlogits"][ts])
    assert np.abs(dl - dl_ref).max() <= 1e-5 * max(1.0, float(np.abs(dl_ref).max()))
    # dx of the sampled tokens: each of their rows through its own expert
    wg, wu, wd = inp["w_gate"], inp["w_up"], inp["w_down"]
    dx_ref = np.zeros((len(toks), w.d))
    row_gate = buf.row_gate.cpu().numpy().astype(np.float64)
    for a, t in enumerate(toks):
        for j in range(w.k):
            p = int(slot[a, j])
            if p < 0:
                continue
            le = int(np.searchsorted(offsets, p, side="right") - 1)
            x_row = to_f64(inp["x"][t:t + 1])
            _, dX, _ = oracle.experts_backward(dy[a:a + 1], np.array([0, 1]), np.array([0]),
                                               row_gate[p:p + 1], np.array([[0]]), x_row,
                                               to_f64(wg[le:le + 1]), to_f64(wu[le:le + 1]),
                                               to_f64(wd[le:le + 1]), 1)
            dx_ref[a] += dX[0]
    assert_close(host(g["dx_experts"][ts]), dx_ref, "bf16", "dx experts (sampled)", scale_atol=True)
    dxr_ref = oracle.router_backward(dl, to_f64(inp["w_router"]))
    assert_close(host(g["dx_router"][ts]), dxr_ref, "bf16", "dx router (sampled)")
