"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: ids, gates, counts, offsets, slots and rows for every token; logits,
expert rows and combined outputs on seeded samples the oracle computes one by
one; LoRA gradients for a sample of experts."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close, bf16_round, check_act_save, check_dispatch, check_route, expert_ref_rows,
                      host, rows_x, run_forward, say, upload)
from sparse_mixture_experts_top_amd import layer
from sparse_mixture_experts_top_amd import binding as B
from sparse_mixture_experts_top_amd.workloads import WORKLOADS, generate, to_f64

pytestmark = pytest.mark.gpu


def sampled_combine(w, buf, gate, tokens):
    """Oracle combine for sampled tokens, fed the GPU's expert rows."""
    slot = host(buf.slot)[tokens]
    rows = np.unique(slot[slot >= 0])
    o = host(buf.y_perm[torch.as_tensor(rows, device="cuda").long()]) if len(rows) else np.zeros((0, w.d))
    remap = -np.ones(max(int(slot.max()) + 1, 1), dtype=np.int64)
    remap[rows] = np.arange(len(rows))
    cslot = np.where(slot >= 0, remap[np.maximum(slot, 0)], -1)
    return oracle.combine(o, cslot, gate[tokens], len(tokens))


def full_case(name, prob=False, act_save=False):
    w = WORKLOADS[name]
    say(f"[case {name}] T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} L={w.L} cap={w.capacity}")
    inp = generate(w, seed=0)
    dev = upload(inp)
    # fused gather and packed weights, as bench.py runs it
    buf = run_forward(w, dev, prob=prob, act_save=act_save, x_perm=False, packed=True)
    rng = np.random.default_rng(123)
    ts = np.sort(rng.choice(w.T, 48, replace=False))
    lg, idx, gate = check_route(w, inp, buf, sample_tokens=ts)
    ref, R = check_dispatch(w, dev, buf, idx, gate)
    rows = np.sort(rng.choice(R, min(R, 384), replace=False))
    lora = {"scale": w.lora_alpha / w.lora_r} if w.lora_r else None
    o_ref = expert_ref_rows(w, inp, buf, rows, lora=lora)
    assert_close(host(buf.y_perm[torch.as_tensor(rows, device="cuda").long()]), o_ref, w.dtype,
                 "expert rows (sampled)", stored_bf16=True)
    tt = np.sort(rng.choice(w.T, 256, replace=False))
    assert_close(host(buf.y[torch.as_tensor(tt, device="cuda").long()]), sampled_combine(w, buf, gate, tt),
                 w.dtype, "combine (sampled tokens)")
    return w, inp, dev, buf, lg, R


@pytest.mark.parametrize("name", ["full_router", "ep64_rank", "skewed_capacity"])
def test_full_size(name):
    full_case(name)


def test_lora_step_full():
    w, inp, dev, buf, lg, R = full_case("lora_step", prob=True, act_save=True)
    B.moe_aux_loss(buf.shape, buf.counts, buf.prob_sum, w.aux_coef, buf.aux)
    p_ref = oracle.softmax_full(lg).sum(0)
    assert np.abs(host(buf.prob_sum) - p_ref).max() <= 1e-5 * np.abs(p_ref).max()
    a_ref = oracle.aux_loss(host(buf.counts), p_ref, w.T, w.k, w.aux_coef)
    say(f"  aux: gpu={buf.aux[0].item():.6e} oracle={a_ref[0]:.6e}")
    assert abs(buf.aux[0].item() - a_ref[0]) <= 1e-5 * abs(a_ref[0])
    L, r, d, f = w.L, w.lora_r, w.d, w.f
    grads = {n: torch.empty(s, dtype=torch.float32, device="cuda") for n, s in
             [("da_up", (L, r, d)), ("db_up", (L, f, r)), ("da_down", (L, r, f)), ("db_down", (L, d, r))]}
    lora = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"])
    xr, xs = layer.x_rows(buf, dev["x"])
    B.moe_lora_bwd(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                   buf.act_save, dev["w_down"], grads["da_up"], grads["db_up"], grads["da_down"],
                   grads["db_down"], buf.ws)
    # the packed variant the benchmark times (W_d^T packed once)
    dgu_p = torch.empty((L, f, d), dtype=torch.bfloat16, device="cuda")
    B.moe_pack_backward_weights(buf.shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
    gp = {n: torch.full_like(g, float("nan")) for n, g in grads.items()}
    B.moe_lora_bwd_packed(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                          buf.act_save, dgu_p, gp["da_up"], gp["db_up"], gp["da_down"], gp["db_down"], buf.ws)
    torch.cuda.synchronize()
    offsets = host(buf.offsets)
    dy64 = to_f64(inp["dy"])
    for le in range(L):        # every local expert
        a, b = int(offsets[le]), int(offsets[le + 1])
        sl = torch.arange(a, b, device="cuda")
        say(f"  expert {le}: {b - a} rows")
        # the saved G | H | U rows against the oracle's own
        parts = check_act_save(w, inp, buf, np.arange(a, b), lora={"scale": w.lora_alpha / r},
                               what=f"act_save[{le}]")
        act = host(buf.act_save[sl])
        lo = {"scale": w.lora_alpha / r,
              **{n: to_f64(inp[n][le:le + 1]) for n in ("a_up", "b_up", "a_down", "b_down")}}
        xe = rows_x(w, inp, buf, np.arange(a, b))
        args = (dy64, xe, np.array([0, b - a]), host(buf.row_src[sl]), buf.row_gate[sl].cpu().numpy())
        # fed the GPU's saved G and H, then the oracle's own: rounded to bf16
        # where act_save stores them and unrounded (max-abs scaled by
        # |ref|inf: neighbouring-bf16 roundings of G or H, and the stored
        # rows' relative rounding, stay in the sums)
        wd = to_f64(inp["w_down"][le:le + 1])
        g_ref = oracle.lora_backward(*args, act[:, :f], act[:, f:2 * f], wd, lo)
        g_own = oracle.lora_backward(*args, bf16_round(parts["G"]), bf16_round(parts["H"]), wd, lo)
        g_own64 = oracle.lora_backward(*args, parts["G"], parts["H"], wd, lo)
        for n in grads:
            assert_close(host(grads[n][le:le + 1]), g_ref[n], "bf16", f"{n}[{le}]")
            assert_close(host(gp[n][le:le + 1]), g_ref[n], "bf16", f"{n}[{le}] (packed)")
            assert_close(host(gp[n][le:le + 1]), g_own[n], "bf16", f"{n}[{le}] (packed, oracle G, H at bf16)",
                         scale_atol=True)
            assert_close(host(gp[n][le:le + 1]), g_own64[n], "bf16", f"{n}[{le}] (packed, oracle G, H unrounded)",
                         scale_atol=True)
