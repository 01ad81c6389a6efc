"""GPU parity of every stage against the oracle, on small shapes that span
several tiles with ragged tails, plus the edge cases. All calls go through the
C ABI (libmoe_mi355x.so)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close, bf16_round, check_act_save, check_dispatch, check_route, expert_ref_rows,
                      host, lora_of, rows_x, run_forward, say, upload)
from sparse_mixture_experts_top_amd import binding as B
from sparse_mixture_experts_top_amd import layer
from sparse_mixture_experts_top_amd.workloads import WORKLOADS, Workload, generate, to_f64

pytestmark = pytest.mark.gpu

W = Workload
SMALL = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    # router: 3 row tiles with a 44-row tail and a partial 40-wide expert tile
    "ragged_bf16": W("ragged_bf16", T=300, d=256, E=40, k=6, f=128),
    # three K steps (d = 192), a local expert range, f = 192 (3 gate/up column tiles)
    "local_bf16": W("local_bf16", T=520, d=192, E=24, k=5, f=192, e_lo=3, e_hi=17),
    # ~384 rows per expert: 3-4 row tiles per expert, 5 FFN column tiles
    "rows_bf16": W("rows_bf16", T=1024, d=128, E=8, k=3, f=320),
    # Zipf-skewed routing with drops
    "capacity_bf16": W("capacity_bf16", T=700, d=128, E=32, k=4, f=64, capacity=30, zipf_s=1.2),
    "capacity_f32": W("capacity_f32", T=200, d=48, E=12, k=3, f=20, e_lo=2, e_hi=10,
                      capacity=25, zipf_s=1.0, dtype="f32"),
    "k_equals_E_bf16": W("k_equals_E_bf16", T=130, d=64, E=8, k=8, f=64),
    "k1_bf16": W("k1_bf16", T=257, d=128, E=16, k=1, f=128),
    # ~300 rows per expert: the 320-row tiles (one row tile per expert, some
    # experts with a second, ragged one), local range
    "wide_bf16": W("wide_bf16", T=1200, d=256, E=16, k=4, f=128, e_lo=2, e_hi=13),
    # 320-row tiles with two K steps (d = 64) and two or more items per
    # workgroup: the weight ring's lead exceeds a workgroup's whole sequence
    "tall_shortk_bf16": W("tall_shortk_bf16", T=8192, d=64, E=64, k=2, f=512),
    # the same with four K steps (packed weights need d % 128 == 0)
    "tall_k128_bf16": W("tall_k128_bf16", T=8192, d=128, E=64, k=2, f=512),
    # ~150 rows per expert: two 128-row tiles per expert, the second ragged,
    # a local range, 3 gate/up column tiles
    "mid_bf16": W("mid_bf16", T=600, d=128, E=16, k=4, f=192, e_lo=1, e_hi=14),
    # capacity 160 under Zipf skew: the hot experts at capacity span two
    # 128-row tiles that share each weight tile
    "mid_capacity_bf16": W("mid_capacity_bf16", T=2000, d=128, E=64, k=4, f=128, capacity=160, zipf_s=1.2),
    # router on 256 x 224 tiles (64 x 4 = 256 of them) with a partial last
    # column tile (880 = 3 x 224 + 208)
    "router_wide_bf16": W("router_wide_bf16", T=16384, d=128, E=880, k=4, f=64),
}


def run_and_check(w, seed=0, x_perm=True, packed=False):
    say(f"[case {w.name}] T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} local=[{w.e_lo},{w.local_hi}) "
        f"cap={w.capacity} dtype={w.dtype} x_perm={x_perm} packed={packed}")
    inp = generate(w, seed=seed)
    dev = upload(inp)
    buf = run_forward(w, dev, x_perm=x_perm, packed=packed)
    lg, idx, gate = check_route(w, inp, buf)
    ref, R = check_dispatch(w, dev, buf, idx, gate)
    rows = np.arange(R)
    o_ref = expert_ref_rows(w, inp, buf, rows)
    o_gpu = host(buf.y_perm[:R]) if R else np.zeros((0, w.d))
    if R:
        assert_close(o_gpu, o_ref, w.dtype, "expert rows", stored_bf16=True)
    y_ref = oracle.combine(o_gpu, host(buf.slot), gate, w.T)
    assert_close(host(buf.y), y_ref, w.dtype, "combine")
    return inp, dev, buf


@pytest.mark.parametrize("name", sorted(SMALL))
def test_stagewise_parity(name):
    run_and_check(SMALL[name])


@pytest.mark.parametrize("name", ["tiny_f32", "ragged_bf16", "local_bf16", "rows_bf16", "capacity_bf16",
                                  "wide_bf16", "mid_capacity_bf16"])
def test_stagewise_parity_fused_gather(name):
    """The expert GEMM reading x through row_src (no x_perm copy)."""
    run_and_check(SMALL[name], seed=7, x_perm=False)


@pytest.mark.parametrize("name", ["tiny_f32", "ragged_bf16", "capacity_bf16"])
def test_end_to_end_from_scratch(name):
    """y against the oracle run from scratch in float64; tokens whose selection
    differs are allowed only when the oracle's k-th / (k+1)-th logit gap is
    within twice the fp32 logit error bound."""
    w = SMALL[name]
    inp = generate(w, seed=1)
    dev = upload(inp)
    buf = run_forward(w, dev)
    f = lambda n: to_f64(inp.get(n))
    ref = oracle.moe_layer(f("x"), f("w_router"), f("w_gate"), f("w_up"), f("w_down"), w.k,
                           bias=f("bias"), e_lo=w.e_lo, e_hi=w.local_hi, capacity=w.capacity)
    idx = host(buf.topk_idx)
    differ = np.nonzero((idx != ref["idx"]).any(1))[0]
    if len(differ):
        from gpu_util import logit_bound
        lb = logit_bound(f("x")[differ], f("w_router"), f("bias")).max(1)
        srt = -np.sort(-ref["logits"][differ], axis=1)
        gap = srt[:, w.k - 1] - srt[:, w.k]
        assert np.all(gap <= 2 * lb), "a selection differs away from a near-tie"
    keep = np.setdiff1d(np.arange(w.T), differ)
    if w.capacity > 0:
        # capacity ranks by gate, so a near-tie anywhere in a capped expert may move a
        # drop; compare only tokens whose kept slots agree
        same = ((host(buf.slot) >= 0) == (ref["slot"] >= 0)).all(1)
        keep = np.intersect1d(keep, np.nonzero(same)[0])
    say(f"  tokens compared: {len(keep)} of {w.T}")
    assert len(keep) >= 0.9 * w.T
    assert_close(host(buf.y)[keep], ref["y"][keep], w.dtype, "y from scratch")


def test_deterministic_bitwise():
    w = SMALL["capacity_bf16"]
    inp = generate(w, seed=2)
    dev = upload(inp)
    a = run_forward(w, dev)
    b = run_forward(w, dev)
    for n in ("topk_idx", "topk_gate", "logits", "counts", "offsets", "slot", "y"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    R = int(a.offsets[-1].item())
    for n in ("row_src", "row_gate", "x_perm", "y_perm"):
        assert torch.equal(getattr(a, n)[:R], getattr(b, n)[:R]), n


def test_zero_input_ties_and_uniform_gates():
    w = W("zeros_bf16", T=70, d=128, E=24, k=5, f=64)
    inp = generate(w, seed=3)
    inp["x"] = torch.zeros_like(inp["x"])
    dev = upload(inp)
    buf = run_forward(w, dev)
    assert (host(buf.topk_idx) == np.arange(5)[None, :]).all()
    assert (buf.topk_gate == 0.2).all()      # exp(0)/5, the fp32 nearest to 1/5 on both sides
    assert (host(buf.y) == 0).all()


def test_capacity_with_every_gate_tied():
    """Zero input: every token picks experts 0..4 with gate 1/5, so each of
    them has T candidates for C places, all tied at g*. The tie rule keeps
    the C lowest tokens, in token order: slot[t, j] = j C + t for t < C,
    else -1 (the capacity search runs all 32 bits here: no prefix ever has
    exactly C candidates at or above it)."""
    C = 20
    w = W("zeros_cap_bf16", T=70, d=128, E=24, k=5, f=64, capacity=C)
    inp = generate(w, seed=3)
    inp["x"] = torch.zeros_like(inp["x"])
    dev = upload(inp)
    buf = run_forward(w, dev)
    slot = host(buf.slot)
    t = np.arange(w.T)[:, None]
    want = np.where(t < C, np.arange(w.k)[None, :] * C + t, -1)
    assert (slot == want).all()
    R = int(host(buf.offsets)[-1])
    assert R == w.k * C
    assert (host(buf.row_src[:R]) == np.tile(np.arange(C), w.k)).all()
    assert (buf.row_gate[:R] == 0.2).all()


def test_empty_batch():
    w = W("empty", T=0, d=128, E=16, k=4, f=64)
    shape = layer.shape_of(w)
    buf = layer.alloc(shape, prob=True)
    buf.counts.fill_(-7)
    buf.offsets.fill_(-7)
    buf.prob_sum.fill_(-7)
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    layer.forward(buf, z(0, 128), z(16, 128), None, z(16, 64, 128), z(16, 64, 128), z(16, 128, 64))
    torch.cuda.synchronize()
    assert (buf.counts == 0).all() and (buf.offsets == 0).all() and (buf.prob_sum == 0).all()


def _bits(t):
    return host(t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny_f32", "ragged_bf16", "local_bf16", "capacity_bf16", "capacity_f32",
                                  "k1_bf16", "router_wide_bf16"])
def test_route_dispatch_fused_equals_separate(name):
    """moe_route_dispatch (histogram folded into the top-k kernel) against
    moe_route + moe_dispatch: every output bitwise equal, on two calls in a
    row on the same workspace (the histogram is cleared by each call)."""
    w = SMALL[name]
    say(f"[case {name}] fused route+dispatch vs separate")
    inp = generate(w, seed=3)
    dev = upload(inp)
    s = layer.shape_of(w)
    sep = layer.alloc(s, logits=True, prob=True, x_perm=True)
    fus = layer.alloc(s, logits=True, prob=True, x_perm=True)
    args = (dev["x"], dev["w_router"], dev.get("bias"))
    B.moe_route(s, *args, sep.topk_idx, sep.topk_gate, sep.logits, sep.prob_sum, sep.ws)
    B.moe_dispatch(s, sep.topk_idx, sep.topk_gate, dev["x"], sep.counts, sep.offsets, sep.slot, sep.row_src,
                   sep.row_gate, sep.x_perm, sep.dropped, sep.ws)
    for rep in range(2):
        fus.ws.fill_(0x5A if rep else 0)
        B.moe_route_dispatch(s, *args, fus.topk_idx, fus.topk_gate, fus.logits, fus.prob_sum, fus.counts,
                             fus.offsets, fus.slot, fus.row_src, fus.row_gate, fus.x_perm, fus.dropped, fus.ws)
        torch.cuda.synchronize()
        R = int(host(sep.offsets)[-1])
        assert int(host(fus.offsets)[-1]) == R
        for n in ("topk_idx", "counts", "offsets", "slot", "dropped"):
            assert (host(getattr(fus, n)) == host(getattr(sep, n))).all(), n
        for n in ("topk_gate", "logits", "prob_sum"):
            assert (_bits(getattr(fus, n)) == _bits(getattr(sep, n))).all(), n
        assert (host(fus.row_src[:R]) == host(sep.row_src[:R])).all()
        assert (_bits(fus.row_gate[:R]) == _bits(sep.row_gate[:R])).all()
        assert (_bits(fus.x_perm[:R]) == _bits(sep.x_perm[:R])).all()


def test_no_local_assignment():
    """Every token prefers experts 0..3 (large bias) while the local range is
    12..15: no rows, y is all zero, slots all -1."""
    w = W("nolocal", T=90, d=64, E=16, k=4, f=64, e_lo=12, e_hi=16, zipf_s=0.0)
    inp = generate(w, seed=4)
    inp["bias"] = torch.tensor([50.0] * 4 + [0.0] * 12)
    dev = upload(inp)
    buf = run_forward(w, dev)
    assert int(buf.offsets[-1].item()) == 0
    assert (buf.slot == -1).all() and (host(buf.y) == 0).all()


def test_lora_no_local_rows_gives_zero_gradients():
    """No token picks a local expert (large bias on experts 0..3, local range
    12..15): the forward has no rows and every adapter gradient element is
    written as exactly 0, through both the plain and the packed backward."""
    w = W("lora_nolocal", T=90, d=128, E=16, k=4, f=128, e_lo=12, e_hi=16, lora_r=16, lora_alpha=32.0,
          lora_b="normal", aux_coef=0.01)
    inp = generate(w, seed=4)
    inp["bias"] = torch.tensor([50.0] * 4 + [0.0] * 12)
    dev = upload(inp)
    buf = run_forward(w, dev, act_save=True, x_perm=False, packed=True)
    assert int(buf.offsets[-1].item()) == 0 and (host(buf.y) == 0).all()
    L, r = w.L, w.lora_r
    lora = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"])
    dgu_p = torch.empty((L, w.f, w.d), dtype=torch.bfloat16, device="cuda")
    B.moe_pack_backward_weights(buf.shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
    xr, xs = layer.x_rows(buf, dev["x"])
    for packed in (False, True):
        g = [torch.full(sz, float("nan"), device="cuda") for sz in ((L, r, w.d), (L, w.f, r), (L, r, w.f), (L, w.d, r))]
        if packed:
            B.moe_lora_bwd_packed(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                                  buf.act_save, dgu_p, *g, buf.ws)
        else:
            B.moe_lora_bwd(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                           buf.act_save, dev["w_down"], *g, buf.ws)
        torch.cuda.synchronize()
        assert all((t == 0).all() for t in g), f"packed={packed}"


def test_capacity_one_everywhere():
    w = W("cap1", T=64, d=64, E=8, k=2, f=64, capacity=1)
    inp = generate(w, seed=5)
    dev = upload(inp)
    buf = run_forward(w, dev)
    lg, idx, gate = check_route(w, inp, buf)
    ref, R = check_dispatch(w, dev, buf, idx, gate)
    assert R == int((ref["counts"] > 0).sum())


@pytest.mark.parametrize("name", ["ragged_bf16", "rows_bf16", "capacity_bf16", "k1_bf16", "wide_bf16",
                                  "tall_k128_bf16", "mid_bf16", "mid_capacity_bf16"])
def test_stagewise_parity_packed_weights(name):
    """Expert weights streamed from their packed copies (fused gather too)."""
    run_and_check(SMALL[name], seed=8, x_perm=False, packed=True)


def test_packed_weights_bitwise_equal_and_permutation():
    """Packing only moves values: the packed buffers hold the same multiset of
    bf16 values, and the packed GEMM reproduces the row-major one bitwise."""
    w = SMALL["rows_bf16"]
    inp = generate(w, seed=9)
    dev = upload(inp)
    shape = layer.shape_of(w)
    gu, dn = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    srt = lambda t: torch.sort(t.float().flatten())[0]
    assert torch.equal(srt(gu), srt(torch.cat([dev["w_gate"], dev["w_up"]], 1)))
    assert torch.equal(srt(dn), srt(dev["w_down"]))
    a = run_forward(w, dev, x_perm=False, packed=False)
    b = run_forward(w, dev, x_perm=False, packed=True)
    R = int(a.offsets[-1].item())
    assert torch.equal(a.y_perm[:R], b.y_perm[:R]) and torch.equal(a.y, b.y)


def _chunk_key(r):
    return (r >> 1) & 3


def test_packed_weights_documented_layout():
    """The packed buffers follow the tile layout the header documents: 8 KB
    tiles of 128 rows x 32 K values, gate/up rows interleaved per 16, chunk c
    of row r at position c ^ key(r). The expected buffers are built on the
    host by index arithmetic from that description."""
    w = SMALL["rows_bf16"]
    dev = upload(generate(w, seed=10))
    shape = layer.shape_of(w)
    gu, dn = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    wg, wu, wd = (dev[n].cpu() for n in ("w_gate", "w_up", "w_down"))
    L, f, d = wg.shape
    jb = torch.arange(128)
    key = _chunk_key(jb)
    c = torch.arange(4)[None, :] ^ key[:, None]                      # [128 rows, 4 slots]
    kk = c[:, :, None] * 8 + torch.arange(8)[None, None, :]          # [128, 4, 8] K offset in step
    # gate/up: tile (le, b, kt); row jb -> 16-row block q = jb // 32, gate if (jb // 16) even
    frag = jb >> 4
    col = (frag >> 1) * 16 + (jb & 15)
    both = torch.stack([wg, wu])                                     # [2, L, f, d]
    nt, nk = f // 64, d // 32
    le = torch.arange(L)[:, None, None, None, None, None]
    b = torch.arange(nt)[None, :, None, None, None, None]
    kt = torch.arange(nk)[None, None, :, None, None, None]
    src = (frag & 1)[None, None, None, :, None, None]
    row = b * 64 + col[None, None, None, :, None, None]
    kidx = kt * 32 + kk[None, None, None]
    exp_gu = both[src, le, row, kidx].reshape(-1)
    assert torch.equal(gu.cpu().reshape(-1), exp_gu)
    # down: tile (le, b < d/128, kt < f/32), rows 128b + jb
    nt, nk = d // 128, f // 32
    b = torch.arange(nt)[None, :, None, None, None, None]
    kt = torch.arange(nk)[None, None, :, None, None, None]
    row = b * 128 + jb[None, None, None, :, None, None]
    exp_dn = wd[le, row, kt * 32 + kk[None, None, None]].reshape(-1)
    assert torch.equal(dn.cpu().reshape(-1), exp_dn)


def test_packed_weights_need_d_multiple_of_128():
    w = SMALL["local_bf16"]            # d = 192
    shape = layer.shape_of(w)
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_pack_expert_weights(shape, z(w.L, w.f, w.d), z(w.L, w.f, w.d), z(w.L, w.d, w.f),
                                  z(w.L, 2 * w.f, w.d), z(w.L, w.d, w.f))
    assert e.value.status == B.MOE_ERR_UNSUPPORTED


# r = 16 carries the adapter terms through the matrix cores (one extra K
# step); other ranks take the fp32 epilogue path. d = f = 192 (not a multiple
# of 128) sends the gradient sums with bf16 rows to the VALU form instead of
# the matrix-core one.
@pytest.mark.parametrize("b_init,x_perm,r,packed,dims", [("normal", True, 16, False, 128),
                                                         ("normal", False, 16, False, 128),
                                                         ("zero", False, 16, False, 128),
                                                         ("normal", False, 8, False, 128),
                                                         ("normal", False, 16, True, 128),
                                                         ("normal", False, 16, False, 192)])
def test_lora_forward_backward_and_aux(b_init, x_perm, r, packed, dims):
    w = W("lora_small", T=256, d=dims, E=12, k=4, f=dims, e_lo=2, e_hi=9, lora_r=r,
          lora_alpha=32.0, lora_b=b_init, aux_coef=0.01)
    check_lora(w, x_perm, packed)


def check_lora(w, x_perm, packed, seed=6):
    """Forward with LoRA (rows, saved G | H | U, softmax sums, aux loss), then
    the adapter gradients against the oracle three ways, plain and packed."""
    b_init, r = w.lora_b, w.lora_r
    say(f"[case {w.name} b={b_init} x_perm={x_perm} r={r} packed={packed} d={w.d} f={w.f}]")
    inp = generate(w, seed=seed)
    dev = upload(inp)
    buf = run_forward(w, dev, prob=True, act_save=True, x_perm=x_perm, packed=packed)
    lg, idx, gate = check_route(w, inp, buf)
    ref, R = check_dispatch(w, dev, buf, idx, gate)
    lo64 = {"scale": w.lora_alpha / w.lora_r}
    o_ref = expert_ref_rows(w, inp, buf, np.arange(R), lora=lo64)
    # with s = alpha / r up to 32 the adapter term can make rows large (|O| ~ 15
    # at r = 1), and the bf16 H fed to the down product carries a relative
    # rounding into them: the max-abs bound scales with max(1, |O|inf)
    assert_close(host(buf.y_perm[:R]), o_ref, "bf16", "expert rows (LoRA)", stored_bf16=True, scale_atol=True)
    # the saved G | H | U rows the backward reads, against the oracle's own
    parts = check_act_save(w, inp, buf, np.arange(R), lora=lo64)
    # aux loss from the GPU counts and probabilities
    B.moe_aux_loss(buf.shape, buf.counts, buf.prob_sum, w.aux_coef, buf.aux)
    p_ref = oracle.softmax_full(lg).sum(0)
    assert np.abs(host(buf.prob_sum) - p_ref).max() <= 1e-5 * np.abs(p_ref).max()
    a_ref = oracle.aux_loss(host(buf.counts), p_ref, w.T, w.k, w.aux_coef)
    assert abs(buf.aux[0].item() - a_ref[0]) <= 1e-5 * abs(a_ref[0]) + 1e-9
    assert abs(buf.aux[1].item() - a_ref[1]) <= 1e-5 * abs(a_ref[1])
    # adapter gradients, oracle fed the GPU's saved G and H
    L, r = w.L, w.lora_r
    grads = {n: torch.empty(s, dtype=torch.float32, device="cuda") for n, s in
             [("da_up", (L, r, w.d)), ("db_up", (L, w.f, r)), ("da_down", (L, r, w.f)),
              ("db_down", (L, w.d, r))]}
    lora = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"])
    xr, xs = layer.x_rows(buf, dev["x"])
    B.moe_lora_bwd(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                   buf.act_save, dev["w_down"], grads["da_up"], grads["db_up"], grads["da_down"],
                   grads["db_down"], buf.ws)
    torch.cuda.synchronize()
    act = host(buf.act_save[:R])
    lo = {"scale": w.lora_alpha / w.lora_r, **{n: to_f64(inp[n]) for n in ("a_up", "b_up", "a_down", "b_down")}}
    g_ref = oracle.lora_backward(to_f64(inp["dy"]), rows_x(w, inp, buf, np.arange(R)), host(buf.offsets),
                                 host(buf.row_src[:R]), buf.row_gate[:R].cpu().numpy(),
                                 act[:, :w.f], act[:, w.f:2 * w.f], to_f64(inp["w_down"]), lo)
    for n in grads:
        assert_close(host(grads[n]), g_ref[n], "bf16", n)
    # the same gradients from the oracle's own G and H (nothing the GPU
    # saved), rounded to bf16 where act_save stores them and unrounded. Both
    # carry a relative rounding into the gradient sums: unrounded, the stored
    # rows' (random-sign sums); rounded, the elements where the GPU's
    # fp32-accumulated G or H rounds to the neighbouring bf16 value. So the
    # max-abs bound scales with |ref|inf for both (the GPU's own G and H above
    # keep the plain one)
    args = (to_f64(inp["dy"]), rows_x(w, inp, buf, np.arange(R)), host(buf.offsets),
            host(buf.row_src[:R]), buf.row_gate[:R].cpu().numpy())
    g_own = oracle.lora_backward(*args, bf16_round(parts["G"]), bf16_round(parts["H"]),
                                 to_f64(inp["w_down"]), lo)
    g_own64 = oracle.lora_backward(*args, parts["G"], parts["H"], to_f64(inp["w_down"]), lo)
    for n in grads:
        assert_close(host(grads[n]), g_own[n], "bf16", n + " (oracle G, H at bf16)", scale_atol=True)
        assert_close(host(grads[n]), g_own64[n], "bf16", n + " (oracle G, H unrounded)", scale_atol=True)
    # the same gradients with W_d^T packed once (the dH product on the DMA
    # engine; the packed transposes need d, f % 128 == 0)
    gp = None
    if w.d % 128 == 0 and w.f % 128 == 0:
        dgu_p = torch.empty((L, w.f, w.d), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_backward_weights(buf.shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
        gp = {n: torch.full_like(g, float("nan")) for n, g in grads.items()}
        B.moe_lora_bwd_packed(buf.shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                              buf.act_save, dgu_p, gp["da_up"], gp["db_up"], gp["da_down"], gp["db_down"], buf.ws)
        torch.cuda.synchronize()
        for n in grads:
            assert_close(host(gp[n]), g_ref[n], "bf16", n + " (packed)")
    if b_init == "zero":
        assert (grads["da_up"] == 0).all() and (grads["da_down"] == 0).all()
        if gp is not None:
            assert (gp["da_up"] == 0).all() and (gp["da_down"] == 0).all()
        frozen = run_forward(w.replace(lora_r=0), dev, x_perm=x_perm)
        assert torch.equal(frozen.y, buf.y)


@pytest.mark.parametrize("r,packed,dims", [(16, True, 128), (16, False, 128), (8, False, 128), (16, False, 192)])
def test_lora_saved_projections(r, packed, dims):
    """z_save: the forward keeps Z_u = X A_up^T and Z_d = H A_down^T (checked
    against float64 products of the rows the GPU used, within the fp32
    accumulation bound), its own outputs unchanged, and the backward reading
    them gives the gradients of the backward that projects again, bitwise."""
    w = W("lora_zsave", T=256, d=dims, E=12, k=4, f=dims, e_lo=2, e_hi=9, lora_r=r,
          lora_alpha=32.0, lora_b="normal", aux_coef=0.01)
    say(f"[case lora z_save r={r} packed={packed} d=f={dims}]")
    inp = generate(w, seed=13)
    dev = upload(inp)
    shape = layer.shape_of(w)
    L, rmax = w.L, B.moe_max_rows(shape)
    pk = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"]) if packed else None
    fwd = lambda b, lo: layer.forward(b, dev["x"], dev["w_router"], dev.get("bias"), dev["w_gate"], dev["w_up"],
                                      dev["w_down"], lo, packed=pk)
    plain = layer.alloc(shape, lora_r=r, act_save=True)
    fwd(plain, lora_of(w, dev))
    z_save = torch.full((2, rmax, r), float("nan"), dtype=torch.float32, device="cuda")
    lo_z = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"], z_save)
    buf = layer.alloc(shape, lora_r=r, act_save=True)
    fwd(buf, lo_z)
    torch.cuda.synchronize()
    R = int(host(buf.offsets)[-1])
    assert R > 0 and torch.equal(buf.y_perm[:R], plain.y_perm[:R]) and torch.equal(buf.act_save[:R], plain.act_save[:R])
    # the kept projections against float64 products of the same rows
    off = host(buf.offsets)
    le_of = np.searchsorted(off, np.arange(R), side="right") - 1
    X = rows_x(w, inp, buf, np.arange(R))
    H = host(buf.act_save[:R])[:, w.f:2 * w.f]
    for part, (rows, A) in enumerate(((X, to_f64(inp["a_up"])), (H, to_f64(inp["a_down"])))):
        ref = np.einsum("pk,pqk->pq", rows, A[le_of])
        # fp32 accumulation over K products (exact in fp32): |err| <= K u sum |x a|
        K = rows.shape[1]
        bound = (K + 8) * 2.0 ** -24 * np.einsum("pk,pqk->pq", np.abs(rows), np.abs(A[le_of])) + 1e-30
        got = host(z_save[part, :R])
        assert np.all(np.abs(got - ref) <= bound), f"z_save[{part}]"
    # gradients: kept projections vs projected again, bitwise
    xr, xs = layer.x_rows(buf, dev["x"])
    shapes = ((L, r, w.d), (L, w.f, r), (L, r, w.f), (L, w.d, r))
    dgu_p = None
    if dims % 128 == 0:
        dgu_p = torch.empty((L, w.f, w.d), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_backward_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
    for bwd_packed in ((False, True) if dgu_p is not None else (False,)):
        out = []
        for lo in (lora_of(w, dev), lo_z):
            g = [torch.full(sz, float("nan"), device="cuda") for sz in shapes]
            if bwd_packed:
                B.moe_lora_bwd_packed(shape, lo, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                                      buf.act_save, dgu_p, *g, buf.ws)
            else:
                B.moe_lora_bwd(shape, lo, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs, buf.act_save,
                               dev["w_down"], *g, buf.ws)
            out.append(g)
        torch.cuda.synchronize()
        for a, b in zip(*out):
            assert torch.equal(a, b), f"bwd_packed={bwd_packed}"


@pytest.mark.parametrize("name", ["rows_bf16", "capacity_bf16"])
def test_forward_graph_replays_match_eager(name):
    """The whole forward captured into one HIP graph: every replay (with eager
    work and synchronisations in between, outputs cleared before each one)
    reproduces the eager forward bitwise."""
    w = SMALL[name]
    say(f"[case graph {name}]")
    dev = upload(generate(w, seed=11))
    shape = layer.shape_of(w)
    buf = layer.alloc(shape, logits=True)
    pk = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    fw = lambda: layer.forward(buf, dev["x"], dev["w_router"], dev.get("bias"), None, None, None,
                               packed=pk)
    fw()
    torch.cuda.synchronize()
    outs = ("topk_idx", "topk_gate", "logits", "counts", "offsets", "slot", "row_src", "row_gate",
            "y_perm", "y")
    R = int(buf.offsets[-1].item())
    rowwise = ("row_src", "row_gate", "y_perm")  # only the R dispatched rows are written
    view = lambda n: getattr(buf, n)[:R] if n in rowwise else getattr(buf, n)
    ref = {n: view(n).clone() for n in outs}
    g = layer.capture(fw)
    for rep in range(3):
        for n in outs:
            getattr(buf, n).fill_(-1 if getattr(buf, n).dtype == torch.int32 else 7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(view(n), ref[n]), (rep, n)
        fw()  # eager work between replays
        torch.cuda.synchronize()


def test_lora_step_deterministic_and_graph_replays_match_eager():
    """The whole LoRA step (forward with adapters and softmax sums, load-balance
    loss, packed adapter backward) gives bitwise equal results on two eager
    runs, and captured as one HIP graph every replay (outputs cleared before
    each, eager work in between) reproduces the eager results bitwise."""
    w = W("lora_graph", T=300, d=256, E=16, k=4, f=128, e_lo=2, e_hi=13, lora_r=16, lora_alpha=32.0,
          lora_b="normal", aux_coef=0.01)
    say("[case lora step graph]")
    inp = generate(w, seed=12)
    dev = upload(inp)
    shape = layer.shape_of(w)
    L, r = w.L, w.lora_r
    buf = layer.alloc(shape, lora_r=r, prob=True, act_save=True)
    pk = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    dgu_p = torch.empty((L, w.f, w.d), dtype=torch.bfloat16, device="cuda")
    B.moe_pack_backward_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_p, None)
    lora = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"])
    grads = [torch.empty(sz, device="cuda") for sz in ((L, r, w.d), (L, w.f, r), (L, r, w.f), (L, w.d, r))]

    def step():
        layer.forward(buf, dev["x"], dev["w_router"], None, None, None, None, lora, packed=pk)
        B.moe_aux_loss(shape, buf.counts, buf.prob_sum, w.aux_coef, buf.aux)
        xr, xs = layer.x_rows(buf, dev["x"])
        B.moe_lora_bwd_packed(shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                              buf.act_save, dgu_p, *grads, buf.ws)

    outs = lambda: [buf.topk_idx, buf.topk_gate, buf.prob_sum, buf.y, buf.aux, *grads]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]
    step()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, outs())):
        assert torch.equal(a, b), f"eager rerun differs in output {i}"
    g = layer.capture(step)
    for rep in range(3):
        for t in outs():
            t.fill_(-1 if t.dtype == torch.int32 else 7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs())):
            assert torch.equal(a, b), (rep, i)
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,need", [(12000, 8192), (20000, 16384)])
def test_capacity_large_expert(T, need):
    """One expert receives nearly every token: more candidates than the
    capacity kernel stages in LDS (> 8192: read from global memory) and, at
    T = 20000, more than one chunk of rounds (> 16384). Dispatch stays
    bit-exact against the oracle."""
    w = W(f"bigcap_{T}", T=T, d=64, E=8, k=1, f=64, capacity=2500, zipf_s=12.0)
    inp, dev, buf = run_and_check(w, seed=3, x_perm=False)
    assert int(buf.counts.max().item()) > need
