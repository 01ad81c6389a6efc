"""Pins for the oracle's full backward of the layer (gradients of
sum(y * dY) + L_aux with respect to the input rows and the router logits):
central finite differences of the independently pinned forward, closed
forms and invariants."""
import math

import numpy as np
import pytest

import oracle

H = 1e-6


def _silu_fd(a):
    return (oracle.silu(a + H) - oracle.silu(a - H)) / (2 * H)


def test_silu_grad_closed_form_and_differences():
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5      # sigma(0) (1 + 0)
    s1 = 1 / (1 + math.exp(-1))
    assert abs(oracle.silu_grad(np.array([1.0]))[0] - s1 * (2 - s1)) < 1e-15
    a = np.linspace(-6, 6, 25)
    assert np.abs(oracle.silu_grad(a) - _silu_fd(a)).max() < 1e-8


def _problem(seed, T=6, d=5, E=5, k=2, f=3, L=None, e_lo=0, capacity=0, lora=False, bias=False):
    rng = np.random.default_rng(seed)
    L = E if L is None else L
    p = {
        "x": rng.normal(size=(T, d)),
        "w_router": rng.normal(size=(E, d)) / math.sqrt(d),
        "w_gate": rng.normal(size=(L, f, d)) / math.sqrt(d),
        "w_up": rng.normal(size=(L, f, d)) / math.sqrt(d),
        "w_down": rng.normal(size=(L, d, f)) / math.sqrt(f),
        "dy": rng.normal(size=(T, d)),
        "k": k, "e_lo": e_lo, "e_hi": e_lo + L, "capacity": capacity,
        "bias": rng.normal(size=E) if bias else None,
        "lora": None,
    }
    if lora:
        r = 2
        p["lora"] = {"scale": 1.5, "a_up": rng.normal(size=(L, r, d)) * 0.3,
                     "b_up": rng.normal(size=(L, f, r)) * 0.3,
                     "a_down": rng.normal(size=(L, r, f)) * 0.3,
                     "b_down": rng.normal(size=(L, d, r)) * 0.3}
    return p


def _forward(p, x, aux_coef):
    return oracle.moe_layer(x, p["w_router"], p["w_gate"], p["w_up"], p["w_down"], p["k"],
                            bias=p["bias"], e_lo=p["e_lo"], e_hi=p["e_hi"], capacity=p["capacity"],
                            lora=p["lora"], aux_coef=aux_coef)


def _loss(fwd, dy):
    return float(np.sum(fwd["y"] * dy)) + float(fwd["aux"][0])


CASES = [
    dict(seed=1),
    dict(seed=2, bias=True),
    dict(seed=3, E=7, L=3, e_lo=2),                      # one rank's local experts
    dict(seed=4, T=10, E=4, k=2, capacity=3),            # capacity drops
    dict(seed=5, lora=True),
    dict(seed=6, k=1),
    dict(seed=7, k=5, E=5),                              # k = E
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{a}{b}" for a, b in c.items()))
@pytest.mark.parametrize("aux_coef", [0.0, 0.3])
def test_dx_matches_central_differences(case, aux_coef):
    p = _problem(**case)
    x, dy, T = p["x"], p["dy"], p["x"].shape[0]
    fwd = _forward(p, x, aux_coef)
    got = oracle.moe_layer_backward(fwd, dy, x, p["w_router"], p["w_gate"], p["w_up"], p["w_down"],
                                    p["k"], T, lora=p["lora"], aux_coef=aux_coef)
    fd = np.zeros_like(x)
    for t in range(T):
        for i in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[t, i] += H
            xm[t, i] -= H
            fp, fm = _forward(p, xp, aux_coef), _forward(p, xm, aux_coef)
            # the selection and the capacity decisions must not move
            assert (fp["idx"] == fwd["idx"]).all() and (fm["idx"] == fwd["idx"]).all()
            assert (fp["slot"] == fwd["slot"]).all() and (fm["slot"] == fwd["slot"]).all()
            fd[t, i] = (_loss(fp, dy) - _loss(fm, dy)) / (2 * H)
    scale = max(1.0, np.abs(fd).max())
    assert np.abs(got["dx"] - fd).max() < 1e-6 * scale


@pytest.mark.parametrize("case", CASES[:5], ids=lambda c: "-".join(f"{a}{b}" for a, b in c.items()))
def test_dlogits_matches_central_differences(case):
    """L(l) = sum_t sum_j [kept] g_tj(l) <dY_t, O_row> + L_aux(l), with the
    expert outputs O fixed and the selection held."""
    p = _problem(**case)
    coef = 0.3
    x, dy, T = p["x"], p["dy"], p["x"].shape[0]
    fwd = _forward(p, x, coef)
    E = p["w_router"].shape[0]
    dg = oracle.gate_backward(dy, fwd["o"], fwd["slot"], fwd["gate"], T)
    got = oracle.logits_backward(dg, fwd["idx"], fwd["gate"], fwd["logits"], fwd["counts"], coef, p["k"])

    def loss_of(l):
        g = oracle.topk_gates(l, fwd["idx"])
        y = oracle.combine(fwd["o"], fwd["slot"], g, T)
        prob_sum = oracle.softmax_full(l).sum(0)
        return float(np.sum(y * dy)) + oracle.aux_loss(fwd["counts"], prob_sum, T, p["k"], coef)[0]

    l0 = fwd["logits"]
    fd = np.zeros_like(l0)
    for t in range(T):
        for e in range(E):
            lp, lm = l0.copy(), l0.copy()
            lp[t, e] += H
            lm[t, e] -= H
            fd[t, e] = (loss_of(lp) - loss_of(lm)) / (2 * H)
    assert np.abs(got - fd).max() < 1e-6 * max(1.0, np.abs(fd).max())


def test_dlogits_rows_sum_to_zero_and_k1_gate_path_vanishes():
    p = _problem(seed=11, T=8, E=6, k=3)
    fwd = _forward(p, p["x"], 0.2)
    dg = oracle.gate_backward(p["dy"], fwd["o"], fwd["slot"], fwd["gate"], 8)
    dl = oracle.logits_backward(dg, fwd["idx"], fwd["gate"], fwd["logits"], fwd["counts"], 0.2, 3)
    # softmax is invariant to a shift of all logits of a token
    assert np.abs(dl.sum(axis=1)).max() < 1e-12
    # k = 1: g = 1 whatever the logits, so the gate path contributes nothing
    p1 = _problem(seed=12, T=8, E=6, k=1)
    f1 = _forward(p1, p1["x"], 0.0)
    dg1 = oracle.gate_backward(p1["dy"], f1["o"], f1["slot"], f1["gate"], 8)
    assert (oracle.logits_backward(dg1, f1["idx"], f1["gate"], f1["logits"]) == 0).all()


def test_lora_with_zero_b_leaves_the_expert_backward_unchanged():
    p = _problem(seed=13, lora=True)
    for n in ("b_up", "b_down"):
        p["lora"][n] = np.zeros_like(p["lora"][n])
    fwd = _forward(p, p["x"], 0.0)
    args = (p["dy"], fwd["offsets"], fwd["row_src"], fwd["row_gate"], fwd["slot"], fwd["x_perm"],
            p["w_gate"], p["w_up"], p["w_down"], 6)
    a = oracle.experts_backward(*args, lora=p["lora"])
    b = oracle.experts_backward(*args)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_dx_is_linear_in_dy_and_zero_rows_for_unrouted_tokens():
    p = _problem(seed=14, E=7, L=2, e_lo=5, T=12)
    fwd = _forward(p, p["x"], 0.0)
    args = (fwd["offsets"], fwd["row_src"], fwd["row_gate"], fwd["slot"], fwd["x_perm"],
            p["w_gate"], p["w_up"], p["w_down"], 12)
    d1 = oracle.experts_backward(p["dy"], *args)[0]
    d2 = oracle.experts_backward(2.5 * p["dy"], *args)[0]
    assert np.abs(d2 - 2.5 * d1).max() < 1e-12 * max(1.0, np.abs(d1).max())
    none = (fwd["slot"] < 0).all(axis=1)
    assert none.any() and (d1[none] == 0).all()
