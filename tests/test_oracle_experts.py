"""Pins for the oracle's expert FFN, combine, load-balance loss and LoRA."""
import math

import numpy as np
import pytest
import torch

import oracle

SILU_1 = 0.7310585786300049      # 1 / (1 + e^-1)
SILU_M1 = -0.2689414213699951    # -1 / (1 + e)
SILU_2 = 1.7615941559557646      # 2 / (1 + e^-2)


def test_silu_constants_are_the_closed_forms():
    assert abs(SILU_1 - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(SILU_M1 + 1 / (1 + math.exp(1))) < 1e-16
    assert abs(SILU_2 - 2 / (1 + math.exp(-2))) < 1e-15
    got = oracle.silu(np.array([1.0, -1.0, 2.0, 0.0]))
    assert np.allclose(got, [SILU_1, SILU_M1, SILU_2, 0.0], rtol=0, atol=1e-16)


def test_expert_ffn_hand_case():
    # x = (1,-1): G = (1,-1), U = (2,-3), H = (2 silu(1), -3 silu(-1)),
    # O = (H0 + H1, H0 - H1)
    x = np.array([[1.0, -1.0]])
    wg = np.array([[1.0, 0.0], [0.0, 1.0]])
    wu = np.array([[2.0, 0.0], [0.0, 3.0]])
    wd = np.array([[1.0, 1.0], [1.0, -1.0]])
    o = oracle.expert_ffn(x, wg, wu, wd)
    h0, h1 = 2 * SILU_1, -3 * SILU_M1
    assert np.allclose(o, [[h0 + h1, h0 - h1]], rtol=0, atol=1e-15)
    # G = (2, 0): the second unit is silenced, H = (silu(2) * 1, 0)
    o2 = oracle.expert_ffn(np.array([[2.0, 0.0]]), wg, np.array([[0.5, 0.0], [0.0, 1.0]]), wd)
    assert np.allclose(o2, [[SILU_2, SILU_2]], rtol=0, atol=1e-15)


def test_hand_moe_layer_one_token():
    # E = 3 one-unit experts (d = 2, f = 1), k = 2, router picks experts 0 and 2
    x = np.array([[1.0, 0.0]])
    wr = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 0.0]])      # logits (1, -1, 0)
    wg = np.array([[[1.0, 0.0]], [[1.0, 0.0]], [[2.0, 0.0]]])  # G = 1, 1, 2
    wu = np.array([[[1.0, 0.0]], [[1.0, 0.0]], [[1.0, 0.0]]])  # U = 1
    wd = np.array([[[1.0], [0.0]], [[0.0], [0.0]], [[0.0], [1.0]]])
    out = oracle.moe_layer(x, wr, wg, wu, wd, k=2)
    e = math.exp(1.0)
    g0, g2 = e / (e + 1), 1 / (e + 1)
    assert out["idx"].tolist() == [[0, 2]]
    assert np.allclose(out["y"], [[g0 * SILU_1, g2 * SILU_2]], rtol=0, atol=1e-15)


def dense_swiglu_torch(x, wg, wu, wd):
    """The dense SwiGLU FFN through torch's own silu and matmul, in float64."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    G = X @ torch.from_numpy(np.asarray(wg, np.float64)).T
    U = X @ torch.from_numpy(np.asarray(wu, np.float64)).T
    return ((torch.nn.functional.silu(G) * U) @ torch.from_numpy(np.asarray(wd, np.float64)).T).numpy()


def tiny_weights(rng, T, d, E, f, L):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / math.sqrt(d)
    wg = rng.standard_normal((L, f, d)) / math.sqrt(d)
    wu = rng.standard_normal((L, f, d)) / math.sqrt(d)
    wd = rng.standard_normal((L, d, f)) / math.sqrt(f)
    return x, wr, wg, wu, wd


def test_k_equals_E_with_identical_experts_is_dense_ffn():
    rng = np.random.default_rng(0)
    T, d, E, f = 9, 12, 6, 5
    x, wr, wg, wu, wd = tiny_weights(rng, T, d, E, f, 1)
    rep = lambda w: np.repeat(w, E, axis=0)
    out = oracle.moe_layer(x, wr, rep(wg), rep(wu), rep(wd), k=E)
    ref = dense_swiglu_torch(x, wg[0], wu[0], wd[0])
    assert np.max(np.abs(out["y"] - ref)) < 1e-13


def test_k1_with_identical_experts_is_the_ffn():
    rng = np.random.default_rng(1)
    T, d, E, f = 7, 8, 5, 6
    x, wr, wg, wu, wd = tiny_weights(rng, T, d, E, f, 1)
    rep = lambda w: np.repeat(w, E, axis=0)
    out = oracle.moe_layer(x, wr, rep(wg), rep(wu), rep(wd), k=1)
    assert (out["gate"] == 1.0).all()
    assert np.max(np.abs(out["y"] - dense_swiglu_torch(x, wg[0], wu[0], wd[0]))) < 1e-13


def test_layer_equals_per_token_sum_over_selected_experts():
    """Dispatch + combine against a direct per-token loop over the selection."""
    rng = np.random.default_rng(2)
    T, d, E, f, k = 11, 8, 7, 4, 3
    for e_lo, e_hi in [(0, 7), (2, 5)]:
        L = e_hi - e_lo
        x, wr, wg, wu, wd = tiny_weights(rng, T, d, E, f, L)
        out = oracle.moe_layer(x, wr, wg, wu, wd, k=k, e_lo=e_lo, e_hi=e_hi)
        l = x @ wr.T
        ref = np.zeros((T, d))
        for t in range(T):
            sel = sorted(range(E), key=lambda e: (-l[t, e], e))[:k]
            z = [math.exp(l[t, e] - l[t, sel[0]]) for e in sel]
            for e, zz in zip(sel, z):
                if e_lo <= e < e_hi:
                    le = e - e_lo
                    ref[t] += zz / sum(z) * dense_swiglu_torch(x[t:t + 1], wg[le], wu[le], wd[le])[0]
        assert np.max(np.abs(out["y"] - ref)) < 1e-13


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(3)
    x, wr, wg, wu, wd = tiny_weights(rng, 5, 8, 6, 4, 6)
    out = oracle.moe_layer(np.zeros_like(x), wr, wg, wu, wd, k=2)
    assert (out["y"] == 0).all()
    assert out["idx"].tolist() == [[0, 1]] * 5       # all-zero logits tie -> lowest ids


def test_combine_is_linear_and_skips_unset_slots():
    rng = np.random.default_rng(4)
    O = rng.standard_normal((6, 3))
    slot = np.array([[0, -1], [2, 1], [-1, -1], [5, 3]])
    g = rng.random((4, 2))
    y = oracle.combine(O, slot, g, 4)
    assert (y[2] == 0).all()
    assert np.allclose(y[0], g[0, 0] * O[0], rtol=0, atol=1e-15)
    assert np.allclose(oracle.combine(2.5 * O, slot, g, 4), 2.5 * y, rtol=0, atol=1e-14)


def test_aux_loss_uniform_and_hand_case():
    E, T, k = 896, 1792, 16          # 32 assignments per expert
    counts = np.full(E, T * k // E)
    prob = np.full(E, T / E)
    val, raw = oracle.aux_loss(counts, prob, T, k, 0.01)
    assert abs(raw - 1.0) < 1e-12 and abs(val - 0.01) < 1e-14
    # 2 experts, T = 4, k = 1: f = (3/4, 1/4), P = (5/8, 3/8): 2 (15/32 + 3/32) = 9/8
    val, raw = oracle.aux_loss([3, 1], [2.5, 1.5], 4, 1, 1.0)
    assert raw == 1.125 and val == 1.125


def lora_case(rng, L, d, f, r, scale, zero_b=False):
    lora = {"scale": scale,
            "a_up": rng.standard_normal((L, r, d)) / math.sqrt(d),
            "a_down": rng.standard_normal((L, r, f)) / math.sqrt(d),
            "b_up": np.zeros((L, f, r)) if zero_b else rng.standard_normal((L, f, r)) * 0.3,
            "b_down": np.zeros((L, d, r)) if zero_b else rng.standard_normal((L, d, r)) * 0.3}
    return lora


def test_lora_forward_equals_merged_weights():
    """[Guide §3]: W' = W0 + (alpha/r) B A applied as one merged weight."""
    rng = np.random.default_rng(5)
    d, f, r = 10, 7, 3
    x = rng.standard_normal((4, d))
    wg, wu = rng.standard_normal((f, d)), rng.standard_normal((f, d))
    wd = rng.standard_normal((d, f))
    lo = lora_case(rng, 1, d, f, r, 2.0)
    one = {key: (v[0] if key != "scale" else v) for key, v in lo.items()}
    got = oracle.expert_ffn(x, wg, wu, wd, one)
    wu_m = wu + 2.0 * one["b_up"] @ one["a_up"]
    wd_m = wd + 2.0 * one["b_down"] @ one["a_down"]
    assert np.max(np.abs(got - dense_swiglu_torch(x, wg, wu_m, wd_m))) < 1e-12


def _loss(x, wr, wg, wu, wd, k, e_lo, e_hi, lora, dy):
    out = oracle.moe_layer(x, wr, wg, wu, wd, k=k, e_lo=e_lo, e_hi=e_hi, lora=lora)
    return float(np.sum(out["y"] * dy)), out


def test_lora_backward_matches_central_differences():
    rng = np.random.default_rng(6)
    T, d, E, f, k, r, e_lo, e_hi = 6, 5, 4, 3, 2, 2, 1, 3
    L = e_hi - e_lo
    x, wr, wg, wu, wd = tiny_weights(rng, T, d, E, f, L)
    lora = lora_case(rng, L, d, f, r, 2.0)
    dy = rng.standard_normal((T, d))
    _, out = _loss(x, wr, wg, wu, wd, k, e_lo, e_hi, lora, dy)
    assert out["offsets"][-1] > 0
    grads = oracle.lora_backward(dy, out["x_perm"], out["offsets"], out["row_src"],
                                 out["row_gate"], out["G"], out["H"], wd, lora)
    h = 1e-6
    for name, gname in [("a_up", "da_up"), ("b_up", "db_up"), ("a_down", "da_down"),
                        ("b_down", "db_down")]:
        num = np.zeros_like(lora[name])
        for pos in np.ndindex(*lora[name].shape):
            keep = lora[name][pos]
            lora[name][pos] = keep + h
            lp, _ = _loss(x, wr, wg, wu, wd, k, e_lo, e_hi, lora, dy)
            lora[name][pos] = keep - h
            lm, _ = _loss(x, wr, wg, wu, wd, k, e_lo, e_hi, lora, dy)
            lora[name][pos] = keep
            num[pos] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - grads[gname])) < 1e-7, name
        assert np.max(np.abs(grads[gname])) > 1e-3, name


def test_lora_zero_b_gives_zero_a_grads_and_frozen_forward():
    rng = np.random.default_rng(7)
    T, d, E, f, k, r = 8, 6, 5, 4, 2, 3
    x, wr, wg, wu, wd = tiny_weights(rng, T, d, E, f, E)
    lora = lora_case(rng, E, d, f, r, 2.0, zero_b=True)
    dy = rng.standard_normal((T, d))
    out = oracle.moe_layer(x, wr, wg, wu, wd, k=k, lora=lora)
    frozen = oracle.moe_layer(x, wr, wg, wu, wd, k=k)
    assert (out["y"] == frozen["y"]).all()
    grads = oracle.lora_backward(dy, out["x_perm"], out["offsets"], out["row_src"],
                                 out["row_gate"], out["G"], out["H"], wd, lora)
    assert (grads["da_up"] == 0).all() and (grads["da_down"] == 0).all()
    assert np.abs(grads["db_up"]).max() > 0 and np.abs(grads["db_down"]).max() > 0
