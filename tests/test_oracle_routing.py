"""Pins for the oracle's router, top-k selection and gates (CPU only).

Each check is against something other than the oracle's own formula: a
pure-Python brute force, a closed form worked by hand, or an identity of the
softmax.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from sparse_mixture_experts_top_amd import workloads


def brute_topk(row, k):
    """Full sort of (-logit, id) pairs: descending logit, ties to the lower id."""
    pairs = sorted(((-float(v) + 0.0, e) for e, v in enumerate(row)))
    return [e for _, e in pairs[:k]]


def check_router_triple_loop():
    w = workloads.WORKLOADS["tiny_f32"].replace(T=12, d=16, E=5)
    inp = workloads.generate(w, seed=3)
    x, wr = workloads.to_f64(inp["x"]), workloads.to_f64(inp["w_router"])
    bias = np.array([0.5, -1.0, 0.0, 2.0, -0.25])
    got = oracle.router_logits(x, wr, bias)
    for t in range(x.shape[0]):
        for e in range(wr.shape[0]):
            acc = 0.0
            for i in range(x.shape[1]):
                acc += x[t, i] * wr[e, i]
            assert abs(got[t, e] - (acc + bias[e])) <= 1e-12 * (1 + abs(acc))


def check_topk_brute_force(seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        T, E = int(rng.integers(1, 6)), int(rng.integers(1, 20))
        k = int(rng.integers(1, E + 1))
        # small integer logits force many ties
        l = rng.integers(-3, 4, size=(T, E)).astype(np.float64)
        idx = oracle.topk_experts(l, k)
        for t in range(T):
            assert list(idx[t]) == brute_topk(l[t], k)


def check_hand_gates():
    # one token, logits (1, 0, -1), k = 2: experts 0 and 1 with gates
    # e/(e+1) and 1/(e+1)
    l = np.array([[1.0, 0.0, -1.0]])
    idx = oracle.topk_experts(l, 2)
    g = oracle.topk_gates(l, idx)
    assert list(idx[0]) == [0, 1]
    e = math.exp(1.0)
    assert abs(g[0, 0] - e / (e + 1)) < 1e-15
    assert abs(g[0, 1] - 1 / (e + 1)) < 1e-15


def test_router_logits_match_triple_loop():
    check_router_triple_loop()


def test_topk_matches_brute_force_with_ties():
    check_topk_brute_force()


def test_topk_signed_zero_ties_to_lower_id():
    l = np.array([[0.0, -0.0, 0.0, -1.0], [-0.0, 0.0, -2.0, -0.0]])
    assert oracle.topk_experts(l, 2).tolist() == [[0, 1], [0, 1]]
    assert oracle.topk_experts(l, 3).tolist() == [[0, 1, 2], [0, 1, 3]]


def test_all_equal_logits_pick_first_k_with_uniform_gates():
    for E, k in [(16, 4), (896, 16), (7, 7)]:
        l = np.zeros((3, E))
        idx = oracle.topk_experts(l, k)
        assert (idx == np.arange(k)[None, :]).all()
        g = oracle.topk_gates(l, idx)
        assert (g == 1.0 / k).all()


def test_hand_computed_gates():
    check_hand_gates()


def test_gates_sum_to_one_and_k1_is_one():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((40, 64)) * 3
    for k in (1, 4, 16, 64):
        idx = oracle.topk_experts(l, k)
        g = oracle.topk_gates(l, idx)
        assert np.all(np.abs(g.sum(1) - 1.0) < 1e-14)
        assert np.all(np.diff(g, axis=1) <= 0)       # descending logits -> descending gates
    g1 = oracle.topk_gates(l, oracle.topk_experts(l, 1))
    assert (g1 == 1.0).all()


def test_gates_equal_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((30, 50)) * 4
    p = oracle.softmax_full(l)
    assert np.all(np.abs(p.sum(1) - 1) < 1e-14)
    idx = oracle.topk_experts(l, 8)
    sel = np.take_along_axis(p, idx, 1)
    ren = sel / sel.sum(1, keepdims=True)
    assert np.max(np.abs(ren - oracle.topk_gates(l, idx))) < 1e-14


def test_selection_is_the_k_largest():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((25, 100))
    idx = oracle.topk_experts(l, 16)
    for t in range(25):
        chosen = set(idx[t].tolist())
        worst_in = min(l[t, e] for e in chosen)
        best_out = max(l[t, e] for e in range(100) if e not in chosen)
        assert worst_in >= best_out


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 6), st.integers(1, 12), st.data())
def test_topk_hypothesis(T, E, data):
    k = data.draw(st.integers(1, E))
    vals = data.draw(st.lists(st.sampled_from([-1.5, -0.0, 0.0, 0.25, 0.25, 3.0]),
                              min_size=T * E, max_size=T * E))
    l = np.array(vals, dtype=np.float64).reshape(T, E)
    idx = oracle.topk_experts(l, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk(l[t], k)
    g = oracle.topk_gates(l, idx)
    assert np.all(np.abs(g.sum(1) - 1) < 1e-14)


def test_capacity_rounding():
    # 1.25 * 8192 * 16 / 896 = 182.857... -> 183
    assert oracle.expert_capacity(1.25, 8192, 16, 896) == 183
    # exact multiples are not rounded up further
    assert oracle.expert_capacity(1.0, 896, 16, 896) == 16
    assert oracle.expert_capacity(1.25, 64, 4, 16) == 20


# ------------------------------------------------------ latent-space router --

def test_latent_router_hand_case():
    # x = [1, 2], W_c = [[1, -1]] -> z = [-1]; W_r = [[2], [-3]], b = [0.5, 0]
    l, z = oracle.latent_router_logits(np.array([[1.0, 2.0]]), np.array([[1.0, -1.0]]),
                                       np.array([[2.0], [-3.0]]), np.array([0.5, 0.0]))
    assert z.tolist() == [[-1.0]]
    assert l.tolist() == [[-1.5, 3.0]]


def test_latent_router_identity_projection_is_the_plain_router():
    rng = np.random.default_rng(11)
    x, wr, b = rng.standard_normal((9, 12)), rng.standard_normal((7, 12)), rng.standard_normal(7)
    l, z = oracle.latent_router_logits(x, np.eye(12), wr, b)
    assert np.array_equal(z, x)
    assert np.allclose(l, oracle.router_logits(x, wr, b), rtol=0, atol=1e-13)


def test_latent_router_equals_merged_weight_and_python_loop():
    # non-square shapes (T=5, d=6, d_c=3, E=4) so a transposed operand fails
    rng = np.random.default_rng(12)
    x, wc, wr = rng.standard_normal((5, 6)), rng.standard_normal((3, 6)), rng.standard_normal((4, 3))
    l, z = oracle.latent_router_logits(x, wc, wr)
    assert np.allclose(l, x @ (wr @ wc).T, rtol=0, atol=1e-12)
    for t in range(5):
        for e in range(4):
            ref = 0.0
            for c in range(3):
                zc = sum(x[t, i] * wc[c, i] for i in range(6))
                ref += zc * wr[e, c]
            assert abs(l[t, e] - ref) <= 1e-12
