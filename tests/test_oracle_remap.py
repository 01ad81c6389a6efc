"""Pins for the oracle's token remapping (dispatch_remap): hand-worked cases,
conservation of the T*k assignments, the capacity and threshold properties,
distinct experts per token, and the reduction to plain dispatch when nothing
overflows."""
import math

import numpy as np
import pytest

import oracle


def routed(logits, k):
    lg = np.asarray(logits, dtype=np.float64)
    ranked = oracle.topk_experts(lg, 2 * k)
    idx, alt = ranked[:, :k], ranked[:, k:]
    return idx, alt, oracle.topk_gates(lg, idx)


def test_hand_case_single_slot():
    # three tokens all pick expert 0 (k = 1, gates exactly 1, C = 1): the
    # lowest token keeps it; the others move to their next-ranked experts
    idx, alt, g = routed([[3, 2, 1, 0], [3, 0, 2, 1], [3, 1, 0, 2]], 1)
    assert idx[:, 0].tolist() == [0, 0, 0] and alt[:, 0].tolist() == [1, 2, 3]
    out = oracle.dispatch_remap(idx, alt, g, 4, capacity=1)
    assert out["expert"][:, 0].tolist() == [0, 2, 3]
    assert out["offsets"].tolist() == [0, 1, 1, 2, 3]
    assert out["row_src"].tolist() == [0, 1, 2]
    assert out["moved"] == 2 and out["dropped"] == 0
    # token 2's next expert is also 2: equal gates, token 1 (lower) wins it
    idx, alt, g = routed([[3, 2, 1, 0], [3, 0, 2, 1], [3, 1, 2, 0]], 1)
    out = oracle.dispatch_remap(idx, alt, g, 4, capacity=1)
    assert out["expert"][:, 0].tolist() == [0, 2, -1]
    assert out["slot"][:, 0].tolist() == [0, 1, -1]
    assert out["moved"] == 1 and out["dropped"] == 1


def test_hand_case_two_overflowing_slots_of_one_token():
    # k = 2, C = 1: token 1 loses both its experts to token 0 (equal gates,
    # lower token first); its first overflowing slot goes to its rank-2
    # expert (4), its second to its rank-3 expert (3); the gates stay
    idx, alt, g = routed([[5, 4, 3, 2, 1], [5, 4, 1, 2, 3]], 2)
    assert idx.tolist() == [[0, 1], [0, 1]] and alt.tolist() == [[2, 3], [4, 3]]
    e = math.e
    assert np.allclose(g, [[e / (e + 1), 1 / (e + 1)]] * 2, rtol=0, atol=1e-15)
    out = oracle.dispatch_remap(idx, alt, g, 5, capacity=1)
    assert out["expert"].tolist() == [[0, 1], [4, 3]]
    assert out["offsets"].tolist() == [0, 1, 2, 2, 3, 4]
    assert out["slot"].tolist() == [[0, 1], [3, 2]]
    assert out["row_src"].tolist() == [0, 0, 1, 1]
    assert np.allclose(out["row_gate"], [e / (e + 1), 1 / (e + 1), 1 / (e + 1), e / (e + 1)], rtol=0, atol=1e-15)
    assert out["moved"] == 2 and out["dropped"] == 0


def skewed_routing(rng, T, E, k, s=1.2):
    """Router logits with a Zipf-shaped per-expert bias (as the skewed workload)."""
    bias = -s * np.log(1 + rng.permutation(E))
    lg = rng.standard_normal((T, E)) + bias[None, :]
    return routed(lg, k)


def check_remap(idx, alt, gate, E, cap, out):
    T, k = idx.shape
    plain = oracle.dispatch(idx, gate, E, 0, E, cap)
    kept1 = plain["slot"] >= 0
    # conservation of the T*k assignments
    assert int(kept1.sum()) + out["moved"] + out["dropped"] == T * k
    expert = out["expert"]
    assert ((expert >= 0) == (out["slot"] >= 0)).all()
    # kept primary assignments stay; the m-th overflowing slot of a token
    # goes to alt[t, m] or nowhere
    assert (expert[kept1] == idx[kept1]).all()
    for t in range(T):
        m = 0
        for j in range(k):
            if not kept1[t, j]:
                assert expert[t, j] in (alt[t, m], -1)
                m += 1
        served = expert[t][expert[t] >= 0]
        assert len(set(served.tolist())) == len(served)          # one row per (token, expert)
    rows = np.diff(out["offsets"])
    assert (rows <= cap).all()                                    # capacity holds
    assert (rows == np.bincount(expert[expert >= 0], minlength=E)).all()
    # per expert: accepted proposals beat rejected ones (gate desc, token asc),
    # and an expert that rejected anything is full
    for e in range(E):
        prop = [(t, j) for t in range(T) for j in range(k) if not kept1[t, j]
                and alt[t, int((~kept1[t, :j]).sum())] == e]
        acc = [(t, j) for t, j in prop if expert[t, j] == e]
        rej = [(t, j) for t, j in prop if expert[t, j] != e]
        if rej:
            assert rows[e] == cap
        if acc and rej:
            worst = min((gate[t, j], -t) for t, j in acc)
            best = max((gate[t, j], -t) for t, j in rej)
            assert worst > best
    # rows: bijection, token-ascending per expert, gates carried
    used = out["slot"][out["slot"] >= 0]
    assert sorted(used.tolist()) == list(range(int(out["offsets"][-1])))
    for e in range(E):
        src = out["row_src"][out["offsets"][e]:out["offsets"][e + 1]]
        assert np.all(np.diff(src) > 0)
    for t in range(T):
        for j in range(k):
            r = out["slot"][t, j]
            if r >= 0:
                assert out["row_src"][r] == t and out["row_gate"][r] == gate[t, j]


@pytest.mark.parametrize("T,E,k,cap,seed", [(60, 12, 3, 14, 0), (200, 24, 4, 30, 1), (90, 10, 5, 40, 2),
                                            (40, 16, 8, 18, 3)])
def test_remap_invariants_on_skewed_routing(T, E, k, cap, seed):
    rng = np.random.default_rng(seed)
    idx, alt, gate = skewed_routing(rng, T, E, k)
    out = oracle.dispatch_remap(idx, alt, gate, E, capacity=cap)
    assert out["moved"] > 0                                      # the cases do overflow
    check_remap(idx, alt, gate, E, cap, out)


def test_remap_with_tied_gates():
    rng = np.random.default_rng(4)
    T, E, k, cap = 80, 10, 3, 20
    idx, alt, _ = skewed_routing(rng, T, E, k)
    gate = rng.choice([0.25, 0.5], size=(T, k))                  # many equal gates
    out = oracle.dispatch_remap(idx, alt, gate, E, capacity=cap)
    check_remap(idx, alt, gate, E, cap, out)


def test_no_overflow_equals_plain_dispatch():
    rng = np.random.default_rng(5)
    idx, alt, gate = skewed_routing(rng, 70, 12, 4)
    cap = int(np.bincount(idx.ravel(), minlength=12).max())
    out = oracle.dispatch_remap(idx, alt, gate, 12, capacity=cap)
    ref = oracle.dispatch(idx, gate, 12, capacity=cap)
    for n in ("counts", "offsets", "slot", "row_src", "row_gate"):
        assert (out[n] == ref[n]).all(), n
    assert out["moved"] == 0 and out["dropped"] == 0


def test_local_range_is_the_full_result_restricted():
    rng = np.random.default_rng(6)
    T, E, k, cap = 150, 20, 4, 22
    idx, alt, gate = skewed_routing(rng, T, E, k)
    full = oracle.dispatch_remap(idx, alt, gate, E, capacity=cap)
    e_lo, e_hi = 5, 13
    loc = oracle.dispatch_remap(idx, alt, gate, E, e_lo, e_hi, capacity=cap)
    lo, hi = full["offsets"][e_lo], full["offsets"][e_hi]
    assert (loc["offsets"] == full["offsets"][e_lo:e_hi + 1] - lo).all()
    assert (loc["row_src"] == full["row_src"][lo:hi]).all()
    inside = (full["expert"] >= e_lo) & (full["expert"] < e_hi)
    assert (loc["slot"][inside] == full["slot"][inside] - lo).all()
    assert (loc["slot"][~inside] == -1).all()
    assert (loc["expert"] == full["expert"]).all()
