"""Pins for the oracle's dispatch (histogram, stable grouping, capacity)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def random_routing(rng, T, E, k, gate_levels=None):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if gate_levels is None:
        gate = rng.random((T, k))
    else:
        gate = rng.choice(np.asarray(gate_levels, dtype=np.float64), size=(T, k))
    return idx, gate


def brute_dispatch(idx, gate, E, e_lo, e_hi, cap):
    """Sort every local assignment by (expert, token) with Python's sort; for an
    overfull expert keep the cap best by (gate desc, token asc)."""
    T, k = idx.shape
    by_e = {e: [] for e in range(e_lo, e_hi)}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e_lo <= e < e_hi:
                by_e[e].append((t, j))
    rows = []
    for e in range(e_lo, e_hi):
        lst = by_e[e]
        if cap > 0 and len(lst) > cap:
            best = sorted(lst, key=lambda tj: (-gate[tj[0], tj[1]], tj[0]))[:cap]
            lst = [tj for tj in lst if tj in best]
        rows.extend(sorted(lst))
    slot = -np.ones((T, k), dtype=np.int64)
    for r, (t, j) in enumerate(rows):
        slot[t, j] = r
    return rows, slot


def check_invariants(idx, gate, E, e_lo, e_hi, cap, out):
    T, k = idx.shape
    L = e_hi - e_lo
    counts = out["counts"]
    assert counts.sum() == T * k
    assert (counts == np.bincount(idx.ravel(), minlength=E)).all()
    local = counts[e_lo:e_hi]
    exp_kept = np.minimum(local, cap) if cap > 0 else local
    assert (out["kept"] == exp_kept).all()
    assert (np.diff(out["offsets"]) == out["kept"]).all() and out["offsets"][0] == 0
    R = out["offsets"][-1]
    slot = out["slot"]
    used = slot[slot >= 0]
    assert sorted(used.tolist()) == list(range(R))              # bijection onto rows
    nonlocal_ = int(((idx < e_lo) | (idx >= e_hi)).sum())
    assert (slot < 0).sum() == nonlocal_ + out["dropped"]       # conservation of T*k
    for le in range(L):
        a, b = out["offsets"][le], out["offsets"][le + 1]
        src = out["row_src"][a:b]
        assert np.all(np.diff(src) > 0)                         # token ascending
        for r in range(a, b):
            t = src[r - a]
            j = int(np.nonzero(idx[t] == e_lo + le)[0][0])
            assert slot[t, j] == r and out["row_gate"][r] == gate[t, j]


@pytest.mark.parametrize("T,E,k,e_lo,e_hi,cap", [
    (20, 8, 3, 0, 8, 0), (20, 8, 3, 2, 5, 0), (40, 6, 4, 0, 6, 9), (33, 10, 5, 1, 9, 7),
    (1, 4, 4, 0, 4, 0), (16, 16, 16, 0, 16, 3)])
def test_dispatch_matches_brute_force(T, E, k, e_lo, e_hi, cap):
    rng = np.random.default_rng(T * 100 + E)
    idx, gate = random_routing(rng, T, E, k, gate_levels=[0.1, 0.2, 0.2, 0.5])
    out = oracle.dispatch(idx, gate, E, e_lo, e_hi, cap)
    rows, slot = brute_dispatch(idx, gate, E, e_lo, e_hi, cap)
    assert (out["slot"] == slot).all()
    assert out["row_src"].tolist() == [t for t, _ in rows]
    check_invariants(idx, gate, E, e_lo, e_hi, cap, out)


def test_capacity_keeps_largest_gates_ties_to_lower_token():
    # expert 0 chosen by 6 tokens with gates (.5,.2,.5,.2,.9,.2), capacity 4:
    # keep .9 (t4), .5 (t0), .5 (t2), then the .2 tie goes to the lowest token t1
    T, E, k = 6, 3, 1
    idx = np.zeros((T, k), dtype=np.int64)
    gate = np.array([[.5], [.2], [.5], [.2], [.9], [.2]])
    out = oracle.dispatch(idx, gate, E, 0, E, capacity=4)
    assert out["row_src"].tolist() == [0, 1, 2, 4]
    assert out["slot"][:, 0].tolist() == [0, 1, 2, -1, 3, -1]
    assert out["dropped"] == 2 and out["kept"].tolist() == [4, 0, 0]


def test_capacity_threshold_property():
    rng = np.random.default_rng(7)
    others = [e for e in range(12) if e != 3]
    idx = np.stack([[3] + list(rng.choice(others, 3, replace=False)) for _ in range(200)])
    gate = rng.random((200, 4))
    cap = 30
    out = oracle.dispatch(idx, gate, 12, 0, 12, cap)
    ts, js = np.nonzero(idx == 3)
    kept = out["slot"][ts, js] >= 0
    assert kept.sum() == cap
    assert gate[ts, js][kept].min() >= gate[ts, js][~kept].max()


def test_infinite_capacity_equals_no_capacity():
    rng = np.random.default_rng(11)
    idx, gate = random_routing(rng, 50, 9, 3)
    a = oracle.dispatch(idx, gate, 9, 0, 9, 0)
    b = oracle.dispatch(idx, gate, 9, 0, 9, 50 * 3)
    for key in ("counts", "kept", "offsets", "slot", "row_src", "row_gate"):
        assert (a[key] == b[key]).all()
    assert b["dropped"] == 0


def test_no_local_assignment_gives_empty_rows():
    idx = np.array([[0, 1], [1, 0]])
    gate = np.full((2, 2), 0.5)
    out = oracle.dispatch(idx, gate, 4, 2, 4, 0)
    assert out["offsets"].tolist() == [0, 0, 0] and (out["slot"] == -1).all()
    assert out["dropped"] == 0 and out["counts"].tolist() == [2, 2, 0, 0]


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 12), st.integers(1, 8), st.data())
def test_dispatch_hypothesis(T, E, data):
    k = data.draw(st.integers(1, E))
    e_lo = data.draw(st.integers(0, E - 1))
    e_hi = data.draw(st.integers(e_lo + 1, E))
    cap = data.draw(st.integers(0, T))
    seed = data.draw(st.integers(0, 1 << 30))
    rng = np.random.default_rng(seed)
    idx, gate = random_routing(rng, T, E, k, gate_levels=[0.25, 0.5])
    out = oracle.dispatch(idx, gate, E, e_lo, e_hi, cap)
    rows, slot = brute_dispatch(idx, gate, E, e_lo, e_hi, cap)
    assert (out["slot"] == slot).all()
    check_invariants(idx, gate, E, e_lo, e_hi, cap, out)
