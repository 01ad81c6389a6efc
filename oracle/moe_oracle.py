"""CPU oracle for the sparse MoE layer y = sum_{i in TopK(x)} g_i(x) * E_i(x).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The library path never
calls it, and it shares no code with the HIP kernels: it is a plain, slow,
float64 NumPy statement of what the layer computes, one step per function.

Pages cited (by title; section in brackets):

* [Guide]   "Adapting Trillion-Parameter MoE Models for LoRA Fine-Tuning:
             A Full-Stack Engineering Guide"
* [DayLvl]  "Day-Level Adaptation and LoRA Fine-Tuning of Ultra-Large-Scale
             Sparse MoE Models"
* [Paths]   "Adapting Ultra-Large MoE Models: Engineering Practices and
             Optimization Pathways"
* [FullOpt] "Trillion-Parameter MoE Model Training Adaptation: Full-Stack
             Optimization Practices"
* [FineTn]  "Fine-Tuning Trillion-Parameter Sparse MoE Models: Challenges and
             Engineering Practices"

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

1. The gate g is the softmax over the router logits, restricted to the k
   selected experts and renormalised ([Guide §2.1] names g only as the
   routing gate score). Selection uses the logits themselves (monotone in the
   softmax), descending, ties to the lower expert id; -0.0 equals +0.0.
2. The expert network E_i is a SwiGLU FFN without biases:
   E(x) = (silu(x W_g^T) * (x W_u^T)) W_d^T, silu(a) = a / (1 + exp(-a)).
3. Capacity ([DayLvl §3.2] expert_capacity; [Paths §3.3] drop overflow):
   an expert with more than C assignments keeps the C with the largest gate,
   equal gates going to the lower token id; the others are dropped and the
   kept gates are not renormalised.
4. Rows of the dispatched matrix are grouped by expert ascending, and within
   an expert by token ascending ([FullOpt §3] permute by routing result).
5. Only experts in [e_lo, e_hi) are computed (one expert-parallel rank's
   share, [FullOpt §4.1]); the other assignments are not drops, they belong to
   other ranks, and tokens with no local expert get y = 0.
6. The load-balance loss ([Guide §2.1], [Paths §3.3]) is the product of
   load and probability, coef * E * sum_e f_e P_e, with f_e the fraction of the T*k assignments
   routed to e (before capacity) and P_e the mean full-softmax probability.
7. LoRA ([Guide §3] eq. W' = W0 + (alpha/r) B A) sits on the up and down
   projections of every local expert; dropout is 0. The backward takes an
   upstream gradient dY of y, i.e. the loss sum(y * dY); routing, gates and
   base weights are frozen ([Guide §3]: do not tune the routing gates), so
   only the four adapter gradients are produced.

8. The full backward of the layer (gradients of sum(y * dY) + L_aux with
   respect to x and the router logits) treats the gates as functions of the
   selected logits only (the selection itself is piecewise constant), the
   load-balance fractions f_e as constants (counts are not differentiable),
   assignments that were dropped or belong to other experts' ranks as
   contributing nothing to y, and the expert and router weights as frozen.

Parity pins: every function here is checked by tests against closed forms,
invariants, brute force or finite differences (tests/test_oracle_*.py).
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


# ---------------------------------------------------------------- routing ---

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """l[t,e] = sum_i x[t,i] * W_r[e,i] (+ b[e]).  [Guide §2.1]: the router
    scores every expert for every token; the bias is the per-expert logit
    offset of the skewed workload."""
    l = _f64(x) @ _f64(w_router).T
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l


def latent_router_logits(x, w_latent, w_router, bias=None):
    """Routing from a low-dimensional projection of the tokens ([DayLvl §2.1]:
    tokens are first mapped to a more stable low-dimensional representation,
    then routed). Reading: a linear map z = x W_c^T to d_c dimensions (no
    bias, no normalisation), then l = z W_r^T (+ b) with W_r [E, d_c].
    Returns (l, z)."""
    z = _f64(x) @ _f64(w_latent).T
    return router_logits(z, w_router, bias), z


def topk_experts(logits, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, descending, ties to the lower
    expert id ([DayLvl §2.1]: each token activates 16 of 896 experts).

    A stable sort of -l keeps equal values in ascending index order, so the
    first k entries are exactly the selection with the tie rule.
    """
    l = _f64(logits)
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_gates(logits, idx) -> np.ndarray:
    """g[t,j] = exp(l[t,idx_j] - m_t) / sum_j' exp(l[t,idx_j'] - m_t): the
    softmax over all experts, renormalised over the selected ones (the full
    denominator cancels). m_t is the largest selected logit."""
    l = _f64(logits)
    sel = np.take_along_axis(l, np.asarray(idx), axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


def softmax_full(logits) -> np.ndarray:
    """p[t,e] = exp(l[t,e]) / sum_e' exp(l[t,e']) over all E experts."""
    l = _f64(logits)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_capacity(capacity_factor: float, T: int, k: int, E: int) -> int:
    """C = ceil(cf * T * k / E): the factor times the even share of the T*k
    assignments ([DayLvl §3.2] expert_capacity=1.25). Rounded up."""
    from fractions import Fraction
    q = Fraction(capacity_factor).limit_denominator(1 << 20) * T * k / E
    return int(-(-q.numerator // q.denominator))


# --------------------------------------------------------------- dispatch ---

def dispatch(idx, gate, E: int, e_lo: int = 0, e_hi: Optional[int] = None,
             capacity: int = 0) -> Dict[str, np.ndarray]:
    """Group the (token, slot) assignments by local expert ([FullOpt §3]:
    tokens are permuted according to the routing results; [Paths §3.3]:
    capacity limit with dropping).

    Returns
      counts   [E]     assignments per expert over all T*k (before capacity)
      kept     [L]     rows kept per local expert
      offsets  [L+1]   exclusive scan of kept
      slot     [T,k]   row of assignment (t,j) or -1 (dropped or not local)
      row_src  [R]     token of each row
      row_gate [R]     gate of each row
      dropped  int     local assignments removed by the capacity rule

    ``gate`` is compared exactly as given (pass the float32 gates a kernel
    produced to reproduce its capacity decisions).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if e_hi is None:
        e_hi = E
    L = e_hi - e_lo
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1

    slot = np.full((T, k), -1, dtype=np.int64)
    rows_src = []
    rows_gate = []
    kept = np.zeros(L, dtype=np.int64)
    offsets = np.zeros(L + 1, dtype=np.int64)
    dropped = 0
    for le in range(L):
        e = e_lo + le
        ts, js = np.nonzero(idx == e)          # row-major: token ascending
        keep = np.ones(len(ts), dtype=bool)
        if capacity > 0 and len(ts) > capacity:
            g = np.asarray(gate)[ts, js]
            # best first: larger gate, then lower token
            order = np.lexsort((ts, -g.astype(F64)))
            keep[:] = False
            keep[order[:capacity]] = True
            dropped += int(len(ts) - capacity)
        ts, js = ts[keep], js[keep]
        offsets[le] = len(rows_src)
        for t, j in zip(ts, js):
            slot[t, j] = len(rows_src)
            rows_src.append(t)
            rows_gate.append(np.asarray(gate)[t, j])
        kept[le] = len(ts)
    offsets[L] = len(rows_src)
    return {
        "counts": counts,
        "kept": kept,
        "offsets": offsets,
        "slot": slot,
        "row_src": np.asarray(rows_src, dtype=np.int64),
        "row_gate": np.asarray(rows_gate, dtype=F64),
        "dropped": dropped,
    }


def dispatch_remap(idx, alt, gate, E: int, e_lo: int = 0, e_hi: Optional[int] = None,
                   capacity: int = 0) -> Dict[str, np.ndarray]:
    """Dispatch with token remapping instead of dropping ([Paths §3.3]:
    tokens above an expert's capacity are remapped or dropped).

    Reading (the pages give no rule):
      1. The capacity rule of ``dispatch`` runs over all E experts: expert e
         keeps its C assignments with the largest gate (ties to the lower
         token); the others overflow.
      2. Each token sends its overflowing assignments, in slot order j, to
         its next-ranked experts outside its selection: the m-th overflowing
         assignment of token t proposes to alt[t, m], where alt[t] lists the
         experts ranked k, k+1, ... by logit (the same order as the
         selection). A token therefore never proposes twice to one expert,
         nor to an expert it already selected.
      3. Expert e accepts proposals into the room its kept assignments left,
         C - kept_e, preferring the larger gate, then the lower token; the
         other proposals are dropped. An accepted assignment keeps its gate
         g[t, j]: the token's combine weights do not change, only the expert
         that serves the slot.
    Rows are grouped by local expert ascending and by token ascending inside
    an expert, as in ``dispatch``.

    Returns the keys of ``dispatch`` (counts = assignments per expert before
    capacity, over the original selection) plus
      expert   [T,k]  the expert serving each assignment (primary or alt),
                      -1 when dropped
      moved    int    accepted proposals on local experts
      dropped  int    rejected proposals to local experts
    """
    idx = np.asarray(idx)
    alt = np.asarray(alt)
    g = np.asarray(gate)
    T, k = idx.shape
    if e_hi is None:
        e_hi = E
    L = e_hi - e_lo
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1
    # 1. the capacity rule over every expert (which assignments overflow)
    primary = dispatch(idx, gate, E, 0, E, capacity)
    kept1 = primary["slot"] >= 0
    kept_per_expert = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if kept1[t, j]:
                kept_per_expert[idx[t, j]] += 1
    # 2. proposals: the m-th overflowing slot of token t goes to alt[t, m]
    target = idx.copy()
    proposal = np.zeros((T, k), dtype=bool)
    for t in range(T):
        m = 0
        for j in range(k):
            if not kept1[t, j]:
                target[t, j] = alt[t, m]
                proposal[t, j] = True
                m += 1
    # 3. each expert fills its room with the best proposals
    accepted = np.zeros((T, k), dtype=bool)
    for e in range(E):
        ts, js = np.nonzero(proposal & (target == e))
        room = max(capacity - int(kept_per_expert[e]), 0) if capacity > 0 else len(ts)
        order = np.lexsort((ts, -g[ts, js].astype(F64)))   # larger gate, then lower token
        for q in order[:room]:
            accepted[ts[q], js[q]] = True
    served = kept1 | accepted
    expert = np.where(served, target, -1)
    # rows: local experts ascending, tokens ascending inside an expert
    slot = np.full((T, k), -1, dtype=np.int64)
    rows_src, rows_gate = [], []
    offsets = np.zeros(L + 1, dtype=np.int64)
    moved = dropped = 0
    for le in range(L):
        e = e_lo + le
        offsets[le] = len(rows_src)
        ts, js = np.nonzero(expert == e)        # row-major: token ascending
        for t, j in zip(ts, js):
            slot[t, j] = len(rows_src)
            rows_src.append(t)
            rows_gate.append(g[t, j])
        moved += int((accepted & (target == e)).sum())
        dropped += int((proposal & ~accepted & (target == e)).sum())
    offsets[L] = len(rows_src)
    return {
        "counts": counts,
        "offsets": offsets,
        "slot": slot,
        "row_src": np.asarray(rows_src, dtype=np.int64),
        "row_gate": np.asarray(rows_gate, dtype=F64),
        "expert": expert,
        "moved": moved,
        "dropped": dropped,
    }


# ----------------------------------------------------------------- experts --

def silu(a):
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def expert_ffn(x_rows, w_gate, w_up, w_down, lora: Optional[dict] = None,
               return_parts: bool = False):
    """One expert on its rows X [n,d]: G = X W_g^T, U = X W_u^T, H = silu(G)*U,
    O = H W_d^T. With LoRA ([Guide §3] W' = W0 + (alpha/r) B A, s = alpha/r):
    U += s (X A_u^T) B_u^T and O += s (H A_d^T) B_d^T.
    ``lora`` holds a_up [r,d], b_up [f,r], a_down [r,f], b_down [d,r], scale."""
    X = _f64(x_rows)
    G = X @ _f64(w_gate).T
    U = X @ _f64(w_up).T
    if lora is not None:
        U = U + lora["scale"] * (X @ _f64(lora["a_up"]).T) @ _f64(lora["b_up"]).T
    H = silu(G) * U
    O = H @ _f64(w_down).T
    if lora is not None:
        O = O + lora["scale"] * (H @ _f64(lora["a_down"]).T) @ _f64(lora["b_down"]).T
    if return_parts:
        return O, {"G": G, "U": U, "H": H}
    return O


def _lora_of(lora, le):
    if lora is None:
        return None
    return {"scale": lora["scale"], "a_up": lora["a_up"][le], "b_up": lora["b_up"][le],
            "a_down": lora["a_down"][le], "b_down": lora["b_down"][le]}


def experts_forward(x_perm, offsets, w_gate, w_up, w_down, lora=None,
                    return_parts: bool = False):
    """Apply local expert le to rows offsets[le]:offsets[le+1] of x_perm."""
    X = _f64(x_perm)
    d = w_down.shape[1]
    O = np.zeros((X.shape[0], d), dtype=F64)
    parts = {"G": [], "U": [], "H": []}
    for le in range(len(offsets) - 1):
        a, b = int(offsets[le]), int(offsets[le + 1])
        if a == b:
            continue
        o, p = expert_ffn(X[a:b], w_gate[le], w_up[le], w_down[le], _lora_of(lora, le),
                          return_parts=True)
        O[a:b] = o
        for key in parts:
            parts[key].append(p[key])
    if return_parts:
        f = w_gate.shape[1]
        cat = {key: (np.concatenate(v, 0) if v else np.zeros((0, f))) for key, v in parts.items()}
        return O, cat
    return O


def combine(o_rows, slot, gate, T: int) -> np.ndarray:
    """y[t] = sum_j [slot[t,j] >= 0] g[t,j] O[slot[t,j]] ([Guide §2.1]: the
    expert outputs are gathered back and summed with the gate weights)."""
    O = _f64(o_rows)
    slot = np.asarray(slot)
    g = _f64(gate)
    y = np.zeros((T, O.shape[1]), dtype=F64)
    for t in range(T):
        for j in range(slot.shape[1]):
            s = slot[t, j]
            if s >= 0:
                y[t] += g[t, j] * O[s]
    return y


def aux_loss(counts, prob_sum, T: int, k: int, coef: float):
    """Load balance as load times probability: f_e = counts_e / (T k), P_e = prob_sum_e / T,
    returns (coef * E * sum f P, E * sum f P)."""
    c = _f64(counts)
    P = _f64(prob_sum) / T
    fr = c / (T * k)
    E = c.shape[0]
    raw = E * float(np.sum(fr * P))
    return coef * raw, raw


# ------------------------------------------------------------------- layer --

def moe_layer(x, w_router, w_gate, w_up, w_down, k: int, bias=None, e_lo: int = 0,
              e_hi: Optional[int] = None, capacity: int = 0, lora=None,
              aux_coef: float = 0.0) -> Dict[str, np.ndarray]:
    """The whole layer from scratch in float64."""
    E = w_router.shape[0]
    T = x.shape[0]
    logits = router_logits(x, w_router, bias)
    idx = topk_experts(logits, k)
    gate = topk_gates(logits, idx)
    disp = dispatch(idx, gate, E, e_lo, e_hi, capacity)
    x_perm = _f64(x)[disp["row_src"]]
    O, parts = experts_forward(x_perm, disp["offsets"], w_gate, w_up, w_down, lora,
                               return_parts=True)
    y = combine(O, disp["slot"], gate, T)
    out = {"logits": logits, "idx": idx, "gate": gate, "x_perm": x_perm, "o": O, "y": y}
    out.update(disp)
    out.update(parts)
    p = softmax_full(logits)
    out["prob_sum"] = p.sum(axis=0)
    out["aux"] = aux_loss(disp["counts"], out["prob_sum"], T, k, aux_coef)
    return out


# ----------------------------------------------------------- LoRA backward --

def lora_backward(dy, x_perm, offsets, row_src, row_gate, G, H, w_down, lora):
    """Adapter gradients of the loss sum(y * dY), per local expert.

    With s = alpha/r, Z_u = X A_u^T, Z_d = H A_d^T and dO[p] = g_p dY[src_p]
    (y = sum g O, so each row's output gradient is its gate times the token's
    upstream gradient):
      dB_d = s dO^T Z_d                 dA_d = s (dO B_d)^T H
      dH   = dO W_d + s (dO B_d) A_d    dU   = dH * silu(G)
      dB_u = s dU^T Z_u                 dA_u = s (dU B_u)^T X
    G and H are the forward's gate pre-activation and SwiGLU output rows.
    Returns fp64 arrays shaped like the adapters.
    """
    s = lora["scale"]
    A_u, B_u = _f64(lora["a_up"]), _f64(lora["b_up"])
    A_d, B_d = _f64(lora["a_down"]), _f64(lora["b_down"])
    dY, X, Gm, Hm = _f64(dy), _f64(x_perm), _f64(G), _f64(H)
    g = _f64(row_gate)
    L = A_u.shape[0]
    da_up, db_up = np.zeros_like(A_u), np.zeros_like(B_u)
    da_down, db_down = np.zeros_like(A_d), np.zeros_like(B_d)
    for le in range(L):
        a, b = int(offsets[le]), int(offsets[le + 1])
        if a == b:
            continue
        dO = g[a:b, None] * dY[np.asarray(row_src[a:b])]
        Xe, Ge, He = X[a:b], Gm[a:b], Hm[a:b]
        Zu = Xe @ A_u[le].T
        Zd = He @ A_d[le].T
        Wd = dO @ B_d[le]
        db_down[le] = s * dO.T @ Zd
        da_down[le] = s * Wd.T @ He
        dH = dO @ _f64(w_down[le]) + s * Wd @ A_d[le]
        dU = dH * silu(Ge)
        db_up[le] = s * dU.T @ Zu
        da_up[le] = s * (dU @ B_u[le]).T @ Xe
    return {"da_up": da_up, "db_up": db_up, "da_down": da_down, "db_down": db_down}


# ---------------------------------------------------------- full backward --
#
# Gradients of the loss sum(y * dY) + L_aux, the full backward pass of the
# layer ([Guide §3]: the adapters are trained through the frozen MoE layer,
# so the upstream layers need dx; [FullOpt §3]: the backward runs the same
# permute / grouped GEMM / unpermute stages in reverse).

def silu_grad(a):
    """d silu(a) / da = sigma(a) (1 + a (1 - sigma(a)))."""
    a = _f64(a)
    sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def gate_backward(dy, o_rows, slot, gate, T: int):
    """dg[t,j] = <dY_t, O[slot[t,j]]> for kept local slots, else 0: y is
    linear in each gate with coefficient the expert's output row."""
    dY, O = _f64(dy), _f64(o_rows)
    slot = np.asarray(slot)
    k = slot.shape[1]
    dg = np.zeros((T, k), dtype=F64)
    for t in range(T):
        for j in range(k):
            s = slot[t, j]
            if s >= 0:
                dg[t, j] = float(np.dot(dY[t], O[s]))
    return dg


def logits_backward(dgate, idx, gate, logits, counts=None, aux_coef: float = 0.0, k: Optional[int] = None,
                    T_total: Optional[int] = None):
    """dL/dl for L = sum(y dY) + L_aux, given dg = dL/dg.

    Gate path: g_j = exp(l_{idx_j}) / sum_i exp(l_{idx_i}) over the k
    selected experts, so dl_{idx_j} = g_j (dg_j - sum_i g_i dg_i) and the
    unselected logits get nothing from it.
    Aux path (with counts): L_aux = coef E sum_e f_e P_e, f_e = counts_e /
    (T k) held constant, P_e = (1/T) sum_t p_te with p_t = softmax(l_t) over
    all E; dP_e/dl_tc = p_te (delta_ec - p_tc) / T, so
    dL_aux/dl_tc = coef E / T * p_tc (f_c - sum_e f_e p_te).
    T_total: the layer's token count when the rows given are a subset of the
    tokens (every row is independent given the counts)."""
    dg, g = _f64(dgate), _f64(gate)
    idx = np.asarray(idx)
    l = _f64(logits)
    T, E = l.shape
    T = T if T_total is None else T_total
    dl = np.zeros(l.shape, dtype=F64)
    inner = (g * dg).sum(axis=1, keepdims=True)
    contrib = g * (dg - inner)
    for t in range(l.shape[0]):
        for j in range(idx.shape[1]):
            dl[t, idx[t, j]] += contrib[t, j]
    if counts is not None and aux_coef != 0.0:
        kk = idx.shape[1] if k is None else k
        fr = _f64(counts) / (T * kk)
        p = softmax_full(l)
        fp = (p * fr[None, :]).sum(axis=1, keepdims=True)
        dl = dl + aux_coef * E / T * p * (fr[None, :] - fp)
    return dl


def experts_backward(dy, offsets, row_src, row_gate, slot, x_perm, w_gate, w_up, w_down, T: int,
                     lora=None):
    """dx through the frozen experts (gates held fixed). Per local expert,
    with dO_p = g_p dY[src_p] and the forward's G, U recomputed from x_perm:
      dH = dO W_d (+ s (dO B_d) A_d)
      dG = dH * U * silu'(G),   dU = dH * silu(G)
      dX = dG W_g + dU W_u (+ s (dU B_u) A_u)
    and dx[t] = sum over the token's kept local slots j (in j order) of
    dX[slot[t,j]] (the unpermute of the backward). Returns (dx [T,d],
    dX rows [R,d], dict of G, U, dG, dU rows)."""
    dY, X = _f64(dy), _f64(x_perm)
    g = _f64(row_gate)
    d = _f64(w_down).shape[1]
    R = X.shape[0]
    f = _f64(w_gate).shape[1]
    dX = np.zeros((R, d), dtype=F64)
    parts = {n: np.zeros((R, f), dtype=F64) for n in ("G", "U", "dG", "dU")}
    for le in range(len(offsets) - 1):
        a, b = int(offsets[le]), int(offsets[le + 1])
        if a == b:
            continue
        lo = _lora_of(lora, le)
        Xe = X[a:b]
        Wg, Wu, Wd = _f64(w_gate[le]), _f64(w_up[le]), _f64(w_down[le])
        G = Xe @ Wg.T
        U = Xe @ Wu.T
        if lo is not None:
            U = U + lo["scale"] * (Xe @ _f64(lo["a_up"]).T) @ _f64(lo["b_up"]).T
        dO = g[a:b, None] * dY[np.asarray(row_src[a:b])]
        dH = dO @ Wd
        if lo is not None:
            dH = dH + lo["scale"] * (dO @ _f64(lo["b_down"])) @ _f64(lo["a_down"])
        dG = dH * U * silu_grad(G)
        dU = dH * silu(G)
        dXe = dG @ Wg + dU @ Wu
        if lo is not None:
            dXe = dXe + lo["scale"] * (dU @ _f64(lo["b_up"])) @ _f64(lo["a_up"])
        dX[a:b] = dXe
        for n, v in (("G", G), ("U", U), ("dG", dG), ("dU", dU)):
            parts[n][a:b] = v
    dx = np.zeros((T, d), dtype=F64)
    slot = np.asarray(slot)
    for t in range(T):
        for j in range(slot.shape[1]):
            s = slot[t, j]
            if s >= 0:
                dx[t] += dX[s]
    return dx, dX, parts


def router_backward(dlogits, w_router):
    """dx contribution of the router: logits = x W_r^T (+ b), so
    dx[t] = sum_e dl[t,e] W_r[e]."""
    return _f64(dlogits) @ _f64(w_router)


def moe_layer_backward(fwd, dy, x, w_router, w_gate, w_up, w_down, k: int, T: int, lora=None,
                       aux_coef: float = 0.0):
    """The layer's full backward from an oracle forward ``fwd`` (moe_layer):
    returns dgate, dlogits and dx = experts part + router part."""
    dg = gate_backward(dy, fwd["o"], fwd["slot"], fwd["gate"], T)
    dl = logits_backward(dg, fwd["idx"], fwd["gate"], fwd["logits"], fwd["counts"], aux_coef, k)
    dx_e, _, _ = experts_backward(dy, fwd["offsets"], fwd["row_src"], fwd["row_gate"], fwd["slot"],
                                  fwd["x_perm"], w_gate, w_up, w_down, T, lora)
    return {"dgate": dg, "dlogits": dl, "dx_experts": dx_e,
            "dx": dx_e + router_backward(dl, w_router)}
