"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them. A mutant that no pin rejects would mean the oracle
could carry that mistake unnoticed."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as mo
import test_oracle_backward as tbwd
import test_oracle_dispatch as tdisp
import test_oracle_experts as texp
import test_oracle_remap as tremap
import test_oracle_routing as trout

F64 = np.float64


def _topk_ties_high(logits, k):
    l = np.asarray(logits, F64)
    E = l.shape[1]
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order)[:, :k]


def _gates_not_renormalised(logits, idx):
    return np.take_along_axis(mo.softmax_full(logits), np.asarray(idx), 1)


def _silu_wrong_sign(a):
    a = np.asarray(a, F64)
    return a / (1.0 + np.exp(a))


def _ffn_drop_lora_up(x_rows, w_gate, w_up, w_down, lora=None, return_parts=False):
    if lora is not None:
        lora = dict(lora)
        lora["b_up"] = np.zeros_like(np.asarray(lora["b_up"], F64))
    return ORIG["expert_ffn"](x_rows, w_gate, w_up, w_down, lora, return_parts)


def _ffn_gate_up_swapped(x_rows, w_gate, w_up, w_down, lora=None, return_parts=False):
    return ORIG["expert_ffn"](x_rows, w_up, w_gate, w_down, lora, return_parts)


def _capacity_keeps_lowest(idx, gate, E, e_lo=0, e_hi=None, capacity=0):
    return ORIG["dispatch"](idx, -np.asarray(gate, F64), E, e_lo, e_hi, capacity)


def _bwd_no_gate(dy, x_perm, offsets, row_src, row_gate, G, H, w_down, lora):
    return ORIG["lora_backward"](dy, x_perm, offsets, row_src, np.ones_like(np.asarray(row_gate, F64)),
                                 G, H, w_down, lora)


def _bwd_wrong_sign_lora_dh(dy, x_perm, offsets, row_src, row_gate, G, H, w_down, lora):
    lo = dict(lora)
    lo["a_down"] = -np.asarray(lora["a_down"], F64)
    out = ORIG["lora_backward"](dy, x_perm, offsets, row_src, row_gate, G, H, w_down, lo)
    out["da_down"] = -out["da_down"]
    return out


def _aux_wrong_norm(counts, prob_sum, T, k, coef):
    return ORIG["aux_loss"](counts, prob_sum, T, 1, coef)


def _silu_grad_is_silu(a):
    return ORIG["silu"](a)


def _dlogits_not_centred(dgate, idx, gate, logits, counts=None, aux_coef=0.0, k=None):
    # drops the - sum_i g_i dg_i term of the softmax Jacobian
    g, dg = np.asarray(gate, F64), np.asarray(dgate, F64)
    out = ORIG["logits_backward"](dgate, idx, gate, logits, counts, aux_coef, k)
    inner = (g * dg).sum(axis=1, keepdims=True)
    np.add.at(out, (np.arange(out.shape[0])[:, None], np.asarray(idx)), g * inner)
    return out


def _dlogits_aux_sign(dgate, idx, gate, logits, counts=None, aux_coef=0.0, k=None):
    return ORIG["logits_backward"](dgate, idx, gate, logits, counts, -aux_coef, k)


def _experts_bwd_gate_up_swapped(dy, offsets, row_src, row_gate, slot, x_perm, w_gate, w_up, w_down, T,
                                 lora=None):
    return ORIG["experts_backward"](dy, offsets, row_src, row_gate, slot, x_perm, w_up, w_gate, w_down, T,
                                    lora)


def _remap_variant(first_alt_only=False, lower_gate_first=False, gate_one=False, room_ignores_kept=False):
    """dispatch_remap with one planted mistake (the rule restated with a flag)."""
    def fn(idx, alt, gate, E, e_lo=0, e_hi=None, capacity=0):
        idx, alt, g = np.asarray(idx), np.asarray(alt), np.asarray(gate, F64)
        T, k = idx.shape
        e_hi = E if e_hi is None else e_hi
        kept1 = ORIG["dispatch"](idx, gate, E, 0, E, capacity)["slot"] >= 0
        kept_e = np.bincount(idx[kept1], minlength=E)
        target, prop = idx.copy(), np.zeros((T, k), bool)
        for t in range(T):
            m = 0
            for j in range(k):
                if not kept1[t, j]:
                    target[t, j] = alt[t, 0 if first_alt_only else m]
                    prop[t, j] = True
                    m += 1
        acc = np.zeros((T, k), bool)
        for e in range(E):
            ts, js = np.nonzero(prop & (target == e))
            room = capacity if room_ignores_kept else max(capacity - int(kept_e[e]), 0)
            order = np.lexsort((ts, g[ts, js] if lower_gate_first else -g[ts, js]))
            for q in order[:room]:
                acc[ts[q], js[q]] = True
        expert = np.where(kept1 | acc, target, -1)
        L = e_hi - e_lo
        slot = np.full((T, k), -1, np.int64)
        src, rg, off = [], [], np.zeros(L + 1, np.int64)
        moved = dropped = 0
        for le in range(L):
            e = e_lo + le
            off[le] = len(src)
            for t, j in zip(*np.nonzero(expert == e)):
                slot[t, j] = len(src)
                src.append(t)
                rg.append(1.0 if (gate_one and acc[t, j]) else g[t, j])
            moved += int((acc & (target == e)).sum())
            dropped += int((prop & ~acc & (target == e)).sum())
        off[L] = len(src)
        return {"counts": np.bincount(idx.ravel(), minlength=E), "offsets": off, "slot": slot,
                "row_src": np.asarray(src, np.int64), "row_gate": np.asarray(rg, F64), "expert": expert,
                "moved": moved, "dropped": dropped}
    return fn


def _latent_projection_negated(x, w_latent, w_router, bias=None):
    return ORIG["latent_router_logits"](-np.asarray(x, F64), w_latent, w_router, bias)


def _latent_bias_dropped(x, w_latent, w_router, bias=None):
    return ORIG["latent_router_logits"](x, w_latent, w_router, None)


ORIG = {n: getattr(mo, n) for n in ("topk_experts", "topk_gates", "silu", "expert_ffn",
                                     "dispatch", "lora_backward", "aux_loss", "silu_grad",
                                     "logits_backward", "experts_backward", "dispatch_remap",
                                     "latent_router_logits")}

MUTANTS = {
    "ties_to_higher_id": ("topk_experts", _topk_ties_high),
    "gates_not_renormalised": ("topk_gates", _gates_not_renormalised),
    "silu_wrong_sign": ("silu", _silu_wrong_sign),
    "lora_up_term_dropped": ("expert_ffn", _ffn_drop_lora_up),
    "gate_and_up_swapped": ("expert_ffn", _ffn_gate_up_swapped),
    "capacity_keeps_lowest_gates": ("dispatch", _capacity_keeps_lowest),
    "backward_ignores_gate": ("lora_backward", _bwd_no_gate),
    "backward_lora_dh_sign": ("lora_backward", _bwd_wrong_sign_lora_dh),
    "aux_loss_drops_k": ("aux_loss", _aux_wrong_norm),
    "silu_grad_is_silu": ("silu_grad", _silu_grad_is_silu),
    "dlogits_not_centred": ("logits_backward", _dlogits_not_centred),
    "dlogits_aux_sign": ("logits_backward", _dlogits_aux_sign),
    "experts_backward_gate_up_swapped": ("experts_backward", _experts_bwd_gate_up_swapped),
    "remap_every_overflow_to_first_alternate": ("dispatch_remap", _remap_variant(first_alt_only=True)),
    "remap_prefers_lower_gates": ("dispatch_remap", _remap_variant(lower_gate_first=True)),
    "remap_drops_the_gate": ("dispatch_remap", _remap_variant(gate_one=True)),
    "remap_room_ignores_kept_rows": ("dispatch_remap", _remap_variant(room_ignores_kept=True)),
    "latent_projection_negated": ("latent_router_logits", _latent_projection_negated),
    "latent_bias_dropped": ("latent_router_logits", _latent_bias_dropped),
}


def _pin_remap_invariants():
    for case in [(60, 12, 3, 14, 0), (200, 24, 4, 30, 1), (40, 16, 8, 18, 3)]:
        tremap.test_remap_invariants_on_skewed_routing(*case)


def _pin_dx_fd_plain():
    tbwd.test_dx_matches_central_differences(tbwd.CASES[0], 0.3)


def _pin_dx_fd_lora_capacity():
    tbwd.test_dx_matches_central_differences(tbwd.CASES[3], 0.0)
    tbwd.test_dx_matches_central_differences(tbwd.CASES[4], 0.0)


def _pin_dlogits_fd():
    tbwd.test_dlogits_matches_central_differences(tbwd.CASES[1])

PINS = [
    trout.test_topk_matches_brute_force_with_ties, trout.test_topk_signed_zero_ties_to_lower_id,
    trout.test_hand_computed_gates, trout.test_gates_sum_to_one_and_k1_is_one,
    trout.test_gates_equal_renormalised_full_softmax,
    tdisp.test_capacity_keeps_largest_gates_ties_to_lower_token,
    tdisp.test_capacity_threshold_property,
    texp.test_silu_constants_are_the_closed_forms, texp.test_expert_ffn_hand_case,
    texp.test_hand_moe_layer_one_token, texp.test_k_equals_E_with_identical_experts_is_dense_ffn,
    texp.test_layer_equals_per_token_sum_over_selected_experts,
    texp.test_aux_loss_uniform_and_hand_case, texp.test_lora_forward_equals_merged_weights,
    texp.test_lora_backward_matches_central_differences,
    tbwd.test_silu_grad_closed_form_and_differences, _pin_dx_fd_plain, _pin_dx_fd_lora_capacity,
    _pin_dlogits_fd, tbwd.test_dlogits_rows_sum_to_zero_and_k1_gate_path_vanishes,
    tremap.test_hand_case_single_slot, tremap.test_hand_case_two_overflowing_slots_of_one_token,
    _pin_remap_invariants, tremap.test_remap_with_tied_gates, tremap.test_no_overflow_equals_plain_dispatch,
    trout.test_latent_router_hand_case, trout.test_latent_router_identity_projection_is_the_plain_router,
    trout.test_latent_router_equals_merged_weight_and_python_loop,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_rejects_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, TypeError) as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"mutant {name} passed every pin"


def test_pins_pass_unmutated():
    for pin in PINS:
        pin()
