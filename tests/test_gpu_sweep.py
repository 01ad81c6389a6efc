"""A seeded sweep of small random layer shapes through the whole forward on
the GPU, each checked stage by stage against the oracle (routing, dispatch,
expert rows, combine): widths, expert counts, k from 1 to E, ragged token
counts, local ranges, capacities with and without skew, bf16 and fp32 (odd
widths), the fused gather and x_perm, row-major and packed weights, and
shapes on both sides of the 320-row tile threshold."""
import numpy as np
import pytest

from sparse_mixture_experts_top_amd.workloads import Workload
from test_gpu_parity import run_and_check

pytestmark = pytest.mark.gpu


def sweep_cases(n_bf16=20, n_f32=6, seed=2024):
    """Shapes drawn from a fixed generator (the draws choose sizes only)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_bf16 + n_f32):
        f32 = i >= n_bf16
        d = int(rng.choice([20, 33, 45, 64])) if f32 else int(rng.choice([64, 128, 192, 256]))
        f = int(rng.choice([7, 19, 32])) if f32 else int(rng.choice([64, 128, 192, 256]))
        E = int(rng.integers(2, 97))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, max(2, 8000 // k)))
        if i % 5 == 4:  # many rows per expert: the 320-row tiles
            E = int(rng.integers(2, 9))
            k = int(rng.integers(1, E + 1))
            T = int(rng.integers(192 * E // k + 1, max(192 * E // k + 2, 6000 // k)))
        e_lo, e_hi = 0, -1
        if rng.random() < 0.4 and E > 2:
            e_lo = int(rng.integers(0, E - 1))
            e_hi = int(rng.integers(e_lo + 1, E + 1))
        cap = 0
        if rng.random() < 0.3:
            cap = max(1, int(T * k / E * rng.uniform(0.3, 1.5)))
        zipf = float(rng.choice([0.0, 0.8, 1.5]))
        w = Workload(f"sweep{i}", T=T, d=d, E=E, k=k, f=f, e_lo=e_lo, e_hi=e_hi, capacity=cap, zipf_s=zipf,
                     dtype="f32" if f32 else "bf16")
        x_perm = bool(rng.random() < 0.5)
        packed = (not f32) and d % 128 == 0 and bool(rng.random() < 0.5)
        cases.append((w, x_perm, packed))
    return cases


CASES = sweep_cases()


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape(i):
    w, x_perm, packed = CASES[i]
    run_and_check(w, seed=100 + i, x_perm=x_perm, packed=packed)


def backward_cases(n=12, seed=2025):
    """Shapes for the backward sweep (T k <= 3000 keeps the float64 checks
    quick); LoRA adapters on some bf16 shapes, packed weights where they fit."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        f32 = i % 4 == 3
        d = int(rng.choice([20, 33, 48])) if f32 else int(rng.choice([64, 128, 192, 256]))
        f = int(rng.choice([7, 19, 32])) if f32 else int(rng.choice([64, 128, 256]))
        E = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, max(2, 3000 // k)))
        e_lo, e_hi = 0, -1
        if rng.random() < 0.4 and E > 2:
            e_lo = int(rng.integers(0, E - 1))
            e_hi = int(rng.integers(e_lo + 1, E + 1))
        cap = max(1, int(T * k / E * rng.uniform(0.5, 1.5))) if rng.random() < 0.3 else 0
        r = 0 if f32 or rng.random() < 0.6 else int(rng.choice([8, 16]))
        w = Workload(f"bsweep{i}", T=T, d=d, E=E, k=k, f=f, e_lo=e_lo, e_hi=e_hi, capacity=cap,
                     zipf_s=float(rng.choice([0.0, 1.0])), dtype="f32" if f32 else "bf16", lora_r=r,
                     lora_alpha=32.0 if r else 0.0, lora_b="normal")
        packed = (not f32) and d % 128 == 0 and f % 128 == 0 and bool(rng.random() < 0.6)
        cases.append((w, packed))
    return cases


BWD_CASES = backward_cases()


@pytest.mark.parametrize("i", range(len(BWD_CASES)))
def test_random_shape_backward(i):
    from test_gpu_backward import check_backward
    w, packed = BWD_CASES[i]
    check_backward(w, packed, seed=200 + i)


def remap_cases(n=8, seed=2026):
    """Shapes for the remapping sweep: capacities below the mean load, so
    assignments overflow (2k <= E and 2k <= 32 for the alternates)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        f32 = i % 4 == 3
        d = int(rng.choice([20, 48])) if f32 else int(rng.choice([64, 128, 192]))
        f = int(rng.choice([7, 32])) if f32 else int(rng.choice([64, 128]))
        E = int(rng.integers(4, 80))
        k = int(rng.integers(1, min(E // 2, 16) + 1))
        T = int(rng.integers(20, max(21, 3000 // k)))
        e_lo, e_hi = 0, -1
        if rng.random() < 0.4:
            e_lo = int(rng.integers(0, E - 1))
            e_hi = int(rng.integers(e_lo + 1, E + 1))
        cap = max(1, int(T * k / E * rng.uniform(0.2, 0.9)))
        w = Workload(f"rsweep{i}", T=T, d=d, E=E, k=k, f=f, e_lo=e_lo, e_hi=e_hi, capacity=cap,
                     zipf_s=float(rng.choice([0.5, 1.2])), dtype="f32" if f32 else "bf16")
        cases.append((w, bool(rng.random() < 0.5)))
    return cases


REMAP_CASES = remap_cases()


@pytest.mark.parametrize("i", range(len(REMAP_CASES)))
def test_random_shape_remap(i):
    from test_gpu_variants import check_remap_case
    w, x_perm = REMAP_CASES[i]
    check_remap_case(w, seed=300 + i, x_perm=x_perm)


def lora_cases(n=10, seed=2027):
    """Shapes for the adapter sweep: ranks from 1 to 64 (the matrix-core
    forms at r <= 16, the extra K step at r = 16, the row loops above),
    zero-initialised B on some, packed weights where d, f % 128 == 0."""
    rng = np.random.default_rng(seed)
    ranks = [1, 5, 8, 12, 16, 16, 24, 32, 48, 64]
    cases = []
    for i in range(n):
        r = int(ranks[i % len(ranks)])
        d = int(rng.choice([64, 128, 192, 256]))
        f = int(rng.choice([64, 128, 192, 256]))
        E = int(rng.integers(2, 41))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, max(2, 2500 // k)))
        e_lo, e_hi = 0, -1
        if rng.random() < 0.5 and E > 2:
            e_lo = int(rng.integers(0, E - 1))
            e_hi = int(rng.integers(e_lo + 1, E + 1))
        cap = max(1, int(T * k / E * rng.uniform(0.5, 1.5))) if rng.random() < 0.25 else 0
        w = Workload(f"lsweep{i}", T=T, d=d, E=E, k=k, f=f, e_lo=e_lo, e_hi=e_hi, capacity=cap,
                     zipf_s=float(rng.choice([0.0, 1.0])), lora_r=r, lora_alpha=float(rng.choice([8.0, 32.0])),
                     lora_b="zero" if rng.random() < 0.2 else "normal", aux_coef=0.01)
        packed = d % 128 == 0 and f % 128 == 0 and bool(rng.random() < 0.5)
        cases.append((w, bool(rng.random() < 0.5), packed))
    return cases


LORA_CASES = lora_cases()


@pytest.mark.parametrize("i", range(len(LORA_CASES)))
def test_random_shape_lora(i):
    from test_gpu_parity import check_lora
    w, x_perm, packed = LORA_CASES[i]
    check_lora(w, x_perm, packed, seed=400 + i)


def latent_cases(n=6, seed=2028):
    """Shapes for the latent-router sweep: latent widths 64 to 256, model
    widths to 512, with and without a logit bias, local ranges."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256, 384, 512]))
        dc = int(rng.choice([64, 128, 192, 256]))
        E = int(rng.integers(2, 201))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, max(2, 3000 // k)))
        e_lo, e_hi = 0, -1
        if rng.random() < 0.4 and E > 2:
            e_lo = int(rng.integers(0, E - 1))
            e_hi = int(rng.integers(e_lo + 1, E + 1))
        cases.append(Workload(f"csweep{i}", T=T, d=d, E=E, k=k, f=int(rng.choice([64, 128])), e_lo=e_lo,
                              e_hi=e_hi, zipf_s=float(rng.choice([0.0, 1.0])), latent_dc=dc))
    return cases


LATENT_CASES = latent_cases()


@pytest.mark.parametrize("i", range(len(LATENT_CASES)))
def test_random_shape_latent(i):
    from test_gpu_variants import check_latent_case
    check_latent_case(LATENT_CASES[i], seed=500 + i)
