"""Seeded sweep of forward shapes on the GPU against the CPU oracle.

The shapes are drawn once from a fixed seed so that together they take every
lane mapping of the row pass (1 to 64 lanes per row), vector and scalar column
loads, padded rows, several microbatches, k up to 32, capacity limits and
both combine paths (the combine kernel, or the scatter summing few row
blocks itself).  Integer outputs bit-exact, floats within 1e-5 relative."""
import numpy as np
import pytest

import load_balancing_statistics_amd as lbs
import oracle
from gpu_helpers import (backward_tolerance, compare_forward, gpu_backward, gpu_forward,
                         oracle_forward)

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([2, 5, 8, 16, 31, 64, 96, 128, 200, 256, 300, 384, 512, 640, 1000]))
        k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32])))
        m = int(rng.choice([1, 1, 2, 3]))
        Tm = int(rng.integers(1, 1200))
        cf = float(rng.choice([0.0, 1.0, 1.25]))
        out.append((Tm * m, E, k, m, cf, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,E,k,m,cf,renorm", _cases(),
                         ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}_cf{c[4]}" for c in _cases()])
def test_forward_sweep(T, E, k, m, cf, renorm):
    print(f"case sweep T={T} E={E} k={k} m={m} cf={cf} renorm={renorm}", flush=True)
    rng = np.random.default_rng(T * 7 + E)
    # logits with a per-expert skew so that capacity limits bite
    L = (rng.standard_normal((T, E)) + rng.normal(0.0, 0.7, E)).astype(np.float32)
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf, renorm=renorm,
                        save_row_stats=True, inv_perm=True)
    g = gpu_forward(p, {"logits": L})
    r = oracle_forward(p, L)
    compare_forward(g, r, p)


@pytest.mark.parametrize("T,E,k,m,cf,renorm", _cases(12, seed=77),
                         ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}" for c in _cases(12, seed=77)])
def test_backward_sweep(T, E, k, m, cf, renorm):
    """The aux-loss gradient over the same kind of shapes, with and without
    the saved row statistics, per-microbatch upstream gradients."""
    print(f"case backward sweep T={T} E={E} k={k} m={m}", flush=True)
    rng = np.random.default_rng(T * 3 + E)
    L = (rng.standard_normal((T, E)) + rng.normal(0.0, 0.7, E)).astype(np.float32)
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf, renorm=renorm,
                        save_row_stats=True, inv_perm=True)
    g = gpu_forward(p, {"logits": L})
    r = oracle_forward(p, L)
    d_aux = np.linspace(0.5, 2.0, m)
    ref = oracle.backward(L, k, r["counts"], n_micro=m, alpha=p.alpha, d_aux=d_aux)
    scale = backward_tolerance(L, r, r["counts"], p, d_aux)
    for stats in (g["row_stats"], None):
        dl = gpu_backward(p, L, g["counts"], row_stats=stats, d_aux=d_aux)
        err = np.abs(dl.astype(np.float64) - ref)
        bound = 1e-5 * np.maximum(np.abs(ref), scale) + 1e-30
        assert (err <= bound).all(), f"{(err > bound).sum()} gradient mismatches"


@pytest.mark.parametrize("T,E,k,m,cf,renorm", _cases(10, seed=314),
                         ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}" for c in _cases(10, seed=314)])
def test_select_bias_sweep(T, E, k, m, cf, renorm):
    """Loss-free balancing: experts ranked by the fp32 sum of logit and
    selection bias (the bias row kernels), weights and statistics unbiased."""
    print(f"case bias sweep T={T} E={E} k={k} m={m}", flush=True)
    rng = np.random.default_rng(T * 5 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    b = rng.normal(0.0, 0.5, E).astype(np.float32)
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf, renorm=renorm,
                        save_row_stats=True, inv_perm=True, select_bias=True)
    g = gpu_forward(p, {"logits": L, "select_bias": b})
    r = oracle_forward(p, L, select_bias=b)
    compare_forward(g, r, p)
