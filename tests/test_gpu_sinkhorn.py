"""Sinkhorn-Knopp flow plan (LoongForge TAOT blog, section 2, Phase 1) on
the GPU against the CPU oracle.  fp64 on both sides; the GPU forms each sum
as four quarter sums of four interleaved partials and exp may differ in the
last ulp, so T, u, v are compared to 1e-10 relative."""
import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
import oracle
from gpu_helpers import DEV, assert_close_rel

pytestmark = pytest.mark.gpu


def _topology(R, per_node, cross):
    """Cost 0 inside a node and `cross` between nodes; the regularisation is
    the cross-node cost, as the page suggests."""
    node = np.arange(R) // per_node
    return np.where(node[:, None] == node[None, :], 0.0, cross)


def _gpu(a, b, C, eps, iters):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(DEV)
    T, u, v = lbs.moe_sinkhorn_plan(t(a), t(b), t(C), eps, iters)
    torch.cuda.synchronize()
    return T.cpu().numpy(), u.cpu().numpy(), v.cpu().numpy()


def _compare(a, b, C, eps, iters):
    g = _gpu(a, b, C, eps, iters)
    r = oracle.sinkhorn(a, b, C, eps, iters)
    for name, x, y in zip(("T", "u", "v"), g, r):
        assert_close_rel(x, y, 1e-10, 1e-300, name)
    return g


@pytest.mark.parametrize("R", [1, 2, 7, 16, 33, 64])
def test_sinkhorn_random(R):
    print(f"case sinkhorn R={R}", flush=True)
    rng = np.random.default_rng(R)
    a = rng.random(R) + 0.05
    b = rng.random(R) + 0.05
    b *= a.sum() / b.sum()
    C = rng.random((R, R)) * 3.0
    _compare(a, b, C, 0.7, 50)


@pytest.mark.parametrize("R,per_node", [(16, 8), (32, 8), (64, 8)])
def test_sinkhorn_taot_like(R, per_node):
    """Hot ranks supply their overload, cold ranks demand their idle
    capacity; intra-node cost 0, cross-node cost lambda = eps."""
    print(f"case sinkhorn taot R={R}", flush=True)
    rng = np.random.default_rng(100 + R)
    load = rng.pareto(1.5, size=R) + 1.0
    mean = load.mean()
    a = np.maximum(load - mean, 0.0)
    b = np.maximum(mean - load, 0.0)
    b *= a.sum() / b.sum()
    lam = 2.0
    T, u, v = _compare(a, b, _topology(R, per_node, lam), lam, 50)
    assert np.all(T[a == 0] == 0.0)            # cold ranks send nothing
    assert np.allclose(T.sum(0), b, rtol=1e-10, atol=1e-12)


def test_sinkhorn_iterations_and_convergence():
    print("case sinkhorn iterations", flush=True)
    rng = np.random.default_rng(7)
    R = 12
    a, b = rng.random(R) + 0.1, rng.random(R) + 0.1
    b *= a.sum() / b.sum()
    C = rng.random((R, R))
    T0, u0, v0 = _compare(a, b, C, 0.4, 0)       # no rounds: T = K
    assert np.allclose(T0, np.exp(-C / 0.4), rtol=1e-14)
    T, _, _ = _compare(a, b, C, 0.4, 2000)
    assert np.allclose(T.sum(1), a, rtol=1e-9) and np.allclose(T.sum(0), b, rtol=1e-12)
