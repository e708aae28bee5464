"""Masked P (page mhpq.cn/news/998159 section 4.4) and the full logits
gradient -- all-token or masked P, plus the gradient through the gate weights
with or without renormalisation -- on the GPU against the CPU oracle.

Forward: integer outputs bit-exact, floating point 1e-5 relative.  Gradient:
per element 1e-5 * (|ref| + scale), where scale = p_i (|G_i| + sum_e |G_e| p_e)
and G = dL/dp is formed here in numpy from the definitions, with the
renormalised weight term taken as (|dW_j| + |D|)/Z (the magnitude of the
terms that cancel in it and in the softmax Jacobian).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
import oracle
from gpu_helpers import DEV, compare_forward, gpu_forward, oracle_forward, params_of

pytestmark = pytest.mark.gpu

# (workload, T override, n_micro override)
SMALL = [("v3_shape", 3000 + 5, 1), ("v4_shape", 4 * 1500, 4), ("zipf_top2", 5000 + 3, 1),
         ("switch_top1", 2048 + 9, 1)]
ODD = [(1500 + 7, 33, 3, 1), (600, 1024, 32, 2), (1200, 250, 5, 3)]


def _masked_case(name, T, m):
    w = replace(WORKLOADS[name], T=T, n_micro=m)
    return w, make_inputs(w, 2)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_masked_forward_small(case):
    name, T, m = case
    print(f"case masked_forward {name} T={T} m={m}", flush=True)
    w, inp = _masked_case(name, T, m)
    p = params_of(w, p_masked=True)
    g = gpu_forward(p, inp)
    r = oracle.route(inp["logits"], w.k, n_micro=w.n_micro, capacity_factor=w.capacity_factor,
                     alpha=w.alpha, renorm=w.renorm, p_masked=True)
    compare_forward(g, r, p)


def test_masked_forward_full_v4():
    w = WORKLOADS["v4_shape"]
    print("case masked_forward_full v4_shape", flush=True)
    inp = make_inputs(w, 0)
    p = params_of(w, p_masked=True)
    g = gpu_forward(p, inp)
    r = oracle.route(inp["logits"], w.k, n_micro=w.n_micro, capacity_factor=w.capacity_factor,
                     alpha=w.alpha, renorm=w.renorm, p_masked=True)
    compare_forward(g, r, p)


def _grad_scale(L, r, counts, k, m, alpha, d_aux, masked, renorm, dW):
    """p_i (|G_i| + sum_e |G_e| p_e) per element, G = dL/dp from the definitions."""
    T, E = L.shape
    Tm = T // m
    p = np.exp(L.astype(np.float64) - r["row_max"][:, None]) / r["row_sum"][:, None]
    g = np.ones(m) if d_aux is None else np.asarray(d_aux, np.float64)
    f = np.repeat(np.asarray(counts, np.float64).reshape(m, E) / (Tm * k), Tm, axis=0)
    gt = np.repeat(g, Tm)[:, None]
    idx = r["topk_idx"].astype(np.int64)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, idx, 1.0, axis=1)
    G = gt * alpha * E * f * (mask / (Tm * k) if masked else 1.0 / Tm)
    if dW is not None:
        pk = np.take_along_axis(p, idx, axis=1)
        if renorm:
            # (dW_j - D)/Z cancels when dW_j ~ D: rounding scales with |dW_j| + |D|
            Z = pk.sum(1, keepdims=True)
            D = (dW * pk).sum(1, keepdims=True) / Z
            add = (np.abs(dW) + np.abs(D)) / Z
        else:
            add = np.abs(dW)
        Gw = np.zeros((T, E))
        np.put_along_axis(Gw, idx, add, axis=1)
        G = np.abs(G) + Gw
    return p * (np.abs(G) + (np.abs(G) * p).sum(1, keepdims=True))


def _check_grad(L, w, p, g, r, masked, renorm, with_w, use_stats, seed):
    T, E, k, m = w.T, w.E, w.k, w.n_micro
    rng = np.random.default_rng(seed)
    d_aux = np.linspace(0.5, 2.0, m)
    dW = rng.standard_normal((T, k)).astype(np.float32) if with_w else None
    ref = oracle.backward(L, k, r["counts"], n_micro=m, alpha=w.alpha, d_aux=d_aux, p_masked=masked,
                          topk_idx=r["topk_idx"], renorm=renorm, d_topk_w=dW)
    dev = torch.device(DEV)
    Lt = torch.from_numpy(L).to(dev)
    dl = torch.full_like(Lt, float("nan"))
    lbs.moe_route_backward(p, Lt, torch.from_numpy(g["counts"]).to(dev), dl,
                           row_stats=torch.from_numpy(g["row_stats"]).to(dev) if use_stats else None,
                           d_aux=torch.from_numpy(d_aux.astype(np.float32)).to(dev),
                           topk_idx=torch.from_numpy(g["topk_idx"]).to(dev),
                           d_topk_w=None if dW is None else torch.from_numpy(dW).to(dev))
    torch.cuda.synchronize()
    got = dl.cpu().numpy().astype(np.float64)
    scale = _grad_scale(L, r, r["counts"], k, m, w.alpha, d_aux, masked, renorm, dW)
    err = np.abs(got - ref)
    bound = 1e-5 * (np.abs(ref) + scale) + 1e-30
    bad = ~(err <= bound)
    assert not bad.any(), (f"{bad.sum()} gradient mismatches; worst ratio {np.nanmax(err / bound)} at "
                           f"{np.unravel_index(np.nanargmax(err / bound), err.shape)}")


@pytest.mark.parametrize("with_w", [False, True])
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_grad_small(case, masked, renorm, with_w):
    name, T, m = case
    print(f"case grad {name} masked={masked} renorm={renorm} w={with_w}", flush=True)
    w, inp = _masked_case(name, T, m)
    w = replace(w, renorm=renorm)
    p = params_of(w, p_masked=masked)
    g = gpu_forward(p, inp)
    r = oracle.route(inp["logits"], w.k, n_micro=w.n_micro, capacity_factor=w.capacity_factor,
                     alpha=w.alpha, renorm=renorm, p_masked=masked)
    compare_forward(g, r, p)
    _check_grad(inp["logits"], w, p, g, r, masked, renorm, with_w, use_stats=True, seed=1)


@pytest.mark.parametrize("shape", ODD, ids=lambda s: "T%d_E%d_k%d_m%d" % s)
def test_grad_odd_shapes(shape):
    T, E, k, m = shape
    print(f"case grad_odd T={T} E={E} k={k} m={m}", flush=True)
    w = replace(WORKLOADS["v3_shape"], T=T, E=E, k=k, n_micro=m, alpha=0.05)
    inp = make_inputs(w, 4)
    for masked, renorm in [(True, True), (False, False)]:
        ww = replace(w, renorm=renorm)
        p = params_of(ww, p_masked=masked)
        g = gpu_forward(p, inp)
        r = oracle.route(inp["logits"], k, n_micro=m, capacity_factor=w.capacity_factor,
                         alpha=w.alpha, renorm=renorm, p_masked=masked)
        compare_forward(g, r, p)
        _check_grad(inp["logits"], ww, p, g, r, masked, renorm, True, use_stats=False, seed=5)


def test_grad_full_v4_masked_weights():
    w = WORKLOADS["v4_shape"]
    print("case grad_full v4_shape masked + weights", flush=True)
    inp = make_inputs(w, 0)
    p = params_of(w, p_masked=True)
    g = gpu_forward(p, inp)
    r = oracle.route(inp["logits"], w.k, n_micro=w.n_micro, capacity_factor=w.capacity_factor,
                     alpha=w.alpha, renorm=w.renorm, p_masked=True)
    _check_grad(inp["logits"], w, p, g, r, True, w.renorm, True, use_stats=True, seed=7)


@pytest.mark.parametrize("T,E,k,m,kind", [(4000, 384, 6, 2, "wide"), (3001, 256, 8, 1, "hot"),
                                          (2500, 64, 4, 1, "hot")])
def test_masked_P_peaked_logits(T, E, k, m, kind):
    """Masked P where picked probabilities span many orders of magnitude:
    router logits N(0, 8^2) ("wide"), or three experts boosted by +30 so that
    every token's remaining picks carry probabilities near 1e-13 ("hot").
    Experts picked only as a low choice then have a tiny P, which must still
    match the oracle within 1e-5 relative."""
    print(f"case masked_P_peaked T={T} E={E} k={k} m={m} kind={kind}", flush=True)
    rng = np.random.default_rng(T + E)
    if kind == "wide":
        L = (8.0 * rng.standard_normal((T, E))).astype(np.float32)
    else:
        L = rng.standard_normal((T, E)).astype(np.float32)
        L[:, rng.choice(E, 3, replace=False)] += 30.0
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=1.0, alpha=0.01, renorm=True,
                        save_row_stats=True, inv_perm=True, p_masked=True)
    g = gpu_forward(p, {"logits": L})
    r = oracle.route(L, k, n_micro=m, capacity_factor=1.0, alpha=0.01, renorm=True, p_masked=True)
    if kind == "hot":
        Pr = r["P"][r["P"] > 0]
        assert Pr.min() < 1e-9 * Pr.max(), "the case must hold experts with tiny masked P"
    compare_forward(g, r, p)
