"""Selection-bias routing (page mhpq.cn/news/998159 section 4.3) and the bias
update step on the GPU against the CPU oracle.

The bias steers the expert choice only (fp32 sums l + b, ties to the lower
expert); weights, P and the statistics use the unbiased softmax.  Integer
outputs must match bit for bit, floating point within 1e-5 relative, and the
bias update (one fp32 add per expert) bit for bit.
"""
import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
import oracle
from gpu_helpers import (DEV, assert_equal, compare_forward, gpu_forward, oracle_forward,
                         params_of)

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["v3_select_bias"]

# (T, E, k, n_micro): v3 and v4 lane mappings, narrow and wide segments, an
# expert count that is not a multiple of 4 (scalar loads), and the maximum E.
SHAPES = [(3000 + 5, 256, 8, 1), (4 * 1500, 384, 6, 4), (5000 + 3, 64, 2, 1),
          (2000 + 1, 8, 1, 1), (1500 + 7, 250, 5, 1), (600, 1024, 32, 2), (777, 33, 3, 1)]


def _case(T, E, k, m, seed, scale=0.5):
    from dataclasses import replace
    w = replace(BASE, T=T, E=E, k=k, n_micro=m, select_bias_scale=scale, alpha=0.01)
    return w, make_inputs(w, seed)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T%d_E%d_k%d_m%d" % s)
def test_bias_forward_small(shape, seed):
    T, E, k, m = shape
    print(f"case bias_forward_small T={T} E={E} k={k} m={m} seed={seed}", flush=True)
    w, inp = _case(T, E, k, m, seed)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"], select_bias=inp["select_bias"])
    compare_forward(g, r, p)


def test_bias_forward_full():
    w = BASE
    print(f"case bias_forward_full T={w.T} E={w.E} k={w.k}", flush=True)
    inp = make_inputs(w, 0)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"], select_bias=inp["select_bias"])
    compare_forward(g, r, p)


def test_bias_zero_equals_unbiased():
    """b = 0 reproduces the unbiased path: same selection, weights, perm."""
    w, inp = _case(3000 + 5, 256, 8, 1, 3)
    inp0 = dict(inp, select_bias=np.zeros(w.E, np.float32))
    print("case bias_zero_equals_unbiased", flush=True)
    gb = gpu_forward(params_of(w), inp0)
    gu = gpu_forward(params_of(w, select_bias=False), {"logits": inp["logits"]})
    for key in ("topk_idx", "counts", "offsets", "perm", "inv_perm", "dropped", "topk_w"):
        assert_equal(gb[key], gu[key], key)
    np.testing.assert_allclose(gb["P"], gu["P"], rtol=1e-6, atol=0)


def test_bias_ties_and_forced_choice():
    """Ties made by fp32 rounding of l + b go to the lower expert; a huge bias
    forces the choice (weights stay the unbiased softmax); constant rows make
    every row a tie and take the overflow path."""
    print("case bias_ties_and_forced_choice", flush=True)
    T, E = 2048 + 3, 64
    rng = np.random.default_rng(5)
    L = (rng.integers(-3, 4, size=(T, E)) / 4).astype(np.float32)
    L[: T // 4] = 1.0                                  # all-equal rows
    b = (rng.integers(-2, 3, size=E) * 2.0 ** -24).astype(np.float32)  # rounds away at |l| >= 1
    b[7] = 2.0 ** -22                                  # representable at 1.0: expert 7 wins ties
    for k in (1, 2, 5):
        w, _ = _case(T, E, k, 1, 0)
        p = params_of(w)
        g = gpu_forward(p, {"logits": L, "select_bias": b})
        r = oracle_forward(p, L, select_bias=b)
        compare_forward(g, r, p)
    bf = np.zeros(E, np.float32)
    bf[11], bf[0] = 1.0e3, -1.0e3
    w, _ = _case(T, E, 3, 1, 0)
    p = params_of(w)
    g = gpu_forward(p, {"logits": L, "select_bias": bf})
    r = oracle_forward(p, L, select_bias=bf)
    compare_forward(g, r, p)
    assert np.all(g["topk_idx"][:, 0] == 11) and not np.any(g["topk_idx"] == 0)


@pytest.mark.parametrize("m", [1, 3])
def test_bias_update_matches_oracle(m):
    """moe_route_bias_update: bit-exact fp32 steps; loads equal to the mean
    (an integer comparison) leave the bias unchanged."""
    print(f"case bias_update m={m}", flush=True)
    E, k, Tm = 300, 4, 750  # mean load m*750*4/300 = 10*m, an integer
    rng = np.random.default_rng(9 + m)
    cnt = rng.multinomial(Tm * k, np.ones(E) / E, size=m).astype(np.int32)
    cnt[:, 5] = 10                                    # exactly at the mean
    b0 = (rng.standard_normal(E) * 100).astype(np.float32)
    want = oracle.bias_update(cnt, T=m * Tm, k=k, gamma=0.125, bias=b0)
    p = lbs.make_params(m * Tm, E, k, n_micro=m)
    bt = torch.from_numpy(b0.copy()).to(DEV)
    ct = torch.from_numpy(cnt).to(DEV)
    lbs.moe_route_bias_update(p, ct, 0.125, bt)
    torch.cuda.synchronize()
    got = bt.cpu().numpy()
    assert_equal(got, want, "bias")
    assert got[5] == b0[5]


def test_bias_training_loop_balances():
    """Forward + update repeated on one batch with a skewed selection bias:
    the loads move toward the mean (CV decreases), every step matching the
    oracle's forward on the GPU's current bias."""
    print("case bias_training_loop", flush=True)
    w, inp = _case(4096, 64, 4, 1, 4, scale=0.0)
    b = np.linspace(-1.0, 1.0, w.E).astype(np.float32)
    p = params_of(w, select_bias=True)
    cvs = []
    bt = torch.from_numpy(b).to(DEV)
    for step in range(6):
        g = gpu_forward(p, {"logits": inp["logits"], "select_bias": bt.cpu().numpy()})
        r = oracle_forward(p, inp["logits"], select_bias=bt.cpu().numpy())
        compare_forward(g, r, p)
        cvs.append(float(g["cv"][0]))
        want = oracle.bias_update(r["counts"], T=w.T, k=w.k, gamma=0.2, bias=bt.cpu().numpy())
        lbs.moe_route_bias_update(p, torch.from_numpy(g["counts"]).to(DEV), 0.2, bt)
        torch.cuda.synchronize()
        assert_equal(bt.cpu().numpy(), want, "bias after step")
    assert cvs[-1] < cvs[0], cvs


# (T, E, k, n_micro): one microbatch with the step inside the scatter (a
# statistics workgroup; the statistics spread over six row blocks), several
# microbatches and the one-launch path (the step by the update kernel)
STEP_SHAPES = [(3000, 256, 8, 1), (30000, 256, 8, 1), (9000, 64, 2, 1), (4000, 300, 4, 2), (2048, 8, 2, 1)]


@pytest.mark.parametrize("shape", STEP_SHAPES, ids=lambda s: "T%d_E%d_k%d_m%d" % s)
def test_route_with_bias_update(shape):
    """moe_route_with_bias_update gives the bytes of moe_route followed by
    moe_route_bias_update, its forward matches the oracle on the bias it
    started from and its bias step matches the oracle's on the counts."""
    T, E, k, m = shape
    print(f"case route_with_bias_update T={T} E={E} k={k} m={m}", flush=True)
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E), dtype=np.float32)
    b0 = (np.round(rng.standard_normal(E) * 4) / 8).astype(np.float32)
    gamma = 0.0625
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=1.25, alpha=0.01, renorm=True,
                        save_row_stats=True, inv_perm=True, select_bias=True)
    dev = torch.device(DEV)
    Lg = torch.from_numpy(L).to(dev)
    res = []
    for fused in (True, False):
        out = lbs.alloc_outputs(p, device=dev)
        ws = lbs.alloc_workspace(p, device=dev)
        bt = torch.from_numpy(b0.copy()).to(dev)
        if fused:
            lbs.moe_route_with_bias_update(p, out, ws, bt, gamma, logits=Lg)
        else:
            lbs.moe_route(p, out, ws, logits=Lg, select_bias=bt)
            lbs.moe_route_bias_update(p, out["counts"], gamma, bt)
        torch.cuda.synchronize()
        res.append(({key: v.cpu().numpy() for key, v in out.items() if v is not None}, bt.cpu().numpy()))
    (g, bias_f), (h, bias_s) = res
    for key in g:
        assert np.array_equal(g[key].view(np.uint8), h[key].view(np.uint8)), key
    assert np.array_equal(bias_f.view(np.uint32), bias_s.view(np.uint32)), "bias"
    compare_forward(g, oracle_forward(p, L, select_bias=b0), p)
    want = oracle.bias_update(g["counts"], T=T, k=k, gamma=gamma, bias=b0)
    assert_equal(bias_f, want, "bias after the step")
    assert not np.array_equal(bias_f, b0)
