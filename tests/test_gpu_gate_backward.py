"""Gate backward dX = dlogits.Wg^T (bf16) and dWg = X^T.dlogits (fp32) on the
GPU against the CPU oracle (fp64 from the same bf16 bits and fp32 dlogits).

Bounds: dX within half a bf16 ulp of the fp64 value (2^-8 relative) plus
1e-5 of sum_e |dl*Wg| for the fp32 accumulation; dWg within 1e-5 of
sum_t |X*dl| (the magnitude of its terms).
"""
import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from load_balancing_statistics_amd.workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
import oracle
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _run(T, d, E, X, W, G, want_dx=True, want_dw=True):
    dev = torch.device(DEV)
    p = lbs.make_params(T, E, min(2, E), d=d)
    Xt = torch.from_numpy(X.view(np.int16)).to(dev)
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    Gt = torch.from_numpy(G).to(dev)
    dX = torch.full((T, d), -1, dtype=torch.int16, device=dev) if want_dx else None
    dW = torch.full((d, E), float("nan"), dtype=torch.float32, device=dev) if want_dw else None
    ws = torch.empty(max(256, lbs.moe_gate_backward_workspace_size(p)), dtype=torch.uint8, device=dev)
    ws.fill_(0xCD)
    lbs.moe_gate_backward(p, Xt, Wt, Gt, dX=dX, dWg=dW, workspace=ws)
    torch.cuda.synchronize()
    return (None if dX is None else dX.cpu().numpy().view(np.uint16),
            None if dW is None else dW.cpu().numpy())


def _check(T, d, E, X, W, G, got_dx, got_dw):
    ref_dx, ref_dw = oracle.gate_backward(X, W, G.astype(np.float64))
    Xf = bf16_bits_to_f32(X).astype(np.float64)
    Wf = bf16_bits_to_f32(W).astype(np.float64)
    Gf = G.astype(np.float64)
    if got_dx is not None:
        dx = bf16_bits_to_f32(got_dx).astype(np.float64)
        mag = np.abs(Gf) @ np.abs(Wf).T
        bound = 2.0 ** -8 * np.abs(ref_dx) + 1e-5 * mag + 1e-38
        bad = ~(np.abs(dx - ref_dx) <= bound)
        assert not bad.any(), f"dX: {bad.sum()} mismatches, first {np.argwhere(bad)[0]}"
    if got_dw is not None:
        mag = np.abs(Xf).T @ np.abs(Gf)
        bound = 1e-5 * mag + 1e-30
        bad = ~(np.abs(got_dw - ref_dw) <= bound)
        assert not bad.any(), f"dWg: {bad.sum()} mismatches, first {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("shape", [(1000 + 7, 256, 8), (777, 128, 16), (300, 64, 33), (129, 72, 64),
                                   (5, 8, 1), (4096, 520, 3), (2000, 200, 12), (64, 1024, 8)],
                         ids=lambda s: "T%d_d%d_E%d" % s)
def test_gate_backward_small(shape):
    T, d, E = shape
    print(f"case gate_backward T={T} d={d} E={E}", flush=True)
    rng = np.random.default_rng(T + d + E)
    X = f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    W = f32_to_bf16_bits(0.02 * rng.standard_normal((d, E), dtype=np.float32))
    G = (1e-3 * rng.standard_normal((T, E))).astype(np.float32)
    dx, dw = _run(T, d, E, X, W, G)
    _check(T, d, E, X, W, G, dx, dw)
    # each output alone
    dx2, _ = _run(T, d, E, X, W, G, want_dw=False)
    _, dw2 = _run(T, d, E, X, W, G, want_dx=False)
    assert np.array_equal(dx2, dx) and np.array_equal(dw2, dw)


def test_gate_backward_full():
    """The gate workload: route, aux-loss backward, then the gate backward of
    the resulting dlogits at T=16384, d=4096, E=8."""
    w = WORKLOADS["gate_top2"]
    print(f"case gate_backward_full T={w.T} d={w.d} E={w.E}", flush=True)
    inp = make_inputs(w, 0)
    rng = np.random.default_rng(3)
    G = (1e-4 * rng.standard_normal((w.T, w.E))).astype(np.float32)
    dx, dw = _run(w.T, w.d, w.E, inp["X"], inp["Wg"], G)
    _check(w.T, w.d, w.E, inp["X"], inp["Wg"], G, dx, dw)


def test_gate_backward_deterministic():
    T, d, E = 2048, 256, 8
    rng = np.random.default_rng(11)
    X = f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    W = f32_to_bf16_bits(0.02 * rng.standard_normal((d, E), dtype=np.float32))
    G = rng.standard_normal((T, E)).astype(np.float32)
    a = _run(T, d, E, X, W, G)
    b = _run(T, d, E, X, W, G)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
