"""The one-launch path for small microbatches (E of 1, 2, 4 or 8, k*E <= 16,
at most 32768 logits a microbatch) against the oracle and against the
multi-kernel path (flag MOE_MULTI_KERNEL) on the same logits: integer outputs
bit-exact with both, floating-point outputs within 1e-5 of the oracle and
1e-6 of the other path (they differ only in the order of a row's sum).
Cases just outside the path (16 experts, k*E above 16) check that both
flags then give the multi-kernel results."""
import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
import oracle
from gpu_helpers import (DEV, INT_KEYS, assert_close_rel, assert_equal, compare_forward, gpu_forward,
                         oracle_forward)

pytestmark = pytest.mark.gpu

FLOAT_KEYS = ("topk_w", "row_stats", "f", "P", "aux_loss", "cv", "max_over_mean", "extra_stats")

# (T, E, k, n_micro, capacity factor, explicit capacity, renorm, p_masked, logits kind)
CASES = [
    (1, 1, 1, 1, 1.0, -1, False, False, "normal"),
    (5000, 1, 1, 2, 1.25, -1, False, False, "normal"),
    (63, 2, 1, 1, 1.0, -1, True, False, "normal"),
    (16384, 2, 2, 1, 1.0, -1, True, True, "quantized"),      # Tm*E = 32768, 16 row blocks
    (1023, 4, 2, 1, 1.25, -1, True, False, "normal"),
    (8192, 4, 3, 1, 1.1, -1, False, True, "normal"),         # 8 row blocks, 8 rows a thread
    (1024, 8, 1, 1, 1.25, -1, False, False, "normal"),       # one row block exactly
    (1025, 8, 2, 1, 1.25, -1, True, False, "normal"),        # one row of a second block
    (4096, 8, 1, 1, 1.25, -1, False, False, "normal"),       # Switch top-1
    (4096, 8, 8, 1, 1.0, -1, True, False, "normal"),         # k*E = 64: multi-kernel
    (4096, 4, 4, 1, 1.0, -1, True, False, "normal"),         # k = E
    (12288, 8, 2, 3, 1.0, -1, True, False, "normal"),        # three microbatches of 4096
    (3000, 8, 4, 1, 1.0, 0, True, False, "normal"),          # capacity 0: all dropped
    (3000, 8, 2, 1, 1.0, 5, True, False, "quantized"),       # explicit capacity, ties
    (3000, 8, 2, 1, 0.0, -1, True, True, "signed_zero"),     # unlimited, -0.0 / +0.0
    (2048, 16, 1, 1, 1.2, -1, False, False, "normal"),       # 16 experts: multi-kernel
    (6144, 8, 2, 3, 1.0, -1, True, True, "quantized"),
    (1500, 8, 2, 1, 1.05, -1, True, False, "equal"),         # every logit equal
    (32768, 1, 1, 1, 1.0, 100, False, False, "normal"),      # 32 rows a thread, drops
]


def _logits(T, E, kind, rng):
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "equal":
        return np.full((T, E), -1.5, np.float32)
    if kind == "quantized":
        return (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    if kind == "signed_zero":
        return rng.choice(np.array([-1.0, -0.0, 0.0, 0.5], np.float32), size=(T, E))
    raise ValueError(kind)


def _params(case, **over):
    T, E, k, m, cf, cap, renorm, masked, _ = case
    kw = dict(n_micro=m, capacity_factor=cf, capacity=cap, alpha=0.02, renorm=renorm,
              save_row_stats=True, inv_perm=True, p_masked=masked)
    kw.update(over)
    return lbs.make_params(T, E, k, **kw)


def _compare_paths(one, multi):
    for key in INT_KEYS + ("inv_perm", "status"):
        assert_equal(one[key], multi[key], key + " (one launch vs multi-kernel)")
    for key in FLOAT_KEYS:
        assert_close_rel(one[key], multi[key], 1e-6, 1e-30, key + " (one launch vs multi-kernel)")


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}_C{c[5]}_{c[8]}"
                                             f"{'_masked' if c[7] else ''}" for c in CASES])
def test_one_launch(case):
    print(f"case one_launch {case}", flush=True)
    T, E = case[0], case[1]
    L = _logits(T, E, case[8], np.random.default_rng(T * 31 + E))
    p = _params(case)
    one = gpu_forward(p, {"logits": L})
    multi = gpu_forward(_params(case, multi_kernel=True), {"logits": L})
    compare_forward(one, oracle_forward(p, L), p)
    _compare_paths(one, multi)
    if case[5] == 0:
        assert one["dropped"].all()


@pytest.mark.parametrize("E,k", [(8, 2), (4, 3)])
def test_one_launch_select_bias(E, k):
    """Selection bias: the choice by l + b_e, with ties the bias creates."""
    print(f"case one_launch bias E={E} k={k}", flush=True)
    T = 3000
    rng = np.random.default_rng(E)
    L = (np.round(rng.standard_normal((T, E)) * 4) / 4).astype(np.float32)
    b = (np.round(rng.standard_normal(E) * 4) / 4).astype(np.float32)
    mk = lambda **o: lbs.make_params(T, E, k, capacity_factor=1.25, alpha=0.01, renorm=True,
                                     save_row_stats=True, inv_perm=True, select_bias=True, **o)
    p = mk()
    one = gpu_forward(p, {"logits": L, "select_bias": b})
    multi = gpu_forward(mk(multi_kernel=True), {"logits": L, "select_bias": b})
    compare_forward(one, oracle_forward(p, L, select_bias=b), p)
    _compare_paths(one, multi)


def test_one_launch_unaligned_logits():
    """Logits at a 4-byte but not 16-byte aligned address: scalar loads."""
    print("case one_launch unaligned", flush=True)
    T, E, k = 2000, 8, 2
    rng = np.random.default_rng(9)
    L = rng.standard_normal((T, E), dtype=np.float32)
    dev = torch.device(DEV)
    buf = torch.empty(T * E + 4, dtype=torch.float32, device=dev)
    Lg = buf[1:1 + T * E].view(T, E)
    Lg.copy_(torch.from_numpy(L).to(dev))
    assert Lg.data_ptr() % 16 != 0
    p = lbs.make_params(T, E, k, capacity_factor=1.0, renorm=True, save_row_stats=True, inv_perm=True)
    out = lbs.alloc_outputs(p, device=dev)
    ws = lbs.alloc_workspace(p, device=dev)
    lbs.moe_route(p, out, ws, logits=Lg)
    torch.cuda.synchronize()
    g = {key: (None if v is None else v.cpu().numpy()) for key, v in out.items()}
    compare_forward(g, oracle_forward(p, L), p)


def test_one_launch_nonfinite():
    """A NaN or +inf row sets the status bit; the other rows are routed
    exactly, and every expert index stays in range."""
    print("case one_launch nonfinite", flush=True)
    T, E, k = 3000, 8, 2
    rng = np.random.default_rng(11)
    for bad in [np.nan, np.inf, -np.inf]:
        L = rng.standard_normal((T, E), dtype=np.float32)
        if bad == -np.inf:
            L[1500, :] = bad  # only -inf in the row
        else:
            L[1500, 3] = bad
        p = lbs.make_params(T, E, k, capacity_factor=1.0, renorm=True, save_row_stats=True, inv_perm=True)
        g = gpu_forward(p, {"logits": L})
        assert g["status"][0] & lbs.MOE_STATUS_NONFINITE
        assert ((g["topk_idx"] >= 0) & (g["topk_idx"] < E)).all()
        ok = np.ones(T, bool)
        ok[1500] = False
        ro = oracle.route(L[ok], k, capacity_factor=0.0, renorm=True)
        assert_equal(g["topk_idx"][ok], ro["topk_idx"], "topk_idx of finite rows")
    g = gpu_forward(lbs.make_params(T, E, k), {"logits": rng.standard_normal((T, E), dtype=np.float32)})
    assert g["status"][0] == 0


def test_one_launch_gate():
    """Gate GEMM followed by the one-launch routing; the same bf16 logits
    through the multi-kernel path give identical integer outputs."""
    from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
    from gpu_helpers import params_of
    w = WORKLOADS["gate_top2"].scaled(T=2048, d=512)
    print(f"case one_launch gate T={w.T} d={w.d} E={w.E}", flush=True)
    inp = make_inputs(w, 0)
    p = params_of(w)
    one = gpu_forward(p, inp)
    multi = gpu_forward(params_of(w, multi_kernel=True), inp)
    assert_equal(one["logits"], multi["logits"], "logits")
    _compare_paths(one, multi)
    compare_forward(one, oracle_forward(params_of(w, d=0), one["logits"]), p)


def _sweep(n=30, seed=77):
    """Shapes and options drawn once inside the one-launch limits: E of 1, 2,
    4 or 8, k*E <= 16, up to 32768 logits a microbatch, 1-5 microbatches."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.integers(1, min(E, 16 // E) + 1))
        m = int(rng.choice([1, 1, 2, 3, 5]))
        Tm = int(rng.integers(1, 32768 // E + 1))
        cf = float(rng.choice([0.0, 0.5, 1.0, 1.1, 1.25]))
        flags = dict(renorm=bool(rng.integers(0, 2)), p_masked=bool(rng.integers(0, 2)),
                     select_bias=bool(rng.integers(0, 4) == 0))
        out.append((Tm * m, E, k, m, cf, flags))
    return out


@pytest.mark.parametrize("case", _sweep(), ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}_cf{c[4]}" for c in _sweep()])
def test_one_launch_sweep(case):
    T, E, k, m, cf, flags = case
    print(f"case one_launch sweep {case}", flush=True)
    rng = np.random.default_rng(T * 13 + E * 7 + k)
    L = (rng.standard_normal((T, E)) + rng.normal(0.0, 0.7, E)).astype(np.float32)
    b = (0.5 * rng.standard_normal(E)).astype(np.float32) if flags["select_bias"] else None
    mk = lambda **o: lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf, alpha=0.01, save_row_stats=True,
                                     inv_perm=True, **flags, **o)
    inputs = {"logits": L}
    if b is not None:
        inputs["select_bias"] = b
    p = mk()
    one = gpu_forward(p, inputs)
    multi = gpu_forward(mk(multi_kernel=True), inputs)
    compare_forward(one, oracle_forward(p, L, select_bias=b), p)
    _compare_paths(one, multi)
