"""HIP path (through the C ABI) against the CPU oracle, on the GPU.

Integer outputs (top-k indices, counts, offsets, perm, inv_perm, drop mask)
must match bit for bit; floating-point outputs within 1e-5 relative (gate
weights, P, aux loss, CV, row sums) -- the bound the routing workloads state.
"""
import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
import oracle
from gpu_helpers import (assert_close_rel, assert_equal, backward_tolerance, check_structure,
                         compare_forward, gpu_backward, gpu_forward, oracle_forward, params_of)

pytestmark = pytest.mark.gpu

# sizes the oracle finishes in well under a second, spanning several row
# blocks and a ragged tail
SMALL = {
    "switch_top1": dict(T=4096 + 37),
    "zipf_top2": dict(T=9000 + 11),
    "v3_shape": dict(T=3000 + 5),
    "v4_shape": dict(T=4 * 1500, n_micro=4),
}


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_small(name, seed):
    w = WORKLOADS[name].scaled(**SMALL[name])
    print(f"case forward_small {name} seed={seed} T={w.T} E={w.E} k={w.k} m={w.n_micro}", flush=True)
    inp = make_inputs(w, seed)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"])
    compare_forward(g, r, p)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["switch_top1", "zipf_top2", "v3_shape", "v4_shape"])
def test_forward_full(name, seed):
    w = WORKLOADS[name]
    print(f"case forward_full {name} seed={seed} T={w.T} E={w.E} k={w.k} m={w.n_micro}", flush=True)
    inp = make_inputs(w, seed)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"])
    compare_forward(g, r, p)


def _check_backward(w, inp, p, g, r, d_aux=None, use_stats=True):
    ref = oracle.backward(inp["logits"], w.k, r["counts"], n_micro=w.n_micro, alpha=w.alpha,
                          d_aux=d_aux)
    dl = gpu_backward(p, inp["logits"], g["counts"],
                      row_stats=g["row_stats"] if use_stats else None, d_aux=d_aux)
    scale = backward_tolerance(inp["logits"], r, r["counts"], p, d_aux)
    err = np.abs(dl.astype(np.float64) - ref)
    bound = 1e-5 * np.maximum(np.abs(ref), scale) + 1e-30
    bad = ~(err <= bound)
    assert not bad.any(), f"{bad.sum()} gradient mismatches, worst ratio {np.max(err / bound)}"


@pytest.mark.parametrize("use_stats", [True, False])
@pytest.mark.parametrize("name", ["v4_shape", "v3_shape", "zipf_top2", "switch_top1"])
def test_backward_small(name, use_stats):
    w = WORKLOADS[name].scaled(**SMALL[name])
    print(f"case backward_small {name} stats={use_stats}", flush=True)
    inp = make_inputs(w, 1)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"])
    d_aux = np.linspace(0.5, 2.0, w.n_micro)
    _check_backward(w, inp, p, g, r, d_aux=d_aux, use_stats=use_stats)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_full_v4(seed):
    w = WORKLOADS["v4_shape"]
    print(f"case backward_full v4_shape seed={seed}", flush=True)
    inp = make_inputs(w, seed)
    p = params_of(w)
    g = gpu_forward(p, inp)
    r = oracle_forward(p, inp["logits"])
    compare_forward(g, r, p)
    _check_backward(w, inp, p, g, r)


# ------------------------------------------------------------- gate GEMM
def _gate_case(w, seed):
    inp = make_inputs(w, seed)
    p = params_of(w)
    g = gpu_forward(p, inp)
    ref_logits = oracle.gate_logits(inp["X"], inp["Wg"])
    err = np.abs(g["logits"].astype(np.float64) - ref_logits)
    assert err.max() <= 2e-2, f"gate logits max error {err.max()}"
    # fp32 accumulation of d bf16 products: error ~ sqrt(d) * eps * |terms|
    assert err.max() <= 1e-4, f"gate logits max error {err.max()} (expected fp32-accumulation level)"
    # selection where the oracle's top-(k+1) values are separated by > 1e-2
    srt = -np.sort(-ref_logits, axis=1)[:, : w.k + 1]
    margin = np.min(srt[:, :-1] - srt[:, 1:], axis=1) if w.k < w.E else np.min(
        srt[:, :-1] - srt[:, 1:], axis=1, initial=np.inf)
    r = oracle.route(ref_logits, w.k, capacity_factor=w.capacity_factor, alpha=w.alpha,
                     renorm=w.renorm)
    sure = margin > 1e-2
    assert_equal(g["topk_idx"][sure], r["topk_idx"][sure], "gate topk_idx (margin > 1e-2)")
    assert_close_rel(g["topk_w"][sure], r["topk_w"][sure], 1e-4, 0, "gate topk_w")
    assert_close_rel(g["P"], r["P"], 1e-4, 0, "gate P")
    check_structure(g, p)
    if sure.all():
        compare_forward(g, r, p)
    # every routing output bit-exact (floats 1e-5) against the oracle routing
    # the very fp32 logits the gate GEMM wrote
    rr = oracle_forward(params_of(w, d=0), g["logits"])
    compare_forward(g, rr, p)
    # the routing behind the gate equals the routing of the logits it wrote
    p2 = params_of(w, d=0)
    g2 = gpu_forward(p2, {"logits": g["logits"]})
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "dropped", "P",
                "aux_loss", "cv", "row_stats"):
        assert_equal(g2[key], g[key], f"gate vs logits path: {key}")
    return inp, p, g, r


def test_gate_small():
    w = WORKLOADS["gate_top2"].scaled(T=1000 + 3, d=512)
    print("case gate_small", flush=True)
    inp, p, g, r = _gate_case(w, 0)


@pytest.mark.parametrize("T,d,E", [(1003, 520, 8), (77, 4096, 16), (130, 264, 12), (1000, 512, 40),
                                   (1, 8, 1), (300, 392, 64), (65, 136, 24)])
def test_gate_logits_shapes(T, d, E):
    """Gate GEMM alone over ragged shapes: T not a multiple of the 64-token
    block, d not a multiple of 32 (nor of the 128-wide k chunk), E = 16 (full
    tile), E = 40 and 64 (three and four expert tiles), E = 12 and 1 (weights
    laid out by the small kernel, E % 8 != 0), a single token and a single
    8-wide k step."""
    print(f"case gate_logits T={T} d={d} E={E}", flush=True)
    rng = np.random.default_rng(T + d + E)
    f32 = rng.standard_normal((T, d)).astype(np.float32)
    w32 = (0.05 * rng.standard_normal((d, E))).astype(np.float32)
    bf = lambda a: ((a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    X, Wg = bf(f32), bf(w32)
    k = min(2, E)
    p = lbs.make_params(T, E, k, d=d, capacity_factor=1.25)
    g = gpu_forward(p, {"X": X, "Wg": Wg})
    ref = oracle.gate_logits(X, Wg)
    err = np.abs(g["logits"].astype(np.float64) - ref)
    assert err.max() <= 1e-4, f"gate logits max error {err.max()}"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gate_full(seed):
    w = WORKLOADS["gate_top2"]
    print(f"case gate_full seed={seed}", flush=True)
    inp, p, g, r = _gate_case(w, seed)
    # backward on the gate logits the forward wrote (the forward on them was
    # compared with the oracle in _gate_case)
    rr = oracle_forward(params_of(w, d=0), g["logits"])
    ref = oracle.backward(g["logits"], w.k, rr["counts"], alpha=w.alpha)
    dl = gpu_backward(p, g["logits"], g["counts"], row_stats=g["row_stats"])
    assert_equal(g["counts"], rr["counts"], "counts of the gate logits")
    scale = backward_tolerance(g["logits"], rr, rr["counts"], params_of(w, d=0))
    err = np.abs(dl.astype(np.float64) - ref)
    assert (err <= 1e-5 * np.maximum(np.abs(ref), scale) + 1e-30).all()


# ------------------------------------------------------------ edge cases
EDGE = [
    # (T, E, k, n_micro, cf, capacity, renorm, kind)
    (1, 8, 2, 1, 1.25, -1, True, "normal"),
    (37, 1, 1, 1, 1.0, -1, False, "normal"),
    (500, 8, 8, 2, 1.0, -1, True, "normal"),
    (300, 16, 16, 1, 1.0, -1, False, "normal"),
    (777, 3, 3, 1, 1.0, -1, True, "normal"),
    (1000, 100, 4, 4, 1.0, -1, True, "normal"),
    (600, 1000, 16, 2, 1.25, -1, True, "normal"),
    (513, 1024, 32, 1, 1.0, -1, True, "normal"),
    (640, 64, 32, 1, 1.0, -1, False, "normal"),
    (2048, 384, 6, 2, 1.0, 0, True, "normal"),       # capacity 0: all dropped
    (2048, 256, 8, 1, 0.0, -1, True, "normal"),      # unlimited
    (2048, 256, 8, 1, 1.0, 17, True, "normal"),      # explicit capacity
    (999, 256, 8, 1, 1.25, -1, True, "equal"),       # every logit equal
    (999, 384, 6, 3, 1.0, -1, True, "quantized"),    # heavy ties
    (1024, 64, 2, 1, 1.0, -1, True, "signed_zero"),  # -0.0 / +0.0 ties
    (1024, 8, 1, 1, 1.25, -1, False, "quantized"),
    (700, 12, 5, 1, 1.0, -1, True, "quantized"),
    (2000, 250, 8, 1, 1.25, -1, True, "normal"),     # 16 lanes x 16 columns, scalar loads
    (3000, 130, 6, 2, 1.0, -1, False, "normal"),     # padded columns, two microbatches
    # top-1 over 9..24 experts: two or four lanes per row
    (3000, 9, 1, 1, 1.25, -1, False, "normal"),
    (3001, 12, 1, 1, 1.1, -1, False, "normal"),
    (4096, 16, 1, 2, 1.2, -1, False, "normal"),
    (2500, 20, 1, 1, 1.05, -1, False, "normal"),
    (2048, 24, 1, 1, 1.0, -1, False, "quantized"),
    (1000, 13, 2, 1, 1.3, -1, True, "normal"),
    # few row blocks in all: the statistics in workgroups of their own, the
    # scatter summing 64 row blocks a microbatch (four groups) or 32 (two)
    (32768, 8, 2, 2, 1.25, -1, True, "normal"),
    (16384, 16, 4, 4, 1.0, -1, True, "quantized"),
    (6000, 64, 2, 3, 1.1, -1, False, "normal"),
    # the scatter folding in up to 16 groups of row blocks (no combine kernel)
    (131072, 8, 1, 1, 1.25, -1, False, "normal"),    # 256 row blocks, 16 groups
    (65536, 16, 4, 1, 1.0, -1, True, "quantized"),   # 16 groups, ties
    (32768, 32, 2, 1, 1.1, -1, True, "normal"),      # 6 groups
    (49152, 8, 2, 3, 1.0, 50, True, "normal"),       # three microbatches, explicit capacity
    # grids too large for statistics workgroups: the statistics spread over a
    # microbatch's first six row blocks (13 a microbatch), or all in block 0
    # (3 a microbatch)
    (81920, 256, 8, 40, 1.25, -1, True, "normal"),
    (102400, 256, 8, 200, 1.0, -1, True, "quantized"),
]


def _edge_logits(T, E, kind, rng):
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "equal":
        return np.full((T, E), 0.75, np.float32)
    if kind == "quantized":
        return (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    if kind == "signed_zero":
        L = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5], np.float32), size=(T, E))
        return L.astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_m{c[3]}_{c[7]}_C{c[5]}" for c in EDGE])
def test_edge(case):
    T, E, k, m, cf, cap, renorm, kind = case
    T = (T // m) * m if T >= m else m
    print(f"case edge {case}", flush=True)
    rng = np.random.default_rng(T * 7 + E)
    L = _edge_logits(T, E, kind, rng)
    p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf, capacity=cap, alpha=0.02,
                        renorm=renorm, save_row_stats=True, inv_perm=True)
    g = gpu_forward(p, {"logits": L})
    r = oracle_forward(p, L)
    compare_forward(g, r, p)
    if cap == 0:
        assert g["dropped"].all()


# (tokens, experts, k, capacity factor as the caller writes it, capacity
# worked by hand from page mhpq.cn/news/998159 section 4.5:
# ceil(factor * ceil(tokens * k / experts)))
RECOMMENDED_CF = [
    (1280, 128, 1, "1.2", 12),
    (5000, 100, 1, "1.1", 55),
    (2000, 100, 1, "1.1", 22),
    (640, 64, 2, "1.1", 22),
    (3000, 100, 1, "1.05", 32),
    (16384, 384, 6, "1.05", 269),
]


@pytest.mark.parametrize("case", RECOMMENDED_CF, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_cf{c[3]}"
                                                      for c in RECOMMENDED_CF])
def test_capacity_at_recommended_factors(case):
    """Drops at the capacity factors the page recommends (1.0-1.05 late in
    training, 1.2-1.5 early): the oracle is given the factor as the caller
    wrote it (text), the library the caller's float; both must cut each
    expert at the page's capacity, including where the product is integral
    (1.2 * 10 = 12, 1.1 * 50 = 55)."""
    T, E, k, cf_text, C = case
    print(f"case capacity T={T} E={E} k={k} cf={cf_text}", flush=True)
    rng = np.random.default_rng(T + E)
    L = (rng.standard_normal((T, E)) + rng.normal(0.0, 0.3, E)).astype(np.float32)
    p = lbs.make_params(T, E, k, capacity_factor=float(cf_text), alpha=0.01, renorm=k > 1,
                        save_row_stats=True, inv_perm=True)
    assert lbs.moe_route_capacity(p) == C
    r = oracle_forward(p, L, capacity_factor=cf_text)
    assert r["capacity"] == C
    g = gpu_forward(p, {"logits": L})
    assert (g["counts"] > C).any(), "the case must drop at the capacity"
    compare_forward(g, r, p)
    assert g["extra_stats"][0, 5] == C


def test_alpha_zero_and_no_renorm():
    w = WORKLOADS["v3_shape"].scaled(T=2000)
    inp = make_inputs(w, 3)
    for alpha, renorm in [(0.0, True), (0.001, False)]:
        p = params_of(w, alpha=alpha, renorm=renorm)
        g = gpu_forward(p, inp)
        r = oracle_forward(p, inp["logits"])
        compare_forward(g, r, p)
        if alpha == 0.0:
            assert g["aux_loss"][0] == 0.0
            dl = gpu_backward(p, inp["logits"], g["counts"])
            assert np.all(dl == 0.0)


@pytest.mark.parametrize("T,E,k", [(300, 64, 2), (4096, 256, 8)])
def test_nonfinite_sets_status(T, E, k):
    """Both ways the status word is formed: few row blocks (the scatter folds
    the combine in and ORs the flags) and many (the combine kernel writes
    it).  The output buffers start poisoned, so a clean call must zero it."""
    print(f"case nonfinite T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(4)
    for bad in [np.nan, np.inf]:
        L = rng.standard_normal((T, E), dtype=np.float32)
        L[123, 7] = bad
        p = lbs.make_params(T, E, k, capacity_factor=1.0, renorm=True, save_row_stats=True)
        g = gpu_forward(p, {"logits": L})
        assert g["status"][0] & lbs.MOE_STATUS_NONFINITE
        # rows other than the bad one are still routed exactly
        ok = np.ones(T, bool)
        ok[123] = False
        ro = oracle.route(L[ok], k, capacity_factor=0.0, renorm=True)
        assert_equal(g["topk_idx"][ok], ro["topk_idx"], "topk_idx of finite rows")
    L = rng.standard_normal((T, E), dtype=np.float32)
    g = gpu_forward(lbs.make_params(T, E, k), {"logits": L})
    assert g["status"][0] == 0


def test_deterministic_repeat():
    w = WORKLOADS["v3_shape"]
    inp = make_inputs(w, 5)
    p = params_of(w)
    a = gpu_forward(p, inp)
    b = gpu_forward(p, inp)
    for key in ("topk_idx", "topk_w", "counts", "perm", "dropped", "P", "aux_loss", "cv",
                "row_stats", "extra_stats"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


def test_errors_leave_outputs_untouched():
    L = torch.zeros((64, 8), device="cuda:0")
    p = lbs.make_params(64, 8, 2)
    out = lbs.alloc_outputs(p, device="cuda:0")
    out["topk_idx"].fill_(-3)
    ws = lbs.alloc_workspace(p, device="cuda:0")
    small = ws[:16]
    with pytest.raises(lbs.MoeRouteError) as ei:
        lbs.moe_route(p, out, small, logits=L)
    assert ei.value.code == lbs.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out["topk_idx"] == -3).all()


@pytest.mark.parametrize("T,E,k,m", [(3000, 256, 8, 1), (2000, 600, 6, 2)])
def test_nullable_outputs(T, E, k, m):
    """f, P, extra_stats, status, row_stats and inv_perm are nullable: with
    them NULL the required outputs are the same bytes as with every output
    present (E=600 takes the 8-wave scatter, two experts per thread)."""
    print(f"case nullable T={T} E={E} k={k} m={m}", flush=True)
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E), dtype=np.float32)
    p_all = lbs.make_params(T, E, k, n_micro=m, capacity_factor=1.0, save_row_stats=True,
                            inv_perm=True)
    full = gpu_forward(p_all, {"logits": L})
    p_min = lbs.make_params(T, E, k, n_micro=m, capacity_factor=1.0)
    dev = torch.device("cuda:0")
    out = lbs.alloc_outputs(p_min, device=dev)
    for key in ("f", "P", "extra_stats", "status", "row_stats", "inv_perm"):
        out[key] = None
    ws = lbs.alloc_workspace(p_min, device=dev)
    lbs.moe_route(p_min, out, ws, logits=torch.from_numpy(L).to(dev))
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm", "dropped", "aux_loss", "cv",
                "max_over_mean"):
        got = out[key].cpu().numpy()
        assert np.array_equal(got.view(np.uint8), full[key].view(np.uint8)), key
