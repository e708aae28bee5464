"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
CPU oracle on the same seeded inputs, and compare element by element."""
import numpy as np
import torch

import load_balancing_statistics_amd as lbs
import oracle

DEV = "cuda:0"

INT_KEYS = ("topk_idx", "counts", "offsets", "perm", "dropped")


def params_of(w, **over):
    kw = dict(T=w.T, E=w.E, k=w.k, n_micro=w.n_micro, d=w.d,
              capacity_factor=w.capacity_factor, alpha=w.alpha, renorm=w.renorm,
              save_row_stats=True, inv_perm=True, select_bias=w.select_bias_scale > 0)
    kw.update(over)
    return lbs.make_params(**kw)


def gpu_forward(params, inputs, out_extra=None):
    """Run moe_route on the GPU; returns numpy copies of all outputs."""
    dev = torch.device(DEV)
    out = lbs.alloc_outputs(params, device=dev)
    for key, t in out.items():  # poison: every required element must be written
        if t is not None:
            t.fill_(float("nan") if t.is_floating_point() else (0xEE if t.dtype == torch.uint8 else -7))
    ws = lbs.alloc_workspace(params, device=dev)
    ws.fill_(0xAB)
    sb = inputs.get("select_bias")
    sb = None if sb is None else torch.from_numpy(np.asarray(sb, np.float32)).to(dev)
    if "logits" in inputs:
        L = torch.from_numpy(inputs["logits"]).to(dev)
        lbs.moe_route(params, out, ws, logits=L, select_bias=sb)
    else:
        X = torch.from_numpy(inputs["X"].view(np.int16)).to(dev)
        W = torch.from_numpy(inputs["Wg"].view(np.int16)).to(dev)
        lbs.moe_route(params, out, ws, X=X, Wg=W, select_bias=sb)
    torch.cuda.synchronize()
    res = {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}
    res["_torch_out"] = out
    return res


def gpu_backward(params, logits, counts, row_stats=None, d_aux=None):
    dev = torch.device(DEV)
    L = logits if isinstance(logits, torch.Tensor) else torch.from_numpy(logits).to(dev)
    cnt = counts if isinstance(counts, torch.Tensor) else torch.from_numpy(counts).to(dev)
    rs = None if row_stats is None else (row_stats if isinstance(row_stats, torch.Tensor)
                                         else torch.from_numpy(row_stats).to(dev))
    g = None if d_aux is None else torch.from_numpy(np.asarray(d_aux, np.float32)).to(dev)
    dl = torch.full_like(L, float("nan"))
    lbs.moe_route_backward(params, L, cnt, dl, row_stats=rs, d_aux=g)
    torch.cuda.synchronize()
    return dl.cpu().numpy()


def oracle_forward(params, logits, select_bias=None, capacity_factor=None):
    """The oracle on the same logits; ``capacity_factor`` is the caller's
    number (a float or a decimal string), by default the float the params
    carry (a double: the caller's float unchanged)."""
    cap = params.capacity
    cf = params.capacity_factor if capacity_factor is None else capacity_factor
    return oracle.route(logits, params.k, n_micro=params.n_micro,
                        capacity_factor=cf, capacity_override=cap,
                        alpha=params.alpha, renorm=bool(params.flags & lbs.MOE_RENORM_TOPK),
                        select_bias=select_bias,
                        p_masked=bool(params.flags & lbs.MOE_P_MASKED))


def assert_close_rel(got, ref, rtol, atol=0.0, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = rtol * np.abs(ref) + atol
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} mismatches; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")


def assert_equal(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")


def compare_forward(g, r, params, check_selection=True):
    """Bit-exact integer outputs, 1e-5 relative floating point."""
    T, k, m, E = params.T, params.k, params.n_micro, params.E
    if check_selection:
        assert_equal(g["topk_idx"], r["topk_idx"], "topk_idx")
        assert_equal(g["counts"], r["counts"], "counts")
        assert_equal(g["offsets"], r["offsets"], "offsets")
        assert_equal(g["perm"], r["perm"], "perm")
        assert_equal(g["inv_perm"], r["inv_perm"], "inv_perm")
        assert_equal(g["dropped"], r["dropped"], "dropped")
        assert_close_rel(g["topk_w"], r["topk_w"], 1e-5, 1e-30, "topk_w")
        assert_close_rel(g["f"], r["f"], 1e-6, 0, "f")
        assert_close_rel(g["aux_loss"], r["aux"], 1e-5, 0, "aux_loss")
        assert_close_rel(g["cv"], r["cv"], 1e-5, 1e-7, "cv")
        assert_close_rel(g["max_over_mean"], r["max_over_mean"], 1e-6, 0, "max_over_mean")
        assert_close_rel(g["extra_stats"], r["extra"], 1e-5, 1e-7, "extra_stats")
    assert_close_rel(g["P"], r["P"], 1e-5, 0, "P")
    assert_close_rel(g["row_stats"][:, 0], r["row_max"], 0, 0, "row max")
    assert_close_rel(g["row_stats"][:, 1], r["row_sum"], 1e-5, 0, "row sum")
    assert g["status"][0] == 0, f"status {g['status'][0]}"


def backward_tolerance(logits, r, counts, params, d_aux=None):
    """Per-element bound 1e-5 * max(|g_ref|, |c| p (f_j + S_t)): the scale of
    the two terms whose difference forms the gradient."""
    T, E, k, m = params.T, params.E, params.k, params.n_micro
    Tm = T // m
    L = np.asarray(logits, np.float64).reshape(m, Tm, E)
    p = np.exp(L - r["row_max"].reshape(m, Tm, 1)) / r["row_sum"].reshape(m, Tm, 1)
    f = np.asarray(counts, np.float64).reshape(m, 1, E) / (Tm * k)
    St = (f * p).sum(axis=2, keepdims=True)
    g = np.ones(m) if d_aux is None else np.asarray(d_aux, np.float64)
    c = np.abs(g * params.alpha * E / Tm).reshape(m, 1, 1)
    return (c * p * (f + St)).reshape(T, E)


def check_structure(g, params):
    """Properties that hold for any valid routing output (used where several
    selections are correct, e.g. near-ties of the bf16 gate logits): counts
    are the histogram of the picks, offsets their prefix, perm the stable
    expert sort, inv_perm its inverse, and an assignment is dropped exactly
    when it sits C or more places past its expert's offset (C from the
    oracle's capacity)."""
    T, E, k, m = params.T, params.E, params.k, params.n_micro
    Tm = T // m
    C = oracle.capacity(Tm, E, k, params.capacity_factor, params.capacity)
    idx = g["topk_idx"].reshape(m, Tm * k)
    for mb in range(m):
        cnt = np.bincount(idx[mb], minlength=E)
        assert np.array_equal(g["counts"][mb], cnt)
        assert np.array_equal(g["offsets"][mb], np.concatenate([[0], np.cumsum(cnt)]))
        seg = g["perm"][mb * Tm * k:(mb + 1) * Tm * k]
        assert np.array_equal(seg, np.argsort(idx[mb], kind="stable") + mb * Tm * k)
        # place of each assignment inside its expert's run
        e_sorted = idx[mb][seg - mb * Tm * k]
        rank = np.arange(Tm * k) - g["offsets"][mb][e_sorted]
        want = (rank >= C) if C >= 0 else np.zeros(Tm * k, bool)
        assert np.array_equal(g["dropped"][seg].astype(bool), want), "dropped"
    assert np.array_equal(g["inv_perm"][g["perm"]], np.arange(T * k))
    assert (np.sort(g["topk_idx"], axis=1)[:, 1:] != np.sort(g["topk_idx"], axis=1)[:, :-1]).all()
