"""C-ABI checks that need no GPU: exported symbols, struct layout, host-side
validation and capacity arithmetic.  No call here reaches a HIP launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")


@pytest.fixture(scope="module")
def lbs():
    import load_balancing_statistics_amd as m
    from load_balancing_statistics_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from load_balancing_statistics_amd import build
        build.build()
    m.load()
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_(?:route|gate|eplb|sinkhorn)\w*)\s*\(", src)))


def test_every_declared_symbol_is_exported(lbs):
    lib = lbs.load()
    names = declared_functions()
    assert set(names) == {"moe_route", "moe_route_noalloc", "moe_route_backward", "moe_route_bias_update",
                          "moe_route_capacity", "moe_route_strerror", "moe_route_workspace_size",
                          "moe_gate_backward", "moe_gate_backward_workspace_size", "moe_eplb_plan",
                          "moe_sinkhorn_plan", "moe_route_with_bias_update"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lbs._binding.LIB_PATH],
                         capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), f"{n} not exported as a text symbol"


def test_struct_layout_matches_header(lbs, tmp_path):
    """Offsets and sizes of the C structs, printed by a gcc-compiled probe,
    equal the ctypes mirrors of the binding."""
    from load_balancing_statistics_amd._binding import moe_route_out, moe_route_params
    fields_p = [f[0] for f in moe_route_params._fields_]
    fields_o = [f[0] for f in moe_route_out._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe_route.h"',
             'int main(void) {',
             'printf("P %zu\\n", sizeof(moe_route_params));',
             'printf("O %zu\\n", sizeof(moe_route_out));']
    for f in fields_p:
        lines.append(f'printf("p.{f} %zu\\n", offsetof(moe_route_params, {f}));')
    for f in fields_o:
        lines.append(f'printf("o.{f} %zu\\n", offsetof(moe_route_out, {f}));')
    lines += ['return 0; }']
    c = tmp_path / "probe.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True,
                                                 text=True).stdout.splitlines())
    assert int(got["P"]) == ctypes.sizeof(moe_route_params)
    assert int(got["O"]) == ctypes.sizeof(moe_route_out)
    for f in fields_p:
        assert int(got[f"p.{f}"]) == getattr(moe_route_params, f).offset, f
    for f in fields_o:
        assert int(got[f"o.{f}"]) == getattr(moe_route_out, f).offset, f


def test_capacity_and_workspace(lbs):
    p = lbs.make_params(1024, 8, 1, capacity_factor=1.25)
    assert lbs.moe_route_capacity(p) == 160
    assert lbs.moe_route_capacity(lbs.make_params(131072, 256, 8, capacity_factor=1.25)) == 5120
    assert lbs.moe_route_capacity(lbs.make_params(262144, 384, 6, n_micro=16)) == 256
    assert lbs.moe_route_capacity(lbs.make_params(100, 8, 2, capacity_factor=0.0)) == -1
    assert lbs.moe_route_capacity(lbs.make_params(100, 8, 2, capacity=7)) == 7
    for T, E, k, m, d in [(1, 1, 1, 1, 0), (4096, 8, 1, 1, 0), (131072, 256, 8, 1, 0),
                          (262144, 384, 6, 16, 0), (16384, 8, 2, 1, 4096), (513, 1024, 32, 1, 0)]:
        n = lbs.moe_route_workspace_size(lbs.make_params(T, E, k, n_micro=m, d=d))
        assert 0 < n < 64 * 1024 * 1024


def test_capacity_at_recommended_factors(lbs):
    """The library's capacity equals the page's formula (mhpq.cn/news/998159
    section 4.5) at the factors the page recommends, as worked by hand in
    tests/golden/capacity_factors.txt: 1280 tokens over 128 experts at 1.2 is
    12, 5000 over 100 at 1.1 is 55 (the double product 55.000000000000007
    must not round up to 56)."""
    path = os.path.join(ROOT, "tests", "golden", "capacity_factors.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        r = dict(tok.split("=") for tok in line.split())
        T, E, k = int(r["tokens"]), int(r["experts"]), int(r["top_k"])
        p = lbs.make_params(T, E, k, capacity_factor=float(r["capacity_factor"]))
        assert lbs.moe_route_capacity(p) == int(r["capacity"]), r
        n += 1
    assert n >= 10


def test_capacity_matches_oracle_over_decimal_factors(lbs):
    """Library (double factor, products within 2^-50 of an integer taken as
    that integer) against the oracle (the caller's decimal, exact integer
    arithmetic) over factors with one to four decimal places and per-expert
    shares from 1 to 5000, microbatches and k > 1 included."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(7)
    factors = sorted({round(x, d) for d in (1, 2, 3, 4)
                      for x in rng.uniform(0.05, 4.0, size=60)} | {1.05, 1.1, 1.15, 1.2, 1.3, 1.5})
    shapes = [(T, E, k, m) for T, E, k, m in [(1, 1, 1, 1), (4096, 8, 1, 1), (65536, 64, 2, 1),
                                               (131072, 256, 8, 1), (262144, 384, 6, 16),
                                               (5000, 100, 1, 1), (3000, 7, 3, 3)]]
    shapes += [(int(s) * 10, 10, 1, 1) for s in rng.integers(1, 5000, size=40)]
    for cf in factors:
        for T, E, k, m in shapes:
            p = lbs.make_params(T, E, k, n_micro=m, capacity_factor=cf)
            want = oracle.capacity(T // m, E, k, cf)
            assert lbs.moe_route_capacity(p) == want, (cf, T, E, k, m)


def test_every_expert_count_and_k_is_supported(lbs):
    """Every E <= MOE_ROUTE_MAX_E and k <= min(E, MOE_ROUTE_MAX_K) is accepted,
    with and without the selection bias and the masked P (top-1 over 9 to 24
    experts once overflowed the row pass's LDS)."""
    for flags in [dict(), dict(select_bias=True, p_masked=True)]:
        bad = []
        for E in range(1, lbs.MOE_ROUTE_MAX_E + 1):
            for k in range(1, min(E, lbs.MOE_ROUTE_MAX_K) + 1):
                try:
                    lbs.moe_route_workspace_size(lbs.make_params(100000, E, k, **flags))
                except lbs.MoeRouteError:
                    bad.append((E, k))
        assert not bad, (flags, bad[:10])


@pytest.mark.parametrize("kw,code", [
    (dict(T=0, E=8, k=1), -1), (dict(T=16, E=8, k=0), -1), (dict(T=16, E=8, k=9), -1),
    (dict(T=15, E=8, k=1, n_micro=2), -1), (dict(T=16, E=2048, k=2), -2),
    (dict(T=16, E=64, k=33), -2), (dict(T=16, E=8, k=1, d=12), -2),
    (dict(T=16, E=100, k=2, d=64), -2), (dict(T=16, E=8, k=1, capacity=-5), -1),
])
def test_invalid_shapes_rejected(lbs, kw, code):
    p = lbs.make_params(**kw)
    with pytest.raises(lbs.MoeRouteError) as ei:
        lbs.moe_route_workspace_size(p)
    assert ei.value.code == code
    assert lbs.moe_route_strerror(code)


def test_moe_route_validates_before_launching(lbs):
    """Missing or misaligned pointers and a short workspace are reported
    without any device work (there is no GPU here)."""
    lib = lbs.load()
    B = lbs._binding
    p = lbs.make_params(64, 8, 2, save_row_stats=True)
    fake = 0x10000  # never dereferenced: validation fails first
    full = {n: fake for n in B._OUT_FIELDS}
    full["logits"] = None

    def call(out_fields, logits=fake, ws=fake, ws_bytes=1 << 20, params=p, bias=None):
        o = B.moe_route_out(*[out_fields.get(n) for n in B._OUT_FIELDS])
        return lib.moe_route(ctypes.byref(params), logits, None, None, bias, ctypes.byref(o),
                             ws, ws_bytes, None)

    for missing in ["topk_idx", "topk_w", "counts", "offsets", "perm", "dropped", "aux_loss",
                    "cv", "max_over_mean", "row_stats"]:
        f = dict(full)
        f[missing] = None
        assert call(f) == B.MOE_ERR_INVALID_ARG, missing
    assert call(full, logits=None) == B.MOE_ERR_INVALID_ARG
    assert call(full, logits=fake + 2) == B.MOE_ERR_INVALID_ARG  # misaligned
    assert call(full, ws=None) == B.MOE_ERR_WORKSPACE
    assert call(full, ws_bytes=16) == B.MOE_ERR_WORKSPACE
    assert call(full, ws=fake + 8) == B.MOE_ERR_WORKSPACE       # not 256-byte aligned
    pi = lbs.make_params(64, 8, 2, inv_perm=True)
    f = dict(full)
    f["inv_perm"] = None
    assert call(f, params=pi) == B.MOE_ERR_INVALID_ARG
    pg = lbs.make_params(64, 8, 2, d=64)
    assert call(full, params=pg) == B.MOE_ERR_INVALID_ARG        # gate path without X/Wg
    assert lib.moe_route(None, None, None, None, None, None, None, 0, None) == B.MOE_ERR_INVALID_ARG
    # selection bias: required with the flag, must be 4-byte aligned
    pb = lbs.make_params(64, 8, 2, select_bias=True)
    assert call(full, params=pb) == B.MOE_ERR_INVALID_ARG
    assert call(full, params=pb, bias=fake + 2) == B.MOE_ERR_INVALID_ARG
    # routing with the bias step: the selection-bias flag, a finite gamma >= 0
    # and a bias pointer are required, and the forward's own checks apply
    def call_step(params, bias=fake, gamma=0.1, logits=fake, ws=fake):
        o = B.moe_route_out(*[full.get(n) for n in B._OUT_FIELDS])
        return lib.moe_route_with_bias_update(ctypes.byref(params), logits, None, None, bias, gamma,
                                              ctypes.byref(o), ws, 1 << 20, None)
    assert call_step(p) == B.MOE_ERR_INVALID_ARG                          # no MOE_SELECT_BIAS
    assert call_step(pb, gamma=-0.1) == B.MOE_ERR_INVALID_ARG
    assert call_step(pb, gamma=float("inf")) == B.MOE_ERR_INVALID_ARG
    assert call_step(pb, bias=None) == B.MOE_ERR_INVALID_ARG
    assert call_step(pb, logits=None) == B.MOE_ERR_INVALID_ARG
    assert call_step(pb, ws=None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route_with_bias_update(None, None, None, None, None, 0.1, None, None, 0,
                                          None) == B.MOE_ERR_INVALID_ARG
    # bias update
    assert lib.moe_route_bias_update(ctypes.byref(p), None, 0.1, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bias_update(ctypes.byref(p), fake, 0.1, None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bias_update(ctypes.byref(p), fake, -0.1, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bias_update(ctypes.byref(p), fake, float("nan"), fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bias_update(ctypes.byref(lbs.make_params(0, 8, 1)), fake, 0.1, fake,
                                     None) == B.MOE_ERR_INVALID_ARG
    # backward
    bwd = lib.moe_route_backward
    assert bwd(ctypes.byref(p), None, None, fake, None, None, None, fake, None) == B.MOE_ERR_INVALID_ARG
    assert bwd(ctypes.byref(p), fake, None, None, None, None, None, fake, None) == B.MOE_ERR_INVALID_ARG
    assert bwd(ctypes.byref(p), fake + 1, None, fake, None, None, None, fake, None) == B.MOE_ERR_INVALID_ARG
    # masked P or a gate-weight gradient need the picks
    pm = lbs.make_params(64, 8, 2, p_masked=True)
    assert bwd(ctypes.byref(pm), fake, None, fake, None, None, None, fake, None) == B.MOE_ERR_INVALID_ARG
    assert bwd(ctypes.byref(p), fake, None, fake, None, None, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert bwd(ctypes.byref(p), fake, None, fake, None, fake + 2, fake, fake, None) == B.MOE_ERR_INVALID_ARG


def test_noalloc_validates_before_any_device_work(lbs):
    """moe_route_noalloc refuses a shape whose workspace exceeds the static
    scratch (4096 microbatches of E=1024 need ~96 MiB) with MOE_ERR_SCRATCH,
    and bad shapes with their usual codes, before touching the device (there
    is no GPU here)."""
    lib = lbs.load()
    B = lbs._binding
    fake = 0x10000
    o = B.moe_route_out(*[fake for _ in B._OUT_FIELDS])
    big = lbs.make_params(1 << 18, 1024, 32, n_micro=4096)
    assert lbs.moe_route_workspace_size(big) > lbs.MOE_ROUTE_SCRATCH_BYTES
    assert lib.moe_route_noalloc(ctypes.byref(big), fake, None, None, None, ctypes.byref(o),
                                 None) == B.MOE_ERR_SCRATCH
    assert "MOE_ROUTE_SCRATCH_BYTES" in lbs.moe_route_strerror(B.MOE_ERR_SCRATCH)
    bad = lbs.make_params(16, 8, 9)
    assert lib.moe_route_noalloc(ctypes.byref(bad), fake, None, None, None, ctypes.byref(o),
                                 None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_noalloc(None, fake, None, None, None, ctypes.byref(o),
                                 None) == B.MOE_ERR_INVALID_ARG


def test_gate_backward_validation(lbs):
    """Shapes, pointers, alignment and workspace of the gate backward are
    checked before any launch."""
    lib = lbs.load()
    B = lbs._binding
    fake = 0x10000
    p = lbs.make_params(64, 8, 2, d=64)
    n = lbs.moe_gate_backward_workspace_size(p)
    assert 0 < n < 64 * 1024 * 1024
    gb = lib.moe_gate_backward
    ok = (fake, fake, fake, fake, fake, fake, 1 << 20, None)
    assert gb(ctypes.byref(lbs.make_params(64, 8, 2, d=0)), *ok) == B.MOE_ERR_INVALID_ARG
    assert gb(ctypes.byref(lbs.make_params(64, 100, 2, d=64)), *ok) == B.MOE_ERR_UNSUPPORTED
    assert gb(ctypes.byref(lbs.make_params(64, 8, 2, d=12)), *ok) == B.MOE_ERR_UNSUPPORTED
    assert gb(ctypes.byref(p), None, fake, fake, fake, fake, fake, 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert gb(ctypes.byref(p), fake, fake, fake, None, None, fake, 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert gb(ctypes.byref(p), fake + 8, fake, fake, fake, fake, fake, 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert gb(ctypes.byref(p), fake, fake, fake, fake + 8, None, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert gb(ctypes.byref(p), fake, fake, fake, None, fake, None, 0, None) == B.MOE_ERR_WORKSPACE
    assert gb(ctypes.byref(p), fake, fake, fake, None, fake, fake, 16, None) == B.MOE_ERR_WORKSPACE


def test_eplb_validation(lbs):
    lib = lbs.load()
    B = lbs._binding
    f = 0x10000
    ok = (f, f, f, f, f, f, f)
    assert lib.moe_eplb_plan(0, 4, 2, *ok, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_eplb_plan(8, 4, 2, *ok, None) == B.MOE_ERR_INVALID_ARG      # num_phys < E
    assert lib.moe_eplb_plan(4, 6, 4, *ok, None) == B.MOE_ERR_INVALID_ARG      # not divisible
    assert lib.moe_eplb_plan(2048, 4096, 2, *ok, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_eplb_plan(4, 8192, 2, *ok, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_eplb_plan(4, 8, 2, None, f, f, f, f, f, f, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_eplb_plan(4, 8, 2, f, f, f, f, f, f, f + 4, None) == B.MOE_ERR_INVALID_ARG  # fp64 alignment


def test_sinkhorn_validation(lbs):
    lib = lbs.load()
    B = lbs._binding
    f = 0x10000
    ok = (f, f, f)
    outs = (f, f, f)
    assert lib.moe_sinkhorn_plan(0, *ok, 1.0, 50, *outs, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_sinkhorn_plan(65, *ok, 1.0, 50, *outs, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_sinkhorn_plan(8, *ok, 0.0, 50, *outs, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_sinkhorn_plan(8, *ok, float("inf"), 50, *outs, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_sinkhorn_plan(8, *ok, 1.0, -1, *outs, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_sinkhorn_plan(8, f, f, None, 1.0, 50, *outs, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_sinkhorn_plan(8, f + 4, f, f, 1.0, 50, *outs, None) == B.MOE_ERR_INVALID_ARG


def test_flag_values_match_header(lbs):
    """Every MOE_* flag and status bit of the header has the binding's value;
    an unknown flag bit is an invalid argument, the known ones are accepted."""
    src = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(MOE_\w+)\s+\(?(-?\d+)u?\)?", src))
    B = lbs._binding
    names = ["MOE_RENORM_TOPK", "MOE_SAVE_ROW_STATS", "MOE_WRITE_INV_PERM", "MOE_SELECT_BIAS",
             "MOE_P_MASKED", "MOE_MULTI_KERNEL", "MOE_STATUS_NONFINITE", "MOE_STATUS_INTERNAL"]
    for n in names:
        assert int(defs[n]) == getattr(B, n), n
    known = 0
    for n in names[:6]:
        known |= getattr(B, n)
    p = lbs.make_params(4096, 8, 1, multi_kernel=True)
    assert lbs.moe_route_workspace_size(p) > 0
    for bit in range(32):
        if known & (1 << bit):
            continue
        q = lbs.make_params(4096, 8, 1)
        q.flags = 1 << bit
        n = ctypes.c_size_t(0)
        assert lbs.load().moe_route_workspace_size(ctypes.byref(q), ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG, bit
