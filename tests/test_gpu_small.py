"""Small single-microbatch batches (E <= 16, T up to 8192) against the
oracle, element by element, on both paths: the one launch (E of 1, 2, 4 or
8 with k*E <= 16) and the multi-kernel path (a few row blocks, the scatter folding the
block combine in; forced with MOE_MULTI_KERNEL): sizes around the 64-row
wave step and the 1024-row marks, expert counts off the vector width, every
option, ties, drops and non-finite rows."""
import numpy as np
import pytest

import load_balancing_statistics_amd as lbs
import oracle
from gpu_helpers import assert_equal, compare_forward, gpu_forward, oracle_forward

pytestmark = pytest.mark.gpu

# T, E, k, capacity_factor, options
CASES = [
    (1, 1, 1, 1.0, ""),
    (1, 16, 8, 1.0, "renorm"),
    (5, 3, 2, 1.25, "renorm"),
    (1023, 8, 2, 1.0, "renorm"),
    (1024, 8, 1, 1.25, ""),
    (1025, 8, 8, 1.0, "renorm"),
    (4096, 8, 1, 1.25, ""),             # the switch workload's shape
    (4096, 8, 2, 0.5, "renorm"),        # many drops
    (8192, 4, 4, 1.0, "renorm"),
    (2048, 16, 8, 1.0, "renorm"),
    (2047, 13, 3, 1.1, "renorm"),       # E off the vector width
    (4096, 5, 2, 1.2, ""),
    (3000, 8, 2, 1.0, "renorm,bias"),
    (2000, 16, 4, 1.25, "renorm,masked"),
    (1500, 6, 3, 1.0, "bias,masked"),
    (4096, 8, 2, 0.0, "renorm"),        # no capacity
]


def _run(T, E, k, cf, opts, seed, logits=None, multi=False):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E), dtype=np.float32) if logits is None else logits
    sb = (0.5 * rng.standard_normal(E)).astype(np.float32) if "bias" in opts else None
    p = lbs.make_params(T, E, k, capacity_factor=cf, alpha=0.01, renorm="renorm" in opts,
                        save_row_stats=True, inv_perm=True, select_bias=sb is not None,
                        p_masked="masked" in opts, multi_kernel=multi)
    inputs = {"logits": L}
    if sb is not None:
        inputs["select_bias"] = sb
    g = gpu_forward(p, inputs)
    r = oracle_forward(p, L, select_bias=sb)
    return p, g, r


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_cf{c[3]}_{c[4] or 'plain'}" for c in CASES])
@pytest.mark.parametrize("multi", [False, True], ids=["default", "multi_kernel"])
def test_small_forward(case, multi):
    T, E, k, cf, opts = case
    print(f"case small T={T} E={E} k={k} cf={cf} {opts} multi={multi}", flush=True)
    for seed in (0, 1):
        p, g, r = _run(T, E, k, cf, opts, seed, multi=multi)
        compare_forward(g, r, p)


@pytest.mark.parametrize("multi", [False, True], ids=["default", "multi_kernel"])
def test_small_ties(multi):
    """Integer logits: most rows hold ties, broken toward the lower expert."""
    T, E, k = 4000, 8, 3
    print(f"case small ties T={T} E={E} k={k} multi={multi}", flush=True)
    rng = np.random.default_rng(7)
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    p, g, r = _run(T, E, k, 1.0, "renorm", 7, logits=L, multi=multi)
    compare_forward(g, r, p)


def test_small_nonfinite():
    T, E, k = 3000, 8, 2
    print(f"case small nonfinite T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(9)
    for bad in [np.nan, np.inf, -np.inf]:
        L = rng.standard_normal((T, E), dtype=np.float32)
        L[1234, 5] = bad
        p = lbs.make_params(T, E, k, capacity_factor=1.0, renorm=True, save_row_stats=True)
        g = gpu_forward(p, {"logits": L})
        if np.isneginf(bad):
            # a -inf logit is a valid zero probability
            assert g["status"][0] == 0
            continue
        assert g["status"][0] & lbs.MOE_STATUS_NONFINITE
        ok = np.ones(T, bool)
        ok[1234] = False
        ro = oracle.route(L[ok], k, capacity_factor=0.0, renorm=True)
        assert_equal(g["topk_idx"][ok], ro["topk_idx"], "topk_idx of finite rows")


def test_small_repeat_and_poisoned_outputs():
    """Two calls give identical bits (outputs start poisoned each time)."""
    T, E, k = 4096, 8, 2
    a = _run(T, E, k, 1.25, "renorm", 3)[1]
    b = _run(T, E, k, 1.25, "renorm", 3)[1]
    for key in ("topk_idx", "topk_w", "perm", "dropped", "counts", "P", "aux_loss", "extra_stats"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key
