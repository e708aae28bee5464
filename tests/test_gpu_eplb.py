"""EPLB placement (page cnvsn.com/news/335486 section 4.1.2) on the GPU
against the CPU oracle: every output bit-exact, including the fp64 pack
loads (same additions in the same order)."""
import os

import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from load_balancing_statistics_amd.workloads import WORKLOADS, make_inputs
import oracle
from gpu_helpers import DEV, assert_equal, gpu_forward, params_of

pytestmark = pytest.mark.gpu

KEYS = ("phy2log", "phy_rank", "logcnt", "pack", "slot", "pack_load")


def _gpu(weight, num_phys, packs):
    w = torch.from_numpy(np.asarray(weight, np.int32)).to(DEV)
    o = lbs.moe_eplb_plan(w, num_phys, packs)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _compare(weight, num_phys, packs):
    g = _gpu(weight, num_phys, packs)
    r = oracle.eplb(np.maximum(np.asarray(weight), 0), num_phys, packs)
    for k in KEYS:
        assert_equal(g[k], r[k], k)
    return g


def test_eplb_worked_example():
    print("case eplb worked example", flush=True)
    g = _compare([9, 7, 5, 3], 4, 2)
    assert list(g["pack"]) == [0, 1, 1, 0] and list(g["pack_load"]) == [12.0, 12.0]


@pytest.mark.parametrize("E,R,packs", [(4, 4, 2), (64, 0, 8), (64, 64, 16), (256, 32, 32),
                                       (384, 64, 64), (1000, 24, 8), (1024, 3072, 1024), (1, 7, 4),
                                       (300, 84, 128)])
def test_eplb_random(E, R, packs):
    print(f"case eplb E={E} R={R} packs={packs}", flush=True)
    rng = np.random.default_rng(E + R)
    w = (rng.pareto(1.2, size=E) * 1000).astype(np.int64).clip(0, 2**31 - 1).astype(np.int32)
    _compare(w, E + R, packs)


def test_eplb_ties_and_zeros():
    print("case eplb ties", flush=True)
    _compare(np.full(96, 50, np.int32), 128, 16)       # equal loads: ties everywhere
    _compare(np.zeros(40, np.int32), 80, 20)           # all idle
    w = np.zeros(64, np.int32)
    w[5] = 1000
    _compare(w, 96, 32)                                # one hot expert takes every copy
    _compare(np.array([3, -2, 7, 0], np.int32), 8, 4)  # negative counts read as 0


def test_eplb_on_routing_counts():
    """The counts a v4_shape forward produces: one microbatch's row, and the
    sum over microbatches, placed on 64 GPUs with 64 redundant replicas."""
    w = WORKLOADS["v4_shape"]
    print("case eplb on v4 counts", flush=True)
    inp = make_inputs(w, 0)
    g = gpu_forward(params_of(w), inp)
    counts = g["counts"]
    _compare(counts[3], w.E + 64, 64)
    _compare(counts.sum(0).astype(np.int32), w.E + 64, 64)
    # the placement lowers the largest per-GPU load below the unreplicated one
    r0 = oracle.eplb(counts[3], w.E, 64)
    r1 = oracle.eplb(counts[3], w.E + 64, 64)
    assert r1["pack_load"].max() < r0["pack_load"].max()


@pytest.mark.parametrize("seed", range(8))
def test_eplb_small_integer_loads(seed):
    """Weights drawn from a handful of small integers: equal per-replica loads
    and equal pack loads at every step, so runs of placements end on ties and
    single placements alternate with runs."""
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 300))
    packs = int(rng.choice([1, 2, 3, 8, 16, 48, 64, 96]))
    per = int(np.ceil(E / packs)) + int(rng.integers(0, 4))
    print(f"case eplb small-int seed={seed} E={E} P={packs * per} packs={packs}", flush=True)
    w = rng.choice([0, 1, 2, 3, 4, 6, 12], size=E).astype(np.int32)
    _compare(w, packs * per, packs)
