"""Seeded synthetic router inputs for the five routing workloads.

This module only draws random inputs (logits, or bf16 activations and gate
weights) with the shapes and value distributions of the workloads; it holds
none of the routing arithmetic.  Both the HIP path's tests/benchmark and the
CPU oracle take their inputs from here.

Workloads (T tokens, E experts, top-k, m microbatches):

* ``switch_top1`` -- Switch-style top-1: T=4096, E=8, logits iid N(0,1),
  alpha 0.01, capacity factor 1.25.
* ``zipf_top2``  -- T=65536, E=64, top-2 with renormalised weights; logits
  N(0,1) plus a per-expert bias log(w_e) with Zipf(s=1) weights
  w_e = 1/(e+1), so hot and cold experts differ by far more than 10x;
  capacity factor 1.0, alpha 0.01.
* ``gate_top2``  -- gate GEMM: X bf16 [16384 x 4096] iid N(0,1), Wg bf16
  [4096 x 8] iid N(0, 0.02^2), logits = X.Wg in fp32, top-2, capacity
  factor 1.25, plus the aux-loss backward.
* ``v3_shape``   -- T=131072, E=256, top-8; logits N(0,1) plus a per-expert
  bias N(0, 0.5^2) fixed per seed; capacity factor 1.25, alpha 0.001.
* ``v4_shape``   -- 16 microbatches of 16384 tokens, E=384, top-6; logits
  N(0,1) with a fresh random hot set of 16 experts per microbatch boosted by
  +2.0; capacity factor 1.0, forward plus aux-loss backward.
* ``v3_select_bias`` -- the v3 shape routed the loss-free way: logits iid
  N(0,1) and a separate per-expert selection bias N(0, 0.5^2) that steers
  the expert choice only, alpha 0 (no aux loss), followed by one bias update
  step (gamma 0.001).

Draw order for a seed: per-expert bias or hot sets first, then the logits
(for the gate workload: X, then Wg), then the selection bias if any.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens in total (= n_micro * Tm)
    E: int                 # experts
    k: int                 # experts per token
    n_micro: int = 1       # microbatches, each routed on its own
    capacity_factor: float = 1.0
    alpha: float = 0.01
    renorm: bool = True    # renormalise the k gate weights to sum to 1
    d: int = 0             # 0: logits given; > 0: gate GEMM with hidden size d
    backward: bool = False # the workload also runs the aux-loss backward
    logits_kind: str = "normal"  # normal | zipf_bias | normal_bias | hot_set
    select_bias_scale: float = 0.0  # > 0: a selection bias N(0, scale^2) per expert
    bias_gamma: float = 0.0         # step of the bias update that follows the forward

    @property
    def Tm(self):
        return self.T // self.n_micro

    def scaled(self, T=None, n_micro=None, d=None):
        """Same distributions at another size (for parity cases)."""
        kw = {}
        if n_micro is not None:
            kw["n_micro"] = n_micro
        if T is not None:
            kw["T"] = T
        if d is not None:
            kw["d"] = d
        return replace(self, **kw)


WORKLOADS = {
    "switch_top1": Workload("switch_top1", T=4096, E=8, k=1, capacity_factor=1.25,
                            alpha=0.01, renorm=False, logits_kind="normal"),
    "zipf_top2": Workload("zipf_top2", T=65536, E=64, k=2, capacity_factor=1.0,
                          alpha=0.01, renorm=True, logits_kind="zipf_bias"),
    "gate_top2": Workload("gate_top2", T=16384, E=8, k=2, capacity_factor=1.25,
                          alpha=0.01, renorm=True, d=4096, backward=True),
    "v3_shape": Workload("v3_shape", T=131072, E=256, k=8, capacity_factor=1.25,
                         alpha=0.001, renorm=True, logits_kind="normal_bias"),
    "v4_shape": Workload("v4_shape", T=262144, E=384, k=6, n_micro=16,
                         capacity_factor=1.0, alpha=0.01, renorm=True,
                         backward=True, logits_kind="hot_set"),
    "v3_select_bias": Workload("v3_select_bias", T=131072, E=256, k=8, capacity_factor=1.25,
                               alpha=0.0, renorm=True, logits_kind="normal",
                               select_bias_scale=0.5, bias_gamma=0.001),
}


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: Workload, seed: int):
    """Draw the inputs of workload ``w`` for ``seed``.

    Returns a dict with ``logits`` (float32 [T,E]) or, for the gate workload,
    ``X`` (uint16 bf16 bits [T,d]) and ``Wg`` (uint16 bf16 bits [d,E]); plus
    ``select_bias`` (float32 [E]) for workloads routed with a selection bias.
    """
    rng = np.random.default_rng(seed)
    if w.d > 0:
        X = f32_to_bf16_bits(rng.standard_normal((w.T, w.d), dtype=np.float32))
        Wg = f32_to_bf16_bits(np.float32(0.02) * rng.standard_normal((w.d, w.E), dtype=np.float32))
        return {"X": X, "Wg": Wg}
    if w.logits_kind == "normal":
        L = rng.standard_normal((w.T, w.E), dtype=np.float32)
    elif w.logits_kind == "zipf_bias":
        # Zipf(s=1) popularity: expert e has rank e+1 and weight 1/(e+1).
        bias = (-np.log(np.arange(1, w.E + 1, dtype=np.float64))).astype(np.float32)
        L = rng.standard_normal((w.T, w.E), dtype=np.float32) + bias[None, :]
    elif w.logits_kind == "normal_bias":
        bias = (np.float32(0.5) * rng.standard_normal(w.E, dtype=np.float32))
        L = rng.standard_normal((w.T, w.E), dtype=np.float32) + bias[None, :]
    elif w.logits_kind == "hot_set":
        n_hot = min(16, w.E)
        hot = [rng.choice(w.E, size=n_hot, replace=False) for _ in range(w.n_micro)]
        L = rng.standard_normal((w.T, w.E), dtype=np.float32)
        Tm = w.Tm
        for mb, h in enumerate(hot):
            L[mb * Tm:(mb + 1) * Tm, h] += np.float32(2.0)
    else:
        raise ValueError(w.logits_kind)
    out = {"logits": np.ascontiguousarray(L, dtype=np.float32)}
    if w.select_bias_scale > 0:
        out["select_bias"] = (np.float32(w.select_bias_scale)
                              * rng.standard_normal(w.E, dtype=np.float32)).astype(np.float32)
    return out
