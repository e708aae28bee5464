"""Row-pass timing events: moe_route launches the row pass with the caller's
events as the kernel's start and stop (hipExtLaunchKernel).  The outputs must
not change, and the events must bracket a positive time no longer than the
whole call."""
import ctypes

import numpy as np
import pytest
import torch

import load_balancing_statistics_amd as lbs
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu

KEYS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "dropped", "P", "aux_loss", "cv",
        "max_over_mean", "extra_stats", "status")


class _Events:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        h = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(h)) == 0
        return h.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, h):
        self.lib.hipEventDestroy(ctypes.c_void_p(h))


def _route(p, L, events=None):
    dev = torch.device(DEV)
    out = lbs.alloc_outputs(p, device=dev)
    ws = lbs.alloc_workspace(p, device=dev)
    lbs.moe_route(p, out, ws, logits=L, row_pass_events=events)
    torch.cuda.synchronize()
    return {k: out[k].cpu().numpy() for k in KEYS if out.get(k) is not None}


@pytest.mark.parametrize("T,E,k", [(8192, 256, 8), (4096, 8, 1), (3000, 384, 6)])
def test_row_pass_events(T, E, k):
    print(f"case events T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(T + E)
    L = torch.from_numpy(rng.standard_normal((T, E), dtype=np.float32)).to(torch.device(DEV))
    p = lbs.make_params(T, E, k, capacity_factor=1.25, renorm=True)
    plain = _route(p, L)
    ev = _Events()
    e0, e1 = ev.create(), ev.create()
    try:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        timed = _route(p, L, events=(e0, e1))
        t1.record()
        torch.cuda.synchronize()
        rows_ms = ev.elapsed_ms(e0, e1)
        call_ms = t0.elapsed_time(t1)
    finally:
        ev.destroy(e0)
        ev.destroy(e1)
    for key in plain:
        assert np.array_equal(plain[key], timed[key], equal_nan=True), key
    assert 0.0 < rows_ms <= call_ms, (rows_ms, call_ms)
