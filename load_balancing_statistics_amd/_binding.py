"""ctypes binding of the C ABI in ``include/moe_route.h`` (same names).

Argument marshalling only: every step of routing runs in the HIP library
``_lib/libmoe_route.so``.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libmoe_route.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5
MOE_ROUTE_SCRATCH_BYTES = 32 * 1024 * 1024

MOE_RENORM_TOPK = 1
MOE_SAVE_ROW_STATS = 2
MOE_WRITE_INV_PERM = 4
MOE_SELECT_BIAS = 8
MOE_P_MASKED = 16
MOE_MULTI_KERNEL = 32

MOE_STATUS_NONFINITE = 1
MOE_STATUS_INTERNAL = 2

MOE_ROUTE_MAX_E = 1024
MOE_ROUTE_MAX_K = 32

EXPORTED = ("moe_route_workspace_size", "moe_route_capacity", "moe_route",
            "moe_route_backward", "moe_route_strerror")


class MoeRouteError(RuntimeError):
    def __init__(self, code, func):
        self.code = code
        super().__init__(f"{func} failed ({code}): {moe_route_strerror(code)}")


class moe_route_params(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_micro", ctypes.c_int32), ("d", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double),
                ("alpha", ctypes.c_float), ("flags", ctypes.c_uint32)]


_OUT_FIELDS = ("topk_idx", "topk_w", "logits", "row_stats", "counts", "offsets", "perm",
               "inv_perm", "dropped", "f", "P", "aux_loss", "cv", "max_over_mean",
               "extra_stats", "status")


class moe_route_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _OUT_FIELDS] + [
        ("row_pass_events", ctypes.c_void_p * 2)]


_lib = None


def load(path=None):
    """Load the HIP routing library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # PyTorch first: its HIP runtime (same soname) then serves this library
    # too, so device pointers and streams are shared by one runtime.
    import torch  # noqa: F401
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP routing library not built: {p} is missing "
                           "(run load_balancing_statistics_amd.build.build())")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(moe_route_params)
    vp = ctypes.c_void_p
    lib.moe_route_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_route_workspace_size.restype = ctypes.c_int
    lib.moe_route_capacity.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.moe_route_capacity.restype = ctypes.c_int
    lib.moe_route.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(moe_route_out), vp, ctypes.c_size_t, vp]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route_noalloc.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(moe_route_out), vp]
    lib.moe_route_noalloc.restype = ctypes.c_int
    lib.moe_route_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_route_backward.restype = ctypes.c_int
    lib.moe_route_bias_update.argtypes = [P, vp, ctypes.c_float, vp, vp]
    lib.moe_route_with_bias_update.argtypes = [P, vp, vp, vp, vp, ctypes.c_float,
                                               ctypes.POINTER(moe_route_out), vp, ctypes.c_size_t, vp]
    lib.moe_route_with_bias_update.restype = ctypes.c_int
    lib.moe_route_bias_update.restype = ctypes.c_int
    lib.moe_gate_backward_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_gate_backward_workspace_size.restype = ctypes.c_int
    lib.moe_gate_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_gate_backward.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.moe_eplb_plan.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_eplb_plan.restype = ctypes.c_int
    lib.moe_sinkhorn_plan.argtypes = [i32, vp, vp, vp, ctypes.c_double, i32, vp, vp, vp, vp]
    lib.moe_sinkhorn_plan.restype = ctypes.c_int
    lib.moe_route_strerror.argtypes = [ctypes.c_int]
    lib.moe_route_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def make_params(T, E, k, n_micro=1, d=0, capacity_factor=1.0, capacity=-1, alpha=0.01,
                renorm=False, save_row_stats=False, inv_perm=False, select_bias=False,
                p_masked=False, multi_kernel=False):
    flags = ((MOE_RENORM_TOPK if renorm else 0) | (MOE_SAVE_ROW_STATS if save_row_stats else 0)
             | (MOE_WRITE_INV_PERM if inv_perm else 0) | (MOE_SELECT_BIAS if select_bias else 0)
             | (MOE_P_MASKED if p_masked else 0) | (MOE_MULTI_KERNEL if multi_kernel else 0))
    return moe_route_params(int(T), int(E), int(k), int(n_micro), int(d), int(capacity),
                            float(capacity_factor), float(alpha), flags)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def moe_route_strerror(code):
    return load().moe_route_strerror(int(code)).decode()


def moe_route_workspace_size(params):
    n = ctypes.c_size_t(0)
    rc = load().moe_route_workspace_size(ctypes.byref(params), ctypes.byref(n))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_workspace_size")
    return n.value


def moe_route_capacity(params):
    c = ctypes.c_int32(0)
    rc = load().moe_route_capacity(ctypes.byref(params), ctypes.byref(c))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_capacity")
    return c.value


def moe_route(params, out, workspace, logits=None, X=None, Wg=None, stream=None,
              row_pass_events=None, select_bias=None):
    """Forward routing; ``out`` maps output names to device tensors (or None).

    ``select_bias``: fp32 [E] device tensor, used when the params carry
    MOE_SELECT_BIAS (expert choice on logits + bias, weights unbiased).

    ``row_pass_events``: optional pair of raw hipEvent_t handles (ints) that the
    library attaches to the row-pass kernel's launch as its start and stop."""
    o = moe_route_out(*[None if out.get(n) is None else out[n].data_ptr() for n in _OUT_FIELDS])
    if row_pass_events is not None:
        o.row_pass_events[0] = row_pass_events[0]
        o.row_pass_events[1] = row_pass_events[1]
    rc = load().moe_route(ctypes.byref(params), _ptr(logits), _ptr(X), _ptr(Wg), _ptr(select_bias),
                          ctypes.byref(o),
                          _ptr(workspace), workspace.numel() * workspace.element_size()
                          if workspace is not None else 0, _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route")


def moe_route_with_bias_update(params, out, workspace, select_bias, gamma, logits=None, X=None, Wg=None,
                               stream=None, row_pass_events=None):
    """One loss-free balancing step: ``moe_route`` with ``select_bias`` (the
    params must carry MOE_SELECT_BIAS), then ``select_bias`` stepped in place
    by ``gamma`` from this call's counts."""
    o = moe_route_out(*[None if out.get(n) is None else out[n].data_ptr() for n in _OUT_FIELDS])
    if row_pass_events is not None:
        o.row_pass_events[0] = row_pass_events[0]
        o.row_pass_events[1] = row_pass_events[1]
    rc = load().moe_route_with_bias_update(ctypes.byref(params), _ptr(logits), _ptr(X), _ptr(Wg),
                                           _ptr(select_bias), float(gamma), ctypes.byref(o), _ptr(workspace),
                                           workspace.numel() * workspace.element_size()
                                           if workspace is not None else 0, _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_with_bias_update")


def moe_route_noalloc(params, out, logits=None, X=None, Wg=None, stream=None, select_bias=None):
    """``moe_route`` with the library's static device scratch as workspace (no
    allocation in the call); calls overlapping on one GPU race."""
    o = moe_route_out(*[None if out.get(n) is None else out[n].data_ptr() for n in _OUT_FIELDS])
    rc = load().moe_route_noalloc(ctypes.byref(params), _ptr(logits), _ptr(X), _ptr(Wg),
                                  _ptr(select_bias), ctypes.byref(o), _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_noalloc")


def moe_route_backward(params, logits, counts, dlogits, row_stats=None, d_aux=None,
                       topk_idx=None, d_topk_w=None, stream=None):
    """dL/dlogits of the aux loss (all-token or masked P, per the params' flags)
    plus, when ``d_topk_w`` is given, of sum d_topk_w * topk_w; into ``dlogits``."""
    rc = load().moe_route_backward(ctypes.byref(params), _ptr(logits), _ptr(row_stats),
                                   _ptr(counts), _ptr(d_aux), _ptr(topk_idx), _ptr(d_topk_w),
                                   _ptr(dlogits), _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_backward")


def moe_route_bias_update(params, counts, gamma, bias, stream=None):
    """One selection-bias step from the forward's counts; ``bias`` is updated in place."""
    rc = load().moe_route_bias_update(ctypes.byref(params), _ptr(counts), float(gamma), _ptr(bias),
                                      _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_route_bias_update")


def moe_gate_backward_workspace_size(params):
    n = ctypes.c_size_t(0)
    rc = load().moe_gate_backward_workspace_size(ctypes.byref(params), ctypes.byref(n))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_gate_backward_workspace_size")
    return n.value


def moe_gate_backward(params, X, Wg, dlogits, dX=None, dWg=None, workspace=None, stream=None):
    """dX = dlogits.Wg^T (bf16 bits) and/or dWg = X^T.dlogits (fp32) into the given tensors."""
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().moe_gate_backward(ctypes.byref(params), _ptr(X), _ptr(Wg), _ptr(dlogits), _ptr(dX),
                                  _ptr(dWg), _ptr(workspace), nbytes, _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_gate_backward")


def moe_eplb_plan(weight, num_phys, num_packs, stream=None):
    """EPLB placement of the experts with loads ``weight`` (int32 device tensor
    [E]); returns a dict of device tensors named like the C outputs."""
    import torch
    E = weight.numel()
    dev = weight.device
    i32 = torch.int32
    o = dict(phy2log=torch.empty(num_phys, dtype=i32, device=dev),
             phy_rank=torch.empty(num_phys, dtype=i32, device=dev),
             logcnt=torch.empty(E, dtype=i32, device=dev),
             pack=torch.empty(num_phys, dtype=i32, device=dev),
             slot=torch.empty(num_phys, dtype=i32, device=dev),
             pack_load=torch.empty(num_packs, dtype=torch.float64, device=dev))
    rc = load().moe_eplb_plan(E, int(num_phys), int(num_packs), _ptr(weight),
                              *[_ptr(o[n]) for n in ("phy2log", "phy_rank", "logcnt", "pack", "slot",
                                                     "pack_load")], _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_eplb_plan")
    return o


def moe_sinkhorn_plan(supply, demand, cost, eps, iters=50, stream=None):
    """Sinkhorn-Knopp plan from fp64 device tensors supply [R], demand [R], cost
    [R,R]; returns (T [R,R], u [R], v [R]) as fp64 device tensors."""
    import torch
    R = supply.numel()
    dev = supply.device
    u = torch.empty(R, dtype=torch.float64, device=dev)
    v = torch.empty(R, dtype=torch.float64, device=dev)
    T = torch.empty((R, R), dtype=torch.float64, device=dev)
    rc = load().moe_sinkhorn_plan(R, _ptr(supply), _ptr(demand), _ptr(cost), float(eps), int(iters),
                                  _ptr(u), _ptr(v), _ptr(T), _stream(stream))
    if rc != MOE_OK:
        raise MoeRouteError(rc, "moe_sinkhorn_plan")
    return T, u, v


def alloc_outputs(params, device="cuda"):
    """Device tensors for every output of ``moe_route`` (plumbing only)."""
    import torch
    T, E, k, m = params.T, params.E, params.k, params.n_micro
    i32, f32 = torch.int32, torch.float32
    out = dict(
        topk_idx=torch.empty((T, k), dtype=i32, device=device),
        topk_w=torch.empty((T, k), dtype=f32, device=device),
        logits=torch.empty((T, E), dtype=f32, device=device) if params.d > 0 else None,
        row_stats=torch.empty((T, 2), dtype=f32, device=device)
        if params.flags & MOE_SAVE_ROW_STATS else None,
        counts=torch.empty((m, E), dtype=i32, device=device),
        offsets=torch.empty((m, E + 1), dtype=i32, device=device),
        perm=torch.empty(T * k, dtype=i32, device=device),
        inv_perm=torch.empty(T * k, dtype=i32, device=device)
        if params.flags & MOE_WRITE_INV_PERM else None,
        dropped=torch.empty(T * k, dtype=torch.uint8, device=device),
        f=torch.empty((m, E), dtype=f32, device=device),
        P=torch.empty((m, E), dtype=f32, device=device),
        aux_loss=torch.empty(m, dtype=f32, device=device),
        cv=torch.empty(m, dtype=f32, device=device),
        max_over_mean=torch.empty(m, dtype=f32, device=device),
        extra_stats=torch.empty((m, 8), dtype=f32, device=device),
        status=torch.empty(1, dtype=i32, device=device),
    )
    return out


def alloc_workspace(params, device="cuda"):
    import torch
    n = moe_route_workspace_size(params)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
