"""ctypes front end of the C oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Arrays in and out are numpy; all floating point is
float64.  See ``moe_oracle.c`` for the definitions and the page citations.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def load_library(path=None):
    """Load (building first if needed) the oracle library; cached."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _build.LIB
    if not os.path.exists(p):
        _build.build(out=p)
    lib = ctypes.CDLL(p)
    ll, d, vp, i = ctypes.c_longlong, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.oracle_capacity.argtypes = [ll, ll, ll, ctypes.c_char_p, ll]
    lib.oracle_capacity.restype = ll
    lib.oracle_gate_logits.argtypes = [vp, vp, ll, ll, ll, vp]
    lib.oracle_gate_logits.restype = None
    lib.oracle_route.argtypes = [vp, ll, ll, ll, ll, ll, d, i, vp, i] + [vp] * 15
    lib.oracle_route.restype = i
    lib.oracle_backward.argtypes = [vp, ll, ll, ll, ll, d, vp, vp, i, vp, i, vp, vp]
    lib.oracle_backward.restype = None
    lib.oracle_gate_backward.argtypes = [vp, vp, vp, ll, ll, ll, vp, vp]
    lib.oracle_gate_backward.restype = None
    lib.oracle_eplb.argtypes = [vp, ll, ll, ll, vp, vp, vp, vp, vp, vp]
    lib.oracle_eplb.restype = i
    lib.oracle_sinkhorn.argtypes = [vp, vp, vp, ll, d, ll, vp, vp, vp]
    lib.oracle_sinkhorn.restype = i
    lib.oracle_bias_update.argtypes = [vp, ll, ll, ll, ll, ctypes.c_float, vp]
    lib.oracle_bias_update.restype = None
    if path is None:
        _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def capacity(Tm, E, k, capacity_factor, capacity_override=-1, lib=None):
    """Per-microbatch capacity C (``-1`` = unlimited).

    ``capacity_factor`` is the caller's number: a string is used as written,
    a float as the shortest decimal that reads back as that float (its
    ``repr``: 1.1 -> "1.1"), so the oracle computes with the decimal the
    caller typed, exactly."""
    lib = lib or load_library()
    text = capacity_factor if isinstance(capacity_factor, str) else repr(float(capacity_factor))
    C = int(lib.oracle_capacity(int(Tm), int(E), int(k), text.encode(), int(capacity_override)))
    if C < -1:
        raise ValueError(f"capacity factor {text!r} is not a decimal number")
    return C


def gate_logits(X_bits, Wg_bits, lib=None):
    """fp64 logits of X[T,d] @ Wg[d,E] from bf16 bit patterns (uint16 arrays)."""
    lib = lib or load_library()
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    W = np.ascontiguousarray(Wg_bits, dtype=np.uint16)
    T, d = X.shape
    d2, E = W.shape
    assert d == d2
    out = np.empty((T, E), np.float64)
    lib.oracle_gate_logits(_p(X), _p(W), T, d, E, _p(out))
    return out


def gate_backward(X_bits, Wg_bits, dlogits, lib=None):
    """(dX [T,d], dWg [d,E]) in float64 for logits = X.Wg, given dL/dlogits [T,E]."""
    lib = lib or load_library()
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    W = np.ascontiguousarray(Wg_bits, dtype=np.uint16)
    T, d = X.shape
    d2, E = W.shape
    assert d == d2
    G = np.ascontiguousarray(dlogits, dtype=np.float64).reshape(T, E)
    dX = np.empty((T, d), np.float64)
    dW = np.empty((d, E), np.float64)
    lib.oracle_gate_backward(_p(X), _p(W), _p(G), T, d, E, _p(dX), _p(dW))
    return dX, dW


def route(logits, k, n_micro=1, capacity_factor=1.0, capacity_override=-1,
          alpha=0.01, renorm=False, select_bias=None, p_masked=False, lib=None):
    """Route ``logits`` [T,E] (any float dtype; widened exactly to float64).

    ``select_bias``: optional float32 [E] added to the logits for the expert
    choice only (fp32 sum); weights and statistics stay unbiased.
    ``p_masked``: P_i over the picked positions, divided by Tm*k.

    Returns a dict of numpy arrays named like the C-ABI outputs, plus
    ``capacity`` (int, -1 = unlimited).
    """
    lib = lib or load_library()
    L = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = L.shape
    m = int(n_micro)
    if T % m:
        raise ValueError("T must be a multiple of n_micro")
    C = capacity(T // m, E, k, capacity_factor, capacity_override, lib=lib)
    o = dict(
        topk_idx=np.empty((T, k), np.int32), topk_w=np.empty((T, k), np.float64),
        row_max=np.empty(T, np.float64), row_sum=np.empty(T, np.float64),
        counts=np.empty((m, E), np.int32), offsets=np.empty((m, E + 1), np.int32),
        perm=np.empty(T * k, np.int32), inv_perm=np.empty(T * k, np.int32),
        dropped=np.empty(T * k, np.uint8), f=np.empty((m, E), np.float64),
        P=np.empty((m, E), np.float64), aux=np.empty(m, np.float64),
        cv=np.empty(m, np.float64), max_over_mean=np.empty(m, np.float64),
        extra=np.empty((m, 8), np.float64))
    b = None if select_bias is None else np.ascontiguousarray(select_bias, dtype=np.float32)
    if b is not None and b.shape != (E,):
        raise ValueError("select_bias must have shape [E]")
    rc = lib.oracle_route(_p(L), T, E, int(k), m, C, float(alpha), int(bool(renorm)), _p(b),
                          int(bool(p_masked)),
                          *[_p(o[n]) for n in ("topk_idx", "topk_w", "row_max", "row_sum",
                                               "counts", "offsets", "perm", "inv_perm",
                                               "dropped", "f", "P", "aux", "cv",
                                               "max_over_mean", "extra")])
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    o["capacity"] = C
    return o


def backward(logits, k, counts, n_micro=1, alpha=0.01, d_aux=None, p_masked=False,
             topk_idx=None, renorm=False, d_topk_w=None, lib=None):
    """dL/dlogits [T,E] (float64) of  sum_mb d_aux[mb]*aux_mb + sum d_topk_w*topk_w,
    with the forward's selection and pre-capacity counts held fixed.
    ``topk_idx`` [T,k] is needed for ``p_masked`` and for ``d_topk_w``."""
    lib = lib or load_library()
    L = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = L.shape
    cnt = np.ascontiguousarray(counts, dtype=np.int32).reshape(n_micro, E)
    g = None if d_aux is None else np.ascontiguousarray(d_aux, dtype=np.float64).reshape(n_micro)
    if (p_masked or d_topk_w is not None) and topk_idx is None:
        raise ValueError("topk_idx is required for p_masked and d_topk_w")
    idx = None if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(T, k)
    dw = None if d_topk_w is None else np.ascontiguousarray(d_topk_w, dtype=np.float64).reshape(T, k)
    out = np.empty((T, E), np.float64)
    lib.oracle_backward(_p(L), T, E, int(k), int(n_micro), float(alpha), _p(cnt), _p(g),
                        int(bool(p_masked)), _p(idx), int(bool(renorm)), _p(dw), _p(out))
    return out


def bias_update(counts, T, k, gamma, bias, lib=None):
    """Selection-bias step after a forward: returns the new float32 [E] bias."""
    lib = lib or load_library()
    cnt = np.ascontiguousarray(counts, dtype=np.int32)
    m, E = cnt.reshape(-1, cnt.shape[-1]).shape
    b = np.array(bias, dtype=np.float32, copy=True)
    if b.shape != (E,):
        raise ValueError("bias must have shape [E]")
    lib.oracle_bias_update(_p(cnt), m, E, int(T), int(k), float(gamma), _p(b))
    return b


def eplb(weight, num_phys, num_packs, lib=None):
    """EPLB placement of E logical experts with loads ``weight`` (ints) onto
    ``num_phys`` physical replicas packed into ``num_packs`` equal packs."""
    lib = lib or load_library()
    w = np.ascontiguousarray(weight, dtype=np.int32).ravel()
    E = w.shape[0]
    o = dict(phy2log=np.empty(num_phys, np.int32), phy_rank=np.empty(num_phys, np.int32),
             logcnt=np.empty(E, np.int32), pack=np.empty(num_phys, np.int32),
             slot=np.empty(num_phys, np.int32), pack_load=np.empty(num_packs, np.float64))
    rc = lib.oracle_eplb(_p(w), E, int(num_phys), int(num_packs),
                         *[_p(o[n]) for n in ("phy2log", "phy_rank", "logcnt", "pack", "slot", "pack_load")])
    if rc != 0:
        raise ValueError("oracle_eplb rejected its arguments")
    return o


def sinkhorn(a, b, C, eps, iters=50, lib=None):
    """Sinkhorn-Knopp plan for supply ``a`` [R], demand ``b`` [R], cost ``C`` [R,R]:
    returns (T [R,R], u [R], v [R]) in float64."""
    lib = lib or load_library()
    a = np.ascontiguousarray(a, dtype=np.float64).ravel()
    b = np.ascontiguousarray(b, dtype=np.float64).ravel()
    R = a.shape[0]
    Cm = np.ascontiguousarray(C, dtype=np.float64).reshape(R, R)
    u, v, T = np.empty(R), np.empty(R), np.empty((R, R))
    if lib.oracle_sinkhorn(_p(a), _p(b), _p(Cm), R, float(eps), int(iters), _p(u), _p(v), _p(T)) != 0:
        raise ValueError("oracle_sinkhorn rejected its arguments")
    return T, u, v
