"""ctypes view of the plain C oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the CPU-baseline leg of bench.py.  The GPU library
never imports it.  All arrays are numpy; the layer is a synth.Layer (any
object with the same attribute names works).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, Q2K, Q8_0, CB2, Q4K = 0, 1, 2, 3, 4, 5

_lib = None


class _OrcLayer(ctypes.Structure):
    _fields_ = [
        ("n_embd", ctypes.c_int32), ("n_expert", ctypes.c_int32), ("n_expert_used", ctypes.c_int32),
        ("n_ff_exp", ctypes.c_int32), ("n_ff_shared", ctypes.c_int32),
        ("gate_fmt", ctypes.c_int32), ("up_fmt", ctypes.c_int32), ("down_fmt", ctypes.c_int32),
        ("shared_fmt", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("route_scale", ctypes.c_double),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.orc_tensor_bytes.restype = I64
        lib.orc_tensor_bytes.argtypes = [ctypes.c_int, I64]
        lib.orc_dequant.argtypes = [ctypes.c_int, P, I64, P, P]
        lib.orc_logits.argtypes = [P, P, I32, P]
        lib.orc_topk.argtypes = [P, I32, I32, I32, D, P, P, P]
        lib.orc_bucket.argtypes = [P, I32, I32, I32, P, P, P, P, P, P]
        lib.orc_moe_forward.argtypes = [P, ctypes.c_int, P, P, I32, P, I32, P, P, P]
        lib.orc_moe_forward_dense.argtypes = [P, ctypes.c_int, P, P, I32, P]
        lib.orc_rmsnorm.argtypes = [P, P, D, I32, I32, P]
        lib.orc_swiglu.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, I32, I32, ctypes.c_int, P, P]
        lib.orc_count_selections.argtypes = [P, I32, I32, I32, I32, P]
        lib.orc_hotlist.restype = I32
        lib.orc_hotlist.argtypes = [P, I32, P]
        lib.orc_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Bound:
    """Keeps the numpy buffers alive while the C struct points at them."""

    def __init__(self, L):
        self.keep = dict(
            router_w=_c(L.router_w, np.float32), router_bias=_c(L.router_bias, np.float32),
            gate=_c(L.gate, np.uint8), up=_c(L.up, np.uint8), down=_c(L.down, np.uint8),
            sh_gate=_c(L.sh_gate, np.uint8), sh_up=_c(L.sh_up, np.uint8), sh_down=_c(L.sh_down, np.uint8),
            codebook=_c(L.codebook, np.int8))
        k = self.keep
        self.s = _OrcLayer(L.n_embd, L.n_expert, L.n_expert_used, L.n_ff_exp, L.n_ff_shared,
                           L.gate_fmt, L.up_fmt, L.down_fmt, L.shared_fmt,
                           _p(k["router_w"]), _p(k["router_bias"]), float(L.route_scale),
                           _p(k["gate"]), _p(k["up"]), _p(k["down"]),
                           _p(k["sh_gate"]), _p(k["sh_up"]), _p(k["sh_down"]), _p(k["codebook"]))

    def ref(self):
        return ctypes.byref(self.s)


def version():
    return _load().orc_version().decode()


def tensor_bytes(fmt, n):
    return _load().orc_tensor_bytes(fmt, n)


def dequant(fmt, src, n, codebook=None):
    src = _c(src, np.uint8)
    cb = _c(codebook, np.int8)
    out = np.empty(n, dtype=np.float32)
    if _load().orc_dequant(fmt, _p(src), n, _p(cb), _p(out)) != 0:
        raise ValueError("oracle: dequant rejected its arguments")
    return out


def input_as_double(x=None, x_bf16=None):
    if x_bf16 is not None:
        b = np.ascontiguousarray(x_bf16, dtype=np.uint16).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)


def logits(L, x=None, x_bf16=None):
    xd = np.ascontiguousarray(input_as_double(x, x_bf16))
    T = xd.shape[0]
    out = np.empty((T, L.n_expert), dtype=np.float64)
    B = _Bound(L)
    _load().orc_logits(B.ref(), _p(xd), T, _p(out))
    return out


def topk(lg, k, route_scale=1.0):
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    gap = np.empty(T, dtype=np.float64)
    if _load().orc_topk(_p(lg), T, E, k, route_scale, _p(idx), _p(w), _p(gap)) != 0:
        raise ValueError("oracle: topk rejected its arguments")
    return idx, w, gap


def route(L, x=None, x_bf16=None):
    """(topk_idx [T][k], topk_w [T][k], decision gap [T]) of the layer's router."""
    return topk(logits(L, x, x_bf16), L.n_expert_used, L.route_scale)


def bucket(idx, E):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    P = T * k
    out = dict(count=np.empty(E, np.int32), offset=np.empty(E + 1, np.int32), perm=np.empty(P, np.int32),
               pos=np.empty(P, np.int32), active=np.empty(E, np.int32), n_active=np.empty(1, np.int32))
    rc = _load().orc_bucket(_p(idx), T, k, E, _p(out["count"]), _p(out["offset"]), _p(out["perm"]),
                            _p(out["pos"]), _p(out["active"]), _p(out["n_active"]))
    if rc != 0:
        raise ValueError("oracle: bucket rejected its arguments")
    return out


def moe_forward(L, x=None, x_bf16=None, rows=None):
    """y [T][D] fp32 (only `rows` filled when given; the rest is NaN), idx, w."""
    mode = BF16 if x_bf16 is not None else F32
    xf = _c(x, np.float32)
    xb = _c(x_bf16, np.uint16)
    T = (xb if xb is not None else xf).shape[0]
    y = np.full((T, L.n_embd), np.nan, dtype=np.float32)
    idx = np.empty((T, L.n_expert_used), np.int32)
    w = np.empty((T, L.n_expert_used), np.float32)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    B = _Bound(L)
    rc = _load().orc_moe_forward(B.ref(), mode, _p(xf), _p(xb), T, _p(r), 0 if r is None else len(r), _p(y),
                                 _p(idx), _p(w))
    if rc != 0:
        raise ValueError("oracle: moe_forward rejected its arguments")
    return y, idx, w


def moe_forward_dense(L, x=None, x_bf16=None):
    mode = BF16 if x_bf16 is not None else F32
    xf = _c(x, np.float32)
    xb = _c(x_bf16, np.uint16)
    T = (xb if xb is not None else xf).shape[0]
    y = np.empty((T, L.n_embd), dtype=np.float32)
    B = _Bound(L)
    if _load().orc_moe_forward_dense(B.ref(), mode, _p(xf), _p(xb), T, _p(y)) != 0:
        raise ValueError("oracle: moe_forward_dense rejected its arguments")
    return y


def rmsnorm(x, gamma, eps=1e-6):
    x = _c(x, np.float32)
    g = _c(gamma, np.float32)
    T, D = x.shape
    out = np.empty_like(x)
    _load().orc_rmsnorm(_p(x), _p(g), eps, T, D, _p(out))
    return out


def count_selections(topk_idx, E, layer, counts):
    """Adds the selections of one layer's routing into counts [n_layer*E] int64 (in place)."""
    idx = _c(topk_idx, np.int32)
    assert counts.dtype == np.int64 and counts.flags.c_contiguous
    T, k = idx.shape
    _load().orc_count_selections(_p(idx), T, k, E, layer, _p(counts))
    return counts


def hotlist(counts):
    """(order, n_hot): indices by hits descending, ties by index; n_hot = positive counts."""
    c = _c(counts, np.int64)
    order = np.empty(c.shape[0], np.int32)
    n_hot = _load().orc_hotlist(_p(c), c.shape[0], _p(order))
    return order, n_hot


def swiglu(fmt_gu, fmt_down, gate, up, down, D, F, x, mode=F32, codebook=None):
    """One SwiGLU FFN on one token in double: W_down (silu(W_gate x) * W_up x)."""
    xd = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(D, dtype=np.float64)
    g, u, d = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    cb = _c(codebook, np.int8)
    if _load().orc_swiglu(fmt_gu, fmt_down, _p(g), _p(u), _p(d), _p(cb), D, F, mode, _p(xd), _p(y)) != 0:
        raise ValueError("oracle: swiglu rejected its arguments")
    return y


def stack_forward(layers, x, eps=1e-6, teacher=None):
    """x_{l+1} = x_l + MoE_l(RMSNorm_l(x_l)), the residual add in fp32.
    teacher: optional list of per-layer inputs to use instead of the oracle's
    own running x (teacher forcing); returns the list of per-layer outputs."""
    outs = []
    cur = np.ascontiguousarray(x, dtype=np.float32)
    for l, L in enumerate(layers):
        xin = cur if teacher is None else np.ascontiguousarray(teacher[l], dtype=np.float32)
        xn = rmsnorm(xin, L.gamma, eps)
        y, _, _ = moe_forward(L, x=xn)
        cur = (xin + y).astype(np.float32)
        outs.append(cur)
    return outs
