"""CPU oracle of the sparse MoE layer (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library and its binding never
load it, and it shares no code with them.

``oracle.c`` holds the arithmetic (plain loops, double accumulation); this
module builds it with gcc and marshals NumPy arrays through ctypes. Every
function cites the passage it follows in the C source.

Parity pins: every oracle function is pinned by tests in
``tests/test_oracle_pins.py`` (hand fixtures, brute-force selection, closed
forms, invariants, reductions to NumPy/IEEE library routines).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OR_F32, OR_BF16, OR_Q2, OR_Q3, OR_Q4 = 0, 1, 2, 3, 4
WTYPE = {"f32": OR_F32, "bf16": OR_BF16, "q2": OR_Q2, "q3": OR_Q3, "q4": OR_Q4}
BITS = {"q2": 2, "q3": 3, "q4": 4}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, strict IEEE, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Q2Matrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scale", C.c_void_p), ("minv", C.c_void_p)]


class Desc(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
        ("inter", C.c_int32), ("shared_inter", C.c_int32), ("renormalize", C.c_int32),
        ("router_t", C.c_int32), ("expert_t", C.c_int32), ("shared_t", C.c_int32),
        ("router_w", C.c_void_p), ("router_bias", C.c_void_p), ("gate_vec", C.c_void_p),
        ("exp_gate", C.c_void_p), ("exp_up", C.c_void_p), ("exp_down", C.c_void_p),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("bias_mode", C.c_int32), ("residual", C.c_int32), ("norm_w", C.c_void_p), ("norm_eps", C.c_double),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = build(force=False)
            L = C.CDLL(path)
            L.oracle_half_to_float.argtypes = [C.c_uint16]
            L.oracle_half_to_float.restype = C.c_float
            L.oracle_float_to_half.argtypes = [C.c_float]
            L.oracle_float_to_half.restype = C.c_uint16
            L.oracle_q2_quantize.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]
            L.oracle_q2_quantize.restype = C.c_int
            L.oracle_q2_dequantize.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p]
            L.oracle_q2_dequantize.restype = None
            L.oracle_qb_quantize.argtypes = [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                             C.c_void_p]
            L.oracle_qb_quantize.restype = C.c_int
            L.oracle_qb_dequantize.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                               C.c_void_p]
            L.oracle_qb_dequantize.restype = None
            L.oracle_route.argtypes = [C.POINTER(Desc), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p]
            L.oracle_route.restype = C.c_int
            L.oracle_layer.argtypes = [C.POINTER(Desc), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_void_p]
            L.oracle_layer.restype = C.c_int
            L.oracle_rmsnorm.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_double, C.c_void_p]
            L.oracle_rmsnorm.restype = None
            L.oracle_max_threads.restype = C.c_int
            L.oracle_set_threads.argtypes = [C.c_int]
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ fp16

def half_to_float(h: int) -> float:
    return float(lib().oracle_half_to_float(int(h)))


def float_to_half(f: float) -> int:
    return int(lib().oracle_float_to_half(float(np.float32(f))))


# -------------------------------------------------------- b-bit blocks

class Q2:
    """Logical b-bit block form of one matrix (codes [rows][cols*b/8], fp16
    scale and min bits [rows][cols/32]); b = 2 unless given."""

    def __init__(self, codes, scale, minv, rows, cols, bits=2):
        self.codes, self.scale, self.minv = codes, scale, minv
        self.rows, self.cols, self.bits = rows, cols, bits
        self.struct = Q2Matrix(codes.ctypes.data, scale.ctypes.data, minv.ctypes.data)


def qb_quantize(w: np.ndarray, bits: int) -> Q2:
    """The b-bit quantizer (oracle.c, oracle_qb_quantize)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.zeros((rows, cols * bits // 8), np.uint8)
    scale = np.zeros((rows, cols // 32), np.uint16)
    minv = np.zeros((rows, cols // 32), np.uint16)
    rc = lib().oracle_qb_quantize(bits, w.ctypes.data, rows, cols, codes.ctypes.data, scale.ctypes.data,
                                  minv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle quantizer rejected the input (non-finite or out of fp16 range)")
    return Q2(codes, scale, minv, rows, cols, bits)


def qb_dequantize(q: Q2) -> np.ndarray:
    out = np.zeros((q.rows, q.cols), np.float32)
    lib().oracle_qb_dequantize(q.bits, q.codes.ctypes.data, q.scale.ctypes.data, q.minv.ctypes.data,
                               q.rows, q.cols, out.ctypes.data)
    return out


def q2_quantize(w: np.ndarray) -> Q2:
    return qb_quantize(w, 2)


def q2_dequantize(q: Q2) -> np.ndarray:
    return qb_dequantize(q)


# ----------------------------------------------------------------- norm

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """u = fp32(x / sqrt(mean(x^2) + eps) * gamma), row by row (oracle.c,
    oracle_rmsnorm)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.reshape(-1, x.shape[-1])
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.zeros_like(rows)
    for r in range(rows.shape[0]):
        lib().oracle_rmsnorm(rows[r].ctypes.data, rows.shape[1], g.ctypes.data, float(eps), out[r].ctypes.data)
    return out.reshape(x.shape)


# ---------------------------------------------------------------- layer

class Layer:
    """Weights of one layer as the oracle reads them.

    router_w [E][H] and gate_vec [H] (f32 values or bf16 bits), optional
    router_bias [E] fp32 (bias_mode 0: in the selection and the weights; 1:
    in the selection only), per-expert matrices (a list of E arrays, or of
    ``Q2`` objects for 2-bit experts; entries may be None for experts that
    are never selected), the shared expert (f32 values or bf16 bits), and
    optionally the pre-MoE RMS norm (norm_w [H] fp32, norm_eps) and the
    residual (y = x + MoE(u)).
    """

    def __init__(self, *, H, E, K, I, Is, router_t, expert_t, shared_t, router_w, gate_vec,
                 router_bias, exp_gate, exp_up, exp_down, sh_gate, sh_up, sh_down, renormalize=1,
                 bias_mode=0, norm_w=None, norm_eps=1e-6, residual=0):
        self.H, self.E, self.K, self.I, self.Is = H, E, K, I, Is
        self._keep = []

        def arr(a, fmt):
            if a is None:
                return None
            dt = np.float32 if fmt == "f32" else np.uint16
            a = np.ascontiguousarray(a, dtype=dt)
            self._keep.append(a)
            return a

        router_w = arr(router_w, router_t)
        gate_vec = arr(gate_vec, router_t)
        if router_bias is not None:
            router_bias = np.ascontiguousarray(router_bias, dtype=np.float32)
            self._keep.append(router_bias)
        sh = [arr(m, shared_t) for m in (sh_gate, sh_up, sh_down)]
        if norm_w is not None:
            norm_w = np.ascontiguousarray(norm_w, dtype=np.float32)
            self._keep.append(norm_w)

        def table(mats):
            t = (C.c_void_p * E)()
            for e, m in enumerate(mats):
                if m is None:
                    t[e] = None
                elif isinstance(m, Q2):
                    self._keep.append(m)
                    t[e] = C.addressof(m.struct)
                else:
                    a = arr(m, expert_t)
                    t[e] = a.ctypes.data
            self._keep.append(t)
            return t

        tg, tu, td = table(exp_gate), table(exp_up), table(exp_down)
        self.desc = Desc(H, E, K, I, Is, renormalize, WTYPE[router_t], WTYPE[expert_t], WTYPE[shared_t],
                         _ptr(router_w), _ptr(router_bias), _ptr(gate_vec),
                         C.addressof(tg), C.addressof(tu), C.addressof(td),
                         _ptr(sh[0]), _ptr(sh[1]), _ptr(sh[2]), int(bias_mode), int(residual), _ptr(norm_w),
                         float(norm_eps))

    def route(self, x: np.ndarray):
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, self.H)
        T = x.shape[0]
        ids = np.zeros((T, self.K), np.int32)
        wts = np.zeros((T, self.K), np.float64)
        gate = np.zeros((T,), np.float64)
        logits = np.zeros((T, self.E), np.float64)
        rc = lib().oracle_route(C.byref(self.desc), x.ctypes.data, T, ids.ctypes.data, wts.ctypes.data,
                                gate.ctypes.data, logits.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_route failed ({rc})")
        return ids, wts, gate, logits

    def forward(self, x: np.ndarray):
        """Returns ids[T][K], wts[T][K] (double), gate[T] (double), y[T][H]
        (fp32, rounded once) and y64[T][H] (double)."""
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, self.H)
        T = x.shape[0]
        ids = np.zeros((T, self.K), np.int32)
        wts = np.zeros((T, self.K), np.float64)
        gate = np.zeros((T,), np.float64)
        y = np.zeros((T, self.H), np.float32)
        y64 = np.zeros((T, self.H), np.float64)
        rc = lib().oracle_layer(C.byref(self.desc), x.ctypes.data, T, ids.ctypes.data, wts.ctypes.data,
                                gate.ctypes.data, y.ctypes.data, y64.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_layer failed ({rc})")
        return ids, wts, gate, y, y64


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())
