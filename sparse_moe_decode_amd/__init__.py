"""Python binding of libmoe.so, the gfx950 sparse MoE layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch provides device memory and streams; tensors are passed to
the C ABI as raw pointers. There is no fallback: if the built library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EALIGN, MOE_EHIP, MOE_ENONFINITE = 0, -1, -2, -3, -4, -5, -6
MOE_F32, MOE_BF16, MOE_Q2B32, MOE_Q3B32, MOE_Q4B32 = 0, 1, 2, 3, 4
MOE_BIAS_SELECT_AND_WEIGH, MOE_BIAS_SELECT_ONLY = 0, 1
WTYPE = {"f32": MOE_F32, "bf16": MOE_BF16, "q2": MOE_Q2B32, "q3": MOE_Q3B32, "q4": MOE_Q4B32}
BITS = {"q2": 2, "q3": 3, "q4": 4}   # code width of the block formats

EXPORTS = ("moe_abi_version", "moe_strerror", "moe_workspace_bytes", "moe_route", "moe_forward",
           "moe_forward_noalloc", "moe_sort_workspace_bytes", "moe_sort_by_expert", "moe_qb_packed_bytes", "moe_qb_pack",
           "moe_qb_unpack", "moe_q2_packed_bytes", "moe_q2_pack", "moe_q2_unpack")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


class LayerDesc(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32), ("inter", C.c_int32),
        ("shared_inter", C.c_int32), ("renormalize", C.c_int32), ("router_t", C.c_int32),
        ("expert_t", C.c_int32), ("shared_t", C.c_int32), ("bias_mode", C.c_int32),
        ("router_w", C.c_void_p), ("router_bias", C.c_void_p), ("shared_gate_w", C.c_void_p),
        ("exp_gate", C.c_void_p), ("exp_up", C.c_void_p), ("exp_down", C.c_void_p),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("norm_w", C.c_void_p), ("norm_eps", C.c_float), ("residual", C.c_int32), ("reserved", C.c_int64),
    ]


_lock = threading.Lock()
_lib = None


def lib():
    """Load libmoe.so (built in-tree by ``sparse_moe_decode_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_moe_decode_amd.build`")
            L = C.CDLL(LIB_PATH)
            vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
            L.moe_abi_version.restype = C.c_uint32
            L.moe_strerror.argtypes = [C.c_int]
            L.moe_strerror.restype = C.c_char_p
            L.moe_workspace_bytes.argtypes = [C.POINTER(LayerDesc), i32]
            L.moe_workspace_bytes.restype = sz
            L.moe_route.argtypes = [C.POINTER(LayerDesc), vp, i32, vp, vp, vp, vp, sz, vp]
            L.moe_route.restype = C.c_int
            L.moe_forward.argtypes = [C.POINTER(LayerDesc), vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            L.moe_forward.restype = C.c_int
            L.moe_forward_noalloc.argtypes = [C.POINTER(LayerDesc), vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
            L.moe_forward_noalloc.restype = C.c_int
            L.moe_sort_workspace_bytes.argtypes = [i32, i32, i32]
            L.moe_sort_workspace_bytes.restype = sz
            L.moe_sort_by_expert.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
            L.moe_sort_by_expert.restype = C.c_int
            L.moe_qb_packed_bytes.argtypes = [i32, i64, i64]
            L.moe_qb_packed_bytes.restype = sz
            L.moe_qb_pack.argtypes = [i32, vp, i64, i64, vp, sz]
            L.moe_qb_pack.restype = C.c_int
            L.moe_qb_unpack.argtypes = [i32, vp, i64, i64, vp, vp]
            L.moe_qb_unpack.restype = C.c_int
            L.moe_q2_packed_bytes.argtypes = [i64, i64]
            L.moe_q2_packed_bytes.restype = sz
            L.moe_q2_pack.argtypes = [vp, i64, i64, vp, sz]
            L.moe_q2_pack.restype = C.c_int
            L.moe_q2_unpack.argtypes = [vp, i64, i64, vp, vp]
            L.moe_q2_unpack.restype = C.c_int
            _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != MOE_OK:
        raise MoEError(rc, where)


def abi_version() -> int:
    return int(lib().moe_abi_version())


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


# ------------------------------------------------------------ packer (host)

def qb_packed_bytes(bits: int, rows: int, cols: int) -> int:
    return int(lib().moe_qb_packed_bytes(bits, rows, cols))


def qb_pack(bits: int, w: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Pack an fp32 [rows][cols] matrix (host) into the b-bit block format."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w: expected a 2-D matrix")
    rows, cols = w.shape
    n = qb_packed_bytes(bits, rows, cols)
    if n == 0:
        raise MoEError(MOE_EINVAL, "moe_qb_pack")
    if out is None:
        out = np.empty(n, np.uint8)
    if not (out.dtype == np.uint8 and out.flags.c_contiguous and out.nbytes >= n):
        raise ValueError("out: expected a contiguous uint8 buffer of moe_qb_packed_bytes bytes")
    _check(lib().moe_qb_pack(bits, w.ctypes.data, rows, cols, out.ctypes.data, out.nbytes), "moe_qb_pack")
    return out


def q2_packed_bytes(rows: int, cols: int) -> int:
    return int(lib().moe_q2_packed_bytes(rows, cols))


def q2_pack(w: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Pack an fp32 [rows][cols] matrix (host) into the 2-bit block format."""
    return qb_pack(2, w, out)


# --------------------------------------------------------------- device calls

def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def workspace_bytes(desc: LayerDesc, T: int) -> int:
    return int(lib().moe_workspace_bytes(C.byref(desc), T))


def _want(t, name, dtype, shape):
    """Host-side checks of a tensor handed to the C ABI as a raw pointer: its
    dtype, shape and contiguity, then that it lives on the GPU."""
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: on {t.device}, expected a GPU tensor")


def _check_ws(ws):
    import torch
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous() or not ws.is_cuda:
        raise ValueError("ws: expected a contiguous GPU tensor")


def _check_rows(desc: LayerDesc, x, y=None, ids=None, wts=None, gate=None, **more):
    import torch
    if x is None or x.dim() != 2:
        raise ValueError("x: expected a [T, hidden] tensor")
    T = x.shape[0]
    H, K = desc.hidden, desc.top_k
    _want(x, "x", torch.float32, (T, H))
    _want(y, "y", torch.float32, (T, H))
    _want(ids, "ids", torch.int32, (T, K))
    _want(wts, "wts", torch.float32, (T, K))
    _want(gate, "gate", torch.float32, (T,))
    for name, t in more.items():
        kind = name.split("_")[0]
        _want(t, name, torch.int32 if kind == "ids" else torch.float32, (T,) if kind == "gate" else (T, K))
    _on_gpu(x=x, y=y, ids=ids, wts=wts, gate=gate, **more)
    return T


def route(desc: LayerDesc, x, ids, wts, gate, ws, stream=None) -> None:
    T = _check_rows(desc, x, ids=ids, wts=wts, gate=gate)
    for name, t in (("ids", ids), ("wts", wts), ("gate", gate)):
        if t is None:
            raise ValueError(f"{name}: required")
    _check_ws(ws)
    _check(lib().moe_route(C.byref(desc), _ptr(x), T, _ptr(ids), _ptr(wts), _ptr(gate), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "moe_route")


def forward(desc: LayerDesc, x, y, ws, ids_in=None, wts_in=None, gate_in=None, ids_out=None, wts_out=None,
            gate_out=None, stream=None) -> None:
    T = _check_rows(desc, x, y, ids_in=ids_in, wts_in=wts_in, gate_in=gate_in, ids_out=ids_out,
                    wts_out=wts_out, gate_out=gate_out)
    if y is None:
        raise ValueError("y: required")
    _check_ws(ws)
    _check(lib().moe_forward(C.byref(desc), _ptr(x), T, _ptr(y), _ptr(ids_in), _ptr(wts_in), _ptr(gate_in),
                             _ptr(ids_out), _ptr(wts_out), _ptr(gate_out), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


NOALLOC_SCRATCH_BYTES = 8 << 20    # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def forward_noalloc(desc: LayerDesc, x, y, ids_in=None, wts_in=None, gate_in=None, ids_out=None, wts_out=None,
                    gate_out=None, stream=None) -> None:
    """moe_forward_noalloc: the layer on the library's own per-GPU scratch
    (no workspace argument, nothing allocated by the call)."""
    T = _check_rows(desc, x, y, ids_in=ids_in, wts_in=wts_in, gate_in=gate_in, ids_out=ids_out,
                    wts_out=wts_out, gate_out=gate_out)
    if y is None:
        raise ValueError("y: required")
    _check(lib().moe_forward_noalloc(C.byref(desc), _ptr(x), T, _ptr(y), _ptr(ids_in), _ptr(wts_in), _ptr(gate_in),
                                     _ptr(ids_out), _ptr(wts_out), _ptr(gate_out), _stream(stream)),
           "moe_forward_noalloc")


def sort_workspace_bytes(T: int, K: int, E: int) -> int:
    return int(lib().moe_sort_workspace_bytes(T, K, E))


def sort_by_expert(ids, E: int, counts, offsets, perm, ws, stream=None) -> None:
    import torch
    if ids is None or ids.dim() != 2:
        raise ValueError("ids: expected a [T, K] tensor")
    T, K = ids.shape
    _want(ids, "ids", torch.int32, (T, K))
    _want(counts, "counts", torch.int32, (E,))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(perm, "perm", torch.int32, (T * K,))
    _on_gpu(ids=ids, counts=counts, offsets=offsets, perm=perm)
    _check_ws(ws)
    _check(lib().moe_sort_by_expert(_ptr(ids), T, K, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), "moe_sort_by_expert")


def qb_unpack(bits: int, packed, rows: int, cols: int, dst, stream=None) -> None:
    import torch
    _want(dst, "dst", torch.float32, (rows, cols))
    _on_gpu(dst=dst)
    if packed.numel() * packed.element_size() < qb_packed_bytes(bits, rows, cols) or not packed.is_contiguous() \
            or not packed.is_cuda:
        raise ValueError("packed: expected a contiguous GPU buffer of moe_qb_packed_bytes(bits, rows, cols) bytes")
    _check(lib().moe_qb_unpack(bits, _ptr(packed), rows, cols, _ptr(dst), _stream(stream)), "moe_qb_unpack")


def q2_unpack(packed, rows: int, cols: int, dst, stream=None) -> None:
    qb_unpack(2, packed, rows, cols, dst, stream)


# ------------------------------------------------------------- layer holder

class Layer:
    """Device-resident weights of one layer and its descriptor.

    Built from host arrays (fp32 values, bf16 bit patterns as uint16, or fp32
    sources of 2-, 3- or 4-bit experts which are packed here by the library
    packer).
    """

    def __init__(self, *, H, E, K, I, Is, router_t, expert_t, shared_t, router_w, gate_vec, router_bias,
                 sh_gate, sh_up, sh_down, exp_gate=None, exp_up=None, exp_down=None, expert_source=None,
                 renormalize=1, bias_mode=0, norm_w=None, norm_eps=1e-6, residual=0, device="cuda"):
        import torch
        self.H, self.E, self.K, self.I, self.Is = H, E, K, I, Is
        self.router_t, self.expert_t, self.shared_t = router_t, expert_t, shared_t
        self.device = device

        def up(a, fmt=None):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            if fmt == "bf16" or a.dtype == np.uint16:
                t = torch.from_numpy(a.view(np.int16)).to(device)
            else:
                t = torch.from_numpy(a).to(device)
            return t

        self.router_w = up(router_w, router_t)
        self.gate_vec = up(gate_vec, router_t)
        self.router_bias = up(None if router_bias is None else np.asarray(router_bias, np.float32))
        self.norm_w = up(None if norm_w is None else np.asarray(norm_w, np.float32))
        self.sh_gate, self.sh_up, self.sh_down = up(sh_gate), up(sh_up), up(sh_down)
        if expert_t in BITS:
            # expert_source(e, mat) -> fp32 [rows][cols]; mat 0 gate, 1 up, 2 down
            self.exp_gate = self._pack_stack(expert_source, 0, I, H)
            self.exp_up = self._pack_stack(expert_source, 1, I, H)
            self.exp_down = self._pack_stack(expert_source, 2, H, I)
        else:
            self.exp_gate, self.exp_up, self.exp_down = up(exp_gate), up(exp_up), up(exp_down)
        self.desc = LayerDesc(H, E, K, I, Is, renormalize, WTYPE[router_t], WTYPE[expert_t], WTYPE[shared_t],
                              int(bias_mode), _ptr(self.router_w), _ptr(self.router_bias), _ptr(self.gate_vec),
                              _ptr(self.exp_gate), _ptr(self.exp_up), _ptr(self.exp_down),
                              _ptr(self.sh_gate), _ptr(self.sh_up), _ptr(self.sh_down), _ptr(self.norm_w),
                              float(norm_eps), int(residual), 0)

    def with_dense(self, *, router_w, gate_vec, router_bias, sh_gate, sh_up, sh_down, norm_w=None) -> "Layer":
        """Another layer of the same shape that shares this layer's routed
        experts but has its own router, gate vector, shared expert (and norm
        gamma, when this layer has a norm)."""
        import torch
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)

        def up(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(self.device)

        other.router_w, other.gate_vec = up(router_w), up(gate_vec)
        other.router_bias = up(None if router_bias is None else np.asarray(router_bias, np.float32))
        other.sh_gate, other.sh_up, other.sh_down = up(sh_gate), up(sh_up), up(sh_down)
        if norm_w is not None:
            other.norm_w = up(np.asarray(norm_w, np.float32))
        d = LayerDesc()
        C.memmove(C.byref(d), C.byref(self.desc), C.sizeof(LayerDesc))
        d.router_w, d.shared_gate_w = _ptr(other.router_w), _ptr(other.gate_vec)
        d.router_bias = _ptr(other.router_bias)
        d.norm_w = _ptr(other.norm_w)
        d.sh_gate, d.sh_up, d.sh_down = _ptr(other.sh_gate), _ptr(other.sh_up), _ptr(other.sh_down)
        other.desc = d
        return other

    def with_expert_copies(self) -> "Layer":
        """The same layer with its routed expert stacks copied to new device
        memory (identical bytes at other addresses), so that layers rotated in
        a benchmark do not share cached expert lines."""
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)
        other.exp_gate, other.exp_up, other.exp_down = (t.clone() for t in (self.exp_gate, self.exp_up,
                                                                            self.exp_down))
        d = LayerDesc()
        C.memmove(C.byref(d), C.byref(self.desc), C.sizeof(LayerDesc))
        d.exp_gate, d.exp_up, d.exp_down = _ptr(other.exp_gate), _ptr(other.exp_up), _ptr(other.exp_down)
        other.desc = d
        return other

    def _pack_stack(self, source, mat, rows, cols):
        import torch
        from concurrent.futures import ThreadPoolExecutor
        bits = BITS[self.expert_t]
        n = qb_packed_bytes(bits, rows, cols)
        host = np.empty((self.E, n), np.uint8)

        def one(e):
            qb_pack(bits, source(e, mat), out=host[e])

        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(one, range(self.E)))
        return torch.from_numpy(host).to(self.device)

    def workspace(self, T: int):
        import torch
        n = workspace_bytes(self.desc, T)
        if n == 0:
            raise MoEError(MOE_EINVAL, "moe_workspace_bytes")
        # no initialization is needed; arbitrary bytes keep that property tested
        return torch.full(((n + 15) // 16 * 16,), 0xA5, dtype=torch.uint8, device=self.device)

    def forward(self, x, y=None, ws=None, routing=None, want_routing=False, stream=None):
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace(T)
        ids = wts = gate = None
        if want_routing:
            ids = torch.empty((T, self.K), dtype=torch.int32, device=self.device)
            wts = torch.empty((T, self.K), dtype=torch.float32, device=self.device)
            gate = torch.empty((T,), dtype=torch.float32, device=self.device)
        if routing is not None:
            forward(self.desc, x, y, ws, ids_in=routing[0], wts_in=routing[1], gate_in=routing[2], stream=stream)
        else:
            forward(self.desc, x, y, ws, ids_out=ids, wts_out=wts, gate_out=gate, stream=stream)
        return (y, ids, wts, gate) if want_routing else y

    def route(self, x, ws=None, stream=None):
        import torch
        T = x.shape[0]
        ids = torch.empty((T, self.K), dtype=torch.int32, device=self.device)
        wts = torch.empty((T, self.K), dtype=torch.float32, device=self.device)
        gate = torch.empty((T,), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace(T)
        route(self.desc, x, ids, wts, gate, ws, stream=stream)
        return ids, wts, gate
