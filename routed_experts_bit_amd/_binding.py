"""ctypes binding of librl_moe.so (C ABI: include/rl_moe.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "librl_moe.so")

RL_OK = 0
RL_QTYPE_Q2B = 1
RL_QTYPE_T1 = 2

# every entry point declared in include/rl_moe.h
EXPORTS = (
    "rl_moe_workspace_bytes",
    "rl_moe_prefill",
    "rl_moe_prefill_timed",
    "rl_moe_decode",
    "rl_moe_group_pairs",
    "rl_moe_dequant",
    "rl_moe_gate_up",
    "rl_moe_route",
    "rl_moe_status",
    "rl_moe_strerror",
)


class RlError(RuntimeError):
    pass


class _Blobs(C.Structure):
    _fields_ = [
        ("arena", C.c_void_p),
        ("desc", C.c_void_p),
        ("desc_host", C.c_void_p),
        ("E", C.c_int32),
        ("H", C.c_int32),
        ("I", C.c_int32),
    ]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load librl_moe.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RlError(f"{_LIB_PATH} is missing: build it with `python -m routed_experts_bit_amd.build`")
    L = C.CDLL(_LIB_PATH)
    P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
    L.rl_moe_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    L.rl_moe_workspace_bytes.restype = SZ
    layer = [P, P, P, C.POINTER(_Blobs), P, I32, I32, P, SZ, P]
    for name in ("rl_moe_prefill", "rl_moe_decode", "rl_moe_gate_up"):
        getattr(L, name).argtypes = layer
        getattr(L, name).restype = C.c_int
    L.rl_moe_prefill_timed.argtypes = layer + [C.POINTER(C.c_void_p)]
    L.rl_moe_prefill_timed.restype = C.c_int
    L.rl_moe_group_pairs.argtypes = [P, I32, I32, I32, P, P, P, P, SZ, P]
    L.rl_moe_group_pairs.restype = C.c_int
    L.rl_moe_dequant.argtypes = [I32, P, C.c_int64, P, P]
    L.rl_moe_dequant.restype = C.c_int
    L.rl_moe_route.argtypes = [P, I32, I32, I32, P, P, P]
    L.rl_moe_route.restype = C.c_int
    L.rl_moe_status.argtypes = [P, P]
    L.rl_moe_status.restype = C.c_int
    L.rl_moe_strerror.argtypes = [C.c_int]
    L.rl_moe_strerror.restype = C.c_char_p
    _lib = L
    return L


def exported_symbols():
    L = lib()
    return {name: hasattr(L, name) for name in EXPORTS}


def strerror(code: int) -> str:
    return lib().rl_moe_strerror(int(code)).decode()


def _check(rc: int, what: str):
    if rc != RL_OK:
        raise RlError(f"{what}: {strerror(rc)} ({rc})")


def _torch():
    import torch

    return torch


def _stream():
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


class DeviceExperts:
    """Packed experts resident on the GPU: arena (uint8) and descriptors, plus the host copy
    of the descriptors that the library reads to choose its type-specialised kernels."""

    def __init__(self, arena_u8, desc_np: np.ndarray, E: int, H: int, I: int, device="cuda"):
        torch = _torch()
        self.E, self.H, self.I = int(E), int(H), int(I)
        if isinstance(arena_u8, np.ndarray):
            n = arena_u8.size
            buf = torch.empty((n + 3) // 4 * 4, dtype=torch.uint8, device=device)
            buf[:n].copy_(torch.from_numpy(np.ascontiguousarray(arena_u8)))
            self.arena = buf
        else:
            self.arena = arena_u8
        self.desc_host = np.ascontiguousarray(desc_np)
        self.desc = torch.from_numpy(self.desc_host.view(np.uint8).copy()).to(device)
        self._blobs = _Blobs(self.arena.data_ptr(), self.desc.data_ptr(), self.desc_host.ctypes.data, self.E, self.H,
                             self.I)

    @classmethod
    def from_workload(cls, experts, device="cuda"):
        return cls(experts.arena, experts.desc, experts.E, experts.H, experts.I, device=device)

    def with_arena(self, arena):
        """Same descriptors over another arena copy (another address, same content)."""
        other = DeviceExperts.__new__(DeviceExperts)
        other.E, other.H, other.I = self.E, self.H, self.I
        other.arena, other.desc_host, other.desc = arena, self.desc_host, self.desc
        other._blobs = _Blobs(arena.data_ptr(), self.desc.data_ptr(), self.desc_host.ctypes.data, self.E, self.H, self.I)
        return other

    @property
    def blobs(self):
        return C.byref(self._blobs)


def workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    n = lib().rl_moe_workspace_bytes(T, k, E, H, I)
    if n == 0:
        raise RlError(f"unsupported sizes T={T} k={k} E={E} H={H} I={I}")
    return int(n)


def alloc_workspace(T: int, k: int, ex: DeviceExperts, device="cuda"):
    torch = _torch()
    n = workspace_bytes(max(T, 1), k, ex.E, ex.H, ex.I)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _layer(fn, x, ids, w, ex: DeviceExperts, out, ws):
    T, k = ids.shape
    rc = fn(_ptr(x), _ptr(ids), _ptr(w), ex.blobs, _ptr(out), T, k, _ptr(ws), ws.numel() if ws is not None else 0,
            _stream())
    return rc


def prefill(x, ids, w, ex: DeviceExperts, out=None, ws=None):
    """x: bf16 [T,H] (torch.bfloat16 or int16 bits), ids int32 [T,k], w float32 [T,k] -> float32 [T,H]."""
    torch = _torch()
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=ids.device)
    if ws is None:
        ws = alloc_workspace(T, ids.shape[1], ex, device=ids.device)
    _check(_layer(lib().rl_moe_prefill, x, ids, w, ex, out, ws), "rl_moe_prefill")
    return out


TIMED_EVENTS = 6  # RL_TIMED_EVENTS


def prefill_timed(x, ids, w, ex: DeviceExperts, out, ws, events):
    """rl_moe_prefill with TIMED_EVENTS torch.cuda.Event (enable_timing) recorded between its
    kernels: grouping (which also splits x) | gate/up | h split | down | combine."""
    T, k = ids.shape
    if len(events) != TIMED_EVENTS:
        raise RlError(f"prefill_timed needs {TIMED_EVENTS} events")
    arr = (C.c_void_p * TIMED_EVENTS)(*[C.c_void_p(e.cuda_event) for e in events])
    rc = lib().rl_moe_prefill_timed(_ptr(x), _ptr(ids), _ptr(w), ex.blobs, _ptr(out), T, k, _ptr(ws), ws.numel(),
                                    _stream(), arr)
    _check(rc, "rl_moe_prefill_timed")
    return out


def decode(x, ids, w, ex: DeviceExperts, out=None, ws=None):
    torch = _torch()
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=ids.device)
    if ws is None:
        ws = alloc_workspace(T, ids.shape[1], ex, device=ids.device)
    _check(_layer(lib().rl_moe_decode, x, ids, w, ex, out, ws), "rl_moe_decode")
    return out


def gate_up(x, ids, w, ex: DeviceExperts, h=None, ws=None):
    """h (fp16 bits as int16) [T*k, I] in sorted-pair order."""
    torch = _torch()
    T, k = ids.shape
    if h is None:
        h = torch.empty((T * k, ex.I), dtype=torch.int16, device=ids.device)
    if ws is None:
        ws = alloc_workspace(T, k, ex, device=ids.device)
    _check(_layer(lib().rl_moe_gate_up, x, ids, w, ex, h, ws), "rl_moe_gate_up")
    return h


def group_pairs(ids, E: int):
    """Returns (offsets[E+1], pair_src[T*k], inv[T*k], workspace) as device tensors; the
    workspace holds the status flags (see status())."""
    torch = _torch()
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pair_src = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(workspace_bytes(max(T, 1), k, E, 256, 64), dtype=torch.uint8, device=dev)
    rc = lib().rl_moe_group_pairs(_ptr(ids), T, k, E, _ptr(offsets), _ptr(pair_src), _ptr(inv), _ptr(ws), ws.numel(),
                                  _stream())
    _check(rc, "rl_moe_group_pairs")
    return offsets, pair_src[: T * k], inv[: T * k], ws


def dequant(qtype: int, blocks_u8, n_values: int, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty(max(n_values, 1), dtype=torch.float32, device=blocks_u8.device)
    _check(lib().rl_moe_dequant(int(qtype), _ptr(blocks_u8), int(n_values), _ptr(out), _stream()), "rl_moe_dequant")
    return out[:n_values]


def route(logits, k: int, ids=None, w=None):
    """Router on the GPU: (topk_ids int32 [T, k], topk_w float32 [T, k]) from fp32 logits [T, E]."""
    torch = _torch()
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().rl_moe_route(_ptr(logits), T, E, int(k), _ptr(ids), _ptr(w), _stream()), "rl_moe_route")
    return ids, w


def status(ws):
    """Device status flags of the last call on `ws` (synchronises the current stream)."""
    torch = _torch()
    torch.cuda.current_stream().synchronize()
    buf = (C.c_int32 * 4)()
    _check(lib().rl_moe_status(_ptr(ws), C.cast(buf, C.c_void_p)), "rl_moe_status")
    return list(buf)
