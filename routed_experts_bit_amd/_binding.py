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
RL_DEC_STRIP = 0
RL_DEC_MFMA_GATEUP = 1
RL_DEC_MFMA_DOWN = 2
RL_DEC_ROWS_GATEUP = 3
RL_DEC_ROWS_DOWN = 4
_BLOCK_BYTES = {RL_QTYPE_Q2B: 74, RL_QTYPE_T1: 57}

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
    "rl_moe_prefill_noalloc",
    "rl_moe_noalloc_status",
    "rl_moe_prefill_block",
    "rl_moe_decode_block",
    "rl_moe_prefill_from_logits",
)
# the bounded expert cache (include/rl_moe.h, rl_cache_*)
CACHE_EXPORTS = (
    "rl_cache_slot_bytes",
    "rl_cache_create",
    "rl_cache_prepare",
    "rl_cache_stats",
    "rl_cache_slot_of",
    "rl_cache_destroy",
)
NOALLOC_SCRATCH_BYTES = 40 << 20  # RL_NOALLOC_SCRATCH_BYTES


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
        ("arena_bytes", C.c_uint64),
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
    for name in ("rl_moe_prefill", "rl_moe_decode"):
        getattr(L, name).argtypes = layer
        getattr(L, name).restype = C.c_int
    L.rl_moe_gate_up.argtypes = [P, P, P, C.POINTER(_Blobs), P, P, P, I32, I32, P, SZ, P]
    L.rl_moe_gate_up.restype = C.c_int
    for name in ("rl_moe_prefill_block", "rl_moe_decode_block"):
        getattr(L, name).argtypes = [P, P, P, C.POINTER(_Blobs), I32, P, P, P, I32, I32, P, SZ, P]
        getattr(L, name).restype = C.c_int
    L.rl_moe_prefill_from_logits.argtypes = [P, P, I32, C.POINTER(_Blobs), I32, P, P, P, P, P, I32, I32, P, SZ, P]
    L.rl_moe_prefill_from_logits.restype = C.c_int
    L.rl_moe_prefill_noalloc.argtypes = [P, P, P, C.POINTER(_Blobs), P, I32, I32, P]
    L.rl_moe_prefill_noalloc.restype = C.c_int
    L.rl_moe_noalloc_status.argtypes = [P]
    L.rl_moe_noalloc_status.restype = C.c_int
    L.rl_moe_prefill_timed.argtypes = layer + [C.POINTER(C.c_void_p)]
    L.rl_moe_prefill_timed.restype = C.c_int
    L.rl_moe_group_pairs.argtypes = [P, I32, I32, I32, P, P, P, P, SZ, P]
    L.rl_moe_group_pairs.restype = C.c_int
    L.rl_moe_dequant.argtypes = [I32, I32, P, C.c_int64, P, P]
    L.rl_moe_dequant.restype = C.c_int
    L.rl_moe_route.argtypes = [P, I32, I32, I32, P, P, P]
    L.rl_moe_route.restype = C.c_int
    L.rl_cache_slot_bytes.argtypes = [I32, I32]
    L.rl_cache_slot_bytes.restype = C.c_uint64
    L.rl_cache_create.argtypes = [P, C.c_uint64, P, I32, I32, I32, P, I32, P, C.POINTER(C.c_void_p)]
    L.rl_cache_create.restype = C.c_int
    L.rl_cache_prepare.argtypes = [P, P, I32, C.POINTER(_Blobs), P]
    L.rl_cache_prepare.restype = C.c_int
    L.rl_cache_stats.argtypes = [P, P]
    L.rl_cache_stats.restype = C.c_int
    L.rl_cache_slot_of.argtypes = [P, I32]
    L.rl_cache_slot_of.restype = I32
    L.rl_cache_destroy.argtypes = [P]
    L.rl_cache_destroy.restype = None
    L.rl_moe_status.argtypes = [P, P]
    L.rl_moe_status.restype = C.c_int
    L.rl_moe_strerror.argtypes = [C.c_int]
    L.rl_moe_strerror.restype = C.c_char_p
    _lib = L
    return L


def exported_symbols():
    L = lib()
    return {name: hasattr(L, name) for name in EXPORTS + CACHE_EXPORTS}


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


def _need(name, t, dtypes, shape=None, device=None):
    """Raise RlError unless `t` is a contiguous CUDA tensor of one of `dtypes`, of `shape` (None
    entries match any size) and on `device`; the library reads and writes these buffers as dense
    arrays of exactly that layout."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise RlError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise RlError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(want is not None and got != want for got, want in zip(t.shape, shape)):
            raise RlError(f"{name}: shape {tuple(t.shape)}, expected {tuple('*' if v is None else v for v in shape)}")
    if not t.is_contiguous():
        raise RlError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise RlError(f"{name}: must be on a CUDA (HIP) device, is on {t.device}")
    if device is not None and t.device != device:
        raise RlError(f"{name}: on {t.device}, the call's other buffers are on {device}")
    return t


def _dt():
    torch = _torch()
    return dict(x=(torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16),
                ids=(torch.int32,), w=(torch.float32,), out=(torch.float32,), ws=(torch.uint8,))


def _check_layer_args(x, ids, w, ex, out, ws, rows=None):
    """Shapes of one layer call: x [T, H] bf16 bits, ids int32 [T, k], w float32 [T, k], out
    float32 [T, H], ws a uint8 buffer of at least workspace_bytes(T, k, ...) bytes."""
    d = _dt()
    _need("topk_ids", ids, d["ids"], (None, None))
    T, k = ids.shape
    if rows is not None and T not in rows:
        raise RlError(f"topk_ids: {T} rows, expected one of {rows}")
    dev = ids.device
    _need("x", x, d["x"], (T, ex.H), dev)
    _need("topk_w", w, d["w"], (T, k), dev)
    if out is not None:
        _need("out", out, d["out"], (T, ex.H), dev)
    _need("workspace", ws, d["ws"], (None,), dev)
    if ex.arena.device != dev or ex.desc.device != dev:
        raise RlError(f"experts: on {ex.arena.device}, the call's buffers are on {dev}")
    need = workspace_bytes(max(T, 1), k, ex.E, ex.H, ex.I)
    if ws.numel() < need:
        raise RlError(f"workspace: {ws.numel()} bytes, the call needs {need}")
    return T, k


class DeviceExperts:
    """Packed experts resident on the GPU: arena (uint8) and descriptors, plus the host copy
    of the descriptors that the library reads to choose its type-specialised kernels.  Every
    descriptor is checked against the arena here (block type known, offsets dword-aligned, each
    matrix inside the arena); the library checks the same again on every call."""

    def __init__(self, arena_u8, desc_np: np.ndarray, E: int, H: int, I: int, device="cuda"):
        torch = _torch()
        self.E, self.H, self.I = int(E), int(H), int(I)
        if isinstance(arena_u8, np.ndarray):
            _check_descriptors(np.ascontiguousarray(desc_np), self.E, self.H, self.I, arena_u8.size)
            _check_t1_digit_bytes(arena_u8, desc_np, self.H, self.I)
            n = arena_u8.size
            buf = torch.zeros((n + 3) // 4 * 4, dtype=torch.uint8, device=device)
            buf[:n].copy_(torch.from_numpy(np.ascontiguousarray(arena_u8)))
            self.arena = buf
        else:
            self.arena = _need("arena", arena_u8, (torch.uint8,), (None,))
        self.desc_host = np.ascontiguousarray(desc_np)
        _check_descriptors(self.desc_host, self.E, self.H, self.I, self.arena.numel())
        self.desc = torch.from_numpy(self.desc_host.view(np.uint8).copy()).to(self.arena.device)
        self._blobs = _Blobs(self.arena.data_ptr(), self.desc.data_ptr(), self.desc_host.ctypes.data, self.E, self.H,
                             self.I, self.arena.numel())

    @classmethod
    def from_workload(cls, experts, device="cuda"):
        return cls(experts.arena, experts.desc, experts.E, experts.H, experts.I, device=device)

    def with_arena(self, arena):
        """Same descriptors over another arena copy (another address, same content)."""
        torch = _torch()
        _need("arena", arena, (torch.uint8,), (None,))
        if arena.numel() < self.arena.numel():
            raise RlError("with_arena: the copy is smaller than the arena the descriptors were checked against")
        other = DeviceExperts.__new__(DeviceExperts)
        other.E, other.H, other.I = self.E, self.H, self.I
        other.arena, other.desc_host, other.desc = arena, self.desc_host, self.desc
        other._blobs = _Blobs(arena.data_ptr(), self.desc.data_ptr(), self.desc_host.ctypes.data, self.E, self.H, self.I,
                              arena.numel())
        return other

    @property
    def blobs(self):
        return C.byref(self._blobs)

    @property
    def qtypes(self) -> np.ndarray:
        return self.desc_host["qtype"]


def _check_descriptors(desc: np.ndarray, E: int, H: int, I: int, arena_bytes: int):
    if desc.shape != (E,) or desc.dtype.itemsize != 32:
        raise RlError(f"descriptors: expected {E} records of 32 bytes, got {desc.shape} x {desc.dtype.itemsize}")
    if H <= 0 or I <= 0 or (H * I) % 256:
        raise RlError(f"experts: H={H} I={I} do not tile into 256-value blocks")
    for e in range(E):
        q = int(desc["qtype"][e])
        if q not in _BLOCK_BYTES:
            raise RlError(f"expert {e}: unknown block type {q}")
        mb = H * I // 256 * _BLOCK_BYTES[q]
        for which in ("gate_off", "up_off", "down_off"):
            off = int(desc[which][e])
            if off % 4 or off + mb > arena_bytes:
                raise RlError(f"expert {e}: {which} {off} (+{mb} bytes) is not a dword-aligned matrix inside the "
                              f"{arena_bytes}-byte arena")


def _check_t1_digit_bytes(arena: np.ndarray, desc: np.ndarray, H: int, I: int):
    """T1 digit bytes hold five base-3 digits, so a valid byte is at most 242.  The kernels do not
    check (a larger byte decodes as five zero weights); an arena given as host memory is checked
    here once, before it is copied to the device."""
    bb = _BLOCK_BYTES[RL_QTYPE_T1]
    nb = H * I // 256
    flat = np.ascontiguousarray(arena).reshape(-1)
    for e in np.nonzero(desc["qtype"] == RL_QTYPE_T1)[0]:
        for which in ("gate_off", "up_off", "down_off"):
            off = int(desc[which][e])
            blocks = flat[off:off + nb * bb].reshape(nb, bb)
            bad = np.nonzero((blocks[:, 5:] > 242).any(axis=1))[0]
            if bad.size:
                b = int(bad[0])
                v = int(blocks[b, 5:].max())
                raise RlError(f"expert {int(e)}: {which[:-4]} block {b} holds the T1 digit byte {v} (at most 242)")


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
    _need("topk_ids", ids, (torch.int32,), (None, None))
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=ids.device)
    if ws is None:
        ws = alloc_workspace(T, ids.shape[1], ex, device=ids.device)
    _check_layer_args(x, ids, w, ex, out, ws)
    _check(_layer(lib().rl_moe_prefill, x, ids, w, ex, out, ws), "rl_moe_prefill")
    return out


def prefill_block(x, ids, w, ex: DeviceExperts, shared: int, gate, residual=None, out=None, ws=None):
    """The MoE block (rl_moe_prefill_block): routed experts in selection order, then the shared
    expert `shared` (a descriptor index) weighted by gate float32 [T], then residual float32 [T, H]
    (None: none).  ids int32 [T, k] / w float32 [T, k] may have k = 0 columns."""
    return _block(lib().rl_moe_prefill_block, "rl_moe_prefill_block", x, ids, w, ex, shared, gate, residual, out, ws)


def decode_block(x, ids, w, ex: DeviceExperts, shared: int, gate, residual=None, out=None, ws=None):
    """rl_moe_decode_block: the MoE block for 1 or 2 rows on the matrix-vector kernels."""
    if ids.shape[0] not in (1, 2):
        raise RlError(f"decode_block: {ids.shape[0]} rows, expected 1 or 2")
    return _block(lib().rl_moe_decode_block, "rl_moe_decode_block", x, ids, w, ex, shared, gate, residual, out, ws)


def _block(fn, name, x, ids, w, ex, shared, gate, residual, out, ws):
    torch = _torch()
    _need("topk_ids", ids, (torch.int32,), (None, None))
    T, k = ids.shape
    dev = ids.device
    d = _dt()
    _need("x", x, d["x"], (T, ex.H), dev)
    _need("topk_w", w, d["w"], (T, k), dev)
    _need("shared_gate", gate, (torch.float32,), (T,), dev)
    if residual is not None:
        _need("residual", residual, (torch.float32,), (T, ex.H), dev)
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=dev)
    _need("out", out, d["out"], (T, ex.H), dev)
    if ws is None:
        ws = torch.empty(workspace_bytes(max(T, 1), k + 1, ex.E, ex.H, ex.I), dtype=torch.uint8, device=dev)
    _need("workspace", ws, d["ws"], (None,), dev)
    rc = fn(_ptr(x), _ptr(ids) if k else None, _ptr(w) if k else None, ex.blobs, int(shared), _ptr(gate),
            _ptr(residual), _ptr(out), T, k, _ptr(ws), ws.numel(), _stream())
    _check(rc, name)
    return out


def prefill_from_logits(x, logits, k: int, ex: DeviceExperts, shared: int = -1, gate=None, residual=None, out=None,
                        ids=None, w=None, ws=None):
    """rl_moe_prefill_from_logits: route every token among the first logits.shape[1] experts (fp32
    logits [T, n_route]) in the grouping's first launch, then the layer (with shared >= 0 the MoE
    block).  Returns (out float32 [T, H], topk_ids int32 [T, k], topk_w float32 [T, k])."""
    torch = _torch()
    _need("logits", logits, (torch.float32,), (None, None))
    T, n_route = logits.shape
    dev = logits.device
    d = _dt()
    _need("x", x, d["x"], (T, ex.H), dev)
    kk = k + (1 if shared >= 0 else 0)
    if shared >= 0:
        _need("shared_gate", gate, (torch.float32,), (T,), dev)
        if residual is not None:
            _need("residual", residual, (torch.float32,), (T, ex.H), dev)
    else:
        gate, residual = None, None
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need("out", out, d["out"], (T, ex.H), dev)
    _need("topk_ids", ids, (torch.int32,), (T, k), dev)
    _need("topk_w", w, (torch.float32,), (T, k), dev)
    if ws is None:
        ws = torch.empty(workspace_bytes(max(T, 1), kk, ex.E, ex.H, ex.I), dtype=torch.uint8, device=dev)
    _need("workspace", ws, d["ws"], (None,), dev)
    rc = lib().rl_moe_prefill_from_logits(_ptr(x), _ptr(logits), n_route, ex.blobs, int(shared), _ptr(gate),
                                          _ptr(residual), _ptr(out), _ptr(ids), _ptr(w), T, int(k), _ptr(ws),
                                          ws.numel(), _stream())
    _check(rc, "rl_moe_prefill_from_logits")
    return out, ids, w


def prefill_noalloc(x, ids, w, ex: DeviceExperts, out):
    """rl_moe_prefill_noalloc: the layer into `out` (float32 [T, H], caller-allocated) with the
    library's static scratch in place of a workspace; nothing is allocated."""
    torch = _torch()
    _need("topk_ids", ids, (torch.int32,), (None, None))
    T, k = ids.shape
    d = _dt()
    dev = ids.device
    _need("x", x, d["x"], (T, ex.H), dev)
    _need("topk_w", w, d["w"], (T, k), dev)
    _need("out", out, d["out"], (T, ex.H), dev)
    rc = lib().rl_moe_prefill_noalloc(_ptr(x), _ptr(ids), _ptr(w), ex.blobs, _ptr(out), T, k, _stream())
    _check(rc, "rl_moe_prefill_noalloc")
    return out


def noalloc_status():
    """Status flags of the last rl_moe_prefill_noalloc on the current device (synchronises)."""
    torch = _torch()
    torch.cuda.current_stream().synchronize()
    buf = (C.c_int32 * 4)()
    _check(lib().rl_moe_noalloc_status(C.cast(buf, C.c_void_p)), "rl_moe_noalloc_status")
    return list(buf)


TIMED_EVENTS = 6  # RL_TIMED_EVENTS


def prefill_timed(x, ids, w, ex: DeviceExperts, out, ws, events):
    """rl_moe_prefill with TIMED_EVENTS torch.cuda.Event (enable_timing) recorded between its
    kernels: grouping (which also splits x) | gate/up | h split | down | combine."""
    T, k = _check_layer_args(x, ids, w, ex, out, ws)
    if len(events) != TIMED_EVENTS:
        raise RlError(f"prefill_timed needs {TIMED_EVENTS} events")
    arr = (C.c_void_p * TIMED_EVENTS)(*[C.c_void_p(e.cuda_event) for e in events])
    rc = lib().rl_moe_prefill_timed(_ptr(x), _ptr(ids), _ptr(w), ex.blobs, _ptr(out), T, k, _ptr(ws), ws.numel(),
                                    _stream(), arr)
    _check(rc, "rl_moe_prefill_timed")
    return out


def decode(x, ids, w, ex: DeviceExperts, out=None, ws=None):
    torch = _torch()
    _need("topk_ids", ids, (torch.int32,), (None, None))
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, ex.H), dtype=torch.float32, device=ids.device)
    if ws is None:
        ws = alloc_workspace(T, ids.shape[1], ex, device=ids.device)
    _check_layer_args(x, ids, w, ex, out, ws, rows=(1, 2))
    _check(_layer(lib().rl_moe_decode, x, ids, w, ex, out, ws), "rl_moe_decode")
    return out


def t1_splits_h(ex: DeviceExperts) -> bool:
    """Whether the layer's T1 gate/up writes h split into hi/lo fp8 rows (I a multiple of 256, at
    most 512), as rl_moe_gate_up documents."""
    return bool(np.any(ex.qtypes == RL_QTYPE_T1)) and ex.I % 256 == 0 and ex.I <= 512


def gate_up(x, ids, w, ex: DeviceExperts, ws=None, h16=None, h8=None, hsc=None):
    """The grouping and gate/up launches of rl_moe_prefill alone.  Returns (h16, h8, hsc): h16
    fp16 bits (int16) [T*k, I] for the rows that gate/up writes in fp16, and for T1 layers whose
    gate/up writes h split for the fp8 down GEMM, h8 uint8 [T*k, 2I] and hsc int32 [T*k] (E8M0
    scale bytes); rows in sorted-pair order.  Buffers the layer does not use are None."""
    torch = _torch()
    _need("topk_ids", ids, (torch.int32,), (None, None))
    T, k = ids.shape
    P, dev = T * k, ids.device
    split = t1_splits_h(ex)
    need16 = bool(np.any(ex.qtypes == RL_QTYPE_Q2B)) or (bool(np.any(ex.qtypes == RL_QTYPE_T1)) and not split)
    if need16 and h16 is None:
        h16 = torch.empty((P, ex.I), dtype=torch.int16, device=dev)
    if split and h8 is None:
        h8 = torch.empty((P, 2 * ex.I), dtype=torch.uint8, device=dev)
    if split and hsc is None:
        hsc = torch.empty((P,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = alloc_workspace(T, k, ex, device=dev)
    _check_layer_args(x, ids, w, ex, None, ws)
    if h16 is not None:
        _need("h16", h16, (torch.int16, torch.float16), (P, ex.I), dev)
    if h8 is not None:
        _need("h8", h8, (torch.uint8,), (P, 2 * ex.I), dev)
    if hsc is not None:
        _need("hsc", hsc, (torch.int32,), (P,), dev)
    rc = lib().rl_moe_gate_up(_ptr(x), _ptr(ids), _ptr(w), ex.blobs, _ptr(h16), _ptr(h8), _ptr(hsc), T, k, _ptr(ws),
                              ws.numel(), _stream())
    _check(rc, "rl_moe_gate_up")
    return h16, h8, hsc


def group_pairs(ids, E: int):
    """Returns (offsets[E+1], pair_src[T*k], inv[T*k], workspace) as device tensors; the
    workspace holds the status flags (see status())."""
    torch = _torch()
    _need("topk_ids", ids, (torch.int32,), (None, None))
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


def dequant(qtype: int, blocks_u8, n_values: int, out=None, decoder: int = RL_DEC_STRIP):
    """Decode n_values values of the blocks starting at blocks_u8's first byte (any alignment)
    with the library's `decoder` (RL_DEC_*); float32 [n_values]."""
    torch = _torch()
    _need("blocks", blocks_u8, (torch.uint8,), (None,))
    nb = n_values // 256
    if n_values % 256 or blocks_u8.numel() < nb * _BLOCK_BYTES.get(int(qtype), 0):
        raise RlError(f"dequant: {blocks_u8.numel()} bytes do not hold {n_values} values of type {qtype}")
    if out is None:
        out = torch.empty(max(n_values, 1), dtype=torch.float32, device=blocks_u8.device)
    _need("out", out, (torch.float32,), (None,), blocks_u8.device)
    if out.numel() < n_values:
        raise RlError("dequant: out is too small")
    _check(lib().rl_moe_dequant(int(qtype), int(decoder), _ptr(blocks_u8), int(n_values), _ptr(out), _stream()),
           "rl_moe_dequant")
    return out[:n_values]


def route(logits, k: int, ids=None, w=None):
    """Router on the GPU: (topk_ids int32 [T, k], topk_w float32 [T, k]) from fp32 logits [T, E]."""
    torch = _torch()
    _need("logits", logits, (torch.float32,), (None, None))
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need("topk_ids", ids, (torch.int32,), (T, k), logits.device)
    _need("topk_w", w, (torch.float32,), (T, k), logits.device)
    _check(lib().rl_moe_route(_ptr(logits), T, E, int(k), _ptr(ids), _ptr(w), _stream()), "rl_moe_route")
    return ids, w


def status(ws):
    """Device status flags of the last call on `ws` (synchronises the current stream)."""
    torch = _torch()
    torch.cuda.current_stream().synchronize()
    buf = (C.c_int32 * 4)()
    _check(lib().rl_moe_status(_ptr(ws), C.cast(buf, C.c_void_p)), "rl_moe_status")
    return list(buf)


class ExpertCache:
    """Bounded expert cache (rl_cache_*): the experts stay in host memory (`host_arena`: a uint8
    tensor, pinned for asynchronous copies, or a numpy array in planning mode) and `n_slots`
    device slots hold the ones a prepare requests.  With plan_only=True nothing touches the GPU:
    the cache tracks residency, hits, misses and evictions only."""

    def __init__(self, host_arena, desc_np: np.ndarray, E: int, H: int, I: int, n_slots: int, plan_only=False,
                 device="cuda"):
        self.E, self.H, self.I, self.n_slots = int(E), int(H), int(I), int(n_slots)
        self.desc_host = np.ascontiguousarray(desc_np)
        self.host_arena = host_arena
        L = lib()
        sb = int(L.rl_cache_slot_bytes(self.H, self.I))
        if sb == 0:
            raise RlError(f"unsupported H={H} I={I}")
        if isinstance(host_arena, np.ndarray):
            hptr, hbytes = host_arena.ctypes.data, host_arena.nbytes
        else:
            hptr, hbytes = host_arena.data_ptr(), host_arena.numel()
        if plan_only:
            self.slots, self.dev_desc = None, None
        else:
            torch = _torch()
            self.slots = torch.empty(self.n_slots * sb, dtype=torch.uint8, device=device)
            self.dev_desc = torch.empty(self.E * 32, dtype=torch.uint8, device=device)
        h = C.c_void_p(0)
        rc = L.rl_cache_create(C.c_void_p(hptr), hbytes, self.desc_host.ctypes.data, self.E, self.H, self.I,
                               _ptr(self.slots), self.n_slots, _ptr(self.dev_desc), C.byref(h))
        _check(rc, "rl_cache_create")
        self._h = h
        self._blobs = _Blobs()

    def prepare(self, ids) -> "CachedExperts":
        """Make the experts of ids (host array-like of ints) resident together; returns the view the
        layer calls take in place of DeviceExperts."""
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
        rc = lib().rl_cache_prepare(self._h, a.ctypes.data if a.size else None, a.size, C.byref(self._blobs),
                                    None if self.slots is None else _stream())
        _check(rc, "rl_cache_prepare")
        return CachedExperts(self)

    def stats(self):
        buf = (C.c_int64 * 4)()
        _check(lib().rl_cache_stats(self._h, C.cast(buf, C.c_void_p)), "rl_cache_stats")
        return dict(prepares=buf[0], hits=buf[1], misses=buf[2], evictions=buf[3])

    def slot_of(self, e: int) -> int:
        return int(lib().rl_cache_slot_of(self._h, int(e)))

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().rl_cache_destroy(self._h)
            self._h = C.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CachedExperts:
    """The device view of an ExpertCache after a prepare (arena = its slots): usable wherever a
    DeviceExperts is, until the next prepare of the same cache."""

    def __init__(self, cache: ExpertCache):
        self.E, self.H, self.I = cache.E, cache.H, cache.I
        self.arena, self.desc = cache.slots, cache.dev_desc
        self._blobs = _Blobs(cache._blobs.arena, cache._blobs.desc, cache._blobs.desc_host, cache._blobs.E,
                             cache._blobs.H, cache._blobs.I, cache._blobs.arena_bytes)
        self.desc_host = cache.desc_host  # block types (the cache keeps each expert's type)
        self._cache = cache

    @property
    def blobs(self):
        return C.byref(self._blobs)

    @property
    def qtypes(self) -> np.ndarray:
        return self.desc_host["qtype"]
