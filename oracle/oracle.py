"""ctypes wrapper of rl_oracle.c (plain C, double precision) -- test infrastructure only.

The parity-unpinned status of each function, if any, is stated in the module docstrings of
the tests that pin it; every function here is pinned by a CPU test.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rl_oracle.c")
_LIB = os.path.join(_HERE, "librl_oracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def default_threads() -> int:
    """Host threads for the oracle: the cores this process may run on (its CPU affinity), capped
    by OMP_NUM_THREADS when that is set (a shared GPU host gives each job a share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no floating-point contraction."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = C.CDLL(_LIB)
    P = C.c_void_p
    lib.orc_fp16_to_double.argtypes = [C.c_uint16]
    lib.orc_fp16_to_double.restype = C.c_double
    lib.orc_bf16_to_double.argtypes = [C.c_uint16]
    lib.orc_bf16_to_double.restype = C.c_double
    lib.orc_dequant.argtypes = [C.c_int, P, C.c_int64, P]
    lib.orc_dequant.restype = C.c_int
    lib.orc_group_pairs.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P, P]
    lib.orc_group_pairs.restype = C.c_int
    lib.orc_moe_prefill.argtypes = [P, P, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, C.c_int, P, P,
                                    C.c_int]
    lib.orc_moe_prefill.restype = C.c_int
    lib.orc_moe_block.argtypes = [P, P, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P,
                                  C.c_int, P, C.c_int]
    lib.orc_moe_block.restype = C.c_int
    lib.orc_route.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P]
    lib.orc_route.restype = C.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def fp16_to_double(bits) -> np.ndarray:
    lib = load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_fp16_to_double(int(v)) for v in b], dtype=np.float64)


def bf16_to_double(bits) -> np.ndarray:
    lib = load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_bf16_to_double(int(v)) for v in b], dtype=np.float64)


def dequant(qtype: int, blocks: np.ndarray, n_values: int) -> np.ndarray:
    lib = load()
    blk = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(max(n_values, 1), dtype=np.float64)
    rc = lib.orc_dequant(int(qtype), _ptr(blk), int(n_values), _ptr(out))
    if rc:
        raise ValueError(f"orc_dequant failed ({rc})")
    return out[:n_values]


def group_pairs(ids: np.ndarray, E: int):
    """Returns (offsets[E+1], pair_src[P], inv[T*k]) as int32 arrays."""
    lib = load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k
    offsets = np.empty(E + 1, np.int32)
    pair_src = np.empty(max(P, 1), np.int32)
    inv = np.empty(max(P, 1), np.int32)
    rc = lib.orc_group_pairs(_ptr(ids), T, k, E, _ptr(offsets), _ptr(pair_src), _ptr(inv))
    if rc:
        raise ValueError(f"orc_group_pairs failed ({rc})")
    return offsets, pair_src[:P], inv[:P]


def moe_prefill(x, ids, w, arena, desc, E, H, I, tokens=None, want_h=False, threads=None):
    """Routed-expert layer output (float64) for `tokens` (default: all); optionally the
    per-pair h [n, k, I]."""
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    arena = np.ascontiguousarray(arena, dtype=np.uint8)
    desc = np.ascontiguousarray(desc)
    T, k = ids.shape
    if tokens is None:
        tok = np.arange(T, dtype=np.int32)
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
    n = tok.size
    out = np.empty((max(n, 1), H), np.float64)
    h = np.empty((max(n, 1), k, I), np.float64) if want_h else None
    nthr = threads or default_threads()
    rc = lib.orc_moe_prefill(_ptr(x), _ptr(ids), _ptr(w), _ptr(arena), _ptr(desc), E, H, I, T, k, _ptr(tok), n,
                             _ptr(out), _ptr(h) if h is not None else None, int(nthr))
    if rc:
        raise ValueError(f"orc_moe_prefill failed ({rc})")
    return (out[:n], h[:n] if h is not None else None) if want_h else out[:n]


def moe_block(x, ids, w, arena, desc, E, H, I, shared, shared_gate, residual=None, tokens=None, threads=None):
    """The MoE block (orc_moe_block): routed sum in selection order, then the shared expert
    `shared` weighted by shared_gate[t], then the residual [T, H] (None: none); float64 [n, H].
    ids / w may have k = 0 columns."""
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    arena = np.ascontiguousarray(arena, dtype=np.uint8)
    desc = np.ascontiguousarray(desc)
    g = np.ascontiguousarray(shared_gate, dtype=np.float32)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    T, k = ids.shape
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.empty((max(tok.size, 1), H), np.float64)
    rc = lib.orc_moe_block(_ptr(x), _ptr(ids) if ids.size else None, _ptr(w) if w.size else None, _ptr(arena),
                           _ptr(desc), E, H, I, T, k, int(shared), _ptr(g), _ptr(res) if res is not None else None,
                           _ptr(tok), tok.size, _ptr(out), int(threads or default_threads()))
    if rc:
        raise ValueError(f"orc_moe_block failed ({rc})")
    return out[: tok.size]


def moe_workload(wl, tokens=None, want_h=False, threads=None):
    ex = wl.experts
    return moe_prefill(wl.x, wl.ids, wl.w, ex.arena, ex.desc, ex.E, ex.H, ex.I, tokens=tokens, want_h=want_h,
                       threads=threads)


def route(logits: np.ndarray, k: int):
    """Router: (ids int32 [T, k], w float64 [T, k]) from fp32 logits [T, E] (orc_route)."""
    lib = load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((max(T, 1), k), np.int32)
    w = np.empty((max(T, 1), k), np.float64)
    rc = lib.orc_route(_ptr(lg), T, E, int(k), _ptr(ids), _ptr(w))
    if rc:
        raise ValueError(f"orc_route failed ({rc})")
    return ids[:T], w[:T]
