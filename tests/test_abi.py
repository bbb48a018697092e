"""The C-ABI library on the CPU: it loads, exports every entry point that include/rl_moe.h
declares, and its host-side validation returns the documented status codes before
launching anything (no compute call is made here)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import routed_experts_bit_amd as rl

    return rl.lib()


def test_exports_match_header(L):
    import routed_experts_bit_amd as rl

    hdr = open(os.path.join(ROOT, "include", "rl_moe.h")).read()
    declared = set(re.findall(r"\b(rl_moe_\w+)\s*\(", hdr))
    assert declared == set(rl._binding.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_workspace_bytes(L):
    # at least one fp16 row of y (H) and of h (I) per pair
    assert L.rl_moe_workspace_bytes(2048, 10, 512, 2048, 512) > 2048 * 10 * (2048 * 2 + 512 * 2)
    assert L.rl_moe_workspace_bytes(64, 2, 8, 256, 64) > 0
    for bad in [(10, 17, 8, 256, 64), (10, 0, 8, 256, 64), (10, 2, 0, 256, 64), (10, 2, 1025, 256, 64),
                (10, 2, 8, 200, 64), (10, 2, 8, 256, 96), (10, 2, 8, 256, 192), (-1, 2, 8, 256, 64)]:
        assert L.rl_moe_workspace_bytes(*bad) == 0, bad


def _blobs(E=8, H=256, I=64, qtype=1):
    import routed_experts_bit_amd as rl
    from workload import DESC_DTYPE

    desc = np.zeros(E, DESC_DTYPE)
    desc["qtype"] = qtype
    b = rl._binding._Blobs(0x1000, 0x2000, desc.ctypes.data, E, H, I)
    return b, desc


def _call(L, fn, b, T=4, k=2, ws=0x10000, ws_bytes=1 << 40, x=0x100, ids=0x200, w=0x300, out=0x400):
    return getattr(L, fn)(C.c_void_p(x), C.c_void_p(ids), C.c_void_p(w), C.byref(b), C.c_void_p(out), T, k,
                          C.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("fn", ["rl_moe_prefill", "rl_moe_gate_up", "rl_moe_decode"])
def test_validation_codes(L, fn):
    RL_EINVAL, RL_ESHAPE, RL_EWORKSPACE, RL_EQTYPE = -1, -2, -3, -5
    dims = dict(H=2048, I=512)
    b, _ = _blobs(**dims)
    T = 2
    assert _call(L, fn, b, T=T, k=17) == RL_ESHAPE
    assert _call(L, fn, b, T=T, k=0) == RL_ESHAPE
    bad, _ = _blobs(E=0, **dims)
    assert _call(L, fn, bad, T=T) == RL_ESHAPE
    bad, _ = _blobs(H=300, I=512)
    assert _call(L, fn, bad, T=T) == RL_ESHAPE
    assert _call(L, fn, b, T=T, x=0) == RL_EINVAL
    assert _call(L, fn, b, T=T, out=0) == RL_EINVAL
    # alignment: x and out 16 bytes, ids and w 4 bytes
    assert _call(L, fn, b, T=T, x=0x108) == RL_EINVAL
    assert _call(L, fn, b, T=T, out=0x404) == RL_EINVAL
    assert _call(L, fn, b, T=T, ids=0x202) == RL_EINVAL
    assert _call(L, fn, b, T=T, w=0x301) == RL_EINVAL
    assert _call(L, fn, b, T=T, ws=0) == RL_EWORKSPACE
    assert _call(L, fn, b, T=T, ws=0x10010) == RL_EWORKSPACE  # not 256-byte aligned
    assert _call(L, fn, b, T=T, ws_bytes=1024) == RL_EWORKSPACE
    badq, _desc = _blobs(qtype=7, **dims)
    assert _call(L, fn, badq, T=T) == RL_EQTYPE
    assert getattr(L, fn)(None, None, None, None, None, 1, 1, None, 0, None) == RL_EINVAL


def test_decode_rows_and_dims(L):
    RL_ESHAPE = -2
    b, _ = _blobs(H=2048, I=512)
    assert _call(L, "rl_moe_decode", b, T=3, k=10) == RL_ESHAPE
    assert _call(L, "rl_moe_decode", b, T=0, k=10) == RL_ESHAPE
    b2, _ = _blobs(H=768, I=512)
    assert _call(L, "rl_moe_decode", b2, T=1, k=10) == RL_ESHAPE


def test_prefill_empty_is_ok(L):
    b, _ = _blobs()
    assert _call(L, "rl_moe_prefill", b, T=0, x=0, ids=0, w=0, out=0, ws=0, ws_bytes=0) == 0


def test_dequant_and_group_codes(L):
    assert L.rl_moe_dequant(3, C.c_void_p(0x100), 256, C.c_void_p(0x200), None) == -1
    assert L.rl_moe_dequant(1, C.c_void_p(0x100), 255, C.c_void_p(0x200), None) == -2
    assert L.rl_moe_dequant(2, None, 0, None, None) == 0
    assert L.rl_moe_dequant(2, None, 256, None, None) == -1
    p = C.c_void_p(0x100)
    ws = C.c_void_p(0x10000)
    assert L.rl_moe_group_pairs(p, 4, 17, 8, p, p, p, ws, 1 << 20, None) == -2
    assert L.rl_moe_group_pairs(p, 4, 2, 1025, p, p, p, ws, 1 << 20, None) == -2
    assert L.rl_moe_group_pairs(p, 4, 2, 8, None, p, p, ws, 1 << 20, None) == -1
    assert L.rl_moe_group_pairs(p, 4, 2, 8, p, p, p, None, 1 << 20, None) == -3
    assert L.rl_moe_group_pairs(p, 4, 2, 8, p, p, p, ws, 16, None) == -3


def test_strerror(L):
    import routed_experts_bit_amd as rl

    for code in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(rl.strerror(code), str) and rl.strerror(code)


def test_route_codes(L):
    p = C.c_void_p(0x100)
    assert L.rl_moe_route(p, 4, 0, 1, p, p, None) == -2      # E < 1
    assert L.rl_moe_route(p, 4, 1025, 2, p, p, None) == -2   # E > 1024
    assert L.rl_moe_route(p, 4, 8, 0, p, p, None) == -2      # k < 1
    assert L.rl_moe_route(p, 4, 64, 17, p, p, None) == -2    # k > 16
    assert L.rl_moe_route(p, 4, 5, 6, p, p, None) == -2      # k > E
    assert L.rl_moe_route(p, -1, 8, 2, p, p, None) == -2     # T < 0
    assert L.rl_moe_route(None, 0, 8, 2, None, None, None) == 0   # T = 0: nothing to do
    assert L.rl_moe_route(None, 4, 8, 2, p, p, None) == -1
    assert L.rl_moe_route(p, 4, 8, 2, p, None, None) == -1
    assert L.rl_moe_route(C.c_void_p(0x102), 4, 8, 2, p, p, None) == -1   # logits not 4-byte aligned
    assert L.rl_moe_route(p, 4, 8, 2, C.c_void_p(0x101), p, None) == -1
