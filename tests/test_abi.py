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
    declared = set(re.findall(r"\b(rl_(?:moe|cache)_\w+)\s*\(", hdr))
    assert declared == set(rl._binding.EXPORTS + rl._binding.CACHE_EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_workspace_bytes(L):
    # at least one fp16 row of y (H) and of h (I) per pair
    assert L.rl_moe_workspace_bytes(2048, 10, 512, 2048, 512) > 2048 * 10 * (2048 * 2 + 512 * 2)
    assert L.rl_moe_workspace_bytes(64, 2, 8, 256, 64) > 0
    for bad in [(10, 17, 8, 256, 64), (10, 0, 8, 256, 64), (10, 2, 0, 256, 64), (10, 2, 1025, 256, 64),
                (10, 2, 8, 200, 64), (10, 2, 8, 256, 96), (10, 2, 8, 256, 192), (-1, 2, 8, 256, 64)]:
        assert L.rl_moe_workspace_bytes(*bad) == 0, bad


def test_workspace_bytes_32bit_offsets(L):
    """Shapes whose activation rows would not fit 32-bit buffer offsets are rejected: the last
    accepted and the first rejected T for x rows (T * 2H bytes, H = 8192) and for h rows
    (T * k * 2I bytes, I = 4096, k = 16); the limit is 2^31 - 2^16 bytes."""
    lim = 2**31 - 2**16
    t_x = lim // (2 * 8192)
    assert L.rl_moe_workspace_bytes(t_x, 1, 8, 8192, 64) > 0
    assert L.rl_moe_workspace_bytes(t_x + 1, 1, 8, 8192, 64) == 0
    t_h = lim // (2 * 4096 * 16)
    assert L.rl_moe_workspace_bytes(t_h, 16, 8, 256, 4096) > 0
    assert L.rl_moe_workspace_bytes(t_h + 1, 16, 8, 256, 4096) == 0
    # the case of the advisory note: 262,144 tokens x top-8 at H 2048, I 512 (2^31 bytes of split h)
    assert L.rl_moe_workspace_bytes(262144, 8, 512, 2048, 512) == 0
    # at the smallest I (64) the offset limit binds just below 2^24 pairs
    t_p = lim // (2 * 64 * 16)
    assert L.rl_moe_workspace_bytes(t_p, 16, 8, 256, 64) > 0
    assert L.rl_moe_workspace_bytes(t_p + 1, 16, 8, 256, 64) == 0


def _matrix_bytes(H, I, qtype):
    return H * I // 256 * (74 if qtype == 1 else 57)


def _blobs(E=8, H=256, I=64, qtype=1, arena_bytes=None):
    """Descriptors of E experts laid out back to back (gate, up, down) in an arena at a fake
    address; no device memory is touched by the validation these tests exercise."""
    import routed_experts_bit_amd as rl
    from workload import DESC_DTYPE

    desc = np.zeros(E, DESC_DTYPE)
    desc["qtype"] = qtype
    mb = _matrix_bytes(H, I, qtype if qtype in (1, 2) else 1)
    mb4 = (mb + 3) // 4 * 4
    for e in range(E):
        desc["gate_off"][e] = (3 * e) * mb4
        desc["up_off"][e] = (3 * e + 1) * mb4
        desc["down_off"][e] = (3 * e + 2) * mb4
    if arena_bytes is None:
        arena_bytes = 3 * E * mb4
    b = rl._binding._Blobs(0x1000, 0x2000, desc.ctypes.data, E, H, I, arena_bytes)
    return b, desc


def _call(L, fn, b, T=4, k=2, ws=0x10000, ws_bytes=1 << 40, x=0x100, ids=0x200, w=0x300, out=0x400):
    if fn == "rl_moe_gate_up":  # h16, h8, hsc in place of out
        return L.rl_moe_gate_up(C.c_void_p(x), C.c_void_p(ids), C.c_void_p(w), C.byref(b), C.c_void_p(out),
                                C.c_void_p(0x800), C.c_void_p(0x900), T, k, C.c_void_p(ws), ws_bytes, None)
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
    if fn != "rl_moe_gate_up":
        assert _call(L, fn, b, T=T, out=0) == RL_EINVAL
        assert _call(L, fn, b, T=T, out=0x404) == RL_EINVAL
    # alignment: x and out 16 bytes, ids and w 4 bytes
    assert _call(L, fn, b, T=T, x=0x108) == RL_EINVAL
    assert _call(L, fn, b, T=T, ids=0x202) == RL_EINVAL
    assert _call(L, fn, b, T=T, w=0x301) == RL_EINVAL
    assert _call(L, fn, b, T=T, ws=0) == RL_EWORKSPACE
    assert _call(L, fn, b, T=T, ws=0x10010) == RL_EWORKSPACE  # not 256-byte aligned
    assert _call(L, fn, b, T=T, ws_bytes=1024) == RL_EWORKSPACE
    badq, _desc = _blobs(qtype=7, **dims)
    assert _call(L, fn, badq, T=T) == RL_EQTYPE
    if fn == "rl_moe_gate_up":
        assert L.rl_moe_gate_up(None, None, None, None, None, None, None, 1, 1, None, 0, None) == RL_EINVAL
    else:
        assert getattr(L, fn)(None, None, None, None, None, 1, 1, None, 0, None) == RL_EINVAL


@pytest.mark.parametrize("qtype", [1, 2])
def test_descriptors_inside_arena(L, qtype):
    """Every expert matrix must lie inside arena_bytes: a descriptor set that fits exactly passes
    the descriptor checks (the call then stops at the too-small workspace, before any launch);
    one byte less of arena, or a matrix offset past the end, or a misaligned offset, is
    RL_EINVAL."""
    RL_EINVAL, RL_EWORKSPACE = -1, -3
    H, I, E = 2048, 512, 4
    b, desc = _blobs(E=E, H=H, I=I, qtype=qtype)
    exact = int(b.arena_bytes)
    assert _call(L, "rl_moe_prefill", b, ws_bytes=16) == RL_EWORKSPACE  # descriptors accepted
    b.arena_bytes = exact - 1
    assert _call(L, "rl_moe_prefill", b, ws_bytes=16) == RL_EINVAL
    b.arena_bytes = exact
    desc["down_off"][E - 1] = exact + 4096  # beyond the arena (no unsigned wrap either)
    assert _call(L, "rl_moe_prefill", b, ws_bytes=16) == RL_EINVAL
    desc["down_off"][E - 1] = 2**64 - 4
    assert _call(L, "rl_moe_prefill", b, ws_bytes=16) == RL_EINVAL
    desc["down_off"][E - 1] = 6
    assert _call(L, "rl_moe_prefill", b, ws_bytes=16) == RL_EINVAL


def test_prefill_rejects_wrapping_offsets(L):
    """The first shape whose split h would exceed 32-bit buffer offsets is RL_ESHAPE before any
    launch (the advisory case: 262,144 tokens x top-8, H 2048, I 512)."""
    b, _ = _blobs(E=8, H=2048, I=512, qtype=2)
    assert _call(L, "rl_moe_prefill", b, T=262144, k=8) == -2
    t_max = (2**31 - 2**16) // (2 * 512 * 8)  # 262,136
    assert _call(L, "rl_moe_prefill", b, T=t_max + 1, k=8) == -2
    assert _call(L, "rl_moe_prefill", b, T=t_max, k=8, ws_bytes=16) == -3  # shape accepted


def test_gate_up_needs_its_h_buffers(L):
    """rl_moe_gate_up: a T1 layer with I <= 512 needs h8 and hsc, a Q2B layer needs h16."""
    RL_EINVAL, RL_EWORKSPACE = -1, -3
    p = C.c_void_p

    def call(b, h16, h8, hsc, ws_bytes=16):
        return L.rl_moe_gate_up(p(0x100), p(0x200), p(0x300), C.byref(b), h16, h8, hsc, 2, 2, p(0x10000), ws_bytes,
                                None)

    t1, _ = _blobs(H=2048, I=512, qtype=2)
    assert call(t1, None, p(0x800), p(0x900)) == RL_EWORKSPACE
    assert call(t1, p(0x400), None, p(0x900)) == RL_EINVAL
    assert call(t1, p(0x400), p(0x800), None) == RL_EINVAL
    q2, _ = _blobs(H=2048, I=512, qtype=1)
    assert call(q2, None, None, None) == RL_EINVAL
    assert call(q2, p(0x400), None, None) == RL_EWORKSPACE
    t1big, _ = _blobs(H=256, I=1024, qtype=2)  # I > 512: fp16 h
    assert call(t1big, None, p(0x800), p(0x900)) == RL_EINVAL
    assert call(t1big, p(0x400), None, None) == RL_EWORKSPACE


def test_decode_rows_and_dims(L):
    RL_ESHAPE = -2
    b, _ = _blobs(H=2048, I=512)
    assert _call(L, "rl_moe_decode", b, T=3, k=10) == RL_ESHAPE
    assert _call(L, "rl_moe_decode", b, T=0, k=10) == RL_ESHAPE
    # more strips per lane than the 1-2 row kernels take (H 256 x 9, 512 x 9; I 256 x 5,
    # 512 x 5) and I below 256: refused on the host
    for H, I in ((2304, 512), (4608, 512), (1024, 1280), (1024, 2560), (1024, 128)):
        b2, _ = _blobs(H=H, I=I)
        assert _call(L, "rl_moe_decode", b2, T=1, k=10) == RL_ESHAPE, (H, I)


def test_prefill_empty_is_ok(L):
    b, _ = _blobs()
    assert _call(L, "rl_moe_prefill", b, T=0, x=0, ids=0, w=0, out=0, ws=0, ws_bytes=0) == 0


def test_dequant_and_group_codes(L):
    v = C.c_void_p
    assert L.rl_moe_dequant(3, 0, v(0x100), 256, v(0x200), None) == -1
    assert L.rl_moe_dequant(1, 5, v(0x100), 256, v(0x200), None) == -1   # unknown decoder
    assert L.rl_moe_dequant(1, -1, v(0x100), 256, v(0x200), None) == -1
    assert L.rl_moe_dequant(1, 0, v(0x100), 255, v(0x200), None) == -2
    assert L.rl_moe_dequant(2, 1, None, 0, None, None) == 0
    assert L.rl_moe_dequant(2, 2, None, 256, None, None) == -1
    # blocks spanning more than 2^32 - 16 bytes from their dword base
    assert L.rl_moe_dequant(2, 1, v(0x101), (2**32 // 57 + 1) * 256, v(0x200), None) == -2
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


# ----------------------------------------------------------------------------- binding checks
def test_binding_rejects_bad_tensors():
    """The Python binding checks dtype, shape, contiguity and device of every buffer before it
    reaches the library (CPU tensors here: each mistake is reported before the device check)."""
    import torch

    import routed_experts_bit_amd as rl
    from routed_experts_bit_amd._binding import _need

    ok = torch.zeros((4, 8), dtype=torch.int32)
    with pytest.raises(rl.RlError, match="dtype"):
        _need("topk_ids", ok.float(), (torch.int32,), (4, 8))
    with pytest.raises(rl.RlError, match="shape"):
        _need("topk_ids", ok, (torch.int32,), (4, 9))
    with pytest.raises(rl.RlError, match="shape"):
        _need("topk_ids", ok, (torch.int32,), (None,))
    with pytest.raises(rl.RlError, match="contiguous"):
        _need("topk_ids", ok.t(), (torch.int32,), (8, 4))
    with pytest.raises(rl.RlError, match="CUDA"):
        _need("topk_ids", ok, (torch.int32,), (4, 8))
    with pytest.raises(rl.RlError, match="torch.Tensor"):
        _need("topk_ids", np.zeros((4, 8), np.int32), (torch.int32,), (4, 8))


def test_binding_checks_descriptors_against_arena():
    import routed_experts_bit_amd as rl
    from routed_experts_bit_amd._binding import _check_descriptors
    from workload import make_experts

    ex = make_experts(3, 256, 64, [1, 2, 1], seed=5)
    _check_descriptors(ex.desc, ex.E, ex.H, ex.I, ex.arena.size)  # the packer's own layout fits
    with pytest.raises(rl.RlError, match="inside"):
        _check_descriptors(ex.desc, ex.E, ex.H, ex.I, int(ex.desc["down_off"][2]) + 100)
    d = ex.desc.copy()
    d["up_off"][1] += 2
    with pytest.raises(rl.RlError, match="dword"):
        _check_descriptors(d, ex.E, ex.H, ex.I, ex.arena.size)
    d = ex.desc.copy()
    d["qtype"][0] = 9
    with pytest.raises(rl.RlError, match="block type"):
        _check_descriptors(d, ex.E, ex.H, ex.I, ex.arena.size)
    with pytest.raises(rl.RlError, match="records"):
        _check_descriptors(ex.desc[:2], ex.E, ex.H, ex.I, ex.arena.size)


def test_noalloc_codes(L):
    """rl_moe_prefill_noalloc validates like rl_moe_prefill and refuses, before any launch, a call
    whose workspace exceeds its static buffer (RL_ETOOBIG)."""
    import routed_experts_bit_amd as rl

    RL_ESHAPE, RL_EINVAL, RL_ETOOBIG = -2, -1, -6
    v = C.c_void_p
    b, _ = _blobs(E=512, H=2048, I=512, qtype=2)

    def call(T, k, x=0x100, out=0x400):
        return L.rl_moe_prefill_noalloc(v(x), v(0x200), v(0x300), C.byref(b), v(out), T, k, None)

    assert L.rl_moe_workspace_bytes(1024, 10, 512, 2048, 512) > rl.NOALLOC_SCRATCH_BYTES
    assert L.rl_moe_workspace_bytes(512, 10, 512, 2048, 512) <= rl.NOALLOC_SCRATCH_BYTES
    assert call(1024, 10) == RL_ETOOBIG
    assert call(4, 17) == RL_ESHAPE
    assert call(4, 10, x=0) == RL_EINVAL
    assert call(0, 10, x=0, out=0) == 0
    assert "scratch" in rl.strerror(RL_ETOOBIG) and "cache" in rl.strerror(RL_ETOOBIG)


def test_t1_digit_bytes_checked_on_load():
    """A T1 digit byte above 242 (more than five base-3 digits) is rejected when a host arena
    is loaded (the kernels themselves decode such a byte as five zero weights, the oracle
    rejects it); a valid arena loads."""
    import routed_experts_bit_amd as rl
    from workload import QTYPE_Q2B, QTYPE_T1, make_experts

    ex = make_experts(4, 256, 64, [QTYPE_Q2B, QTYPE_T1, QTYPE_T1, QTYPE_Q2B], seed=5, threads=1)
    rl.DeviceExperts(ex.arena, ex.desc, ex.E, ex.H, ex.I, device="cpu")
    bad = ex.arena.copy()
    off = int(ex.desc["up_off"][2]) + 3 * 57 + 5 + 17  # expert 2 (T1), up matrix, block 3, a digit byte
    bad[off] = 243
    with pytest.raises(rl.RlError, match="expert 2: up block 3"):
        rl.DeviceExperts(bad, ex.desc, ex.E, ex.H, ex.I, device="cpu")
    # Q2B code bytes take every value
    ok = ex.arena.copy()
    ok[int(ex.desc["gate_off"][0]) + 20] = 255
    rl.DeviceExperts(ok, ex.desc, ex.E, ex.H, ex.I, device="cpu")


def test_kernel_resource_rules():
    """The build's check of the compiler's kernel-resource-usage remarks: the tuned matrix kernels
    (hand-counted load waits, two waves per SIMD) and the 1-2 row kernels may not use scratch, and
    the tuned ones must keep two waves per SIMD; other kernels are only reported."""
    from routed_experts_bit_amd import build as hb

    def remark(fn, scratch, occ, vgprs=256):
        loc = "/x/rl_kernels.h:1:1: remark: "
        tail = " [-Rpass-analysis=kernel-resource-usage]"
        return "\n".join([loc + f"Function Name: {fn}" + tail, " 1 | __global__ void k() {", "   | ^",
                          loc + f"    VGPRs: {vgprs}" + tail, loc + f"    ScratchSize [bytes/lane]: {scratch}" + tail,
                          loc + f"    Occupancy [waves/SIMD]: {occ}" + tail])

    text = "\n".join([
        remark("_ZN2rl7k_t1_f8ILi0ELi2ELb1EEEvNS_6GuArgsE", 0, 2),
        remark("_ZN2rl7k_t1_dnENS_6GuArgsE", 0, 2, 226),
        remark("_ZN2rl9k_gv_downILi2ELi32ELi1ELi256EEEvNS_6GvArgsE", 0, 5, 84),
        remark("_ZN2rl6k_downILi1ELi256ELi4ELi4EEEvNS_8DownArgsE", 1404, 2),  # untuned path: reported only
    ])
    res = hb.kernel_resources(text)
    assert res["_ZN2rl7k_t1_dnENS_6GuArgsE"] == {"vgprs": 226, "scratch": 0, "occupancy": 2}
    assert len(res) == 4 and hb.check_resources(res) == []
    bad = hb.kernel_resources("\n".join([remark("_ZN2rl7k_q2_mmILi0ELi2ELb1EEEvNS_6GuArgsE", 84, 2),
                                         remark("_ZN2rl7k_t1_f8ILi0ELi2ELb0EEEvNS_6GuArgsE", 0, 1),
                                         remark("_ZN2rl11k_gv_gateupILi1ELi64ELi2ELi256EEEvNS_6GvArgsE", 8, 4)]))
    msgs = hb.check_resources(bad)
    assert len(msgs) == 3 and "84 bytes" in msgs[0] and "1 wave" in msgs[1] and "8 bytes" in msgs[2]
