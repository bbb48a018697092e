"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: bit-exact for the block decode and the pair grouping; relative L2 <= 2e-3 (float64,
over the whole output) for the fp16 h of the gate/up stage and for the layer output.
"""
import numpy as np
import pytest

from gpu_util import log, rel_l2, to_device
from workload import QTYPE_Q2B, QTYPE_T1, BLOCK_BYTES, make_experts, make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


# ----------------------------------------------------------------------------- decode
def _decode_blocks(qtype, nb=3159):
    """Blocks that cover, at every byte position, every digit byte (T1: 0..242) or code byte
    (Q2B: 0..255), at every sub-block every sub-scale, and the special block scales d = +0, -0,
    the smallest and a mid fp16 subnormal (both signs) and the fp16 maximum; the other d are
    random normal fp16 values.  nb is a multiple of 243 (13 * 243) above 3,000."""
    rng = np.random.default_rng(100 + qtype)
    bb = BLOCK_BYTES[qtype]
    blk = np.zeros((nb, bb), np.uint8)
    d = (rng.standard_normal(nb) * 0.01).astype(np.float16).view(np.uint16)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0155, 0x8155, 0x7BFF, 0xFBFF], np.uint16)
    d[np.arange(nb) % 97 < special.size] = special[(np.arange(nb) % 97)[np.arange(nb) % 97 < special.size]]
    blk[:, 0] = d & 255
    blk[:, 1] = d >> 8
    b = np.arange(nb)[:, None]
    if qtype == QTYPE_T1:
        sub = (b + np.arange(8)[None, :]) % 8                      # every sub-scale at every sub-block
        word = np.sum(sub.astype(np.uint32) << (3 * np.arange(8, dtype=np.uint32))[None, :], axis=1)
        blk[:, 2], blk[:, 3], blk[:, 4] = word & 255, (word >> 8) & 255, (word >> 16) & 255
        blk[:, 5:] = (b + 37 * np.arange(52)[None, :]) % 243       # every digit byte at every position
    else:
        sub = (b + np.arange(16)[None, :]) % 16
        blk[:, 2:10] = sub[:, 0::2] | (sub[:, 1::2] << 4)
        blk[:, 10:] = (b + 37 * np.arange(64)[None, :]) % 256      # every code byte at every position
    return blk


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
@pytest.mark.parametrize("decoder", ["strip", "mfma_gateup", "mfma_down", "rows_gateup", "rows_down"])
def test_dequant_bit_exact(orc, rl, qtype, decoder):
    """Each of the library's device decoders, run as the kernels run it (the MFMA ones with their
    selector and fp8 / 16-bit tables built on the device, windows cut at the block's byte
    misalignment, operands written at their k-map positions; the 1-2 row ones with their unit
    tables copied from device data, at the three strip widths), equals the oracle's decode bit for
    bit: every product d * s * c is exact in fp32.  Blocks at all four byte misalignments."""
    import torch

    dec = {"strip": rl.RL_DEC_STRIP, "mfma_gateup": rl.RL_DEC_MFMA_GATEUP, "mfma_down": rl.RL_DEC_MFMA_DOWN,
           "rows_gateup": rl.RL_DEC_ROWS_GATEUP, "rows_down": rl.RL_DEC_ROWS_DOWN}[decoder]
    blk = _decode_blocks(qtype)
    nb = blk.shape[0]
    ref_all = orc.dequant(qtype, blk.reshape(-1), nb * 256)
    # the 1-2 row decoders cut block b of a call into strips of 64, 32 or 16 values by b % 3:
    # three calls starting one block apart give every block every strip width
    shifts = range(3) if decoder.startswith("rows") else range(1)
    for sh in shifts:
        flat = blk[sh:].reshape(-1)
        ref = ref_all[256 * sh:]
        for mis in range(4):
            log(f"dequant qtype={qtype} decoder={decoder} blocks={nb - sh} misalignment={mis}")
            buf = torch.zeros(flat.size + 8, dtype=torch.uint8, device="cuda")
            buf[mis:mis + flat.size].copy_(torch.from_numpy(flat))
            got = rl.dequant(qtype, buf[mis:mis + flat.size], (nb - sh) * 256, decoder=dec).cpu().numpy()
            assert np.array_equal(got.astype(np.float64), ref), f"first block {sh}, misalignment {mis}"


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
def test_dequant_real_matrix(orc, rl, qtype):
    ex = make_experts(2, 2048, 512, qtype, seed=3)
    import torch

    arena = torch.from_numpy(ex.arena).cuda()
    for which in ("gate", "down"):
        off = int(ex.desc[which + "_off"][1])
        n = 2048 * 512
        ref = orc.dequant(qtype, ex.matrix(1, which), n)
        mb = n // 256 * BLOCK_BYTES[qtype]
        for dec in (rl.RL_DEC_STRIP, rl.RL_DEC_MFMA_GATEUP, rl.RL_DEC_MFMA_DOWN, rl.RL_DEC_ROWS_GATEUP,
                    rl.RL_DEC_ROWS_DOWN):
            got = rl.dequant(qtype, arena[off:off + mb], n, decoder=dec).cpu().numpy()
            assert np.array_equal(got.astype(np.float64), ref)


# ----------------------------------------------------------------------------- grouping
@pytest.mark.parametrize(
    "T,k,E,kind",
    [(1, 1, 1, "uniform"), (64, 2, 8, "uniform"), (2048, 10, 512, "uniform"), (1090, 10, 512, "skewed"),
     (300, 16, 1024, "dup"), (4096, 8, 64, "uniform"), (5, 3, 1024, "uniform"), (8192, 10, 512, "skewed"),
     (777, 13, 3, "uniform"), (3277, 10, 1000, "uniform"), (4095, 8, 1024, "skewed")],
)
def test_group_pairs_bit_exact(orc, rl, T, k, E, kind):
    import torch

    rng = np.random.default_rng(T * 31 + k)
    if kind == "skewed":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    elif kind == "dup":
        ids = rng.integers(0, 7, size=(T, k)).astype(np.int32)  # duplicates inside rows, most experts empty
    else:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    log(f"group T={T} k={k} E={E} {kind}")
    offsets, src, inv, ws = rl.group_pairs(torch.from_numpy(ids).cuda(), E)
    o2, s2, i2 = orc.group_pairs(ids, E)
    assert np.array_equal(offsets.cpu().numpy(), o2)
    assert np.array_equal(src.cpu().numpy(), s2)
    assert np.array_equal(inv.cpu().numpy(), i2)
    assert rl.status(ws)[0] == 0


def test_group_pairs_flags_bad_id(rl):
    import torch

    ids = np.array([[0, 1], [5, 2], [3, -1]], np.int32)
    offsets, src, inv, ws = rl.group_pairs(torch.from_numpy(ids).cuda(), 4)
    assert rl.status(ws)[0] & 1
    inv = inv.cpu().numpy()
    assert inv[2] == -1 and inv[5] == -1
    good = [0, 1, 3, 4]
    assert sorted(inv[good].tolist()) == [0, 1, 2, 3]
    assert offsets.cpu().numpy()[-1] == 4


# ----------------------------------------------------------------------------- layer
def _medium(name, seed, T=256, E=32, H=2048, I=512, k=10, types=None):
    over = dict(E=E, H=H, I=I, k=k)
    if types:
        over["types"] = types
    return make_workload(name, seed=seed, T=T, **over)


CASES = {
    "tiny_q2b": lambda: make_workload("tiny", seed=21),
    "tiny_t1": lambda: make_workload("tiny", seed=22, types="t1"),
    "med_q2b": lambda: _medium("q2b_1090", 23, types="q2b"),
    "med_t1": lambda: _medium("t1_2048", 24),
    "med_mixed": lambda: _medium("mixed_2048", 25),
    "i128_t1": lambda: _medium("t1_2048", 26, T=96, E=16, H=1024, I=128, k=4),
    "i64_q2b": lambda: _medium("q2b_1090", 27, T=80, E=12, H=512, I=64, k=3),
    "i256_mixed_k1": lambda: _medium("mixed_2048", 28, T=130, E=8, H=768, I=256, k=1),
    # I > 512: h split by its own kernel and down on the streamed-activation kernel
    "i1024_t1": lambda: _medium("t1_2048", 29, T=64, E=8, H=1024, I=1024, k=3),
    "i1024_q2b": lambda: _medium("q2b_1090", 33, T=64, E=8, H=1024, I=1024, k=3, types="q2b"),
    # the largest k and E: many experts with no or few pairs
    "k16_e1024_mixed": lambda: _medium("mixed_2048", 31, T=96, E=1024, H=256, I=256, k=16),
    # one token
    "t1_one_token": lambda: _medium("t1_2048", 32, T=1, E=64, H=2048, I=512, k=10),
    # the largest supported hidden size and expert intermediate size, both block types
    "max_h_mixed": lambda: _medium("mixed_2048", 34, T=40, E=6, H=8192, I=256, k=2),
    "max_i_mixed": lambda: _medium("mixed_2048", 35, T=40, E=4, H=256, I=4096, k=2),
}


@pytest.fixture(scope="module")
def cases():
    return {}


def _case(cases, name):
    if name not in cases:
        cases[name] = CASES[name]()
    return cases[name]


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(orc, rl, cases, name):
    wl = _case(cases, name)
    log(f"prefill {name} T={wl.T} k={wl.k} E={wl.experts.E} H={wl.experts.H} I={wl.experts.I}")
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, ids, w, ex, ws=ws).cpu().numpy()
    assert rl.status(ws)[0] == 0
    ref = orc.moe_workload(wl)
    err = rel_l2(out, ref)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("I", [256, 512])
def test_prefill_t1_row_scales(orc, rl, I):
    """T1 experts with I <= 512 hand h to the down kernel as hi/lo fp8 under one power-of-two
    scale per row, block and k-group pair.  Token rows scaled by 2^e, e in [-4, 3] (h then spans
    ~14 binades across rows, and y stays in fp16's normal range): every output row must meet the
    bar against its own norm, which a scale shared across rows, or taken from the wrong rows or
    k-groups, would miss."""
    import dataclasses

    wl = make_workload("t1_2048", seed=37 + I, T=64, E=16, H=1024, I=I, k=4)
    e = np.random.default_rng(I).integers(-4, 4, size=wl.T)
    xf = (wl.x.astype(np.uint32) << 16).view(np.float32) * np.exp2(e)[:, None].astype(np.float32)
    wl = dataclasses.replace(wl, x=(xf.view(np.uint32) >> 16).astype(np.uint16))  # exact: powers of two
    log(f"prefill t1 row scales I={I} T={wl.T} k={wl.k} E={wl.experts.E} H={wl.experts.H}")
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, ids, w, ex, ws=ws).cpu().numpy().astype(np.float64)
    assert rl.status(ws)[0] == 0
    ref = orc.moe_workload(wl)
    per_row = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    log(f"  rel_l2 per row: max {per_row.max():.3e} median {np.median(per_row):.3e}")
    assert per_row.max() <= TOL


def _e4m3(b):
    """OCP FP8 E4M3 (the MFMA's fp8 operand format) to float64: bias 7, exponent field 0 is
    subnormal (m/8 * 2^-6), S.1111.111 is NaN, no infinities."""
    b = np.asarray(b, np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, s * v)


def _t1_kmap(g, j):
    return np.where(j < 60, 60 * g + j, 240 + 4 * g + (j - 60))


def unsplit_h(h8, hsc, I):
    """h rows [P, I] from the split rows the T1 gate/up writes for the fp8 down GEMM (layout in
    include/rl_moe.h, rl_moe_gate_up), plus the per-(row, block, lane-group pair) exponents
    [P, I/256, 2] and the scaled values (hi + lo) [P, I]."""
    P = h8.shape[0]
    nkb = I // 256
    h = np.zeros((P, I))
    scaled = np.zeros((P, I))
    ex = np.zeros((P, nkb, 2), np.int64)
    sc = hsc.astype(np.int64) & 0xFFFFFFFF
    for kb in range(nkb):
        for hh in range(2):
            for g in range(4):
                o = 512 * kb + 256 * hh + 64 * g
                hi, lo = _e4m3(h8[:, o:o + 32]), _e4m3(h8[:, o + 32:o + 64])
                e = (sc >> (8 * (2 * kb + (g >> 1)))) & 255
                ex[:, kb, g >> 1] = e
                cols = 256 * kb + _t1_kmap(g, 32 * hh + np.arange(32))
                scaled[:, cols] = hi + lo
                h[:, cols] = (hi + lo) * np.exp2(e - 127.0)[:, None]
    return h, ex, scaled


@pytest.mark.parametrize("name", ["tiny_q2b", "med_t1", "med_mixed", "i64_q2b", "i256_mixed_k1", "i1024_t1"])
def test_gate_up_h_parity(orc, rl, cases, name):
    """h after the fused decode + gate/up + SwiGLU, as the production path leaves it for the down
    GEMM: fp16 rows (Q2B experts; T1 with I > 512 or < 256) within the layer bar; and for T1 with
    I a multiple of 256 up to 512, the split rows (hi/lo e4m3 bytes + one E8M0 exponent per row,
    block and lane-group pair) decoded on the host and checked element by element:
      |h_gpu - h_oracle| <= 2^-8 |h_oracle| + 2^-12 G
    (G = the largest |h_oracle| of the element's 128-column group: hi + lo keeps 8 significant
    bits, |x - (hi + lo)| <= 2^-8 |x| + 2^-10 in scaled units where the group maximum is >= 128;
    the fp32 GEMM itself is ~1e-6 off); every group's scaled maximum in [127, 256]; no NaN byte."""
    wl = _case(cases, name)
    x, ids, w, ex = to_device(wl)
    h16, h8, hsc = rl.gate_up(x, ids, w, ex)
    _, ref_h = orc.moe_workload(wl, want_h=True)  # [T, k, I]
    _, src, _ = orc.group_pairs(wl.ids, wl.experts.E)
    ref_sorted = ref_h.reshape(wl.T * wl.k, -1)[src]
    qt = wl.experts.desc["qtype"][wl.ids.reshape(-1)[src]]
    I = wl.experts.I
    split = rl.t1_splits_h(ex)
    t1_rows = (qt == QTYPE_T1) if split else np.zeros(qt.shape, bool)
    got = np.zeros_like(ref_sorted)
    if h16 is not None:
        got[~t1_rows] = h16.cpu().numpy().view(np.float16).astype(np.float64)[~t1_rows]
    if split:
        hb = h8.cpu().numpy()[t1_rows]
        hs = hsc.cpu().numpy().view(np.uint32)[t1_rows]
        assert not np.any((hb & 0x7F) == 0x7F), "NaN byte in split h"
        hv, _, scaled = unsplit_h(hb, hs, I)
        got[t1_rows] = hv
        ref_t1 = ref_sorted[t1_rows]
        # G: the maximum over each (block, lane-group pair) group of columns, taken through the layout
        G = np.zeros_like(ref_t1)
        for kb in range(I // 256):
            for p in range(2):
                cols = np.concatenate([256 * kb + _t1_kmap(g, np.arange(64)) for g in (2 * p, 2 * p + 1)])
                gm = np.abs(ref_t1[:, cols]).max(axis=1, keepdims=True)
                G[:, cols] = gm
                sm = np.abs(scaled[:, cols]).max(axis=1)
                live = gm[:, 0] > 0
                assert np.all((sm[live] >= 127) & (sm[live] <= 256)), (kb, p, sm[live].min(), sm[live].max())
        err = np.abs(hv - ref_t1)
        bound = 2.0**-8 * np.abs(ref_t1) + 2.0**-12 * G
        worst = float(np.max(err / np.maximum(bound, 1e-300)))
        log(f"gate_up {name}: split h rows {int(t1_rows.sum())}, worst error / bound {worst:.3f}")
        assert np.all(err <= bound)
    err = rel_l2(got, ref_sorted)
    log(f"gate_up {name} rel_l2={err:.3e}")
    assert err <= TOL


def test_prefill_deterministic_and_invariants(orc, rl, cases):
    import torch

    wl = _case(cases, "med_mixed")
    x, ids, w, ex = to_device(wl)
    a = rl.prefill(x, ids, w, ex)
    b = rl.prefill(x, ids, w, ex)
    assert torch.equal(a, b)
    # doubling all weights doubles the output exactly
    c = rl.prefill(x, ids, w * 2, ex)
    assert torch.equal(c, 2 * a)
    # a zero-weight pair contributes nothing, whichever expert it names
    w0 = w.clone()
    w0[:, 3] = 0
    d1 = rl.prefill(x, ids, w0, ex)
    ids2 = ids.clone()
    ids2[:, 3] = (ids2[:, 3] + 5) % wl.experts.E
    d2 = rl.prefill(x, ids2, w0, ex)
    assert torch.equal(d1, d2)
    # x = 0 gives exactly 0
    z = rl.prefill(torch.zeros_like(x), ids, w, ex)
    assert torch.count_nonzero(z).item() == 0


def test_back_to_back_calls_no_sync(orc, rl, cases):
    """Two calls with different routing, different workspaces, one stream, no host sync in
    between: both correct (per-call tables never live in shared library buffers)."""
    import torch

    wl = _case(cases, "med_t1")
    x, ids, w, ex = to_device(wl)
    ids_b = torch.flip(ids, dims=[1]).contiguous()
    w_b = torch.flip(w, dims=[1]).contiguous()
    ws1 = rl.alloc_workspace(wl.T, wl.k, ex)
    ws2 = rl.alloc_workspace(wl.T, wl.k, ex)
    o1 = rl.prefill(x, ids, w, ex, ws=ws1)
    o2 = rl.prefill(x, ids_b, w_b, ex, ws=ws2)
    o3 = rl.prefill(x, ids, w, ex, ws=ws1)
    torch.cuda.synchronize()
    ref = orc.moe_workload(wl)
    assert rel_l2(o1.cpu().numpy(), ref) <= TOL
    ex_np = wl.experts
    ref_b = orc.moe_prefill(wl.x, wl.ids[:, ::-1].copy(), wl.w[:, ::-1].copy(), ex_np.arena, ex_np.desc, ex_np.E,
                            ex_np.H, ex_np.I)
    assert rel_l2(o2.cpu().numpy(), ref_b) <= TOL
    assert torch.equal(o1, o3)


@pytest.mark.parametrize("name", ["med_t1", "med_mixed"])
def test_repeated_calls_identical(rl, cases, name):
    """Ten calls in a row on one workspace (experts of more than 64 pairs, so work items span
    several chunks): every output finite and bit-identical to the first.  Catches reads of
    staged data before its loads complete, which show up as run-to-run differences."""
    import torch

    wl = _case(cases, name)
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    first = rl.prefill(x, ids, w, ex, ws=ws).clone()
    # the hook writes only the rows its layer uses: zeroed buffers, reused by every call
    bufs = [None if t is None else torch.zeros_like(t) for t in rl.gate_up(x, ids, w, ex, ws=ws)]
    rl.gate_up(x, ids, w, ex, ws=ws, h16=bufs[0], h8=bufs[1], hsc=bufs[2])
    h0 = [None if t is None else t.clone() for t in bufs]
    assert torch.isfinite(first).all()
    for _ in range(10):
        assert torch.equal(rl.prefill(x, ids, w, ex, ws=ws), first)
        rl.gate_up(x, ids, w, ex, ws=ws, h16=bufs[0], h8=bufs[1], hsc=bufs[2])
        for a_, b_ in zip(h0, bufs):
            assert (a_ is None and b_ is None) or torch.equal(a_, b_)


@pytest.mark.parametrize("name", ["med_t1", "tiny_q2b"])
def test_timed_hook_matches_prefill(rl, cases, name):
    """rl_moe_prefill_timed: the same output bits as rl_moe_prefill, and its events recorded in
    order on the call's stream (every interval non-negative)."""
    import torch

    wl = _case(cases, name)
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    ref = rl.prefill(x, ids, w, ex, ws=ws).clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(rl.TIMED_EVENTS)]
    stream = torch.cuda.current_stream()
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    rl.prefill_timed(x, ids, w, ex, out, ws, evs)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    gaps = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)]
    assert all(g >= 0.0 for g in gaps), gaps


@pytest.mark.parametrize("types", ["t1", "q2b"])
@pytest.mark.parametrize("shape", [dict(), dict(T=32, E=4, H=256, I=256, k=2), dict(T=16, E=3, H=256, I=1024, k=2)])
def test_large_y_exact_range(orc, rl, shape, types):
    """Down outputs far beyond the fp16 range are carried exactly in range: y waits for the
    ordered combine as fp16 under a power-of-two scale per (pair, 64-column tile), so the layer
    still meets the bar and stays finite.  Every down block of expert 0 is replaced (T1: d = 1e4,
    sub-scales 7, digits +1, weights 7e4; Q2B: d = 1e4, sub-scales 15, codes 3, weights 2.25e5),
    so a token's k outputs differ by ~10 orders of magnitude.  Shapes: the tiny layer (I = 64),
    I = 256 (down with activations in LDS) and I = 1024 (streamed down)."""
    wl = make_workload("tiny", seed=30, types=types, **shape)
    ex = wl.experts
    arena = ex.arena.copy()
    nblk = ex.H * ex.I // 256
    d = np.frombuffer(np.float16(6.0e4).tobytes(), np.uint8)
    if types == "t1":
        blk = np.concatenate([d, np.full(3, 0xFF, np.uint8), np.full(52, 242, np.uint8)])
        assert blk.size == BLOCK_BYTES[QTYPE_T1]
    else:
        blk = np.concatenate([d, np.full(72, 0xFF, np.uint8)])
        assert blk.size == BLOCK_BYTES[QTYPE_Q2B]
    off = int(ex.desc["down_off"][0])
    arena[off:off + nblk * blk.size] = np.tile(blk, nblk)
    import dataclasses

    big = dataclasses.replace(ex, arena=arena)
    wl = dataclasses.replace(wl, experts=big)
    x, ids, w, dev = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, dev)
    out = rl.prefill(x, ids, w, dev, ws=ws).cpu().numpy().astype(np.float64)
    assert rl.status(ws)[0] == 0
    ref = orc.moe_workload(wl)
    assert np.all(np.isfinite(out))
    log(f"large y {types} {shape}: max |out| {np.abs(ref).max():.3e}")
    assert np.abs(ref).max() > 1e5  # far beyond fp16 (65504)
    assert rel_l2(out, ref) <= TOL
    # tokens that did not use expert 0 are unaffected by it: each within the bar on its own
    clean = ~np.any(wl.ids == 0, axis=1)
    if clean.any():
        assert rel_l2(out[clean], ref[clean]) <= TOL


def test_empty_input(rl, cases):
    import torch

    wl = _case(cases, "tiny_q2b")
    _, _, _, ex = to_device(wl)
    ids = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    out = rl.prefill(x, ids, w, ex)
    assert out.shape == (0, 256)


def test_bad_expert_id_flagged(orc, rl, cases):
    wl = _case(cases, "tiny_q2b")
    x, ids, w, ex = to_device(wl)
    ids[5, 1] = wl.experts.E + 3
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, ids, w, ex, ws=ws).cpu().numpy()
    assert rl.status(ws)[0] & 1
    ref = orc.moe_workload(wl)
    keep = np.ones(wl.T, bool)
    keep[5] = False
    assert rel_l2(out[keep], ref[keep]) <= TOL


# ----------------------------------------------------------------------------- 1-2 rows
@pytest.mark.parametrize("types", ["t1", "q2b", "mixed"])
def test_decode_rows_parity_and_bit_identity(orc, rl, types):
    import torch

    ex_np = make_experts(64, 2048, 512, {"t1": QTYPE_T1, "q2b": QTYPE_Q2B, "mixed": [QTYPE_Q2B] * 32 + [QTYPE_T1] * 32}[types], seed=40)
    wl = make_workload("decode_t1", seed=41, T=2, experts=ex_np, E=64)
    wl.ids[1, :3] = wl.ids[0, :3]  # the two rows share some experts
    x, ids, w, ex = to_device(wl)
    log(f"decode {types}")
    two = rl.decode(x, ids, w, ex)
    one0 = rl.decode(x[:1], ids[:1], w[:1], ex)
    one1 = rl.decode(x[1:], ids[1:], w[1:], ex)
    assert torch.equal(two[0], one0[0])
    assert torch.equal(two[1], one1[0])
    ref = orc.moe_workload(wl)
    err = rel_l2(two.cpu().numpy(), ref)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
    # the matrix-vector path and the prefill path agree within the same bar
    pre = rl.prefill(x, ids, w, ex)
    assert rel_l2(two.cpu().numpy(), pre.cpu().numpy()) <= TOL


@pytest.mark.parametrize("H,I", [(8192, 256), (256, 4096), (1280, 768), (3584, 1536), (1792, 512), (3072, 3072)])
def test_decode_rows_max_dims(orc, rl, H, I):
    """The 1-2 row path at the largest hidden and intermediate sizes and at sizes whose columns
    per lane make an odd number of strips of 16 or 32 (mixed block types)."""
    import torch

    ex_np = make_experts(6, H, I, [QTYPE_Q2B] * 3 + [QTYPE_T1] * 3, seed=42)
    wl = make_workload("decode_t1", seed=43, T=2, experts=ex_np, E=6, H=H, I=I, k=3)
    x, ids, w, ex = to_device(wl)
    log(f"decode max dims H={H} I={I}")
    two = rl.decode(x, ids, w, ex)
    one1 = rl.decode(x[1:], ids[1:], w[1:], ex)
    assert torch.equal(two[1], one1[0])
    err = rel_l2(two.cpu().numpy(), orc.moe_workload(wl))
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL



@pytest.mark.parametrize("H,I", [(2304, 512), (4608, 256), (1024, 1280), (1024, 2560), (1024, 128)])
def test_decode_rows_refuses_sizes(rl, H, I):
    """Sizes outside the 1-2 row kernels' strip counts (H > 8 strips per lane, I > 4, I < 256)
    are refused on the host before any launch."""
    ex_np = make_experts(2, H, I, [QTYPE_Q2B, QTYPE_T1], seed=44)
    wl = make_workload("decode_t1", seed=45, T=1, experts=ex_np, E=2, H=H, I=I, k=2)
    x, ids, w, ex = to_device(wl)
    log(f"decode refuses H={H} I={I}")
    with pytest.raises(rl.RlError, match="size outside"):
        rl.decode(x, ids, w, ex)

# ----------------------------------------------------------------------------- full size
FULL = {
    "q2b_1090": dict(),
    "t1_2048": dict(),
    "mixed_2048": dict(),
    "ep8_2048": dict(),  # one GPU's expert share: 64 experts x ~320 pairs
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_parity(orc, rl, name):
    """Full-size layer on the GPU (the bench's launch configuration) against the oracle over every
    token: relative L2 over the whole output within the bar, and the worst token reported."""
    wl = make_workload(name, seed=7)
    cnt = np.bincount(wl.ids.ravel(), minlength=wl.experts.E)
    log(f"full {name} T={wl.T} pairs/expert min={cnt.min()} max={cnt.max()}")
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, ids, w, ex, ws=ws).cpu().numpy().astype(np.float64)
    assert rl.status(ws)[0] == 0
    ref = orc.moe_workload(wl)
    err = rel_l2(out, ref)
    per_tok = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    log(f"  rel_l2={err:.3e} worst token {per_tok.max():.3e}")
    assert err <= TOL
    assert np.all(np.isfinite(out))


def test_duplicate_ids_in_a_row(orc, rl):
    """Rows that name one expert more than once: each (token, slot) is its own pair, summed in
    selection order (the grouping orders equal experts by token, then slot).  Mixed block types;
    some rows name a single expert k times."""
    wl = make_workload("tiny", seed=51, T=200, H=512, E=16, I=256, k=6, types="mixed")
    rng = np.random.default_rng(52)
    ids = wl.ids.copy()
    dup = rng.random(wl.T) < 0.5
    ids[dup, 1] = ids[dup, 0]
    ids[dup, 4] = ids[dup, 2]
    ids[::17] = ids[::17, :1]  # every 17th row: one expert six times
    import dataclasses

    wl = dataclasses.replace(wl, ids=ids)
    x, dids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, dids, w, ex, ws=ws).cpu().numpy()
    assert rl.status(ws)[0] == 0
    err = rel_l2(out, orc.moe_workload(wl))
    log(f"duplicate ids rel_l2={err:.3e}")
    assert err <= TOL
    # the 1-2 row path on the first two rows (both with duplicates)
    two = rl.decode(x[:2].contiguous(), dids[:2].contiguous(), w[:2].contiguous(), ex).cpu().numpy()
    ref2 = orc.moe_prefill(wl.x[:2], ids[:2], wl.w[:2], wl.experts.arena, wl.experts.desc, wl.experts.E,
                           wl.experts.H, wl.experts.I)
    assert rel_l2(two, ref2) <= TOL


@pytest.mark.parametrize("R", [1, 2])
def test_decode_full_size(orc, rl, R):
    """The 1-2 row path at the bench's shape (512 T1 experts, H 2048, I 512, top-10), several
    seeded steps, each against the oracle."""
    import torch

    from workload.gen import _routing, gen_x

    wl = make_workload("t1_2048", seed=7)
    ex = rl.DeviceExperts.from_workload(wl.experts)
    e = wl.experts
    for s in range(4):
        i_np, w_np = _routing(R, e.E, wl.k, 900 + s)
        x_np = gen_x(R, e.H, 950 + s)
        out = rl.decode(torch.from_numpy(x_np.view(np.int16).copy()).cuda(), torch.from_numpy(i_np).cuda(),
                        torch.from_numpy(w_np).cuda(), ex).cpu().numpy()
        ref = orc.moe_prefill(x_np, i_np, w_np, e.arena, e.desc, e.E, e.H, e.I)
        err = rel_l2(out, ref)
        log(f"decode full size R={R} step {s} rel_l2={err:.3e}")
        assert err <= TOL


def test_decode_graph_replay(rl):
    """The 1-2 row path captured in a HIP graph (it records kernel launches only): several steps
    in one graph, replayed three times with eager calls and synchronisations in between; every
    replay gives the eager outputs bit for bit."""
    import torch

    from workload.gen import _routing, gen_x

    ex_np = make_experts(64, 2048, 512, [QTYPE_Q2B] * 32 + [QTYPE_T1] * 32, seed=44)
    ex = rl.DeviceExperts.from_workload(ex_np)
    steps = []
    for s in range(4):
        R = 1 + s % 2
        i_np, w_np = _routing(R, 64, 8, 700 + s)
        steps.append((torch.from_numpy(gen_x(R, 2048, 750 + s).view(np.int16).copy()).cuda(),
                      torch.from_numpy(i_np).cuda(), torch.from_numpy(w_np).cuda()))
    wss = [rl.alloc_workspace(2, 8, ex) for _ in steps]
    eager = [rl.decode(x, i, w, ex, ws=ws).clone() for (x, i, w), ws in zip(steps, wss)]
    outs = [torch.full_like(e, float("nan")) for e in eager]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (x, i, w), ws, o in zip(steps, wss, outs):
            rl.decode(x, i, w, ex, out=o, ws=ws)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for s, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (rep, s)
        x, i, w = steps[rep % len(steps)]
        rl.decode(x, i, w, ex)  # eager work between replays
        torch.cuda.synchronize()
    log("decode graph replays bit-identical")


@pytest.mark.parametrize("name", ["med_mixed", "i1024_t1"])
def test_prefill_graph_replay(rl, cases, name):
    """rl_moe_prefill captured in a HIP graph (it records kernel launches only: no allocation, no
    memset, no host synchronisation) with two calls on their own workspaces, replayed three times
    with eager calls in between: every replay gives the eager outputs bit for bit."""
    import torch

    wl = _case(cases, name)
    x, ids, w, ex = to_device(wl)
    ids2 = torch.flip(ids, dims=[1]).contiguous()
    w2 = torch.flip(w, dims=[1]).contiguous()
    wss = [rl.alloc_workspace(wl.T, wl.k, ex) for _ in range(2)]
    eager = [rl.prefill(x, i, ww, ex, ws=ws).clone() for (i, ww), ws in zip(((ids, w), (ids2, w2)), wss)]
    outs = [torch.full_like(e, float("nan")) for e in eager]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (i, ww), ws, o in zip(((ids, w), (ids2, w2)), wss, outs):
            rl.prefill(x, i, ww, ex, out=o, ws=ws)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for s, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (rep, s)
        rl.prefill(x, ids, w, ex)  # eager work between replays
        torch.cuda.synchronize()
    log(f"prefill graph replays bit-identical ({name})")


def test_gateup_matrices_far_apart(rl):
    """T1 experts whose gate and up matrices lie more than 2 GiB apart in the arena take the
    gate/up kernel whose windows use one buffer resource per matrix (the spanning resource needs
    both within 2^31 bytes): same experts, same inputs, bit-identical output to the compact layout
    (itself checked against the oracle by the other tests)."""
    import torch

    from workload import DESC_DTYPE

    wl = make_workload("t1_2048", seed=71, T=80, E=4, H=1024, I=256, k=2)
    x, ids, w, ex = to_device(wl)
    near = rl.prefill(x, ids, w, ex)
    e_np = wl.experts
    mb = e_np.H * e_np.I // 256 * BLOCK_BYTES[QTYPE_T1]
    far = 1 << 31
    desc = np.zeros(e_np.E, DESC_DTYPE)
    desc["qtype"] = QTYPE_T1
    src = torch.from_numpy(np.ascontiguousarray(e_np.arena)).cuda()
    arena = torch.zeros(far + 4 * e_np.E * mb + 64, dtype=torch.uint8, device="cuda")
    for e in range(e_np.E):
        g0 = 4 * e * mb
        u0 = far + 4 * e * mb  # up more than 2 GiB after gate
        d0 = g0 + 2 * mb
        for (which, dst) in (("gate_off", g0), ("up_off", u0), ("down_off", d0)):
            so = int(e_np.desc[which][e])
            arena[dst:dst + mb].copy_(src[so:so + mb])
            desc[which][e] = dst
    ex_far = rl.DeviceExperts(arena, desc, e_np.E, e_np.H, e_np.I)
    far_out = rl.prefill(x, ids, w, ex_far)
    assert torch.equal(near, far_out)
    log("gate/up with matrices 2 GiB apart: bit-identical")
    del arena, ex_far


def test_chunked_layer_bit_identical_to_one_call(orc, rl):
    """A layer taken as consecutive calls of at most 128 tokens (the 8,192-token workload runs as
    four 2,048-token calls) gives bit-identical outputs to one call over all its tokens: every
    output row's arithmetic (its decode, MFMA accumulation, scales, ordered combine) depends only
    on its own pairs, never on which rows share its tiles.  Mixed block types, a ragged last
    chunk; also checked against the oracle."""
    import torch

    from workload import make_workload

    wl = make_workload("tiny", seed=21, T=600, H=512, E=64, I=256, k=6, types="mixed")
    x, ids, w, dev = to_device(wl)
    T, H = wl.T, wl.experts.H
    log(f"chunked layer T={T} H={H} E={wl.experts.E} I={wl.experts.I} k={wl.k} chunks of 128")
    ws = rl.alloc_workspace(T, wl.k, dev)
    whole = rl.prefill(x, ids, w, dev, ws=ws).cpu().numpy()
    assert rl.status(ws)[0] == 0
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws_c = rl.alloc_workspace(128, wl.k, dev)
    for c0 in range(0, T, 128):
        c1 = min(T, c0 + 128)
        rl.prefill(x[c0:c1], ids[c0:c1], w[c0:c1], dev, out=out[c0:c1], ws=ws_c)
    chunked = out.cpu().numpy()
    assert rl.status(ws_c)[0] == 0
    assert np.array_equal(chunked.view(np.uint32), whole.view(np.uint32))
    err = rel_l2(chunked, orc.moe_workload(wl))
    log(f"  rel_l2 vs oracle {err:.3e}")
    assert err <= TOL
