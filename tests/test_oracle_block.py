"""Pins of the oracle's MoE block (orc_moe_block): the routed experts' ordered sum, then the shared
expert weighted by its per-token gate, then the residual (CPU only).

  * the shared expert alone (k = 0) is g_t times one plain dense SwiGLU FFN -- checked against
    numpy float64 matrix products on the decoded weights (a library primitive, another summation
    order), for Q2B and T1 shared experts;
  * the whole block (routed, shared, residual; some tokens also route to the shared expert)
    against a numpy brute force;
  * special cases exact in double: a zero gate leaves the routed layer bit for bit; zero routed
    weights and a zero gate leave the residual exactly.
"""
import numpy as np
import pytest

from workload import QTYPE_Q2B, QTYPE_T1, make_experts, make_workload, gen_x


def _dense(orc, ex, e):
    H, I = ex.H, ex.I
    q = int(ex.desc["qtype"][e])
    Wg = orc.dequant(q, ex.matrix(e, "gate"), I * H).reshape(I, H)
    Wu = orc.dequant(q, ex.matrix(e, "up"), I * H).reshape(I, H)
    Wd = orc.dequant(q, ex.matrix(e, "down"), H * I).reshape(H, I)
    return Wg, Wu, Wd


def _xf(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ffn(orc, ex, e, xf):
    Wg, Wu, Wd = _dense(orc, ex, e)
    g, u = xf @ Wg.T, xf @ Wu.T
    return (g / (1.0 + np.exp(-g)) * u) @ Wd.T


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
def test_shared_alone_is_dense_ffn(orc, qtype):
    ex = make_experts(4, 256, 128, [QTYPE_T1, QTYPE_Q2B, QTYPE_T1, qtype], seed=71)
    T = 11
    x = gen_x(T, 256, 72)
    g = np.random.default_rng(73).uniform(0.1, 1.0, T).astype(np.float32)
    ids = np.zeros((T, 0), np.int32)
    w = np.zeros((T, 0), np.float32)
    got = orc.moe_block(x, ids, w, ex.arena, ex.desc, 4, 256, 128, shared=3, shared_gate=g)
    ref = g.astype(np.float64)[:, None] * _ffn(orc, ex, 3, _xf(x))
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_block_matches_numpy(orc):
    wl = make_workload("tiny", seed=74, T=30, E=8, k=3, types="mixed")
    ex = wl.experts
    ids = wl.ids.copy()
    ids[::4, 1] = 7  # some tokens also route to the shared expert (an independent pair)
    shared = 7
    rng = np.random.default_rng(75)
    g = rng.uniform(0.0, 1.0, wl.T).astype(np.float32)
    r = rng.standard_normal((wl.T, ex.H)).astype(np.float32)
    got = orc.moe_block(wl.x, ids, wl.w, ex.arena, ex.desc, ex.E, ex.H, ex.I, shared=shared, shared_gate=g, residual=r)
    xf = _xf(wl.x)
    ref = np.zeros((wl.T, ex.H))
    for t in range(wl.T):
        for j in range(wl.k):
            ref[t] += float(wl.w[t, j]) * _ffn(orc, ex, int(ids[t, j]), xf[t:t + 1])[0]
    ref += g.astype(np.float64)[:, None] * _ffn(orc, ex, shared, xf)
    ref += r
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_zero_gate_leaves_routed_layer(orc):
    wl = make_workload("tiny", seed=76, T=20, E=8, k=2, types="mixed")
    ex = wl.experts
    routed = orc.moe_workload(wl)
    got = orc.moe_block(wl.x, wl.ids, wl.w, ex.arena, ex.desc, ex.E, ex.H, ex.I, shared=5,
                        shared_gate=np.zeros(wl.T, np.float32))
    assert np.array_equal(got, routed)


def test_zero_weights_leave_residual(orc):
    wl = make_workload("tiny", seed=77, T=9, E=8, k=2)
    ex = wl.experts
    r = np.random.default_rng(78).standard_normal((wl.T, ex.H)).astype(np.float32)
    got = orc.moe_block(wl.x, wl.ids, np.zeros_like(wl.w), ex.arena, ex.desc, ex.E, ex.H, ex.I, shared=0,
                        shared_gate=np.zeros(wl.T, np.float32), residual=r)
    assert np.array_equal(got, r.astype(np.float64))


def test_block_rejects_bad_shared(orc):
    wl = make_workload("tiny", seed=79, T=4)
    ex = wl.experts
    for bad in (-1, ex.E):
        with pytest.raises(ValueError):
            orc.moe_block(wl.x, wl.ids, wl.w, ex.arena, ex.desc, ex.E, ex.H, ex.I, shared=bad,
                          shared_gate=np.ones(wl.T, np.float32))
