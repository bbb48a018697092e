"""Pins of the oracle's pair grouping, per-pair FFN and ordered combine (CPU only).

  * grouping: brute force against Python's sorted() on (expert, token, slot) and the
    invariants (permutation of all pairs, offsets = exclusive scan of the histogram);
  * FFN: with k = 1 and weight 1 the layer is one plain dense SwiGLU FFN -- checked against
    numpy float64 matrix products on the decoded weights (a library primitive, another
    summation order); the whole tiny layer against a numpy brute force over tokens;
  * combine invariants, exact in double: x = 0 gives 0; a zero-weight pair contributes
    nothing whatever expert it names; doubling every weight doubles the output; a consistent
    relabelling of experts and blobs changes nothing; results do not depend on threads.
"""
import numpy as np
import pytest

from workload import DESC_DTYPE, QTYPE_Q2B, QTYPE_T1, Experts, make_experts, make_workload


def _brute_group(ids, E):
    T, k = ids.shape
    pairs = sorted(range(T * k), key=lambda p: (int(ids.flat[p]), p // k, p % k))
    counts = np.bincount(ids.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inv = np.empty(T * k, np.int32)
    inv[np.array(pairs, dtype=np.int64)] = np.arange(T * k)
    return offsets, np.array(pairs, np.int32), inv


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 3, 5, 1), (40, 10, 16, 2), (33, 2, 64, 3), (0, 4, 8, 4)])
def test_group_pairs_brute_force(orc, T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, max(E // 3, 1), size=(T, k)).astype(np.int32)  # many empty experts and duplicates
    offsets, src, inv = orc.group_pairs(ids, E)
    o2, s2, i2 = _brute_group(ids, E)
    assert np.array_equal(offsets, o2)
    assert np.array_equal(src, s2)
    assert np.array_equal(inv, i2)
    assert sorted(src.tolist()) == list(range(T * k))
    assert np.array_equal(src[inv], np.arange(T * k))


def test_group_pairs_rejects_bad_ids(orc):
    ids = np.array([[0, 3]], np.int32)
    with pytest.raises(ValueError):
        orc.group_pairs(ids, 3)
    with pytest.raises(ValueError):
        orc.group_pairs(np.array([[-1]], np.int32), 3)


def _dense(ex, e):
    H, I = ex.H, ex.I
    q = int(ex.desc["qtype"][e])
    import oracle

    Wg = oracle.dequant(q, ex.matrix(e, "gate"), I * H).reshape(I, H)
    Wu = oracle.dequant(q, ex.matrix(e, "up"), I * H).reshape(I, H)
    Wd = oracle.dequant(q, ex.matrix(e, "down"), H * I).reshape(H, I)
    return Wg, Wu, Wd


def _xf(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _numpy_layer(wl):
    ex = wl.experts
    dense = {e: _dense(ex, e) for e in np.unique(wl.ids)}
    xf = _xf(wl.x)
    out = np.zeros((wl.T, ex.H))
    for j in range(wl.k):
        for e in np.unique(wl.ids[:, j]):
            rows = np.nonzero(wl.ids[:, j] == e)[0]
            Wg, Wu, Wd = dense[e]
            g = xf[rows] @ Wg.T
            u = xf[rows] @ Wu.T
            h = g / (1.0 + np.exp(-g)) * u
            out[rows] += wl.w[rows, j].astype(np.float64)[:, None] * (h @ Wd.T)
    return out


@pytest.fixture(scope="module")
def tiny():
    return make_workload("tiny", seed=11)


def test_tiny_layer_matches_numpy(orc, tiny):
    got = orc.moe_workload(tiny)
    ref = _numpy_layer(tiny)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_single_expert_weight_one_is_dense_ffn(orc):
    ex = make_experts(3, 256, 128, [QTYPE_T1, QTYPE_Q2B, QTYPE_T1], seed=5)
    from workload import gen_x

    x = gen_x(9, 256, 6)
    for e in range(3):
        ids = np.full((9, 1), e, np.int32)
        w = np.ones((9, 1), np.float32)
        got = orc.moe_prefill(x, ids, w, ex.arena, ex.desc, 3, 256, 128)
        Wg, Wu, Wd = _dense(ex, e)
        xf = _xf(x)
        g, u = xf @ Wg.T, xf @ Wu.T
        ref = (g / (1 + np.exp(-g)) * u) @ Wd.T
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_zero_input_gives_zero(orc, tiny):
    ex = tiny.experts
    out = orc.moe_prefill(np.zeros_like(tiny.x), tiny.ids, tiny.w, ex.arena, ex.desc, ex.E, ex.H, ex.I)
    assert np.all(out == 0.0)


def test_zero_weight_pair_contributes_nothing(orc, tiny):
    ex = tiny.experts
    w = tiny.w.copy()
    w[:, 1] = 0.0
    a = orc.moe_prefill(tiny.x, tiny.ids, w, ex.arena, ex.desc, ex.E, ex.H, ex.I)
    ids2 = tiny.ids.copy()
    ids2[:, 1] = (ids2[:, 1] + 3) % ex.E
    b = orc.moe_prefill(tiny.x, ids2, w, ex.arena, ex.desc, ex.E, ex.H, ex.I)
    assert np.array_equal(a, b)
    # and equals the k = 1 layer of the remaining pair
    c = orc.moe_prefill(tiny.x, tiny.ids[:, :1].copy(), w[:, :1].copy(), ex.arena, ex.desc, ex.E, ex.H, ex.I)
    assert np.array_equal(a, c)


def test_doubling_weights_doubles_output(orc, tiny):
    ex = tiny.experts
    a = orc.moe_prefill(tiny.x, tiny.ids, tiny.w, ex.arena, ex.desc, ex.E, ex.H, ex.I)
    b = orc.moe_prefill(tiny.x, tiny.ids, tiny.w * 2, ex.arena, ex.desc, ex.E, ex.H, ex.I)
    assert np.array_equal(b, 2 * a)


def test_relabelling_experts(orc, tiny):
    ex = tiny.experts
    perm = np.random.default_rng(1).permutation(ex.E)  # new label of old expert e is perm[e]
    desc2 = np.zeros(ex.E, DESC_DTYPE)
    desc2[perm] = ex.desc
    ex2 = Experts(ex.arena, desc2, ex.E, ex.H, ex.I)
    a = orc.moe_workload(tiny)
    b = orc.moe_prefill(tiny.x, perm[tiny.ids].astype(np.int32), tiny.w, ex2.arena, ex2.desc, ex.E, ex.H, ex.I)
    assert np.array_equal(a, b)


def test_thread_count_and_token_subset(orc):
    wl = make_workload("tiny", seed=12, T=40, E=16, k=4)
    a = orc.moe_workload(wl, threads=1)
    b = orc.moe_workload(wl, threads=8)
    assert np.array_equal(a, b)
    sub = np.array([39, 0, 17], np.int32)
    c = orc.moe_workload(wl, tokens=sub, threads=3)
    assert np.array_equal(c, a[sub])


def test_selection_order_matters_only_by_rounding(orc):
    # Reversing the selection order changes the summation order; the result moves by
    # rounding only (the combine is a sum), never by more.
    wl = make_workload("tiny", seed=13, T=16, E=8, k=4)
    ex = wl.experts
    a = orc.moe_workload(wl)
    b = orc.moe_prefill(wl.x, wl.ids[:, ::-1].copy(), wl.w[:, ::-1].copy(), ex.arena, ex.desc, ex.E, ex.H, ex.I)
    assert np.max(np.abs(a - b)) <= 1e-14 * np.max(np.abs(a))


def test_pair_h_output(orc, tiny):
    out, h = orc.moe_workload(tiny, want_h=True)
    ex = tiny.experts
    t, j = 5, 1
    e = int(tiny.ids[t, j])
    Wg, Wu, _ = _dense(ex, e)
    xf = _xf(tiny.x[t])
    g, u = Wg @ xf, Wu @ xf
    ref = g / (1 + np.exp(-g)) * u
    assert np.max(np.abs(h[t, j] - ref)) <= 1e-12 * np.max(np.abs(ref))
