"""The seeded workloads have the load shapes their descriptions state (input recipe checks,
CPU): the 1,090-token layer's Zipf-biased routing is skewed (~20-40 pairs per expert for the
middle of the distribution, a long tail, no empty expert), the 2,048-token layer's uniform routing
gives ~40 pairs per expert with no empty expert, and every routing row selects k distinct experts."""
import numpy as np

from workload import CONFIGS, zipf_bias
from workload.gen import _routing

SEED = 1234  # the seed bench.py uses


def _route(name):
    """The routing make_workload(name, SEED) draws (seed + 2, Zipf permutation seed + 3),
    without building the experts."""
    cfg = CONFIGS[name]
    bias = zipf_bias(cfg["E"], SEED + 3) if cfg.get("bias") == "zipf" else None
    return _routing(cfg["T"], cfg["E"], cfg["k"], SEED + 2, bias)


def _counts(name):
    ids, _ = _route(name)
    return np.bincount(ids.ravel(), minlength=CONFIGS[name]["E"])


def test_q2b_1090_is_skewed():
    c = _counts("q2b_1090")
    assert c.sum() == 10900 and c.min() > 0
    p25, med, p75 = np.percentile(c, [25, 50, 75])
    assert 15 <= p25 and p75 <= 40 and 18 <= med <= 30
    assert c.max() >= 2.5 * med  # a long tail of hot experts


def test_t1_2048_is_uniform():
    c = _counts("t1_2048")
    assert c.sum() == 20480 and c.min() > 0
    assert abs(np.median(c) - 40) <= 2 and c.max() <= 2 * 40


def test_ep8_share_has_320_pairs_per_expert():
    c = _counts("ep8_2048")
    assert c.sum() == 20480 and CONFIGS["ep8_2048"]["E"] == 64
    assert abs(np.median(c) - 320) <= 20 and c.min() >= 240 and c.max() <= 400


def test_rows_select_distinct_experts_in_descending_weight():
    for name in ("q2b_1090", "t1_2048", "tiny", "ep8_2048"):
        ids, w = _route(name)
        assert all(len(set(r)) == CONFIGS[name]["k"] for r in ids.tolist())
        assert np.all(np.diff(w, axis=1) <= 0)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
