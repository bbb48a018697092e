"""A seeded sweep of layer shapes: the GPU prefill (and, on a third of the cases, the MoE block
and the 1-2 row path on the first rows) against the oracle, through the C ABI.

Each case draws its hidden size H (multiples of 256 up to 2048), intermediate size I (64, 128 and
multiples of 256 up to 1024, i.e. the three down kernels and both h layouts), expert count E,
top-k (up to 16, at most E), token count T (up to 256, with T * k at most 1,024 so the oracle
finishes in about a second), block types (Q2B, T1 or both), routing (uniform or Zipf-skewed, so
that some experts exceed 96 pairs and are cut into several records) and, on every fifth case,
rows that name one expert more than once.  Bar: relative L2 <= 2e-3 (float64, whole output), the
status word clear."""
import dataclasses

import numpy as np
import pytest

from gpu_util import log, rel_l2, to_device
from workload import make_block_workload, make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-3
N_CASES = 24
HS = [256, 512, 768, 1024, 1536, 2048]
IS = [64, 128, 256, 512, 768, 1024]
TYPES = ["q2b", "t1", "mixed"]


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


def _shape(i):
    rng = np.random.default_rng(9000 + i)
    H = int(rng.choice(HS))
    I = int(rng.choice(IS))
    E = int(rng.integers(1, 65))
    k = int(rng.integers(1, min(16, E) + 1))
    T = int(rng.integers(1, min(256, 1024 // k) + 1))
    return dict(T=T, E=E, k=k, H=H, I=I, types=TYPES[i % 3], bias="zipf" if i % 4 == 3 else None,
                dup=i % 5 == 4, block=i % 3 == 1)


def _rows_dim_ok(d, max_strips):
    """The sizes the 1-2 row call takes, as its declaration states: a multiple of 256 whose d/16
    columns per lane split into at most max_strips strips of 64, 32 or 16 columns."""
    if d < 256 or d % 256:
        return False
    per_lane = d // 16
    strip = 64 if per_lane % 64 == 0 else (32 if per_lane % 32 == 0 else 16)
    return per_lane // strip <= max_strips


def _dups(wl, seed):
    """Rows naming one expert twice (half the rows) or k times (every 7th row)."""
    if wl.k < 2:
        return wl
    rng = np.random.default_rng(seed)
    ids = wl.ids.copy()
    half = rng.random(wl.T) < 0.5
    ids[half, 1] = ids[half, 0]
    ids[::7] = ids[::7, :1]
    return dataclasses.replace(wl, ids=ids)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_prefill(orc, rl, i):
    s = _shape(i)
    over = {key: s[key] for key in ("E", "k", "H", "I", "types", "bias")}
    wl = make_workload("t1_2048", seed=9100 + i, T=s["T"], **over)
    if s["dup"]:
        wl = _dups(wl, 9200 + i)
    log(f"sweep {i}: T={wl.T} k={wl.k} E={wl.experts.E} H={wl.experts.H} I={wl.experts.I} types={s['types']} "
        f"bias={s['bias']} dup={s['dup']} max pairs/expert={np.bincount(wl.ids.ravel()).max()}")
    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    out = rl.prefill(x, ids, w, ex, ws=ws).cpu().numpy()
    assert rl.status(ws)[0] == 0
    err = rel_l2(out, orc.moe_workload(wl))
    log(f"  prefill rel_l2={err:.3e}")
    assert err <= TOL
    if s["block"]:
        # the 1-2 row path on the first rows; sizes it does not cover must be refused
        R = min(2, wl.T)
        if not (_rows_dim_ok(wl.experts.H, 8) and _rows_dim_ok(wl.experts.I, 4)):
            with pytest.raises(rl.RlError, match="size outside"):
                rl.decode(x[:R].contiguous(), ids[:R].contiguous(), w[:R].contiguous(), ex)
            log(f"  {R}-row call refused (H={wl.experts.H}, I={wl.experts.I})")
            return
        rows = rl.decode(x[:R].contiguous(), ids[:R].contiguous(), w[:R].contiguous(), ex).cpu().numpy()
        ref = orc.moe_prefill(wl.x[:R], wl.ids[:R], wl.w[:R], wl.experts.arena, wl.experts.desc, wl.experts.E,
                              wl.experts.H, wl.experts.I)
        e_rows = rel_l2(rows, ref)
        log(f"  {R}-row rel_l2={e_rows:.3e}")
        assert e_rows <= TOL


@pytest.mark.parametrize("i", [j for j in range(N_CASES) if _shape(j)["block"]])
def test_sweep_block(orc, rl, i):
    import torch

    s = _shape(i)
    over = {key: s[key] for key in ("E", "k", "H", "I", "types", "bias")}
    bw = make_block_workload("t1_2048", seed=9300 + i, T=s["T"], **over)
    wl = bw.wl
    log(f"sweep block {i}: T={wl.T} k={wl.k}+shared E={wl.experts.E} H={wl.experts.H} I={wl.experts.I}")
    ex = rl.DeviceExperts.from_workload(wl.experts)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = rl.prefill_block(dev(wl.x.view(np.int16)), dev(wl.ids), dev(wl.w), ex, bw.shared, dev(bw.gate),
                           dev(bw.residual)).cpu().numpy().astype(np.float64)
    ref = orc.moe_block(wl.x, wl.ids, wl.w, wl.experts.arena, wl.experts.desc, wl.experts.E, wl.experts.H,
                        wl.experts.I, shared=bw.shared, shared_gate=bw.gate, residual=bw.residual)
    res = bw.residual.astype(np.float64)
    err = rel_l2(out - res, ref - res)
    log(f"  block rel_l2={err:.3e}")
    assert err <= TOL
