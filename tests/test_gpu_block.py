"""GPU parity of the MoE block (rl_moe_prefill_block: routed experts in selection order, then the
shared expert weighted by its per-token gate, then the residual) against the oracle's
orc_moe_block, through the C ABI.  Bar: relative L2 <= 2e-3 (float64, whole output) of the block
without the residual, and of the full block; special cases bit-exact: a zero gate and no residual
give rl_moe_prefill's output bit for bit."""
import numpy as np
import pytest

from gpu_util import log, rel_l2
from workload import make_block_workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


def _dev(bw):
    import torch

    import routed_experts_bit_amd as rl

    wl = bw.wl
    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    ids = torch.from_numpy(wl.ids.copy()).cuda()
    w = torch.from_numpy(wl.w.copy()).cuda()
    g = torch.from_numpy(bw.gate.copy()).cuda()
    r = torch.from_numpy(bw.residual.copy()).cuda()
    ex = rl.DeviceExperts.from_workload(wl.experts)
    return x, ids, w, g, r, ex


def _oracle(orc, bw, residual=True, ids=None, w=None, gate=None):
    wl = bw.wl
    ex = wl.experts
    return orc.moe_block(wl.x, wl.ids if ids is None else ids, wl.w if w is None else w, ex.arena, ex.desc, ex.E,
                         ex.H, ex.I, shared=bw.shared, shared_gate=bw.gate if gate is None else gate,
                         residual=bw.residual if residual else None)


CASES = {
    "tiny_q2b": lambda: make_block_workload("tiny", seed=81),
    "med_t1": lambda: make_block_workload("t1_2048", seed=82, T=256, E=32),
    "med_mixed": lambda: make_block_workload("mixed_2048", seed=83, T=200, E=24),
    "i1024_q2b": lambda: make_block_workload("q2b_1090", seed=84, T=64, E=8, H=1024, I=1024, k=3, bias=None),
    "i128_t1": lambda: make_block_workload("t1_2048", seed=85, T=96, E=16, H=1024, I=128, k=4),
    "k15": lambda: make_block_workload("mixed_2048", seed=86, T=40, E=64, H=256, I=256, k=15),
}


@pytest.mark.parametrize("name", list(CASES))
def test_block_parity(orc, rl, name):
    bw = CASES[name]()
    wl = bw.wl
    log(f"block {name}: T={wl.T} k={wl.k}+shared E={wl.experts.E} H={wl.experts.H} I={wl.experts.I}")
    x, ids, w, g, r, ex = _dev(bw)
    out = rl.prefill_block(x, ids, w, ex, bw.shared, g, r).cpu().numpy().astype(np.float64)
    ref = _oracle(orc, bw)
    res = bw.residual.astype(np.float64)
    e_block = rel_l2(out - res, ref - res)
    e_all = rel_l2(out, ref)
    log(f"  rel_l2 block {e_block:.3e}, with residual {e_all:.3e}")
    assert e_block <= TOL and e_all <= TOL
    nores = rl.prefill_block(x, ids, w, ex, bw.shared, g).cpu().numpy()
    assert rel_l2(nores, _oracle(orc, bw, residual=False)) <= TOL


def test_block_zero_gate_is_prefill(rl):
    """With a zero gate and no residual the block is the routed layer, bit for bit (the shared
    pairs add exactly 0 at the end of each token's ordered sum)."""
    import torch

    bw = CASES["med_mixed"]()
    x, ids, w, g, r, ex = _dev(bw)
    a = rl.prefill_block(x, ids, w, ex, bw.shared, torch.zeros_like(g))
    b = rl.prefill(x, ids, w, ex)
    assert torch.equal(a, b)


def test_block_shared_alone(orc, rl):
    """k = 0: every token is its shared expert's pair alone (the hottest possible expert: one
    pair per token, split into many work records)."""
    import torch

    bw = make_block_workload("t1_2048", seed=87, T=300, E=16, H=1024, I=512)
    x, _, _, g, r, ex = _dev(bw)
    T = bw.wl.T
    ids0 = torch.zeros((T, 0), dtype=torch.int32, device="cuda")
    w0 = torch.zeros((T, 0), dtype=torch.float32, device="cuda")
    out = rl.prefill_block(x, ids0, w0, ex, bw.shared, g, r).cpu().numpy().astype(np.float64)
    ref = _oracle(orc, bw, ids=np.zeros((T, 0), np.int32), w=np.zeros((T, 0), np.float32))
    res = bw.residual.astype(np.float64)
    err = rel_l2(out - res, ref - res)
    log(f"block shared alone T={T}: rel_l2 {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name", ["t1_2048", "q2b_1090"])
def test_block_full_size(orc, rl, name):
    """The full-size layers with a shared expert (2,048 or 1,090 of its pairs, one per token) and
    the residual, against the oracle over every token."""
    bw = make_block_workload(name, seed=7)
    wl = bw.wl
    x, ids, w, g, r, ex = _dev(bw)
    import torch

    ws = torch.empty(rl.workspace_bytes(wl.T, wl.k + 1, ex.E, ex.H, ex.I), dtype=torch.uint8, device="cuda")
    out = rl.prefill_block(x, ids, w, ex, bw.shared, g, r, ws=ws).cpu().numpy().astype(np.float64)
    assert rl.status(ws)[0] == 0
    ref = _oracle(orc, bw)
    res = bw.residual.astype(np.float64)
    err = rel_l2(out - res, ref - res)
    log(f"block full {name}: T={wl.T} rel_l2 {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("types", ["t1", "mixed"])
def test_decode_block(orc, rl, types):
    """The 1-2 row path with the shared expert and the residual: against the oracle, each row of a
    2-row call bit-identical to a 1-row call, and within the bar of the prefill block."""
    import torch

    name = {"t1": "t1_2048", "mixed": "mixed_2048"}[types]
    bw = make_block_workload(name, seed=88, T=2, E=64)
    wl = bw.wl
    wl.ids[1, :3] = wl.ids[0, :3]  # the rows share some experts
    x, ids, w, g, r, ex = _dev(bw)
    two = rl.decode_block(x, ids, w, ex, bw.shared, g, r)
    one0 = rl.decode_block(x[:1].contiguous(), ids[:1].contiguous(), w[:1].contiguous(), ex, bw.shared,
                           g[:1].contiguous(), r[:1].contiguous())
    one1 = rl.decode_block(x[1:].contiguous(), ids[1:].contiguous(), w[1:].contiguous(), ex, bw.shared,
                           g[1:].contiguous(), r[1:].contiguous())
    assert torch.equal(two[0], one0[0]) and torch.equal(two[1], one1[0])
    got = two.cpu().numpy().astype(np.float64)
    ref = _oracle(orc, bw)
    res = bw.residual.astype(np.float64)
    err = rel_l2(got - res, ref - res)
    log(f"decode block {types}: rel_l2 {err:.3e}")
    assert err <= TOL
    pre = rl.prefill_block(x, ids, w, ex, bw.shared, g, r).cpu().numpy().astype(np.float64)
    assert rel_l2(got - res, pre - res) <= TOL
