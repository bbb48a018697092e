"""GPU parity of the router (rl_moe_route) against the CPU oracle's router, through the C ABI.

Bars: the selected ids are bit-exact (both sides decide on the fp32 logits themselves, ties to
the lower id); the weights agree with the oracle's double-precision weights to 4e-6 relative
per weight.  Derivation: the kernel computes exp(l_j - m) in fp32 (the subtraction of two fp32
logits rounds to at most half an ulp of |l_j - m| < 32, i.e. <= 1.9e-6 absolute, and expf is
within about 2 ulp), sums k <= 16 terms in fp32 (<= 16 x 6e-8) and divides once (6e-8): about
3e-6 relative in the worst case, 4e-6 with margin.
"""
import numpy as np
import pytest

from gpu_util import log
from workload import gen_logits, zipf_bias

pytestmark = pytest.mark.gpu

WTOL = 4e-6


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


def _run(rl, lg, k):
    import torch

    ids, w = rl.route(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize(
    "T,E,k,bias",
    [(64, 8, 2, False), (1090, 512, 10, True), (2048, 512, 10, False), (33, 1024, 16, False), (7, 13, 13, False),
     (5, 1, 1, False), (130, 100, 3, False), (50, 200, 7, False), (17, 700, 12, False)],
)
def test_route_parity(orc, rl, T, E, k, bias):
    log(f"route parity T={T} E={E} k={k} bias={bias}")
    lg = gen_logits(T, E, seed=2000 + E + k, bias=zipf_bias(E, 77) if bias else None)
    ids, w = _run(rl, lg, k)
    rids, rw = orc.route(lg, k)
    assert np.array_equal(ids, rids)
    rel = np.abs(w.astype(np.float64) - rw) / rw
    log(f"  max relative weight error {rel.max():.3e}")
    assert rel.max() <= WTOL


def test_route_ties(orc, rl):
    rng = np.random.default_rng(11)
    lg = rng.integers(-3, 4, size=(300, 64)).astype(np.float32)  # many equal logits per row
    ids, w = _run(rl, lg, 8)
    rids, rw = orc.route(lg, 8)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw) / rw) <= WTOL


def test_route_empty(rl):
    import torch

    ids, w = rl.route(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 4)
    assert ids.shape == (0, 4) and w.shape == (0, 4)


def test_route_then_layer_matches_oracle_routing(orc, rl):
    """The layer fed by the GPU router equals the layer fed by the oracle's router: same ids,
    and weights within the router bar, so the outputs agree to far below the layer bar."""
    import torch

    from gpu_util import rel_l2
    from workload import make_workload

    wl = make_workload("tiny", seed=5)
    lg = gen_logits(wl.T, wl.experts.E, seed=9)
    ids, w = rl.route(torch.from_numpy(lg).cuda(), wl.k)
    rids, rw = orc.route(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    dev = rl.DeviceExperts.from_workload(wl.experts)
    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    ws = rl.alloc_workspace(wl.T, wl.k, dev)
    out = rl.prefill(x, ids, w, dev, ws=ws).cpu().numpy()
    ref = orc.moe_prefill(wl.x, rids, rw.astype(np.float32), wl.experts.arena, wl.experts.desc, wl.experts.E,
                          wl.experts.H, wl.experts.I)
    err = rel_l2(out, ref)
    log(f"  routed tiny layer rel_l2 {err:.3e}")
    assert err <= 2e-3 and rl.status(ws)[0] == 0


@pytest.mark.parametrize("k", [5, 7, 9])
def test_routed_layer_other_k(orc, rl, k):
    """Router then layer for k values that the other layer tests do not use (one combine
    instance per k): E = 16 experts, H = 256, I = 64 (Q2B), 80 tokens."""
    import torch

    from gpu_util import rel_l2
    from workload import make_experts

    T, E, H, I = 80, 16, 256, 64
    ex = make_experts(E, H, I, 1, seed=40 + k)
    from workload import gen_x

    x = gen_x(T, H, seed=50 + k)
    lg = gen_logits(T, E, seed=60 + k)
    ids, w = rl.route(torch.from_numpy(lg).cuda(), k)
    rids, rw = orc.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    dev = rl.DeviceExperts.from_workload(ex)
    ws = rl.alloc_workspace(T, k, dev)
    out = rl.prefill(torch.from_numpy(x.view(np.int16).copy()).cuda(), ids, w, dev, ws=ws).cpu().numpy()
    ref = orc.moe_prefill(x, rids, rw.astype(np.float32), ex.arena, ex.desc, E, H, I)
    err = rel_l2(out, ref)
    log(f"  k={k} routed layer rel_l2 {err:.3e}")
    assert err <= 2e-3 and rl.status(ws)[0] == 0


# ----------------------------------------------------------------------------- router fused with the grouping
@pytest.mark.parametrize(
    "name,T,E,k,shared,ties",
    [("tiny", 64, 8, 2, False, False), ("t1_2048", 300, 64, 10, False, False), ("mixed_2048", 257, 48, 7, True, False),
     ("t1_2048", 2048, 512, 10, False, False), ("q2b_1090", 1090, 512, 10, True, False),
     ("mixed_2048", 199, 32, 16, False, True)],
)
def test_prefill_from_logits(orc, rl, name, T, E, k, shared, ties):
    """rl_moe_prefill_from_logits routes in the grouping's first launch: its topk_ids equal the
    oracle router's bit for bit (weights within 4e-6, and bit-identical to rl_moe_route's), and its
    layer output is bit-identical to rl_moe_prefill (or rl_moe_prefill_block) on that routing --
    the pairs' sorted order is unique, so the token-aligned grouping tiles change nothing."""
    import torch

    from workload import make_block_workload

    bw = make_block_workload(name, seed=300 + k, T=T, E=E, k=k)
    wl = bw.wl
    ex = rl.DeviceExperts.from_workload(wl.experts)
    if ties:
        lg = np.random.default_rng(301).integers(-2, 3, size=(T, E)).astype(np.float32)
    else:
        lg = gen_logits(T, E, seed=302 + E, bias=zipf_bias(E, 303) if name == "q2b_1090" else None)
    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    lgd = torch.from_numpy(lg).cuda()
    g = torch.from_numpy(bw.gate).cuda()
    r = torch.from_numpy(bw.residual).cuda()
    sh = bw.shared if shared else -1
    log(f"from logits {name} T={T} E={E}(+shared) k={k} shared={shared} ties={ties}")
    out, ids, w = rl.prefill_from_logits(x, lgd, k, ex, shared=sh, gate=g, residual=r)
    rids, rw = orc.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert (np.abs(w.cpu().numpy().astype(np.float64) - rw) / rw).max() <= WTOL
    ids2, w2 = rl.route(lgd, k)
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    if shared:
        ref = rl.prefill_block(x, ids, w, ex, bw.shared, g, r)
    else:
        ref = rl.prefill(x, ids, w, ex)
    assert torch.equal(out, ref)
