"""The bounded expert cache on the GPU (rl_cache_*): layers run on a cache's slots give the same
bits as on the whole resident arena (decoded weights are exact, and every output row's arithmetic
depends only on its own pairs), through many prepares with evictions.  The 2-row verify prepares
the union of both rows' experts once, then runs each row with its own selection order."""
import numpy as np
import pytest

from gpu_util import log, rel_l2
from workload import make_block_workload
from workload.gen import _routing, gen_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


@pytest.fixture(scope="module")
def layer(rl):
    import torch

    bw = make_block_workload("mixed_2048", seed=95, T=64)  # 512 routed experts (half Q2B, half T1) + shared
    ex = bw.wl.experts
    full = rl.DeviceExperts.from_workload(ex)
    host = torch.from_numpy(ex.arena).pin_memory()  # the model in pinned host memory
    return bw, full, host


def test_decode_verify_steps_through_cache(rl, layer):
    import torch

    bw, full, host = layer
    ex = bw.wl.experts
    cache = rl.ExpertCache(host, ex.desc, ex.E, ex.H, ex.I, n_slots=48)
    k = 10
    for step in range(40):
        R = 1 + step % 2
        ids_np, w_np = _routing(R, 512, k, 500 + step)  # routed experts 0..511
        x = torch.from_numpy(gen_x(R, ex.H, 600 + step).view(np.int16).copy()).cuda()
        ids = torch.from_numpy(ids_np).cuda()
        w = torch.from_numpy(w_np).cuda()
        g = torch.from_numpy(bw.gate[:R].copy()).cuda()
        r = torch.from_numpy(bw.residual[:R].copy()).cuda()
        # one prepare of the union of both rows' experts (and the shared expert)
        view = cache.prepare(np.concatenate([ids_np.ravel(), [bw.shared]]))
        got = rl.decode_block(x, ids, w, view, bw.shared, g, r)
        ref = rl.decode_block(x, ids, w, full, bw.shared, g, r)
        assert torch.equal(got, ref), step
        got2 = rl.decode(x, ids, w, view)
        assert torch.equal(got2, rl.decode(x, ids, w, full)), step
    st = cache.stats()
    log(f"cache after 40 steps: {st}")
    assert st["evictions"] > 0 and st["hits"] > 0


def test_prefill_chunks_through_cache(rl, layer):
    """64-token chunks: the union of a chunk's experts prepared, then the prefill on the slots;
    bit-identical to the whole arena."""
    import torch

    bw, full, host = layer
    ex = bw.wl.experts
    cache = rl.ExpertCache(host, ex.desc, ex.E, ex.H, ex.I, n_slots=400)
    wl = bw.wl
    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    for c0 in range(0, wl.T, 32):
        ids_np = wl.ids[c0:c0 + 32]
        view = cache.prepare(ids_np)
        ids = torch.from_numpy(ids_np.copy()).cuda()
        w = torch.from_numpy(wl.w[c0:c0 + 32].copy()).cuda()
        got = rl.prefill(x[c0:c0 + 32], ids, w, view)
        assert torch.equal(got, rl.prefill(x[c0:c0 + 32], ids, w, full)), c0
    log(f"prefill chunks: {cache.stats()}")


def test_union_larger_than_cache_refused(rl, layer):
    bw, full, host = layer
    ex = bw.wl.experts
    cache = rl.ExpertCache(host, ex.desc, ex.E, ex.H, ex.I, n_slots=12)
    ids_np, _ = _routing(2, 512, 10, 700)
    if len(set(ids_np.ravel().tolist())) > 12:
        with pytest.raises(rl.RlError, match="cache slots"):
            cache.prepare(ids_np)
    # each row alone fits
    cache.prepare(ids_np[:1])
