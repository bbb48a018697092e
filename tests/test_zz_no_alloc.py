"""rl_moe_prefill_noalloc (the entry point for callers that cannot allocate device memory)
through the C ABI: bit-identical to rl_moe_prefill with its own workspace, on two calls in a row
(the second smaller, with other shapes, so it runs on what the first left in the shared static
buffer), both within the layer bar against the oracle; sizes beyond the buffer are refused."""
import numpy as np
import pytest

from gpu_util import log, rel_l2, to_device
from workload import make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def rl():
    import torch

    import routed_experts_bit_amd as rl

    assert torch.cuda.is_available()
    rl.lib()
    return rl


def _check_call(orc, rl, wl, name):
    import torch

    x, ids, w, ex = to_device(wl)
    ws = rl.alloc_workspace(wl.T, wl.k, ex)
    ref = rl.prefill(x, ids, w, ex, ws=ws)
    assert rl.status(ws)[0] == 0
    out = torch.full((wl.T, wl.experts.H), float("nan"), dtype=torch.float32, device="cuda")
    rl.prefill_noalloc(x, ids, w, ex, out)
    assert rl.noalloc_status()[0] == 0
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.cpu().numpy().view(np.uint32)), name
    err = rel_l2(got, orc.moe_workload(wl))
    log(f"noalloc {name}: T={wl.T} H={wl.experts.H} E={wl.experts.E} I={wl.experts.I} k={wl.k} rel_l2={err:.3e}")
    assert err <= TOL


def test_noalloc_matches_prefill_two_calls(orc, rl):
    # first call: 512 tokens of the 512-expert, top-10, H 2048, I 512 layer, mixed block types
    # (the largest chunk the buffer is sized for)
    big = make_workload("mixed_2048", seed=61, T=512)
    _check_call(orc, rl, big, "first (512 tokens, mixed)")
    # second call, smaller and with other shapes: T1 experts, I = 256, k = 4
    small = make_workload("t1_2048", seed=62, T=96, E=24, H=1024, I=256, k=4)
    _check_call(orc, rl, small, "second (96 tokens)")


def test_noalloc_refuses_beyond_buffer(rl):
    import torch

    wl = make_workload("t1_2048", seed=63, T=1024)  # needs ~75 MiB of workspace
    x, ids, w, ex = to_device(wl)
    assert rl.workspace_bytes(wl.T, wl.k, ex.E, ex.H, ex.I) > rl.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((wl.T, ex.H), dtype=torch.float32, device="cuda")
    with pytest.raises(rl.RlError, match="no-allocation scratch"):
        rl.prefill_noalloc(x, ids, w, ex, out)
    assert torch.count_nonzero(out).item() == 0  # nothing was launched


def test_noalloc_graph_replay(rl):
    """The allocation-free call captured in a HIP graph (its intended use: the call records only
    kernel launches, no allocation and no memset) and replayed three times, with eager calls of
    other shapes on the shared buffer between the replays: every replay gives the eager output
    bit for bit."""
    import torch

    wl = make_workload("t1_2048", seed=64, T=128, E=64)
    x, ids, w, ex = to_device(wl)
    ref = torch.empty((wl.T, ex.H), dtype=torch.float32, device="cuda")
    rl.prefill_noalloc(x, ids, w, ex, ref)
    other = make_workload("mixed_2048", seed=65, T=48, E=32, H=1024, I=512, k=6)
    xo, io, wo, exo = to_device(other)
    outo = torch.empty((other.T, exo.H), dtype=torch.float32, device="cuda")
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rl.prefill_noalloc(x, ids, w, ex, out)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        rl.prefill_noalloc(xo, io, wo, exo, outo)  # eager work on the same buffer between replays
        torch.cuda.synchronize()
    assert rl.noalloc_status()[0] == 0
    log("noalloc graph replays bit-identical")
