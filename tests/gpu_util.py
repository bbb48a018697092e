"""Helpers shared by the GPU tests: move a synthetic workload to the device."""
import numpy as np


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def to_device(wl, ex_dev=None):
    import torch

    import routed_experts_bit_amd as rl

    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    ids = torch.from_numpy(wl.ids.copy()).cuda()
    w = torch.from_numpy(wl.w.copy()).cuda()
    if ex_dev is None:
        ex_dev = rl.DeviceExperts.from_workload(wl.experts)
    return x, ids, w, ex_dev


def log(msg):
    print(msg, flush=True)
