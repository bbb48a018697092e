"""Build the HIP library librl_moe.so (gfx950 only) in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "rl_moe.hip"), os.path.join(PKG, "csrc", "rl_cache.hip")]
LIB = os.path.join(PKG, "librl_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Kernels whose step loops count their outstanding buffer-to-LDS loads by hand (s_waitcnt with
# fixed counts) and are tuned for two waves per SIMD: they must compile with no scratch (spill
# code would add vector-memory operations to those loops and cost what the tuning bought) and
# keep two waves per SIMD.  The 1-2 row kernels must have no scratch either.
TUNED = ("k_t1_f8ILi0E", "k_q2_mmILi0E", "k_t1_dn", "k_q2_dn")
NO_SCRATCH = TUNED + ("k_gv_gateup", "k_gv_down")


def kernel_resources(remarks: str) -> dict:
    """Per kernel (mangled name): {"scratch": bytes per lane, "occupancy": waves per SIMD,
    "vgprs": VGPRs}, from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in body:
            key, val = (t.strip() for t in body.rsplit(":", 1))
            name = {"ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy", "VGPRs": "vgprs"}.get(key)
            if name is not None:
                out[cur][name] = int(val)
    return out


def check_resources(res: dict) -> list:
    """The violations of the rules above (empty when the build is acceptable)."""
    bad = []
    for fn, r in res.items():
        if any(k in fn for k in NO_SCRATCH) and r.get("scratch", 0) != 0:
            bad.append(f"{fn}: {r['scratch']} bytes of scratch per lane")
        if any(k in fn for k in TUNED) and r.get("occupancy", 2) < 2:
            bad.append(f"{fn}: {r['occupancy']} wave(s) per SIMD")
    return bad


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(PKG, "csrc"), "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    diag = "\n".join(l for l in proc.stderr.splitlines() if "kernel-resource-usage" not in l and l.strip()
                     and not l.lstrip().startswith(("|", "^")) and not l.lstrip()[:1].isdigit())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr[-4000:]}")
    if verbose and diag:
        print(diag, flush=True)
    res = kernel_resources(proc.stderr)
    bad = check_resources(res)
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernel resources out of bounds:\n  " + "\n  ".join(bad))
    if verbose:
        spill = sorted(fn for fn, r in res.items() if r.get("scratch", 0))
        print(f"{len(res)} kernels; with scratch (untuned paths): {len(spill)}", flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
