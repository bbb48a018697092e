"""The HIP library's block decoder (rl_decode.h, host+device code) run on the CPU through a
small harness, against the oracle, bit-exactly: every strip width the kernels use (64-value
strips of gate/up rows, 16/32-value strips of short down rows), bf16 and fp16 operands, and
block addresses at every alignment mod 4.  Catches indexing mistakes before any GPU run."""
import ctypes as C
import os
import subprocess

import numpy as np
import pytest

from workload import QTYPE_Q2B, QTYPE_T1, BLOCK_BYTES, make_experts

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("hd") / "libhd.so")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "routed_experts_bit_amd", "csrc"),
           os.path.join(HERE, "host", "host_decode.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    L = C.CDLL(out)
    L.hd_decode.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int64, C.c_void_p]
    L.hd_decode.restype = C.c_int
    L.hd_t1f8.argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
    L.hd_t1f8.restype = C.c_int
    L.hd_q2w.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
    L.hd_q2w.restype = C.c_int
    return L


def _blocks(qtype, nb, seed):
    ex = make_experts(1, 256, 64, qtype, seed=seed, threads=1)  # 3 matrices of 64 blocks each
    raw = ex.matrix(0, "gate")
    blk = np.concatenate([raw, ex.matrix(0, "down")])
    nb = min(nb, blk.size // BLOCK_BYTES[qtype])
    blk = blk[: nb * BLOCK_BYTES[qtype]].copy()
    rng = np.random.default_rng(seed)
    # make sure extreme fields appear: all scales, every code / digit byte value
    bb = BLOCK_BYTES[qtype]
    view = blk.reshape(nb, bb)
    if qtype == QTYPE_Q2B:
        view[:, 2:10] = rng.integers(0, 256, size=(nb, 8))
        view[:, 10:] = rng.integers(0, 256, size=(nb, 64))
    else:
        view[:, 2:5] = rng.integers(0, 256, size=(nb, 3))
        view[:, 5:56] = rng.integers(0, 243, size=(nb, 51))
        view[:, 56] = rng.integers(0, 3, size=nb)
    return blk, nb


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
@pytest.mark.parametrize("f16", [0, 1])
@pytest.mark.parametrize("strip", [16, 32, 64])
@pytest.mark.parametrize("mis", [0, 1, 2, 3])
def test_strip_decoder_matches_oracle(orc, harness, qtype, f16, strip, mis):
    blk, nb = _blocks(qtype, 40, seed=100 + qtype)
    # the decoder reads whole aligned dwords around each block: keep the buffer 4-aligned and
    # padded, and place the blocks at every misalignment
    buf = np.zeros(blk.size + 32, np.uint8)
    buf[mis : mis + blk.size] = blk
    out = np.empty(nb * 256, np.float32)
    base = buf.ctypes.data
    rc = harness.hd_decode(qtype, f16, strip, base + mis, nb, out.ctypes.data)
    assert rc == 0
    ref = orc.dequant(qtype, blk, nb * 256)
    assert np.array_equal(out.astype(np.float64), ref), np.nonzero(out != ref)[0][:10]


@pytest.mark.parametrize("mis", [0, 1, 2, 3])
def test_t1_fp8_byte_strips(orc, harness, mis):
    """The fp8 operands of the T1 path: every block position is covered exactly once through
    t1_kmap, with the right digit and sub-scale (per-dword table choice, tail bytes), at every
    block misalignment; zero-scale blocks decode to zero."""
    blk, nb = _blocks(QTYPE_T1, 40, seed=77)
    blk = blk.reshape(nb, BLOCK_BYTES[QTYPE_T1]).copy()
    blk[5, 0:2] = 0  # d = 0 (fp16 +0) with non-zero digits and sub-scales
    blk = blk.ravel()
    buf = np.zeros(blk.size + 32, np.uint8)
    buf[mis: mis + blk.size] = blk
    out = np.full(nb * 256, np.nan, np.float32)
    assert harness.hd_t1f8(buf.ctypes.data + mis, nb, out.ctypes.data) == 0
    ref = orc.dequant(QTYPE_T1, blk, nb * 256)
    assert not np.isnan(out).any()
    assert np.array_equal(out.astype(np.float64), ref), np.nonzero(out != ref)[0][:10]


@pytest.mark.parametrize("f16", [0, 1])
@pytest.mark.parametrize("mis", [0, 1, 2, 3])
def test_q2b_16bit_strips(orc, harness, f16, mis):
    """The bf16 / fp16 operands of the Q2B path on the 16-bit MFMA: every block position is
    covered exactly once through q2_kmap, with the right code and sub-scale, at every block
    misalignment (a 4-aligned matrix only has 0 and 2); zero-scale blocks decode to zero."""
    blk, nb = _blocks(QTYPE_Q2B, 40, seed=78 + f16)
    blk = blk.reshape(nb, BLOCK_BYTES[QTYPE_Q2B]).copy()
    blk[7, 0:2] = 0  # d = 0 (fp16 +0) with non-zero codes and sub-scales
    blk[8, 0:2] = [0x00, 0x80]  # d = -0
    blk = blk.ravel()
    buf = np.zeros(blk.size + 32, np.uint8)
    buf[mis: mis + blk.size] = blk
    out = np.full(nb * 256, np.nan, np.float32)
    assert harness.hd_q2w(buf.ctypes.data + mis, nb, f16, out.ctypes.data) == 0
    ref = orc.dequant(QTYPE_Q2B, blk, nb * 256)
    assert not np.isnan(out).any()
    assert np.array_equal(out.astype(np.float64), ref), np.nonzero(out != ref)[0][:10]
