"""Pins of the oracle's scalar conversions and block decoders (CPU only).

What pins them, none of which re-types the oracle's own formula:
  * fp16 -> double over all 65,536 patterns against numpy's float16, bf16 -> double over all
    patterns against torch's bfloat16 conversion (independent library code);
  * hand-worked Q2B and T1 blocks (tests/golden/*.json): literal expected values;
  * round trips through the packers (independent code in the encoding direction) of values
    that lie exactly on the quantisation grid;
  * bijection invariants: every T1 byte 0..242 decodes to the five digits whose base-3 value,
    least significant first, is that byte; every Q2B code byte decodes to the four codes whose
    base-4 value, least significant first, is that byte; each sub-scale only touches its own
    16 / 32 values.
"""
import json
import os

import numpy as np
import pytest
import torch

from workload import QTYPE_Q2B, QTYPE_T1, pack_q2b, pack_t1

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_fp16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.fp16_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.bf16_to_double(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref, equal_nan=True)


def _golden(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_t1_golden_block(orc):
    g = _golden("t1_block.json")
    blk = np.full(57, g["digit_bytes_default"], np.uint8)
    blk[0:5] = g["bytes_0_4"]
    for i, v in g["digit_bytes_override"].items():
        blk[5 + int(i)] = v
    vals = orc.dequant(QTYPE_T1, blk, 256)
    for o, want in g["expected"].items():
        assert vals[int(o)] == want, (o, vals[int(o)], want)


def test_q2b_golden_block(orc):
    g = _golden("q2b_block.json")
    blk = np.full(74, g["code_bytes_default"], np.uint8)
    blk[0:10] = g["bytes_0_9"]
    for i, v in g["code_bytes_override"].items():
        blk[10 + int(i)] = v
    vals = orc.dequant(QTYPE_Q2B, blk, 256)
    for o, want in g["expected"].items():
        assert vals[int(o)] == want, (o, vals[int(o)], want)


def test_t1_digit_bijection(orc):
    # d = 1.0, every sub-scale 1: decoded value = digit - 1.  Put byte b in digit slot 0.
    seen = set()
    for b in range(243):
        blk = np.full(57, 121, np.uint8)
        blk[0:2] = [0x00, 0x3C]
        sc = sum(1 << (3 * j) for j in range(8))
        blk[2:5] = [sc & 255, (sc >> 8) & 255, sc >> 16]
        blk[5] = b
        v = orc.dequant(QTYPE_T1, blk, 256)
        digits = [int(v[i]) + 1 for i in range(5)]
        assert all(0 <= dg <= 2 for dg in digits)
        assert sum(dg * 3**i for i, dg in enumerate(digits)) == b
        seen.add(tuple(digits))
        assert np.all(v[5:] == 0.0)
    assert len(seen) == 243


def test_t1_rejects_bytes_above_242(orc):
    blk = np.full(57, 121, np.uint8)
    blk[20] = 243
    with pytest.raises(ValueError):
        orc.dequant(QTYPE_T1, blk, 256)


def test_q2b_code_bijection(orc):
    # d = 2.0 and s = 1 everywhere: value = 2*(q - 1.5) = 2q - 3.
    for b in range(256):
        blk = np.full(74, 0x55, np.uint8)
        blk[0:2] = [0x00, 0x40]
        blk[2:10] = 0x11
        blk[10 + 7] = b  # values 28..31
        v = orc.dequant(QTYPE_Q2B, blk, 256)
        q = [(int(v[28 + i]) + 3) // 2 for i in range(4)]
        assert all(2 * qi - 3 == v[28 + i] for i, qi in enumerate(q))
        assert sum(qi * 4**i for i, qi in enumerate(q)) == b


@pytest.mark.parametrize("qtype,sub,bytes_", [(QTYPE_Q2B, 16, 74), (QTYPE_T1, 32, 57)])
def test_subscale_locality(orc, qtype, sub, bytes_):
    nsub = 256 // sub
    for j in range(nsub):
        blk = np.zeros(bytes_, np.uint8)
        blk[0:2] = [0x00, 0x3C]
        if qtype == QTYPE_Q2B:
            blk[2 + j // 2] = 5 << (4 * (j % 2))
            blk[10:] = 0xFF  # q = 3 everywhere
            want = 5 * 1.5
        else:
            sc = 3 << (3 * j)
            blk[2:5] = [sc & 255, (sc >> 8) & 255, sc >> 16]
            blk[5:] = 242  # digit 2 everywhere
            blk[56] = 2
            want = 3.0
        v = orc.dequant(qtype, blk, 256)
        inside = np.zeros(256, bool)
        inside[j * sub : (j + 1) * sub] = True
        assert np.all(v[inside] == want)
        assert np.all(v[~inside] == 0.0)


def _grid_values(rng, qtype, nb):
    """Values exactly on the quantisation grid whose packer output is unambiguous: every
    sub-block holds its largest magnitude at least once, so the packer recovers s and d."""
    if qtype == QTYPE_Q2B:
        d = np.float32(2.0**-7)
        s = rng.integers(1, 16, size=(nb, 16))
        s[:, 0] = 15
        q = rng.integers(0, 4, size=(nb, 16, 16))
        q[:, :, 0] = 3
        return (d * s[:, :, None] * (q - 1.5)).astype(np.float32).reshape(-1)
    d = np.float32(2.0**-6)
    s = rng.integers(1, 8, size=(nb, 8))
    s[:, 0] = 7
    t = rng.integers(-1, 2, size=(nb, 8, 32))
    t[:, :, 0] = 1
    return (d * s[:, :, None] * t).astype(np.float32).reshape(-1)


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
def test_packer_round_trip(orc, qtype):
    rng = np.random.default_rng(7)
    vals = _grid_values(rng, qtype, 24)
    blocks = pack_q2b(vals) if qtype == QTYPE_Q2B else pack_t1(vals)
    dec = orc.dequant(qtype, blocks.reshape(-1), vals.size)
    assert np.array_equal(dec, vals.astype(np.float64))


@pytest.mark.parametrize("qtype", [QTYPE_Q2B, QTYPE_T1])
def test_quantised_gaussian_close(orc, qtype):
    # A sanity bound on the packers (amax scaling: ternary rounds most Gaussian values to 0).
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(256 * 64) * 0.02).astype(np.float32)
    blocks = pack_q2b(w) if qtype == QTYPE_Q2B else pack_t1(w)
    dec = orc.dequant(qtype, blocks.reshape(-1), w.size)
    rel = np.linalg.norm(dec - w) / np.linalg.norm(w)
    assert rel < (0.45 if qtype == QTYPE_Q2B else 0.7)
