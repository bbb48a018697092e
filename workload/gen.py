"""Seeded generators for the routed-expert MoE workloads.

Block formats (the pages name ~1.75-bit and ~2.3-bit i-quants for the experts but never
give their bit layout; the two synthetic formats below stand in for them, with the
plainest byte layout the format description supports):

Q2B, 256 values per block, 74 bytes (2.3125 bits/weight)
    bytes 0..1    d, IEEE half, little-endian
    bytes 2..9    16 sub-scales of 4 bits; sub-block j (values 16j..16j+15) uses the
                  low nibble of byte 2 + j//2 when j is even, the high nibble when odd
    bytes 10..73  2-bit codes q; value o sits in byte 10 + o//4 at bits 2*(o%4)
    value         w = d * s_j * (q - 1.5)

T1, 256 values per block, 57 bytes (1.78125 bits/weight)
    bytes 0..1    d, IEEE half, little-endian
    bytes 2..4    24-bit little-endian word of 8 sub-scales of 3 bits; sub-block j
                  (values 32j..32j+31) uses bits 3j..3j+2
    bytes 5..56   ternary digits, five per byte, least significant first: value o is
                  base-3 digit o%5 of byte 5 + o//5 (byte 56 holds only value 255)
    value         w = d * s_j * (digit - 1)

A matrix of R rows x C columns (rows are output features, the input dimension is
contiguous) is flattened row-major and cut into consecutive 256-value blocks.

Nothing here decodes blocks or computes any part of the expert layer.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

QTYPE_Q2B = 1
QTYPE_T1 = 2
BLOCK_VALUES = 256
BLOCK_BYTES = {QTYPE_Q2B: 74, QTYPE_T1: 57}
MATRIX_ALIGN = 256

DESC_DTYPE = np.dtype(
    [("qtype", "<i4"), ("reserved", "<i4"), ("gate_off", "<u8"), ("up_off", "<u8"), ("down_off", "<u8")]
)
assert DESC_DTYPE.itemsize == 32


# ----------------------------------------------------------------------------- bf16 inputs
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_x(T: int, H: int, seed: int) -> np.ndarray:
    """Activations x ~ N(0,1), rounded to bf16 before either path sees them."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


# ----------------------------------------------------------------------------- routing
def zipf_bias(E: int, seed: int, alpha: float = 1.1, beta: float = 0.1) -> np.ndarray:
    """Per-expert logit bias beta*ln(r^-alpha) for a seeded rank permutation r of 1..E."""
    rng = np.random.Generator(np.random.PCG64(seed))
    r = rng.permutation(E) + 1
    return beta * (-alpha * np.log(r.astype(np.float64)))


def route_softmax_topk(logits: np.ndarray, k: int):
    """Softmax over experts, top-k by descending probability (ties to the lower id), then the
    k probabilities renormalised to sum to one (summed in selection order).

    Column j of the returned ids is the j-th selection; that column order is the order in
    which the layer sums its experts.
    """
    lg = np.asarray(logits, dtype=np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    ptop = np.take_along_axis(p, order, axis=1)
    tot = np.zeros(ptop.shape[0])
    for j in range(k):
        tot = tot + ptop[:, j]
    w = ptop / tot[:, None]
    return order.astype(np.int32), w.astype(np.float32)


# ----------------------------------------------------------------------------- packers
def _fp16_bytes(d: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(d.astype(np.float16)).view(np.uint8).reshape(-1, 2)


def pack_q2b(w: np.ndarray) -> np.ndarray:
    """Quantise float values (length a multiple of 256) to Q2B blocks; returns uint8 [nb, 74]."""
    v = np.asarray(w, dtype=np.float32).reshape(-1, 16, 16)
    nb = v.shape[0]
    ideal = np.abs(v).max(axis=2) / np.float32(1.5)  # per sub-block scale that maps amax to 1.5
    d16 = (ideal.max(axis=1) / np.float32(15.0)).astype(np.float16)
    d = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d[:, None] > 0, np.rint(ideal / d[:, None]), 0.0)
    s = np.clip(s, 0, 15).astype(np.uint8)
    step = d[:, None] * s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(step[..., None] > 0, np.floor(v / step[..., None] + 2.0), 1.0)
    q = np.clip(q, 0, 3).astype(np.uint8).reshape(nb, 256)
    out = np.zeros((nb, 74), dtype=np.uint8)
    out[:, 0:2] = _fp16_bytes(d16)
    out[:, 2:10] = s[:, 0::2] | (s[:, 1::2] << 4)
    qq = q.reshape(nb, 64, 4)
    out[:, 10:74] = qq[:, :, 0] | (qq[:, :, 1] << 2) | (qq[:, :, 2] << 4) | (qq[:, :, 3] << 6)
    return out


_POW3 = np.array([1, 3, 9, 27, 81], dtype=np.uint16)


def pack_t1(w: np.ndarray) -> np.ndarray:
    """Quantise float values (length a multiple of 256) to T1 blocks; returns uint8 [nb, 57]."""
    v = np.asarray(w, dtype=np.float32).reshape(-1, 8, 32)
    nb = v.shape[0]
    ideal = np.abs(v).max(axis=2)
    d16 = (ideal.max(axis=1) / np.float32(7.0)).astype(np.float16)
    d = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d[:, None] > 0, np.rint(ideal / d[:, None]), 0.0)
    s = np.clip(s, 0, 7).astype(np.uint32)
    step = d[:, None] * s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(step[..., None] > 0, np.rint(v / step[..., None]), 0.0)
    digit = (np.clip(t, -1, 1) + 1).astype(np.uint16).reshape(nb, 256)
    out = np.zeros((nb, 57), dtype=np.uint8)
    out[:, 0:2] = _fp16_bytes(d16)
    sc = np.zeros(nb, dtype=np.uint32)
    for j in range(8):
        sc |= s[:, j] << (3 * j)
    out[:, 2] = sc & 0xFF
    out[:, 3] = (sc >> 8) & 0xFF
    out[:, 4] = (sc >> 16) & 0xFF
    dd = np.zeros((nb, 260), dtype=np.uint16)
    dd[:, :256] = digit
    out[:, 5:57] = (dd.reshape(nb, 52, 5) * _POW3).sum(axis=2).astype(np.uint8)
    # the last byte covers values 255..259 of which only 255 exists; the padding digits are 0
    return out


def pack_matrix(w: np.ndarray, qtype: int) -> np.ndarray:
    flat = np.asarray(w, dtype=np.float32).reshape(-1)
    if flat.size % BLOCK_VALUES:
        raise ValueError("matrix size must be a multiple of 256 values")
    if qtype == QTYPE_Q2B:
        return pack_q2b(flat).reshape(-1)
    if qtype == QTYPE_T1:
        return pack_t1(flat).reshape(-1)
    raise ValueError(f"unknown qtype {qtype}")


def matrix_bytes(rows: int, cols: int, qtype: int) -> int:
    return (rows * cols // BLOCK_VALUES) * BLOCK_BYTES[qtype]


def _align(n: int, a: int = MATRIX_ALIGN) -> int:
    return (n + a - 1) // a * a


# ----------------------------------------------------------------------------- experts
@dataclass
class Experts:
    """Packed experts: one uint8 arena plus a 32-byte descriptor per expert.

    gate and up are [I x H] (row = intermediate feature), down is [H x I] (row = hidden
    feature); each starts at a 256-byte aligned offset of the arena.
    """

    arena: np.ndarray
    desc: np.ndarray
    E: int
    H: int
    I: int

    @property
    def qtypes(self) -> np.ndarray:
        return self.desc["qtype"]

    def matrix(self, e: int, which: str) -> np.ndarray:
        q = int(self.desc["qtype"][e])
        rows, cols = (self.H, self.I) if which == "down" else (self.I, self.H)
        off = int(self.desc[which + "_off"][e])
        return self.arena[off : off + matrix_bytes(rows, cols, q)]


def _layout(qtypes, H, I):
    desc = np.zeros(len(qtypes), dtype=DESC_DTYPE)
    off = 0
    for e, q in enumerate(qtypes):
        desc[e]["qtype"] = q
        for which, (r, c) in (("gate_off", (I, H)), ("up_off", (I, H)), ("down_off", (H, I))):
            desc[e][which] = off
            off = _align(off + matrix_bytes(r, c, q))
    return desc, off


def make_experts(E: int, H: int, I: int, qtypes, seed: int, std: float = 0.02, threads: int | None = None) -> Experts:
    """Weights ~ N(0, std^2) per matrix, quantised to each expert's block type.

    Each (expert, matrix) has its own PCG64 stream keyed by (seed, expert, matrix), so the
    result does not depend on the thread count.
    """
    qtypes = np.broadcast_to(np.asarray(qtypes, dtype=np.int32), (E,)).copy()
    desc, total = _layout(qtypes, H, I)
    arena = np.zeros(total, dtype=np.uint8)

    def one(e: int):
        q = int(qtypes[e])
        for mi, (which, (r, c)) in enumerate((("gate_off", (I, H)), ("up_off", (I, H)), ("down_off", (H, I)))):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, e, mi])))
            w = rng.standard_normal(r * c, dtype=np.float32) * np.float32(std)
            b = pack_matrix(w, q)
            o = int(desc[e][which])
            arena[o : o + b.size] = b

    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr <= 1 or E == 1:
        for e in range(E):
            one(e)
    else:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, range(E)))
    return Experts(arena=arena, desc=desc, E=E, H=H, I=I)


# ----------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    x: np.ndarray  # uint16 bf16 bits [T, H]
    ids: np.ndarray  # int32 [T, k]
    w: np.ndarray  # float32 [T, k]
    experts: Experts
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def k(self):
        return self.ids.shape[1]


def gen_logits(T: int, E: int, seed: int, bias=None) -> np.ndarray:
    """Router logits as fp32 [T, E]: N(0,1) (+ a per-expert bias), the inputs of the router row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((T, E))
    if bias is not None:
        logits = logits + bias[None, :]
    return logits.astype(np.float32)


def _routing(T, E, k, seed, bias=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((T, E))
    if bias is not None:
        logits = logits + bias[None, :]
    return route_softmax_topk(logits, k)


# Shapes and recipes of the synthetic workloads (hidden H, experts E, intermediate I, top-k).
CONFIGS = {
    "tiny": dict(T=64, H=256, E=8, I=64, k=2, types="q2b", bias=None),
    "q2b_1090": dict(T=1090, H=2048, E=512, I=512, k=10, types="q2b", bias="zipf"),
    "t1_2048": dict(T=2048, H=2048, E=512, I=512, k=10, types="t1", bias=None),
    "mixed_2048": dict(T=2048, H=2048, E=512, I=512, k=10, types="mixed", bias=None),
    # 8,192 tokens taken as four consecutive 2,048-token calls (chunk: tokens per call)
    "mixed_8192": dict(T=8192, H=2048, E=512, I=512, k=10, types="mixed", bias=None, chunk=2048),
    "decode_t1": dict(T=2, H=2048, E=512, I=512, k=10, types="t1", bias=None),
    # one GPU's share of the 512-expert T1 layer sharded by expert over 8 GPUs with 2,048 tokens
    # per GPU: 64 experts, ~320 pairs each (the received rows stand in as 2,048 tokens x top-10 of
    # the 64 local experts)
    "ep8_2048": dict(T=2048, H=2048, E=64, I=512, k=10, types="t1", bias=None),
}


def _qtypes(kind: str, E: int):
    if kind == "q2b":
        return np.full(E, QTYPE_Q2B, np.int32)
    if kind == "t1":
        return np.full(E, QTYPE_T1, np.int32)
    if kind == "mixed":  # the lower half of the expert ids Q2B, the upper half T1
        return np.where(np.arange(E) < E // 2, QTYPE_Q2B, QTYPE_T1).astype(np.int32)
    raise ValueError(kind)


def make_workload(name: str, seed: int = 1234, T: int | None = None, experts: Experts | None = None, **over) -> Workload:
    """Build one of CONFIGS (optionally with T or shape overrides).  Seeds: weights `seed`,
    x `seed+1`, routing `seed+2`."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if T is not None:
        cfg["T"] = T
    T, H, E, I, k = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["k"]
    if experts is None:
        experts = make_experts(E, H, I, _qtypes(cfg["types"], E), seed)
    x = gen_x(T, H, seed + 1)
    bias = zipf_bias(E, seed + 3) if cfg.get("bias") == "zipf" else None
    ids, w = _routing(T, E, k, seed + 2, bias)
    return Workload(name=name, x=x, ids=ids, w=w, experts=experts, seed=seed, meta=cfg)


@dataclass
class BlockWorkload:
    """A layer workload plus the rest of the MoE block: the shared expert (descriptor `shared` of
    wl.experts, after the routed experts 0..shared-1 that wl.ids route to), its per-token gate and
    the residual stream."""

    wl: Workload
    shared: int
    gate: np.ndarray      # float32 [T], the shared expert's weight per token
    residual: np.ndarray  # float32 [T, H]


def make_block_workload(name: str, seed: int = 1234, T: int | None = None, **over) -> BlockWorkload:
    """Workload `name` with one more expert, the shared one, of the block type of the last routed
    expert (weights from the same per-(seed, expert, matrix) streams, so the routed experts equal
    make_workload's), a gate sigmoid(N(0,1)) per token (seed+4) and a residual N(0,1) fp32
    (seed+5)."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if T is not None:
        cfg["T"] = T
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    qt = _qtypes(cfg["types"], E)
    experts = make_experts(E + 1, H, I, np.concatenate([qt, qt[-1:]]), seed)
    routed = make_workload(name, seed=seed, experts=experts, **{k_: v for k_, v in cfg.items() if k_ in ("T", "H", "E", "I", "k", "types")})
    Tn = routed.T
    rng = np.random.Generator(np.random.PCG64(seed + 4))
    gate = (1.0 / (1.0 + np.exp(-rng.standard_normal(Tn)))).astype(np.float32)
    residual = np.random.Generator(np.random.PCG64(seed + 5)).standard_normal((Tn, H), dtype=np.float32)
    return BlockWorkload(wl=routed, shared=E, gate=gate, residual=residual)
