"""Seeded synthetic inputs for the routed top-k MoE layer on codebook-quantized experts.

This module is the only code shared by the oracle side and the HIP side.  It draws
random numbers and lays random bytes out in the stream layouts; it contains none of
the method's arithmetic (no grid expansion, no dequantization, no routing).

Random numbers come from one counter-based generator: output ``i`` of stream
``(seed, tag)`` is the SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) applied to ``key + (i + 1) * golden``,
with ``key`` itself a finalised hash of ``seed`` and the FNV-1a hash of ``tag``.
Every value is therefore a pure function of (seed, tag, index).

Stream layouts (one quantized matrix of ``rows x cols``, ``cols % 256 == 0``;
blocks run along the input dimension, NB = cols/256 super-blocks, NG = cols/8 groups):

IQ2_XS-like (qtype 1), 70 bytes per 256 weights:
  qs  u16[rows][NG]  bits 0-8 grid index, bits 9-15 sign of weights 0-6 (1 = negative);
                     weight 7's sign is the parity of bits 9-15
  sc  u32[rows][NB]  nibble i = 4-bit scale of the 32-weight sub-block i
  d   u16[rows][NB]  IEEE binary16 super-block scale (finite, normal, > 0)

IQ1_M-like (qtype 2), 56 bytes per 256 weights:
  ql  u8[rows][NG]     grid index bits 0-7
  qh  u8[rows][NG/2]   group g uses nibble (g & 1) of byte g/2: bits 0-2 = index
                       bits 8-10, bit 3 = delta sign (1 = minus)
  sd  u64[rows][NB]    bits 0-15 binary16 d; bits 16+3i..18+3i = 3-bit scale of the
                       16-weight sub-block i

IQ1_S-like (qtype 4), 50 bytes per 256 weights, the same 2048 x 8 ternary grid:
  ql  u8[rows][NG]     grid index bits 0-7
  qh  u16[rows][NG/4]  one word per 32-weight sub-block: bits 3i..3i+2 = index bits
                       8-10 of the sub-block's group i (i = 0..3), bits 12-14 = 3-bit
                       scale, bit 15 = delta sign of the whole sub-block (1 = minus)
  d   u16[rows][NB]    binary16 super-block scale

Compact grids: one u16 per grid row, symbol j (0, 1 or 2) in bits 2j..2j+1.
IQ2_XS-like: 512 distinct rows; IQ1_M-like: 2048 distinct rows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

QTYPE_IQ2XS = 1
QTYPE_IQ1M = 2
QTYPE_IQ1S = 4
QTYPE_NAMES = {QTYPE_IQ2XS: "iq2xs", QTYPE_IQ1M: "iq1m", QTYPE_IQ1S: "iq1s"}

GRID_ROWS = {QTYPE_IQ2XS: 512, QTYPE_IQ1M: 2048}

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Default seeds, echoed by every test and benchmark line that uses them.
SEED_GRIDS = 20240601
SEED_BANK = 7
SEED_INPUT = 11


def _fnv1a64(tag: str) -> int:
    h = 0xCBF29CE484222325
    for b in tag.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, tag: str) -> np.uint64:
    s = np.array([(seed * 0x9E3779B97F4A7C15 ^ _fnv1a64(tag)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(s)[0]


def u64(seed: int, tag: str, n: int, start: int = 0) -> np.ndarray:
    """Outputs ``start .. start+n-1`` of stream (seed, tag) as uint64."""
    k = _key(seed, tag)
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(k + i * _GOLDEN)


def uniform(seed: int, tag: str, n: int) -> np.ndarray:
    """float64 uniform on the open interval (0, 1): 53 high bits, centred."""
    v = u64(seed, tag, n) >> np.uint64(11)
    return (v.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, tag: str, n: int) -> np.ndarray:
    """float32 N(0, 1) by the Box-Muller transform (cosine branch)."""
    u1 = uniform(seed, tag + "/bm1", n)
    u2 = uniform(seed, tag + "/bm2", n)
    return (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)).astype(np.float32)


def random_bytes(seed: int, tag: str, nbytes: int) -> np.ndarray:
    words = (nbytes + 7) // 8
    return u64(seed, tag, words).view(np.uint8)[:nbytes].copy()


# ----------------------------------------------------------------------------- grids

def grid_compact(qtype: int, seed: int = SEED_GRIDS) -> np.ndarray:
    """Seeded compact grid: distinct rows of 8 symbols drawn uniformly from {0, 1, 2}.

    Row r, attempt a uses generator output r*64 + a; a row equal to an earlier one is
    rejected and the next attempt is drawn.  Symbol j is byte j of the output mod 3.
    """
    rows = GRID_ROWS[qtype]
    draws = u64(seed, "grid/" + QTYPE_NAMES[qtype], rows * 64)
    seen = set()
    out = np.zeros(rows, dtype=np.uint16)
    for r in range(rows):
        for a in range(64):
            v = int(draws[r * 64 + a])
            code = 0
            for j in range(8):
                code |= (((v >> (8 * j)) & 0xFF) % 3) << (2 * j)
            if code not in seen:
                seen.add(code)
                out[r] = code
                break
        else:  # pragma: no cover - 64 consecutive duplicates cannot happen for these sizes
            raise RuntimeError("grid generation failed")
    return out


# ----------------------------------------------------------------------------- matrices

def stream_bytes(qtype: int, rows: int, cols: int) -> tuple[int, int, int]:
    """Byte sizes of the three streams of one rows x cols matrix."""
    if cols % 256 or rows <= 0 or cols <= 0:
        raise ValueError("cols must be a positive multiple of 256")
    ng, nb = cols // 8, cols // 256
    if qtype == QTYPE_IQ2XS:
        return rows * ng * 2, rows * nb * 4, rows * nb * 2
    if qtype == QTYPE_IQ1M:
        return rows * ng, rows * ng // 2, rows * nb * 8
    if qtype == QTYPE_IQ1S:
        return rows * ng, rows * (ng // 4) * 2, rows * nb * 2
    raise ValueError(f"unknown qtype {qtype}")


def matrix_bytes(qtype: int, rows: int, cols: int) -> int:
    return sum(stream_bytes(qtype, rows, cols))


# d0 * U(0.75, 1.25) with d0 = C / sqrt(cols) puts the weight RMS near 1/sqrt(cols).
_D_CONST = {QTYPE_IQ2XS: 3.29e-4 * math.sqrt(2048.0), QTYPE_IQ1M: 2.90e-3 * math.sqrt(2048.0),
            QTYPE_IQ1S: 2.90e-3 * math.sqrt(2048.0)}


def _fp16_scales(seed: int, tag: str, n: int, qtype: int, cols: int) -> np.ndarray:
    d0 = _D_CONST[qtype] / math.sqrt(cols)
    u = uniform(seed, tag + "/d", n)
    return (d0 * (0.75 + 0.5 * u)).astype(np.float16).view(np.uint16)


def qbank(qtype: int, n: int, rows: int, cols: int, seed: int, tag: str) -> list[np.ndarray]:
    """``n`` matrices of one shape, each stream as a uint8 array [n][stream_bytes]."""
    b0, b1, b2 = stream_bytes(qtype, rows, cols)
    s0 = random_bytes(seed, tag + "/s0", n * b0).reshape(n, b0)
    s1 = random_bytes(seed, tag + "/s1", n * b1).reshape(n, b1)
    nb_total = n * rows * (cols // 256)
    if qtype in (QTYPE_IQ2XS, QTYPE_IQ1S):
        s2 = _fp16_scales(seed, tag, nb_total, qtype, cols).view(np.uint8).reshape(n, b2).copy()
    else:
        raw = random_bytes(seed, tag + "/s2", n * b2).view(np.uint64).copy()
        d = _fp16_scales(seed, tag, nb_total, qtype, cols).astype(np.uint64)
        raw = (raw & np.uint64(0xFFFFFFFFFFFF0000)) | d
        s2 = raw.view(np.uint8).reshape(n, b2)
    return [s0, s1, s2]


@dataclass
class Bank:
    """Experts [first, first+n) of one layer, all in one format."""
    qtype: int
    first: int
    n: int
    gate: list
    up: list
    down: list


@dataclass
class Layer:
    hidden: int
    inter: int
    n_experts: int          # routed experts E; the shared expert, if any, has id E
    has_shared: int
    banks: list = field(default_factory=list)

    def bank_of(self, e: int) -> tuple[Bank, int]:
        for b in self.banks:
            if b.first <= e < b.first + b.n:
                return b, e - b.first
        raise KeyError(e)

    def expert_bytes(self, e: int) -> int:
        b, _ = self.bank_of(e)
        return 2 * matrix_bytes(b.qtype, self.inter, self.hidden) + matrix_bytes(b.qtype, self.hidden, self.inter)


def make_layer(qtypes, hidden: int = 2048, inter: int = 512, n_experts: int = 512,
               has_shared: int = 1, seed: int = SEED_BANK, tag: str = "layer0") -> Layer:
    """A layer whose experts are split into banks.

    ``qtypes`` is a list of (qtype, count) covering the E routed experts in id order;
    the shared expert (id E) takes the format of the last bank and joins it.
    """
    layer = Layer(hidden, inter, n_experts, has_shared)
    first = 0
    for bi, (qt, cnt) in enumerate(qtypes):
        n = cnt + (has_shared if bi == len(qtypes) - 1 else 0)
        t = f"{tag}/bank{bi}"
        layer.banks.append(Bank(qt, first, n,
                                qbank(qt, n, inter, hidden, seed, t + "/gate"),
                                qbank(qt, n, inter, hidden, seed, t + "/up"),
                                qbank(qt, n, hidden, inter, seed, t + "/down")))
        first += cnt
    if first != n_experts:
        raise ValueError("bank counts must cover the routed experts")
    return layer


# ----------------------------------------------------------------------------- activations

def activations(T: int, H: int, seed: int = SEED_INPUT, tag: str = "x") -> np.ndarray:
    return normal(seed, tag, T * H).reshape(T, H)


def logits(T: int, E: int, seed: int = SEED_INPUT, tag: str = "logits", zipf_alpha: float = 0.0) -> np.ndarray:
    """Router logits N(0, 1); with ``zipf_alpha`` > 0 expert e gets the bias
    -alpha * ln(rank_e), rank_e in 1..E its position under a seeded permutation."""
    z = normal(seed, tag, T * E).reshape(T, E)
    if zipf_alpha > 0.0:
        keys = u64(seed, tag + "/perm", E)
        rank = np.empty(E, dtype=np.float64)
        rank[np.argsort(keys, kind="stable")] = np.arange(1, E + 1)
        z = (z.astype(np.float64) - zipf_alpha * np.log(rank)[None, :]).astype(np.float32)
    return np.ascontiguousarray(z)


def tie_logits(kind: str, T: int, E: int, seed: int = SEED_INPUT, tag: str = "ties") -> np.ndarray:
    """Router logits [T][E] full of ties, for the selection's tie rule:
    few_values: N(0,1)/2 rounded to integers -- long runs of equal logits; rounding the
      small negatives leaves -0.0 next to +0.0;
    signed_zeros: every logit <= -0.5 except 12 per token, set to +0.0 or -0.0 at seeded
      positions, so the selection is decided among zeros of both signs;
    all_zero: every logit +0.0 or -0.0 (seeded signs)."""
    z = normal(seed, tag, T * E).reshape(T, E)
    neg = (u64(seed, tag + "/sign", T * E).reshape(T, E) & np.uint64(1)).astype(bool)
    if kind == "few_values":
        return np.round(z * 0.5).astype(np.float32)
    if kind == "all_zero":
        return np.where(neg, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    if kind == "signed_zeros":
        out = (-np.abs(z) - 0.5).astype(np.float32)
        for t in range(T):
            pos = np.argsort(u64(seed, f"{tag}/zpos/{t}", E), kind="stable")[:12]
            out[t, pos] = np.where(neg[t, pos], np.float32(-0.0), np.float32(0.0))
        return out
    raise ValueError(kind)


def router_weights(E: int, H: int, seed: int = SEED_BANK, tag: str = "router") -> np.ndarray:
    """fp32 router matrix [E][H] with entries N(0, 1/H): for activations ~N(0, 1) the
    logits are then about N(0, 1), the distribution the routed-layer workloads use."""
    w = normal(seed, tag, E * H).astype(np.float64) / math.sqrt(H)
    return np.ascontiguousarray(w.astype(np.float32).reshape(E, H))


def shared_gate_weights(H: int, seed: int = SEED_BANK, tag: str = "router/shared-gate") -> np.ndarray:
    """fp32 gate vector [H] of the shared expert, entries N(0, 1/H)."""
    return router_weights(1, H, seed, tag).reshape(H)
