"""Pins for the oracle's grid expansion and dequantization (CPU only).

The pages fix the grid shapes and symbol values ("Red Lite dev10 — standalone native
Metal path", section "Quant grids"); the stream layouts are documented in ``synth``.
Here the bytes are built by an *encoder* written from that layout description
(semantic fields -> bytes) and the oracle has to decode them back, exhaustively over
every code, and the decoded values must satisfy the invariants of the format.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def facts():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- grids

def test_grid_shapes_and_alphabets(ogrids):
    f = facts()
    g2, g1 = ogrids.iq2_array(), ogrids.iq1_array()
    assert g2.shape == (f["iq2xs_grid"]["rows"], f["iq2xs_grid"]["cols"])
    assert g1.shape == (f["iq1m_grid"]["rows"], f["iq1m_grid"]["cols"])
    assert set(np.unique(g2).tolist()) == set(f["iq2xs_grid"]["symbol_values"])
    assert set(np.unique(g1).tolist()) == set(f["iq1m_grid"]["symbol_values"])
    assert [int(h, 16) for h in f["iq2xs_grid"]["symbol_values_hex"]] == f["iq2xs_grid"]["symbol_values"]
    # distinct rows
    assert len({r.tobytes() for r in g2}) == 512
    assert len({r.tobytes() for r in g1}) == 2048


def test_grid_round_trip(grids_compact, ogrids):
    """compact -> expand (oracle) -> recompact with the pages' symbol order == compact."""
    f = facts()
    c2, c1 = grids_compact
    for comp, vals, table in ((c2, ogrids.iq2_array(), f["iq2xs_grid"]["symbol_values"]),
                              (c1, ogrids.iq1_array(), f["iq1m_grid"]["symbol_values"])):
        sym = np.vectorize(table.index)(vals.astype(np.int64))
        re = np.zeros(len(comp), dtype=np.uint32)
        for j in range(8):
            re |= sym[:, j].astype(np.uint32) << (2 * j)
        np.testing.assert_array_equal(re.astype(np.uint16), comp)


def test_grid_rejects_symbol_3(grids_compact):
    c2, c1 = (a.copy() for a in grids_compact)
    c2[17] |= 3 << 6
    with pytest.raises(ValueError):
        O.grids(c2, c1)


def test_f16_decode_matches_numpy_for_every_pattern():
    """IEEE binary16 decode vs numpy's conversion, all 65536 bit patterns."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(int(p)) for p in pats], dtype=np.float32)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(np.isinf(got), np.isinf(ref))


# ----------------------------------------------------------------------------- encoders

def encode_iq2(idx, signs7, scales, d16):
    """Semantic fields -> IQ2_XS-like streams.

    idx, signs7: [rows][NG] (signs7 bit j = sign of weight j, j < 7); scales: [rows][NB][8]
    nibbles; d16: [rows][NB] binary16 bit patterns."""
    qs = (idx.astype(np.uint32) | (signs7.astype(np.uint32) << 9)).astype(np.uint16)
    sc = np.zeros(scales.shape[:2], dtype=np.uint32)
    for i in range(8):
        sc |= scales[:, :, i].astype(np.uint32) << (4 * i)
    return [qs.view(np.uint8).ravel(), sc.view(np.uint8).ravel(), d16.astype(np.uint16).view(np.uint8).ravel()]


def encode_iq1(idx11, dneg, scales, d16):
    """idx11, dneg: [rows][NG]; scales: [rows][NB][16] 3-bit values; d16: [rows][NB]."""
    rows, ng = idx11.shape
    ql = (idx11 & 0xFF).astype(np.uint8)
    nib = ((idx11 >> 8) & 7) | (dneg.astype(np.int64) << 3)
    qh = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sd = d16.astype(np.uint64)
    for i in range(16):
        sd |= scales[:, :, i].astype(np.uint64) << np.uint64(16 + 3 * i)
    return [ql.ravel(), qh.ravel(), sd.view(np.uint8).ravel()]


def test_iq2_exhaustive_codes_and_scales(ogrids):
    """Every 16-bit code under every 4-bit scale: a 4096 x 2048 matrix."""
    rows, cols = 4096, 2048
    ng, nb = cols // 8, cols // 256
    code = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 65536
    idx, signs7 = code & 511, code >> 9
    # scale of sub-block i of super-block b in row r: (r // 256 + b + i + r) % 16, so that
    # across the 16 copies of the code space every code meets every scale.
    r_ = np.arange(rows)[:, None, None]
    b_ = np.arange(nb)[None, :, None]
    i_ = np.arange(8)[None, None, :]
    scales = (r_ // 256 + b_ + i_ + r_) % 16
    d = np.full((rows, nb), 0x3C00, dtype=np.uint16)   # 1.0
    m = O.qmat(O.IQ2XS, rows, cols, encode_iq2(idx, signs7, scales, d))
    W = O.dequant(m, ogrids)
    g2 = ogrids.iq2_array()

    grp = W.reshape(rows, ng, 8)
    s_of_group = np.repeat(scales, 4, axis=2).reshape(rows, ng)        # 4 groups per sub-block
    unit = (2 * s_of_group + 1).astype(np.float32) * np.float32(0.125)
    q = grp / unit[:, :, None]                                          # exact: w = unit * (+/-G)
    assert np.array_equal(q * unit[:, :, None], grp)
    # magnitudes are the grid row the index names
    np.testing.assert_array_equal(np.abs(q).astype(np.int64), g2[idx].astype(np.int64))
    # explicit signs of weights 0..6
    neg = q < 0
    for j in range(7):
        np.testing.assert_array_equal(neg[:, :, j], ((signs7 >> j) & 1).astype(bool))
    # parity sign: an even number of negatives in every group
    assert np.all(neg.sum(axis=2) % 2 == 0)
    # every (code, scale) pair occurs
    pairs = np.unique(code.ravel() * 16 + s_of_group.ravel())
    assert len(pairs) == 65536 * 16


def test_iq1_exhaustive_codes_and_scales(ogrids):
    """Every (11-bit index, delta sign) code under every 3-bit scale: 128 x 2048."""
    rows, cols = 128, 2048
    ng, nb = cols // 8, cols // 256
    code = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 4096
    idx11, dneg = code & 2047, code >> 11
    r_ = np.arange(rows)[:, None, None]
    b_ = np.arange(nb)[None, :, None]
    i_ = np.arange(16)[None, None, :]
    scales = (r_ // 16 + b_ + i_ + r_) % 8
    d = np.full((rows, nb), 0x3C00, dtype=np.uint16)
    m = O.qmat(O.IQ1M, rows, cols, encode_iq1(idx11, dneg, scales, d))
    W = O.dequant(m, ogrids)
    g1 = ogrids.iq1_array()
    grp = W.reshape(rows, ng, 8)
    s_of_group = np.repeat(scales, 2, axis=2).reshape(rows, ng)        # 2 groups per sub-block
    unit = (2 * s_of_group + 1).astype(np.float32)
    q = grp / unit[:, :, None]
    assert np.array_equal(q * unit[:, :, None], grp)
    delta = np.where(dneg.astype(bool), -0.125, 0.125)
    np.testing.assert_array_equal(q - delta[:, :, None], g1[idx11].astype(np.float32))
    pairs = np.unique(code.ravel() * 8 + s_of_group.ravel())
    assert len(pairs) == 4096 * 8


def encode_iq1s(idx11, dneg32, scales32, d16):
    """idx11: [rows][NG]; dneg32, scales32: [rows][NG/4] (one per 32-weight sub-block);
    d16: [rows][NB]."""
    rows, ng = idx11.shape
    ql = (idx11 & 0xFF).astype(np.uint8)
    hi = (idx11 >> 8) & 7
    qh = (hi[:, 0::4] | (hi[:, 1::4] << 3) | (hi[:, 2::4] << 6) | (hi[:, 3::4] << 9)
          | (scales32.astype(np.int64) << 12) | (dneg32.astype(np.int64) << 15)).astype(np.uint16)
    return [ql.ravel(), qh.view(np.uint8).ravel(), d16.astype(np.uint16).view(np.uint8).ravel()]


def test_iq1s_exhaustive_codes_and_scales(ogrids):
    """Every 11-bit index under every (3-bit scale, delta sign) of its sub-block: the
    weights are d * (2s + 1) * (grid value +/- 1/8), one scale and sign per 32 weights."""
    rows, cols = 128, 2048
    ng, nb = cols // 8, cols // 256
    idx11 = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 2048   # depends on (row % 8, group)
    # (scale, sign) of sub-block sb of row r: (r // 8 + sb) % 16, so that each index, met
    # once per 8 rows, sees all 16 combinations over the 128 rows
    combo = (np.arange(rows)[:, None] // 8 + np.arange(ng // 4)[None, :]) % 16
    scales32, dneg32 = combo & 7, combo >> 3
    d = np.full((rows, nb), 0x3C00, dtype=np.uint16)
    m = O.qmat(O.IQ1S, rows, cols, encode_iq1s(idx11, dneg32, scales32, d))
    W = O.dequant(m, ogrids)
    g1 = ogrids.iq1_array()
    grp = W.reshape(rows, ng, 8)
    s_of_group = np.repeat(scales32, 4, axis=1)
    n_of_group = np.repeat(dneg32, 4, axis=1)
    unit = (2 * s_of_group + 1).astype(np.float32)
    q = grp / unit[:, :, None]
    assert np.array_equal(q * unit[:, :, None], grp)
    delta = np.where(n_of_group.astype(bool), -0.125, 0.125)
    np.testing.assert_array_equal(q - delta[:, :, None], g1[idx11].astype(np.float32))
    # every index meets every (scale, sign)
    triples = np.unique((idx11 * 16 + s_of_group * 2 + n_of_group).ravel())
    assert len(triples) == 2048 * 16


def test_iq1s_equals_iq1m_with_repeated_fields(ogrids):
    """An IQ1_S-like matrix and the IQ1_M-like matrix whose per-16 scales and per-8 delta
    signs repeat the per-32 ones dequantize to the same bits (the two formats share the
    grid and the formula; IQ1_S-like is the coarser packing)."""
    rows, cols = 32, 512
    s = synth.qbank(synth.QTYPE_IQ1S, 1, rows, cols, 5, "iq1s-vs-iq1m")
    ql, qh, d = (a[0] for a in s)
    ng, nb = cols // 8, cols // 256
    qh16 = qh.view(np.uint16).reshape(rows, ng // 4).astype(np.int64)
    idx11 = ql.reshape(rows, ng).astype(np.int64) | (np.stack([(qh16 >> (3 * i)) & 7 for i in range(4)], 2)
                                                       .reshape(rows, ng) << 8)
    dneg = np.repeat((qh16 >> 15) & 1, 4, axis=1)
    sc16 = np.repeat((qh16 >> 12) & 7, 2, axis=1).reshape(rows, nb, 16)
    m_s = O.qmat(O.IQ1S, rows, cols, [ql, qh, d])
    m_m = O.qmat(O.IQ1M, rows, cols, encode_iq1(idx11, dneg, sc16, d.view(np.uint16).reshape(rows, nb)))
    np.testing.assert_array_equal(O.dequant(m_s, ogrids), O.dequant(m_m, ogrids))


@pytest.mark.parametrize("qtype", [synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M, synth.QTYPE_IQ1S])
def test_seeded_weights_alphabet_and_exactness(ogrids, qtype):
    """Seeded matrices: values lie in the scaled alphabet, fp32 == fp64 weight (exactness),
    and doubling every super-block scale doubles every weight bit-exactly."""
    rows, cols = 64, 512
    s = synth.qbank(qtype, 1, rows, cols, 3, "alpha")
    streams = [a[0] for a in s]
    m = O.qmat(qtype, rows, cols, streams)
    W = O.dequant(m, ogrids)
    for r in (0, 17, 63):
        for c in (0, 255, 256, 511):
            assert float(W[r, c]) == O.weight_f64(m, ogrids, r, c)
    # double d: binary16 exponent + 1 (all d are normal and far from the top)
    s2 = streams[2].copy()
    if qtype in (synth.QTYPE_IQ2XS, synth.QTYPE_IQ1S):
        dd = s2.view(np.uint16)
        dd += np.uint16(1 << 10)
    else:
        dd = s2.view(np.uint64)
        dd += np.uint64(1 << 10)
    W2 = O.dequant(O.qmat(qtype, rows, cols, [streams[0], streams[1], s2]), ogrids)
    np.testing.assert_array_equal(W2, 2 * W)
    # alphabet
    if qtype == synth.QTYPE_IQ2XS:
        d = np.repeat(streams[2].view(np.float16).astype(np.float32).reshape(rows, cols // 256), 256, axis=1)
        sc = streams[1].view(np.uint32).reshape(rows, cols // 256)
        nib = np.stack([(sc >> (4 * i)) & 15 for i in range(8)], axis=2)
        s_ = np.repeat(nib.reshape(rows, -1), 32, axis=1)
        q = W / (d * (2 * s_ + 1) * 0.125)
        assert set(np.unique(np.abs(q)).tolist()) <= {8.0, 25.0, 43.0}
    elif qtype == synth.QTYPE_IQ1S:
        d = np.repeat(streams[2].view(np.float16).astype(np.float32).reshape(rows, cols // 256), 256, axis=1)
        qh = streams[1].view(np.uint16).reshape(rows, cols // 32).astype(np.int64)
        s_ = np.repeat((qh >> 12) & 7, 32, axis=1)
        q = W / (d * (2 * s_ + 1))
        assert set(np.unique(q).tolist()) <= {-1.125, -0.875, -0.125, 0.125, 0.875, 1.125}
    else:
        sd = streams[2].view(np.uint64).reshape(rows, cols // 256)
        d = np.repeat((sd & np.uint64(0xFFFF)).astype(np.uint16).view(np.float16).astype(np.float32), 256, axis=1)
        nib = np.stack([(sd >> np.uint64(16 + 3 * i)) & np.uint64(7) for i in range(16)], axis=2).astype(np.int64)
        s_ = np.repeat(nib.reshape(rows, -1), 16, axis=1)
        q = W / (d * (2 * s_ + 1))
        assert set(np.unique(q).tolist()) <= {-1.125, -0.875, -0.125, 0.125, 0.875, 1.125}
