"""Pins for the oracle's mat-vec, SiLU and expert FFN (CPU only).

Mat-vec: a one-hot input returns the dequantized column bit-exactly (one nonzero
product); scaling the input by 2 doubles the output bit-exactly; the fp32 result lies
within Higham's bound gamma_n * sum|w||x| (Higham, "Accuracy and Stability of Numerical
Algorithms", 2nd ed., section 3.1) of numpy's float64 product of the same matrix.
SiLU: closed forms and the logistic function from scipy.  FFN: numpy float64 on the
dequantized matrices.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle as O
import synth

U32 = 2.0 ** -24


def gamma(n):
    return n * U32 / (1 - n * U32)


@pytest.fixture(scope="module")
def mats():
    out = {}
    for qt in (synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M):
        for rows, cols in ((48, 512), (40, 768)):
            s = synth.qbank(qt, 1, rows, cols, 5, f"lin/{qt}/{rows}")
            out[(qt, rows, cols)] = O.qmat(qt, rows, cols, [a[0] for a in s])
    return out


def test_one_hot_columns_bit_exact(mats, ogrids):
    for m in mats.values():
        W = O.dequant(m, ogrids)
        for c in (0, 1, 7, 8, 255, 256, m.cols - 1):
            x = np.zeros(m.cols, dtype=np.float32)
            x[c] = 1.0
            np.testing.assert_array_equal(O.matvec(m, ogrids, x), W[:, c])


def test_scaling_input_by_two_is_exact(mats, ogrids):
    x = synth.activations(1, 768, tag="lin/x")[0]
    for m in mats.values():
        xx = x[: m.cols]
        np.testing.assert_array_equal(O.matvec(m, ogrids, 2 * xx), 2 * O.matvec(m, ogrids, xx))


def test_matvec_within_higham_bound(mats, ogrids):
    x = synth.activations(1, 768, tag="lin/x2")[0]
    for m in mats.values():
        W = O.dequant(m, ogrids).astype(np.float64)
        xx = x[: m.cols].astype(np.float64)
        ref = W @ xx
        y = O.matvec(m, ogrids, x[: m.cols]).astype(np.float64)
        bound = gamma(m.cols) * (np.abs(W) @ np.abs(xx))
        assert np.all(np.abs(y - ref) <= bound)
        # the fp64 twin agrees with numpy to rounding of double sums
        y64 = O.matvec_f64(m, ogrids, xx)
        assert np.all(np.abs(y64 - ref) <= 1e-13 * (np.abs(W) @ np.abs(xx)))


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    v = O.silu(-1e30)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0          # g -> -inf gives -0
    assert O.silu(100.0) == 100.0                               # sigmoid rounds to 1
    xs = np.linspace(-30, 30, 4001).astype(np.float32)
    got = np.array([O.silu(float(a)) for a in xs], dtype=np.float32)
    ref = xs.astype(np.float64) * expit(xs.astype(np.float64))
    # three rounded steps (libm expf within 1 ulp, the add, the divide): at most 3 ulp
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 3 * ulp + 1e-45)
    for a in (-3.0, -0.5, 0.25, 2.0):
        assert abs(O.silu_f64(a) - a * expit(a)) <= 1e-15 * max(1.0, abs(a))


@pytest.mark.parametrize("qtype", [synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M])
def test_expert_ffn_vs_numpy_float64(ogrids, qtype):
    layer = synth.make_layer([(qtype, 2)], hidden=512, inter=256, n_experts=2, has_shared=0, tag=f"ffn{qtype}")
    tab = O.ExpertTable(layer)
    x = synth.activations(1, 512, tag="ffn/x")[0]
    for e in range(2):
        Wg = O.dequant(tab.qmat(e, "gate"), ogrids).astype(np.float64)
        Wu = O.dequant(tab.qmat(e, "up"), ogrids).astype(np.float64)
        Wd = O.dequant(tab.qmat(e, "down"), ogrids).astype(np.float64)
        g = Wg @ x.astype(np.float64)
        u = Wu @ x.astype(np.float64)
        h = g * expit(g) * u
        ref = Wd @ h
        y, hh = O.expert_ffn(tab, e, ogrids, x, want_h=True)
        np.testing.assert_allclose(hh, h, rtol=0, atol=1e-5 * np.abs(h).max())
        assert np.abs(y - ref).max() <= 1e-5 * np.linalg.norm(ref)
        y64 = O.expert_ffn_f64(tab, e, ogrids, x)
        assert np.abs(y64 - ref).max() <= 1e-12 * np.linalg.norm(ref)
