"""Pins of the oracle's router projection (logits = x W_r^T, optional sigmoid gate of the
shared expert), each against something other than the oracle's own formula:

- one-hot activations pick one column of the router matrix, exactly;
- permutation rows of the router matrix pick single activations, exactly;
- small-integer operands give exact integer dot products (numpy int64 matmul);
- scaling x by a power of two scales every logit by it, exactly;
- the fp32 sums stay within the textbook bound n * 2^-24 * sum|x w| of the fp64 ones;
- the gate is 1/2 at zero, s(z) + s(-z) = 1, and tends to 0 / 1 at the ends.

A dropped term, a transposed operand or a wrong row stride fails the first three.
"""
import numpy as np
import pytest

import oracle as O
import synth

H, E = 256, 48


def test_one_hot_columns():
    wr = synth.router_weights(E, H, tag="pin/router/w")
    wsg = synth.shared_gate_weights(H, tag="pin/router/g")
    for c in (0, 1, 77, H - 1):
        x = np.zeros((1, H), np.float32)
        x[0, c] = 1.0
        lg, sw = O.router(x, wr, wsg)
        np.testing.assert_array_equal(lg[0], wr[:, c])
        np.testing.assert_allclose(sw[0], 1.0 / (1.0 + np.exp(-np.float64(wsg[c]))), rtol=3e-7)  # fp32 expf


def test_permutation_rows():
    rng = np.random.default_rng(3)
    cols = rng.permutation(H)[:E]
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), cols] = 1.0
    x = synth.activations(3, H, tag="pin/router/x")
    lg, sw = O.router(x, wr)
    assert sw is None
    np.testing.assert_array_equal(lg, x[:, cols])


def test_integer_operands_exact():
    rng = np.random.default_rng(5)
    x = rng.integers(-7, 8, size=(4, H)).astype(np.float32)
    wr = rng.integers(-5, 6, size=(E, H)).astype(np.float32)
    want = (x.astype(np.int64) @ wr.astype(np.int64).T).astype(np.float64)
    lg, _ = O.router(x, wr)
    l64, _ = O.router_f64(x, wr)
    np.testing.assert_array_equal(lg.astype(np.float64), want)
    np.testing.assert_array_equal(l64, want)


def test_power_of_two_scaling():
    x = synth.activations(2, H, tag="pin/router/x2")
    wr = synth.router_weights(E, H, tag="pin/router/w2")
    a, _ = O.router(x, wr)
    b, _ = O.router(4.0 * x, wr)
    np.testing.assert_array_equal(b, 4.0 * a)


@pytest.mark.parametrize("Hn", [256, 2048])
def test_fp32_within_bound_of_fp64(Hn):
    x = synth.activations(3, Hn, tag="pin/router/x3")
    wr = synth.router_weights(E, Hn, tag="pin/router/w3")
    lg, _ = O.router(x, wr)
    l64, _ = O.router_f64(x, wr)
    scale = O.dot_abs(x, wr)
    # the brute-force magnitude sum agrees with numpy's
    np.testing.assert_allclose(scale, np.abs(x.astype(np.float64))[:, None, :].__mul__(
        np.abs(wr.astype(np.float64))[None, :, :]).sum(-1), rtol=1e-12)
    bound = Hn * 2.0 ** -24 * scale
    assert np.all(np.abs(lg - l64) <= bound)
    # and the fp64 sums match numpy's matmul to double rounding
    np.testing.assert_allclose(l64, x.astype(np.float64) @ wr.astype(np.float64).T, rtol=0, atol=1e-12 * scale.max())


def test_gate_identities():
    x = np.zeros((1, 4), np.float32)
    wsg = np.zeros(4, np.float32)
    _, s0 = O.router(x, np.zeros((1, 4), np.float32), wsg)
    assert s0[0] == 0.5
    x = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    for z in (0.25, 1.5, 6.0):
        _, sp = O.router_f64(x, np.zeros((1, 4), np.float32), np.array([z, 0, 0, 0], np.float32))
        _, sn = O.router_f64(x, np.zeros((1, 4), np.float32), np.array([-z, 0, 0, 0], np.float32))
        assert abs(sp[0] + sn[0] - 1.0) < 1e-15 and sp[0] > 0.5
    _, lo = O.router(x, np.zeros((1, 4), np.float32), np.array([-200.0, 0, 0, 0], np.float32))
    _, hi = O.router(x, np.zeros((1, 4), np.float32), np.array([200.0, 0, 0, 0], np.float32))
    assert lo[0] == 0.0 and hi[0] == 1.0


def test_generated_logits_are_standard_normal_like():
    x = synth.activations(16, 2048, tag="pin/router/x4")
    wr = synth.router_weights(512, 2048, tag="pin/router/w4")
    lg, _ = O.router(x, wr)
    assert 0.9 < lg.std() < 1.1 and abs(lg.mean()) < 0.05
