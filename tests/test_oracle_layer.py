"""Pins for the oracle's whole routed layer (CPU only).

The four layer invariants: a single expert with router weight 1.0 equals that
expert's FFN bit-exactly; identical experts with weights summing to one give that
expert's output; permuting the selected list leaves the result bit-identical (the
accumulation order is canonical); dequantized values stay in the alphabets (in
test_oracle_dequant).  Plus brute force against numpy float64 / scipy on a tiny layer,
the fp64 shadow, RMSNorm closed forms and a short residual chain of layers ("Red Lite
dev16 — complete full-attention parity": post-attention RMSNorm, routed MoE plus
shared expert, residual).
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle as O
import synth


@pytest.fixture(scope="module")
def small():
    layer = synth.make_layer([(synth.QTYPE_IQ2XS, 4), (synth.QTYPE_IQ1M, 4)], hidden=512, inter=256,
                             n_experts=8, has_shared=1, tag="small")
    return layer, O.ExpertTable(layer)


def test_single_expert_weight_one_is_its_ffn(small, ogrids):
    layer, tab = small
    x = synth.activations(2, 512, tag="one")
    for e in (0, 5, 8):
        if e == 8:
            continue
        r = O.moe_layer(tab, ogrids, x, 1, False, ids=np.array([[e], [e]], np.int32),
                        w=np.ones((2, 1), np.float32))
        for t in range(2):
            np.testing.assert_array_equal(r["acc"][t], O.expert_ffn(tab, e, ogrids, x[t]))


def test_identical_experts_weights_sum_to_one(ogrids):
    layer = synth.make_layer([(synth.QTYPE_IQ1M, 6)], hidden=512, inter=256, n_experts=6, has_shared=0,
                             tag="ident")
    b = layer.banks[0]
    for mat in (b.gate, b.up, b.down):
        for s in mat:
            s[:] = s[0][None, :]
    tab = O.ExpertTable(layer)
    x = synth.activations(1, 512, tag="ident/x")
    lg = synth.logits(1, 6, tag="ident/l")
    k = 5
    r = O.moe_layer(tab, ogrids, x, k, False, logits=lg)
    y = O.expert_ffn(tab, 0, ogrids, x[0])
    ulp = np.spacing(np.abs(y))
    assert np.all(np.abs(r["acc"][0] - y) <= 2 * k * ulp)


def test_permuting_selected_list_is_bit_identical(small, ogrids):
    layer, tab = small
    x = synth.activations(3, 512, tag="perm")
    ids = np.array([[1, 6, 3, 0], [7, 2, 5, 4], [4, 0, 7, 3]], np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.3, 0.2], [0.7, 0.1, 0.1, 0.1]], np.float32)
    base = O.moe_layer(tab, ogrids, x, 4, True, ids=ids, w=w)["acc"]
    rng = np.random.default_rng(0)
    for _ in range(4):
        p = np.stack([rng.permutation(4) for _ in range(3)])
        got = O.moe_layer(tab, ogrids, x, 4, True, ids=np.take_along_axis(ids, p, 1),
                          w=np.take_along_axis(w, p, 1))["acc"]
        np.testing.assert_array_equal(got, base)


@pytest.mark.parametrize("banks", [[(synth.QTYPE_IQ2XS, 2), (synth.QTYPE_IQ1M, 2)],
                                   [(synth.QTYPE_IQ1S, 2), (synth.QTYPE_IQ2XS, 2)]])
def test_tiny_layer_brute_force_numpy(ogrids, banks):
    """H = I = 256, E = 4, every expert selected: numpy float64 / scipy softmax reference."""
    layer = synth.make_layer(banks, hidden=256, inter=256, n_experts=4, has_shared=1, tag="tiny")
    tab = O.ExpertTable(layer)
    T, k = 5, 3
    x = synth.activations(T, 256, tag="tiny/x")
    lg = synth.logits(T, 4, tag="tiny/l")
    acc0 = synth.activations(T, 256, tag="tiny/acc")
    r = O.moe_layer(tab, ogrids, x, k, True, logits=lg, acc=acc0)
    ref = acc0.astype(np.float64).copy()
    for t in range(T):
        sel = np.lexsort((np.arange(4), -lg[t].astype(np.float64)))[:k]
        p = softmax(lg[t].astype(np.float64))[sel]
        p = p / p.sum()
        for e, wt in list(zip(sel, p)) + [(4, 1.0)]:
            Wg, Wu, Wd = (O.dequant(tab.qmat(e, n), ogrids).astype(np.float64) for n in ("gate", "up", "down"))
            g = Wg @ x[t]
            h = g * expit(g) * (Wu @ x[t])
            ref[t] += wt * (Wd @ h)
    for t in range(T):
        assert np.abs(r["acc"][t] - ref[t]).max() <= 2e-6 * np.linalg.norm(ref[t])


def test_fp64_shadow(small, ogrids):
    layer, tab = small
    x = synth.activations(4, 512, tag="shadow")
    lg = synth.logits(4, 8, tag="shadow/l")
    r = O.moe_layer(tab, ogrids, x, 3, True, logits=lg)
    r64 = O.moe_layer_f64(tab, ogrids, x, 3, True, logits=lg)
    for t in range(4):
        assert np.abs(r["acc"][t] - r64["acc"][t]).max() <= 1e-6 * np.linalg.norm(r64["acc"][t])


def test_threads_do_not_change_results(small, ogrids):
    layer, tab = small
    x = synth.activations(2, 512, tag="thr")
    lg = synth.logits(2, 8, tag="thr/l")
    a = O.moe_layer(tab, ogrids, x, 3, True, logits=lg, n_threads=1)
    b = O.moe_layer(tab, ogrids, x, 3, True, logits=lg, n_threads=4)
    for key in ("acc", "y", "w", "ids"):
        np.testing.assert_array_equal(a[key], b[key])


def test_rmsnorm_closed_forms():
    H = 2048
    h = np.full((1, H), 3.0, np.float32)
    np.testing.assert_allclose(O.rmsnorm(h), 3.0 / np.sqrt(9.0 + 1e-6), rtol=2e-7)
    z = O.rmsnorm(np.zeros((1, H), np.float32))
    assert np.all(z == 0)
    v = synth.activations(3, H, tag="rms")
    ref = v / np.sqrt((v.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(O.rmsnorm(v), ref, rtol=2e-6, atol=0)
    np.testing.assert_allclose(O.rmsnorm_f64(v.astype(np.float64)), ref, rtol=1e-14)
    # scale invariance (eps is negligible at this magnitude)
    np.testing.assert_allclose(O.rmsnorm(4 * v), O.rmsnorm(v), rtol=1e-6)


def test_residual_chain_is_stable(ogrids):
    """Three layers of h <- h + MoE(RMSNorm(h)) against the fp64 chain."""
    H, I, E, k = 512, 256, 8, 2
    layers = [O.ExpertTable(synth.make_layer([(qt, E)], hidden=H, inter=I, n_experts=E, has_shared=1,
                                             tag=f"chain{li}"))
              for li, qt in enumerate((synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M, synth.QTYPE_IQ1M))]
    h = synth.activations(2, H, tag="chain/h")
    h64 = h.astype(np.float64)
    for li, tab in enumerate(layers):
        lg = synth.logits(2, E, tag=f"chain/l{li}")
        h = O.moe_layer(tab, ogrids, O.rmsnorm(h), k, True, logits=lg, acc=h)["acc"]
        h64 = O.moe_layer_f64(tab, ogrids, O.rmsnorm_f64(h64), k, True, logits=lg, acc=h64)["acc"]
    assert np.all(np.isfinite(h))
    for t in range(2):
        assert np.abs(h[t] - h64[t]).max() <= 1e-5 * np.linalg.norm(h64[t])


@pytest.mark.parametrize("banks", [[(synth.QTYPE_IQ2XS, 2), (synth.QTYPE_IQ1M, 2)]])
def test_fp64_shadow_brute_force_numpy(ogrids, banks):
    """The fp64 shadow of the layer against the same numpy float64 brute force, at the
    bound of float64 summation order (measured ~1e-16 of the norm; fp32 sits near 1e-7), not
    the fp32 one: pins the shadow independently of its fp32 twin."""
    layer = synth.make_layer(banks, hidden=256, inter=256, n_experts=4, has_shared=1, tag="tiny64")
    tab = O.ExpertTable(layer)
    T, k = 4, 3
    x = synth.activations(T, 256, tag="tiny64/x")
    lg = synth.logits(T, 4, tag="tiny64/l")
    acc0 = synth.activations(T, 256, tag="tiny64/acc")
    r = O.moe_layer_f64(tab, ogrids, x, k, True, logits=lg, acc=acc0)
    ref = acc0.astype(np.float64).copy()
    for t in range(T):
        sel = np.lexsort((np.arange(4), -lg[t].astype(np.float64)))[:k]
        p = softmax(lg[t].astype(np.float64))[sel]
        p = p / p.sum()
        for e, wt in list(zip(sel, p)) + [(4, 1.0)]:
            Wg, Wu, Wd = (O.dequant(tab.qmat(e, n), ogrids).astype(np.float64) for n in ("gate", "up", "down"))
            g = Wg @ x[t].astype(np.float64)
            h = g * expit(g) * (Wu @ x[t].astype(np.float64))
            ref[t] += wt * (Wd @ h)
    for t in range(T):
        assert np.abs(r["acc"][t] - ref[t]).max() <= 1e-13 * np.linalg.norm(ref[t])
