"""Pins for the oracle's routing and grouping (CPU only).

Routing ("Red Metal dev8 — resident routed top-k layer": positive router weights that
sum to about one; top-10 of 512 per "Red Lite dev9", section "Inspect the real
Qwen3-Next model"): the selected ids equal a brute-force full sort by (logit
descending, id ascending); the weights equal scipy's softmax over all E logits
renormalised over the selected set; relabelling the experts relabels the selection.
Grouping: numpy's stable argsort of the ids.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O
import synth


def brute_topk(l, k):
    order = np.lexsort((np.arange(len(l)), -l.astype(np.float64)))
    return order[:k]


@pytest.mark.parametrize("E,k", [(16, 4), (16, 16), (8, 1), (512, 10), (513, 17)])
def test_route_matches_full_sort_and_softmax(E, k):
    T = 32
    lg = synth.logits(T, E, tag=f"rt{E}")
    ids, w = O.route(lg, k, add_shared=False)
    for t in range(T):
        np.testing.assert_array_equal(ids[t], brute_topk(lg[t], k))
        p = softmax(lg[t].astype(np.float64))
        ref = p[ids[t]] / p[ids[t]].sum()
        np.testing.assert_allclose(w[t], ref, rtol=4 * k * 2.0 ** -24, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * 2.0 ** -24 + 2.0 ** -24
        assert np.all(w[t] > 0)


def test_route_ties_go_to_lower_id():
    l = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, 2.0, 2.0, -1.0]], dtype=np.float32)
    ids, w = O.route(l, 5, add_shared=False)
    np.testing.assert_array_equal(ids[0], [1, 2, 4, 5, 6])
    assert w[0, 0] == w[0, 1] == w[0, 2] and w[0, 3] == w[0, 4]


def test_route_relabel_invariance():
    T, E, k = 16, 64, 10
    lg = synth.logits(T, E, tag="relabel")
    perm = np.argsort(synth.u64(3, "perm", E), kind="stable")   # new column j holds old expert perm[j]
    ids, w = O.route(lg, k, False)
    ids2, w2 = O.route(lg[:, perm], k, False)
    inv = np.empty(E, dtype=np.int64)
    inv[perm] = np.arange(E)
    # distinct logits, so the selection is unique
    np.testing.assert_array_equal(perm[ids2], ids)
    np.testing.assert_array_equal(w2, w)


def test_route_shared_slot():
    lg = synth.logits(3, 512, tag="shared")
    ids, w = O.route(lg, 10, add_shared=True)
    assert ids.shape == (3, 11)
    assert np.all(ids[:, 10] == 512) and np.all(w[:, 10] == 1.0)
    ids0, w0 = O.route(lg, 10, add_shared=False)
    np.testing.assert_array_equal(ids[:, :10], ids0)
    np.testing.assert_array_equal(w[:, :10], w0)


def test_route_fp64_twin_close():
    lg = synth.logits(8, 512, tag="r64")
    ids, w = O.route(lg, 10, True)
    ids64, w64 = O.route_f64(lg, 10, True)
    np.testing.assert_array_equal(ids, ids64)
    np.testing.assert_allclose(w, w64, rtol=4e-7)


@pytest.mark.parametrize("T,E,k,shared", [(1, 512, 10, True), (8, 512, 10, True), (256, 512, 10, False),
                                          (37, 16, 4, False), (64, 40, 16, True)])
def test_group_is_stable_sort(T, E, k, shared):
    lg = synth.logits(T, E, tag=f"grp{T}")
    ids, _ = O.route(lg, k, shared)
    n_ids = E + int(shared)
    counts, offsets, ss, sp = O.group(ids, n_ids)
    flat = ids.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=n_ids))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(ss, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(sp[ss], np.arange(len(flat)))
    assert offsets[-1] == T * (k + int(shared))


@pytest.mark.parametrize("kind", ["few_values", "signed_zeros", "all_zero"])
@pytest.mark.parametrize("E,k", [(512, 10), (1023, 16), (16, 4)])
def test_route_signed_zero_and_heavy_ties(kind, E, k):
    """-0.0 and +0.0 compare equal, so they tie and the lower id goes first; long runs of
    equal logits select the lowest ids of the run.  Checked against the brute-force sort
    (numpy orders -0.0 and +0.0 as equal), and the weights of tied experts are equal."""
    T = 24
    lg = synth.tie_logits(kind, T, E, tag=f"edge/{kind}/{E}")
    assert np.signbit(lg).any() and (lg == 0).any()
    ids, w = O.route(lg, k, add_shared=False)
    for t in range(T):
        np.testing.assert_array_equal(ids[t], brute_topk(lg[t], k))
        sel = lg[t, ids[t]]
        for a in range(k):
            for b in range(k):
                if sel[a] == sel[b]:
                    assert w[t, a] == w[t, b]
    if kind == "all_zero":
        np.testing.assert_array_equal(ids, np.tile(np.arange(k), (T, 1)))
        assert np.all(w == np.float32(1.0) / np.float32(k))


def test_route_fp64_against_full_sort_and_scipy():
    """The fp64 shadow of the router top-k against a full float64 sort (ties to the lower
    id) and scipy's softmax renormalised over the selection, to float64 rounding: pins
    the shadow independently of its fp32 twin."""
    from scipy.special import softmax
    lg = synth.logits(16, 512, tag="r64/sort")
    ids64, w64 = O.route_f64(lg, 10, True)
    for t in range(16):
        sel = np.lexsort((np.arange(512), -lg[t].astype(np.float64)))[:10]
        p = softmax(lg[t].astype(np.float64))[sel]
        np.testing.assert_array_equal(ids64[t, :10], sel)
        np.testing.assert_allclose(w64[t, :10], p / p.sum(), rtol=1e-14, atol=0)
        assert ids64[t, 10] == 512 and w64[t, 10] == 1.0


def test_accumulate_fp64_exact_on_dyadic_values():
    """acc + sum of w * y over the slots in ascending id, on values whose products and
    partial sums are exact in float64 (small dyadic rationals): the shadow must return
    the exact rational sum, and the order of the slots in the list must not matter."""
    from fractions import Fraction
    rng = np.random.default_rng(7)
    T, kp, H = 3, 5, 16
    ids = np.stack([rng.permutation(9)[:kp] for _ in range(T)]).astype(np.int32)
    w = rng.integers(-8, 9, size=(T, kp)) / 16.0
    y = rng.integers(-1000, 1001, size=(T * kp, H)) / 64.0
    acc = rng.integers(-50, 51, size=(T, H)) / 4.0
    got = O.accumulate_f64(y, w, ids, acc)
    for t in range(T):
        for c in range(H):
            exact = Fraction(acc[t, c]) + sum(Fraction(w[t, j]) * Fraction(y[t * kp + j, c]) for j in range(kp))
            assert Fraction(got[t, c]) == exact
    perm = rng.permutation(kp)
    rows = (np.arange(T)[:, None] * kp + perm[None, :]).reshape(-1)
    again = O.accumulate_f64(y[rows], w[:, perm], ids[:, perm], acc)
    np.testing.assert_array_equal(again, got)
