"""Pins of the oracle's router: exact logits, selection rule and weights."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import codecs
from oracle.layer import route, select_topk


def _rn32_rational(xs, ws):
    S = sum((Fraction(a) * Fraction(b) for a, b in zip(xs, ws)), Fraction(0))
    c = np.float32(float(S))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - S),
                                     int(np.float32(v).view(np.uint32)) & 1))


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_logits_are_correctly_rounded_exact_dots(cfg):
    D = synth.config(cfg).dims
    x = synth.make_activations(cfg, 0, T=min(D.T, 4))
    wr, _ = synth.make_router(cfg, 0, with_skew=False)
    got = route(x, wr, None, D.top_k)["logits"]
    X, W = codecs.bf16_to_f64(x), codecs.bf16_to_f64(wr)
    rng = np.random.default_rng(cfg)
    for _ in range(12):
        t, e = int(rng.integers(X.shape[0])), int(rng.integers(W.shape[0]))
        assert got[t, e] == float(_rn32_rational(X[t].tolist(), W[e].tolist()))
    # math.fsum agrees on many more samples (fsum is exactly rounded to f64 first)
    for _ in range(400):
        t, e = int(rng.integers(X.shape[0])), int(rng.integers(W.shape[0]))
        assert got[t, e] == float(np.float32(math.fsum((X[t] * W[e]).tolist())))


def test_logits_certificate_fallback():
    """Cancellation that plain float64 summation gets wrong must still round exactly."""
    x = synth.bf16_bits_from_f32(np.array([[1.0, 2.0 ** -60, -1.0, 0.0]], dtype=np.float32))
    w = synth.bf16_bits_from_f32(np.array([[1.0, 1.0, 1.0, 1.0],
                                           [2.0 ** 70, 1.0, 2.0 ** 70, 0.5]], dtype=np.float32))
    lg = route(x, w, None, 2)["logits"]
    assert lg[0, 0] == 2.0 ** -60
    assert lg[0, 1] == 2.0 ** -60


def test_topk_equals_full_sort():
    for cfg in (0, 1, 3):
        D = synth.config(cfg).dims
        x = synth.make_activations(cfg, 1, T=min(D.T, 8))
        wr, _ = synth.make_router(cfg, 1, with_skew=False)
        rt = route(x, wr, None, D.top_k)
        for t in range(x.shape[0]):
            lg = rt["logits"][t].tolist()
            ref = sorted(range(len(lg)), key=lambda e: (-lg[e], e))[:D.top_k]
            assert rt["idx"][t].tolist() == ref


def test_zero_input_ties_to_lower_index():
    D = synth.config(1).dims
    x = np.zeros((3, D.d), dtype=np.uint16)
    wr, _ = synth.make_router(1, 0, with_skew=False)
    rt = route(x, wr, None, D.top_k)
    assert np.all(rt["logits"] == 0)
    for t in range(3):
        assert rt["idx"][t].tolist() == list(range(D.top_k))
        np.testing.assert_allclose(rt["w"][t], 1.0 / D.top_k, rtol=0, atol=1e-16)


def test_signed_zero_logits_tie():
    """+0 and -0 compare equal: the lower index wins whatever the sign."""
    lg = np.array([[-0.0, 0.0, -0.0, 0.0, -0.0, 0.0, -1.0, -0.0]])
    idx, w = select_topk(lg, 5)
    assert idx[0].tolist() == [0, 1, 2, 3, 4]
    lg = np.array([[0.5, -0.0, 0.5, 0.25, 0.5, 0.0]])
    assert select_topk(lg, 4)[0][0].tolist() == [0, 2, 4, 3]
    # through the router: x = 0 with a signed-zero bias still selects 0..k-1
    E, d = 16, 8
    bias = np.where(np.arange(E) % 3 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    rt = route(np.zeros((1, d), dtype=np.uint16), np.zeros((E, d), dtype=np.uint16), bias, 5)
    assert rt["idx"][0].tolist() == [0, 1, 2, 3, 4]


def test_k1_weight_is_one():
    D = synth.config(0).dims
    x = synth.make_activations(0, 0)
    wr, _ = synth.make_router(0, 0)
    rt = route(x, wr, None, 1)
    assert np.all(rt["w"] == 1.0)


def test_bias_selects_chosen_set():
    D = synth.config(1).dims
    x = synth.make_activations(1, 0, T=4)
    wr, _ = synth.make_router(1, 0, with_skew=False)
    chosen = [5, 77, 130, 200, 311, 312, 400, 401, 499, 511]
    bias = np.zeros(D.n_experts, dtype=np.float32)
    bias[chosen] = 100.0
    rt = route(x, wr, bias, D.top_k)
    for t in range(4):
        assert sorted(rt["idx"][t].tolist()) == chosen


def test_weights_invariants_and_two_way_closed_form():
    D = synth.config(1).dims
    x = synth.make_activations(3, 0, T=64)
    wr, _ = synth.make_router(3, 0)
    rt = route(x, wr, None, D.top_k)
    w = rt["w"]
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)
    rt2 = route(x, wr, None, 2)
    l0 = np.take_along_axis(rt2["logits"], rt2["idx"][:, :1], 1)[:, 0]
    l1 = np.take_along_axis(rt2["logits"], rt2["idx"][:, 1:2], 1)[:, 0]
    np.testing.assert_allclose(rt2["w"][:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-15)


def test_skewed_verify_calibration():
    """The stored biases put exactly 48 of the 80 picks in groups 0-1."""
    tab = synth.skew_bias_table()
    assert (0, 0) in tab
    D = synth.config(2).dims
    for (seed, layer) in sorted(tab):
        x = synth.make_activations(2, seed)
        wr, bias = synth.make_router(2, seed, layer)
        idx = route(x, wr, bias, D.top_k)["idx"]
        assert int(np.sum(idx < 128)) == 48


def test_bias_add_rounds_twice_closed_form():
    """The bias is added to the already rounded fp32 logit and the sum is
    rounded again (two roundings, each to nearest-even).

    x = [1, 2^-30, 0, ...], W_r row = [1, 1, 0, ...], bias = 2^-24:
    RN32(1 + 2^-30) = 1 exactly, then 1 + 2^-24 sits halfway between 1 and
    1 + 2^-23 and ties to the even 1.  One rounding of the whole sum would
    give 1 + 2^-23; no rounding after the add would leave 1 + 2^-24.  The
    negated token with bias -2^-24 checks the same tie below -1.
    """
    d, E = 8, 4
    xf = np.zeros((2, d), dtype=np.float32)
    xf[0, 0], xf[0, 1] = 1.0, 2.0 ** -30
    xf[1, 0], xf[1, 1] = -1.0, -(2.0 ** -30)
    wf = np.zeros((E, d), dtype=np.float32)
    wf[0, 0] = wf[0, 1] = 1.0
    wf[1, 0] = wf[1, 1] = 1.0
    x = synth.bf16_bits_from_f32(xf)
    w = synth.bf16_bits_from_f32(wf)
    assert codecs.bf16_to_f64(x)[0, 1] == 2.0 ** -30
    bias = np.zeros(E, dtype=np.float32)
    bias[0] = np.float32(2.0 ** -24)
    bias[1] = np.float32(-(2.0 ** -24))
    lg = route(x, w, bias, 2)["logits"]
    assert lg[0, 0] == 1.0
    assert lg[1, 1] == -1.0
    # without a tie the bias shows: -1 + 2^-24 is exact (spacing below 1 is
    # 2^-24), and 1 + 1.5 * 2^-24 rounds up to 1 + 2^-23
    assert lg[1, 0] == -1.0 + 2.0 ** -24
    bias[0] = np.float32(3 * 2.0 ** -25)
    assert route(x, w, bias, 2)["logits"][0, 0] == 1.0 + 2.0 ** -23
