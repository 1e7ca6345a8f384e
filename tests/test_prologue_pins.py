"""Pins for the prologue oracle (oracle/prologue.py): short convolution, Swish, L2 normalisation
and the gate activations of the Kimi Linear summary page, section "Kimi Linear model
composition".

Each pin checks a hand-derived value or a property the readings fix (a one-tap filter reduces
the convolution to the identity, a shifted tap delays the sequence, segments joined through the
carried state equal one run, packed sequences equal separate runs, unit norms, the softplus
and sigmoid identities); planted mistakes in the oracle fail them."""
import json
import os

import numpy as np
import pytest

from oracle import prologue as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prologue_hand.json")


def _golden_err(mutant=0):
    g = json.load(open(GOLDEN))
    a = {k: np.array(v, dtype=np.float64) for k, v in g.items() if isinstance(v, list) and k != "derivation"}
    q, k, v, gg, b, st = P.prologue(a["q_raw"], a["k_raw"], a["v_raw"], a["wq"], a["wk"], a["wv"], a["g_raw"],
                                    a["beta_raw"], [(0, 2)], conv_state=a["conv_state"], eps=g["eps"], _mutant=mutant)
    errs = [np.abs(x - a["expected_" + n]).max() for x, n in
            ((q, "q"), (k, "k"), (v, "v"), (gg, "g"), (b, "beta"), (st, "state"))]
    return max(errs), g["tolerance"]


def rand_case(seed, T=40, H=2, dk=8, dv=6, W=4):
    rng = np.random.default_rng(seed)
    q, k, g = (rng.standard_normal((T, H, dk)) for _ in range(3))
    v = rng.standard_normal((T, H, dv))
    b = rng.standard_normal((T, H))
    wq, wk = (rng.standard_normal((H, dk, W)) for _ in range(2))
    wv = rng.standard_normal((H, dv, W))
    return q, k, v, wq, wk, wv, g, b


def test_golden_hand_example():
    err, tol = _golden_err()
    assert err <= tol


def _swish(x):
    return x / (1.0 + np.exp(-x))


def test_one_tap_filter_is_identity_convolution():
    q, k, v, wq, wk, wv, g, b = rand_case(1)
    unit = lambda w: np.concatenate([np.zeros(w.shape[:-1] + (w.shape[-1] - 1,)), np.ones(w.shape[:-1] + (1,))], -1)
    qo, ko, vo, *_ = P.prologue(q, k, v, unit(wq), unit(wk), unit(wv), g, b, [(0, 40)], eps=0.0)
    sq, sk = _swish(q), _swish(k)
    assert np.allclose(qo, sq / np.linalg.norm(sq, axis=-1, keepdims=True), rtol=1e-13, atol=1e-15)
    assert np.allclose(ko, sk / np.linalg.norm(sk, axis=-1, keepdims=True), rtol=1e-13, atol=1e-15)
    assert np.allclose(vo, _swish(v), rtol=1e-13, atol=1e-15)


def test_first_tap_only_delays_by_width_minus_one():
    q, k, v, wq, wk, wv, g, b = rand_case(2)
    first = lambda w: np.concatenate([np.full(w.shape[:-1] + (1,), 2.0), np.zeros(w.shape[:-1] + (w.shape[-1] - 1,))], -1)
    qo, ko, vo, *_ = P.prologue(q, k, v, first(wq), first(wk), first(wv), g, b, [(0, 40)], eps=1e-6)
    assert np.array_equal(vo[:3], np.zeros_like(vo[:3]))  # zero before the sequence start
    assert np.allclose(vo[3:], _swish(2.0 * v[:-3]), rtol=1e-13, atol=1e-15)


def segment_error(mutant=0):
    q, k, v, wq, wk, wv, g, b = rand_case(3)
    full = P.prologue(q, k, v, wq, wk, wv, g, b, [(0, 40)], _mutant=mutant)
    a = P.prologue(q[:17], k[:17], v[:17], wq, wk, wv, g[:17], b[:17], [(0, 17)], _mutant=mutant)
    c = P.prologue(q[17:], k[17:], v[17:], wq, wk, wv, g[17:], b[17:], [(0, 23)], conv_state=a[5], _mutant=mutant)
    return max(np.abs(np.concatenate([a[i], c[i]]) - full[i]).max() for i in range(5)) + np.abs(c[5] - full[5]).max()


def test_segments_joined_through_the_state_equal_one_run():
    assert segment_error() <= 1e-14


def test_packed_sequences_equal_separate_runs():
    q, k, v, wq, wk, wv, g, b = rand_case(4)
    bounds = [(0, 0), (0, 1), (1, 15), (16, 24)]
    packed = P.prologue(q, k, v, wq, wk, wv, g, b, bounds)
    for n, (s, L) in enumerate(bounds):
        one = P.prologue(q[s:s + L], k[s:s + L], v[s:s + L], wq, wk, wv, g[s:s + L], b[s:s + L], [(0, L)])
        for i in range(5):
            assert np.array_equal(one[i], packed[i][s:s + L])
        assert np.array_equal(one[5][0], packed[5][n])


def test_unit_norms_and_activation_identities():
    q, k, v, wq, wk, wv, g, b = rand_case(5)
    qo, ko, _, go, bo, _ = P.prologue(q, k, v, wq, wk, wv, g, b, [(0, 40)], eps=0.0)
    assert np.allclose(np.linalg.norm(qo, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(np.linalg.norm(ko, axis=-1), 1.0, atol=1e-14)
    gn, bn = P.prologue(q, k, v, wq, wk, wv, -g, -b, [(0, 40)])[3:5]
    assert np.allclose(go - gn, -g, atol=1e-13)  # softplus(x) - softplus(-x) = x
    assert np.allclose(bo + bn, 1.0, atol=1e-15)  # sigmoid(x) + sigmoid(-x) = 1
    assert np.all(go < 0)


def test_bf16_raw_inputs_are_decoded():
    bits = np.array([[[0x3F80, 0xC020]]], dtype=np.uint16)  # 1.0, -2.5
    one = np.array([[[0.0, 1.0], [0.0, 1.0]]])  # identity filters, W = 2
    q, *_ = P.prologue(bits, bits, bits, one, one, one, np.zeros((1, 1, 2)), np.zeros((1, 1)), [(0, 1)], eps=0.0)
    s = _swish(np.array([1.0, -2.5]))
    assert np.allclose(q[0, 0], s / np.linalg.norm(s), rtol=1e-15)


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5])
def test_planted_mistakes_are_caught(mutant):
    err, tol = _golden_err(mutant)
    assert err > 1e3 * tol
    if mutant == 5:  # state ignored: segments no longer join
        assert segment_error(mutant) > 1e-3
