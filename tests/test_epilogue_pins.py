"""Pins for the output-epilogue oracle (oracle/epilogue.py): per-head RMSNorm and the output
gate of the Kimi Linear summary page, section "Kimi Linear model composition".

None of these re-types the oracle's formula: each checks a value derived by hand or a
property the reading fixes (unit RMS, scale invariance, the gate's symmetry), and planted
mistakes in the oracle are shown to fail them."""
import json
import os

import numpy as np
import pytest

from oracle import epilogue

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "norm_gate_hand.json")


def _golden(mutant=0):
    g = json.load(open(GOLDEN))
    out = epilogue.norm_gate(np.array(g["o"]), np.array(g["gate"]), np.array(g["weight"]), g["eps"], _mutant=mutant)
    return np.abs(out - np.array(g["expected"])).max(), g["tolerance"]


def _rows(seed, shape=(3, 4, 128), scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


def test_golden_hand_example():
    err, tol = _golden()
    assert err <= tol


def unit_rms_error(mutant=0):
    o = _rows(1, scale=5.0)
    out = epilogue.norm_gate(o, np.full(o.shape, 40.0), np.ones(o.shape[-1]), 0.0, _mutant=mutant)
    return np.abs(np.mean(out * out, axis=-1) - 1.0).max()


def test_unit_rms_per_head():
    # sigmoid(40) = 1 - 4e-18, w = 1, eps = 0: every (token, head) row has unit RMS
    assert unit_rms_error() <= 1e-12


def test_scale_invariance_and_sign():
    o, z, w = _rows(2), _rows(3), 1.0 + 0.1 * _rows(4, (128,))
    base = epilogue.norm_gate(o, z, w, 0.0)
    assert np.allclose(epilogue.norm_gate(3.7 * o, z, w, 0.0), base, rtol=1e-13, atol=0)
    assert np.array_equal(epilogue.norm_gate(-o, z, w, 0.0), -base)


def gate_symmetry_error(mutant=0):
    o, z, w = _rows(5), _rows(6, scale=3.0), 1.0 + 0.1 * _rows(7, (128,))
    a = epilogue.norm_gate(o, z, w, 1e-6, _mutant=mutant)
    b = epilogue.norm_gate(o, -z, w, 1e-6, _mutant=mutant)
    half = epilogue.norm_gate(o, np.zeros_like(z), w, 1e-6, _mutant=mutant)
    return np.abs(a + b - 2.0 * half).max()


def test_gate_symmetry():
    # sigmoid(z) + sigmoid(-z) = 1 and sigmoid(0) = 1/2
    assert gate_symmetry_error() <= 1e-13


def test_zero_row_with_eps_is_zero():
    o = np.zeros((2, 2, 64))
    out = epilogue.norm_gate(o, _rows(8, (2, 2, 64)), np.ones(64), 1e-6)
    assert np.array_equal(out, np.zeros_like(out))


def test_bf16_bit_decoding():
    bits = np.array([0x3F80, 0xC020, 0x0000, 0x3E80], dtype=np.uint16)  # 1.0, -2.5, 0.0, 0.25
    assert np.array_equal(epilogue.as_f64(bits), np.array([1.0, -2.5, 0.0, 0.25]))


@pytest.mark.parametrize("mutant", [1, 2, 3, 4])
def test_planted_mistakes_are_caught(mutant):
    err, tol = _golden(mutant)
    assert err > 1e3 * tol
    if mutant == 1:  # sum instead of mean
        assert unit_rms_error(mutant) > 1e-3
    if mutant == 3:  # swish instead of sigmoid
        assert gate_symmetry_error(mutant) > 1e-3
