"""Pins for the general-DPLR comparator oracle (``oracle.dplr_fwd``).

Kimi Linear summary page, "Less compute than general DPLR" section: KDA is the DPLR
transition with both low-rank vectors tied to the key.  Checks: (1) with a = -beta k,
b = e^{g} k and write key beta k the DPLR oracle reproduces the (separately pinned) KDA
oracle; (2) dense transition matrices (Diag(e^g) + a b^T) iterated explicitly; (3) the
four-matrix chunkwise form in oracle/chunkwise.py reaches the recurrence; (4) linearity in
(v, S0); (5) a planted mistake is caught.
"""
import numpy as np
import pytest

import oracle
from oracle import chunkwise


def rand_dplr(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = (0.5 * rng.standard_normal((B, T, H, dk))).astype(np.float32)
    a = (0.3 * rng.standard_normal((B, T, H, dk))).astype(np.float32)
    b = (0.3 * rng.standard_normal((B, T, H, dk))).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return q, k, v, a, b, g, S0


def test_kda_is_the_key_tied_special_case():
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 2, 40, 2, 8, 6
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    o_kda, f_kda = oracle.fwd(q, k, v, g, beta, initial_state=S0, scale=0.8)
    # DPLR inputs are float32: a = -beta k, b = e^g k and the write key beta k are rounded
    # to float32, so compare at float32 level
    a = (-beta[..., None] * k).astype(np.float32)
    b = (np.exp(g.astype(np.float64)) * k).astype(np.float32)
    kw = (beta[..., None] * k).astype(np.float32)
    o_d, f_d = oracle.dplr_fwd(q, kw, v, a, b, g, initial_state=S0, scale=0.8)
    np.testing.assert_allclose(o_d, o_kda, rtol=0, atol=2e-6 * np.abs(o_kda).max())
    np.testing.assert_allclose(f_d, f_kda, rtol=0, atol=2e-6 * np.abs(f_kda).max())


def dense_run(q, k, v, a, b, g, S0, scale):
    S = S0.copy()
    O = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        M = np.diag(np.exp(g[t])) + np.outer(a[t], b[t])
        S = M @ S + np.outer(k[t], v[t])
        O[t] = scale * S.T @ q[t]
    return O, S


def f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def test_explicit_transition_matrices():
    rng = np.random.default_rng(2)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 1, 23, 1, 6, 5)
    o, fin = oracle.dplr_fwd(q, k, v, a, b, g, initial_state=S0, scale=1.3)
    O, S = dense_run(*f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], g[0, :, 0], S0[0, 0]), 1.3)
    np.testing.assert_allclose(o[0, :, 0], O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], S, rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_four_matrix_chunk_form_equals_recurrence(chunk):
    rng = np.random.default_rng(3 + chunk)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 1, 75, 1, 8, 6)
    o, fin = oracle.dplr_fwd(q, k, v, a, b, g, initial_state=S0, scale=0.9)
    O, S = chunkwise.dplr_fwd_one(*f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], g[0, :, 0]),
                                  S0[0, 0].astype(np.float64), chunk, scale=0.9)
    np.testing.assert_allclose(O, o[0, :, 0], rtol=0, atol=1e-10 * max(1, np.abs(o).max()))
    np.testing.assert_allclose(S, fin[0, 0], rtol=0, atol=1e-10 * max(1, np.abs(fin).max()))


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(4)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 1, 30, 2, 4, 4)
    v2 = rng.standard_normal(v.shape).astype(np.float32)
    S2 = rng.standard_normal(S0.shape).astype(np.float32)
    o1, f1 = oracle.dplr_fwd(q, k, v, a, b, g, initial_state=S0)
    o2, f2 = oracle.dplr_fwd(q, k, v2, a, b, g, initial_state=S2)
    o3, f3 = oracle.dplr_fwd(q, k, (v + v2).astype(np.float64).astype(np.float32), a, b, g,
                             initial_state=(S0.astype(np.float64) + S2).astype(np.float32))
    # v + v2 and S0 + S2 rounded to float32: compare at that level
    np.testing.assert_allclose(o3, o1 + o2, rtol=0, atol=1e-5 * np.abs(o3).max())
    np.testing.assert_allclose(f3, f1 + f2, rtol=0, atol=1e-5 * np.abs(f3).max())


def test_packed_sequences_equal_separate_runs():
    rng = np.random.default_rng(5)
    lens = [5, 0, 17, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, v, a, b, g, _ = rand_dplr(rng, 1, int(cu[-1]), 2, 4, 3)
    S0 = (0.5 * rng.standard_normal((len(lens), 2, 4, 3))).astype(np.float32)
    o, fin = oracle.dplr_fwd(q, k, v, a, b, g, initial_state=S0, cu_seqlens=cu)
    for n in range(len(lens)):
        s = slice(cu[n], cu[n + 1])
        o1, f1 = oracle.dplr_fwd(q[:, s], k[:, s], v[:, s], a[:, s], b[:, s], g[:, s], initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[:, s], o1)
        np.testing.assert_array_equal(fin[n], f1[0])


def test_planted_mistake_is_caught(tmp_path):
    path = str(tmp_path / "libkda_oracle_m21.so")
    oracle.build(path, mutant=21)
    rng = np.random.default_rng(2)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 1, 23, 1, 6, 5)
    o, fin = oracle.dplr_fwd(q, k, v, a, b, g, initial_state=S0, scale=1.3, lib_path=path)
    O, S = dense_run(*f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], g[0, :, 0], S0[0, 0]), 1.3)
    assert np.abs(o[0, :, 0] - O).max() > 1e-6
