"""Pins for the KDA oracle: checks against what the pages and the mathematics fix.

None of these retypes the oracle's update: each compares it with a special case
that has its own closed form or textbook form, an invariant, brute force on tiny
inputs, or the independent chunkwise form.  Sources are the Kimi Linear summary
page ("From linear attention to Gated DeltaNet", "Kimi Delta Attention:
fine-grained memory control", "Chunkwise parallel algorithm", "Kimi Linear model
composition").  The last test rebuilds the oracle with planted mistakes and
checks that the pins catch every one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunkwise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, T, dk, dv, *, H=1, B=1, g_scale=1.0, unit_k=True, unit_q=True, s0=True):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    if unit_q:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H, dk)))) * g_scale).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    return q, k, v, g, beta, S0


def exact_unit_keys(rng, shape):
    """Keys whose fp32 values have norm exactly 1: four entries of +-0.5, the rest 0."""
    *lead, dk = shape
    k = np.zeros(shape, dtype=np.float32)
    flat = k.reshape(-1, dk)
    for row in flat:
        idx = rng.choice(dk, size=4, replace=False)
        row[idx] = 0.5 * rng.choice([-1.0, 1.0], size=4)
    return k


def f64(*xs):
    return [None if x is None else np.asarray(x, dtype=np.float64) for x in xs]


# ---------------------------------------------------------------- golden ----

def test_golden_hand_worked_example():
    """Hand-derived two-token example (tests/golden/kda_hand_d2.json)."""
    gd = json.load(open(os.path.join(GOLDEN, "kda_hand_d2.json")))
    arr = lambda key, shape: np.asarray(gd[key], dtype=np.float32).reshape(shape)
    T, dk, dv = 2, gd["dk"], gd["dv"]
    o, fin = oracle.fwd(arr("q", (1, T, 1, dk)), arr("k", (1, T, 1, dk)), arr("v", (1, T, 1, dv)),
                        arr("g", (1, T, 1, dk)), arr("beta", (1, T, 1)), scale=gd["scale"])
    np.testing.assert_allclose(o[0, :, 0], np.asarray(gd["expected_o"]), atol=gd["tolerance"], rtol=0)
    np.testing.assert_allclose(fin[0, 0], np.asarray(gd["expected_final_state"]), atol=gd["tolerance"], rtol=0)


# ------------------------------------------------------------------- P1 -----

def explicit_matrix_run(q, k, v, g, beta, S0):
    """Brute force: form M_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) as a dense matrix
    and iterate S <- M_t S + beta_t k_t v_t^T."""
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else S0.copy()
    O = np.zeros((T, v.shape[1]))
    for t in range(T):
        M = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
        S = M @ S + beta[t] * np.outer(k[t], v[t])
        O[t] = S.T @ q[t]
    return O, S


@pytest.mark.parametrize("dk,dv,T", [(4, 3, 17), (8, 8, 32), (16, 5, 9)])
def test_p1_explicit_transition_matrices(dk, dv, T):
    rng = np.random.default_rng(dk * 100 + dv)
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv, unit_k=False)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    qq, kk, vv, gg, bb, ss = f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0])
    O_ref, S_ref = explicit_matrix_run(qq, kk, vv, gg, bb, ss)
    np.testing.assert_allclose(o[0, :, 0], O_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fin[0, 0], S_ref, atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P2 -----

def test_p2_unit_gate_is_deltanet_online_gradient_descent():
    """alpha == 1 (g = 0): the update is one online gradient step with step size beta on
    the reconstruction loss L(S) = 0.5 ||S^T k - v||^2, whose gradient is k (S^T k - v)^T."""
    rng = np.random.default_rng(2)
    T, dk, dv = 40, 12, 7
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    g[:] = 0.0
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    qq, kk, vv, bb, S = f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0])
    O = np.zeros((T, dv))
    for t in range(T):
        grad = np.outer(kk[t], S.T @ kk[t] - vv[t])
        S = S - bb[t] * grad
        O[t] = S.T @ qq[t]
    np.testing.assert_allclose(o[0, :, 0], O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fin[0, 0], S, atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P3 -----

def test_p3_channel_uniform_gate_is_gated_deltanet():
    """Channel-uniform alpha_t (a scalar per token): Gated DeltaNet's scalar-gate form
    S <- alpha_t (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T (the scalar commutes)."""
    rng = np.random.default_rng(3)
    T, dk, dv = 50, 10, 6
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    gs = -np.log1p(np.exp(rng.standard_normal(T))).astype(np.float32)
    g[0, :, 0, :] = gs[:, None]
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    qq, kk, vv, bb, S, a = f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0], np.exp(gs.astype(np.float64)))
    O = np.zeros((T, dv))
    for t in range(T):
        S = a[t] * (S - bb[t] * np.outer(kk[t], kk[t] @ S)) + bb[t] * np.outer(kk[t], vv[t])
        O[t] = S.T @ qq[t]
    np.testing.assert_allclose(o[0, :, 0], O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fin[0, 0], S, atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P4 -----

def test_p4_zero_beta_is_pure_gated_decay():
    """beta == 0: S_t = Diag(exp(G_t)) S_0 with G = cumsum(g), o_t = S_0^T (q_t * exp(G_t))."""
    rng = np.random.default_rng(4)
    T, dk, dv = 33, 9, 5
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    beta[:] = 0.0
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g[0, :, 0].astype(np.float64), axis=0)
    S0d = S0[0, 0].astype(np.float64)
    O = (q[0, :, 0].astype(np.float64) * np.exp(G)) @ S0d
    np.testing.assert_allclose(o[0, :, 0], O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fin[0, 0], np.exp(G[-1])[:, None] * S0d, atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P5 -----

def test_p5_full_step_writes_value_exactly():
    """beta = 1 and ||k|| = 1: after the update the memory returns v_t for k_t exactly
    (S_t^T k_t = v_t) whatever the gate; with q_t = k_t the output is v_t."""
    rng = np.random.default_rng(5)
    T, dk, dv = 30, 16, 8
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    k = exact_unit_keys(rng, k.shape)
    beta[:] = 1.0
    o, _ = oracle.fwd(k, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0].astype(np.float64), atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P6 -----

def test_p6_householder_reflection_preserves_norm():
    """alpha == 1, beta = 2, ||k|| = 1, v = 0: S <- (I - 2 k k^T) S is a Householder
    reflection, so the Frobenius norm of the state never changes."""
    rng = np.random.default_rng(6)
    T, dk, dv = 25, 8, 8
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    k = exact_unit_keys(rng, k.shape)
    g[:] = 0.0
    beta[:] = 2.0
    v[:] = 0.0
    n0 = np.linalg.norm(S0[0, 0].astype(np.float64))
    for t_end in (1, 7, T):
        _, fin = oracle.fwd(q[:, :t_end], k[:, :t_end], v[:, :t_end], g[:, :t_end], beta[:, :t_end],
                            initial_state=S0)
        assert abs(np.linalg.norm(fin[0, 0]) - n0) <= 1e-12 * max(1.0, n0)
    # and it is a reflection, not the identity: the state itself moved
    assert np.abs(fin[0, 0] - S0[0, 0]).max() > 1e-3


# ------------------------------------------------------------------- P7 -----

def test_p7_basis_keys_decouple_into_scalar_ema():
    """k_t = e_{c_t}: each row of the state is a first-order filter.  Row c gets decay
    w_t = (1 - beta_t [c_t = c]) alpha_{t,c} and input beta_t [c_t = c] v_t, so
    row_c(T) = prod_t w_t row_c(0) + sum_t (prod_{s>t} w_s) beta_t [c_t = c] v_t."""
    rng = np.random.default_rng(7)
    T, dk, dv = 24, 6, 4
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    cs = rng.integers(0, dk, size=T)
    k[:] = 0.0
    k[0, np.arange(T), 0, cs] = 1.0
    _, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    a = np.exp(g[0, :, 0].astype(np.float64))
    bb = beta[0, :, 0].astype(np.float64)
    vv = v[0, :, 0].astype(np.float64)
    S_ref = np.zeros((dk, dv))
    for c in range(dk):
        hit = (cs == c).astype(np.float64)
        w = (1.0 - bb * hit) * a[:, c]
        row = np.prod(w) * S0[0, 0, c].astype(np.float64)
        for t in range(T):
            row = row + np.prod(w[t + 1:]) * bb[t] * hit[t] * vv[t]
        S_ref[c] = row
    np.testing.assert_allclose(fin[0, 0], S_ref, atol=1e-12, rtol=0)


# ------------------------------------------------------------------- P8 -----

def test_p8_linear_in_values_and_initial_state():
    rng = np.random.default_rng(8)
    T, dk, dv = 40, 8, 6
    q, k, v1, g, beta, S1 = rand_case(rng, T, dk, dv)
    # values on a 2^-12 grid: 0.5 x + (-2) y is then exact in fp32, so the combined
    # inputs carry no rounding of their own
    grid = lambda x: (np.round(x * 4096.0) / 4096.0).astype(np.float32)
    v1, S1 = grid(v1), grid(S1)
    v2 = grid(rng.standard_normal(v1.shape))
    S2 = grid(rng.standard_normal(S1.shape))
    a, b = 0.5, -2.0
    o1, f1 = oracle.fwd(q, k, v1, g, beta, initial_state=S1)
    o2, f2 = oracle.fwd(q, k, v2, g, beta, initial_state=S2)
    o3, f3 = oracle.fwd(q, k, (a * v1 + b * v2).astype(np.float32), g, beta,
                        initial_state=(a * S1 + b * S2).astype(np.float32))
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-11, rtol=0)
    np.testing.assert_allclose(f3, a * f1 + b * f2, atol=1e-11, rtol=0)


# ------------------------------------------------------------------- P9 -----

def test_p9_split_and_state_passing():
    """Running [0, T1) and then [T1, T) from its final state equals one run (the chunk
    algorithm's state passing); this needs the final state rounded only at fp32, so
    the split run re-enters through an fp32 state and the bound is fp32-sized."""
    rng = np.random.default_rng(9)
    T, T1, dk, dv = 60, 23, 8, 8
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    oa, fa = oracle.fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], initial_state=S0)
    ob, fb = oracle.fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:],
                        initial_state=fa.astype(np.float32))
    np.testing.assert_allclose(oa, o[:, :T1], atol=1e-13, rtol=0)
    np.testing.assert_allclose(ob, o[:, T1:], atol=1e-6, rtol=0)
    np.testing.assert_allclose(fb, fin, atol=1e-6, rtol=0)


def test_p9_packed_varlen_equals_separate_runs():
    rng = np.random.default_rng(10)
    lens = [5, 0, 17, 1, 33]
    dk, dv, H = 8, 6, 3
    T = sum(lens)
    q, k, v, g, beta, _ = rand_case(rng, T, dk, dv, H=H)
    S0 = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s = slice(cu[n], cu[n + 1])
        if L == 0:
            np.testing.assert_array_equal(fin[n], S0[n].astype(np.float64))
            continue
        on, fn = oracle.fwd(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[:, s], on)
        np.testing.assert_array_equal(fin[n], fn[0])


def test_head_subset_matches_full_run():
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_case(rng, 20, 8, 8, H=4, B=2)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    o2, fin2 = oracle.fwd(q, k, v, g, beta, initial_state=S0, heads=[3, 1])
    np.testing.assert_array_equal(o2[:, :, 0], o[:, :, 3])
    np.testing.assert_array_equal(o2[:, :, 1], o[:, :, 1])
    np.testing.assert_array_equal(fin2[:, 0], fin[:, 3])


def test_bf16_bits_are_read_exactly():
    """bf16 inputs given as raw bits must give exactly what their fp32 values give."""
    torch = pytest.importorskip("torch")
    import kda_inputs
    inp = kda_inputs.make_inputs(2, 19, 2, 16, 8, "bf16", seed=3)
    args = [kda_inputs.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
    assert args[0].dtype == np.uint16
    o_b, f_b = oracle.fwd(*args, inp.g.numpy(), inp.beta.numpy(), initial_state=inp.s0.numpy())
    args32 = [x.float().numpy() for x in (inp.q, inp.k, inp.v)]
    o_f, f_f = oracle.fwd(*args32, inp.g.numpy(), inp.beta.numpy(), initial_state=inp.s0.numpy())
    np.testing.assert_array_equal(o_b, o_f)
    np.testing.assert_array_equal(f_b, f_f)


# ------------------------------------------------------------------ P10 -----

@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("anchor", ["none", "subchunk"])
def test_p10_chunkwise_form_equals_recurrence(chunk, anchor):
    rng = np.random.default_rng(100 + chunk)
    T, dk, dv = 203, 16, 12
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv, g_scale=0.3)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0, scale=0.75)
    qq, kk, vv, gg, bb, ss = f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0])
    O, S = chunkwise.fwd_one(qq, kk, vv, gg, bb, ss, chunk, scale=0.75, anchor=anchor, sub=4 if chunk >= 16 else 1)
    np.testing.assert_allclose(O, o[0, :, 0], atol=1e-10, rtol=0)
    np.testing.assert_allclose(S, fin[0, 0], atol=1e-10, rtol=0)


def test_p10_forward_substitution_is_the_inverse():
    """Special case that reduces to a library routine: row-by-row forward substitution
    equals LAPACK's inverse of a unit lower-triangular matrix."""
    rng = np.random.default_rng(12)
    M = np.eye(20) + np.tril(rng.standard_normal((20, 20)) * 0.3, -1)
    np.testing.assert_allclose(chunkwise.forward_substitution_inverse(M), np.linalg.inv(M), atol=1e-12, rtol=0)


# ------------------------------------------------------------------ P11 -----

def test_p11_repeated_decode_equals_forward():
    rng = np.random.default_rng(13)
    T, dk, dv, N, H = 9, 8, 8, 3, 2
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv, B=N, H=H)
    S0 = rng.standard_normal((N, H, dk, dv)).astype(np.float32)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0)
    S = S0.astype(np.float64)
    for t in range(T):
        ot, S = oracle.decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S.astype(np.float32))
        # the state re-enters through fp32 each step: compare at fp32 size
        np.testing.assert_allclose(ot, o[:, t], atol=1e-5, rtol=0)
    np.testing.assert_allclose(S, fin, atol=1e-5, rtol=0)
    o1, s1 = oracle.decode(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0)
    np.testing.assert_array_equal(o1, o[:, 0])


# ------------------------------------------------------------------ P12 -----

def test_p12_state_norm_bound():
    """With ||k|| = 1, beta in [0, 1] and alpha in (0, 1], I - beta k k^T has eigenvalues
    in [1 - beta, 1] and Diag(alpha) is a contraction, so ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||
    (the L2-normalisation of q and k is there for this eigenvalue stability)."""
    rng = np.random.default_rng(14)
    T, dk, dv = 30, 8, 8
    q, k, v, g, beta, S0 = rand_case(rng, T, dk, dv)
    prev = np.linalg.norm(S0[0, 0].astype(np.float64), 2)
    for t in range(1, T + 1):
        _, fin = oracle.fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], initial_state=S0)
        cur = np.linalg.norm(fin[0, 0], 2)
        bound = prev + float(beta[0, t - 1, 0]) * np.linalg.norm(v[0, t - 1, 0].astype(np.float64))
        assert cur <= bound + 1e-12
        prev = cur


# ------------------------------------------------------- planted mistakes ----

def _pin_suite_results(lib_path):
    """Evaluate a few pins against an oracle library; return the names that fail."""
    failed = []
    gd = json.load(open(os.path.join(GOLDEN, "kda_hand_d2.json")))
    arr = lambda key, shape: np.asarray(gd[key], dtype=np.float32).reshape(shape)
    o, fin = oracle.fwd(arr("q", (1, 2, 1, 2)), arr("k", (1, 2, 1, 2)), arr("v", (1, 2, 1, 2)),
                        arr("g", (1, 2, 1, 2)), arr("beta", (1, 2, 1)), lib_path=lib_path)
    if not (np.allclose(o[0, :, 0], gd["expected_o"], atol=1e-6) and
            np.allclose(fin[0, 0], gd["expected_final_state"], atol=1e-6)):
        failed.append("golden")
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = rand_case(rng, 17, 6, 6, unit_k=False)
    o, fin = oracle.fwd(q, k, v, g, beta, initial_state=S0, lib_path=lib_path)
    O_ref, S_ref = explicit_matrix_run(*f64(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0]))
    if not (np.allclose(o[0, :, 0], O_ref, atol=1e-12) and np.allclose(fin[0, 0], S_ref, atol=1e-12)):
        failed.append("p1")
    return failed


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5])
def test_planted_mistakes_are_caught(tmp_path, mutant):
    path = str(tmp_path / f"libkda_oracle_m{mutant}.so")
    oracle.build(path, mutant=mutant)
    assert _pin_suite_results(path), f"planted mistake {mutant} was not caught by the pins"


def test_unmutated_oracle_passes_the_same_checks():
    assert _pin_suite_results(oracle.LIB_PATH) == []
