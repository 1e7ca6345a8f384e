"""Pins for the oracle's backward (``oracle.bwd``): the gradients of the token recurrence.

The pages give no gradient formulas; the backward is fixed by the forward (already pinned
in test_oracle_pins.py) and calculus.  Each check here compares ``oracle.bwd`` with
something computed another way:

* brute force: central finite differences of the forward oracle on tiny inputs, over
  every input element (q, k, v, g, beta, the initial state);
* Euler's theorem: the outputs are linear in (v, S0) and in q, so the loss equals
  <dv, v> + <dS0, S0> and sum <dO, o> equals <dq, q>;
* beta == 0 (pure gated decay, Kimi Linear summary page, "Kimi Delta Attention:
  fine-grained memory control"): closed-form gradients of o_t = S0^T (q_t * e^{G_t});
* state passing and packing: a split run and packed sequences give the same gradients.

The last tests rebuild the oracle with planted backward mistakes and check the pins
catch each of them.
"""
import numpy as np
import pytest

import oracle


def rand_case(rng, B, T, H, dk, dv, *, unit_k=True, s0=True, dsf=True):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    N = B
    S0 = (0.5 * rng.standard_normal((N, H, dk, dv))).astype(np.float32) if s0 else None
    do = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dsf_ = (0.5 * rng.standard_normal((N, H, dk, dv))).astype(np.float32) if dsf else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, do=do, dsf=dsf_)


def loss(c, lib_path=oracle.LIB_PATH, **kw):
    o, fin = oracle.fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], initial_state=c["S0"], lib_path=lib_path, **kw)
    L = float(np.sum(o * c["do"].astype(np.float64)))
    if c["dsf"] is not None:
        L += float(np.sum(fin * c["dsf"].astype(np.float64)))
    return L


def grads(c, lib_path=oracle.LIB_PATH, **kw):
    return oracle.bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], initial_state=c["S0"],
                      d_final_state=c["dsf"], lib_path=lib_path, **kw)


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "d_initial_state"}


def finite_difference(c, name, idx, eps=1e-3, lib_path=oracle.LIB_PATH, **kw):
    """Central difference of the loss in one float32 input element (the realised float32
    step sizes are used, so the quotient is exact up to the O(eps^2) truncation)."""
    x = c[name]
    x0 = float(x[idx])
    h = eps * max(1.0, abs(x0))
    xp, xm = np.float32(x0 + h), np.float32(x0 - h)
    x[idx] = xp
    lp = loss(c, lib_path, **kw)
    x[idx] = xm
    lm = loss(c, lib_path, **kw)
    x[idx] = np.float32(x0)
    return (lp - lm) / (float(xp) - float(xm))


def fd_max_error(c, lib_path=oracle.LIB_PATH, names=tuple(GRAD_OF), max_elems=None, rng=None, **kw):
    """Largest |analytic - finite difference| / max(1, |analytic|) over the checked elements."""
    gr = grads(c, lib_path, **kw)
    worst = 0.0
    for name in names:
        x = c[name]
        if x is None:
            continue
        gx = gr[GRAD_OF[name]]
        idxs = list(np.ndindex(x.shape))
        if max_elems is not None and len(idxs) > max_elems:
            pick = rng.choice(len(idxs), size=max_elems, replace=False)
            idxs = [idxs[i] for i in pick]
        for idx in idxs:
            fd = finite_difference(c, name, idx, lib_path=lib_path, **kw)
            an = float(gx[idx])
            worst = max(worst, abs(an - fd) / max(1.0, abs(an)))
    return worst


# ----------------------------------------------------------- brute force ----

@pytest.mark.parametrize("B,T,H,dk,dv,unit_k,scale", [
    (2, 6, 2, 4, 3, True, 1.0),
    (1, 9, 1, 3, 5, False, 0.7),
])
def test_bwd_matches_finite_differences_everywhere(B, T, H, dk, dv, unit_k, scale):
    rng = np.random.default_rng(11 + T)
    c = rand_case(rng, B, T, H, dk, dv, unit_k=unit_k)
    assert fd_max_error(c, scale=scale) < 2e-6


def test_bwd_matches_finite_differences_packed_sequences():
    rng = np.random.default_rng(5)
    cu = np.array([0, 3, 3, 8], dtype=np.int64)  # includes an empty sequence
    c = rand_case(rng, 1, 8, 2, 4, 4)
    c["S0"] = (0.5 * rng.standard_normal((3, 2, 4, 4))).astype(np.float32)
    c["dsf"] = (0.5 * rng.standard_normal((3, 2, 4, 4))).astype(np.float32)
    assert fd_max_error(c, cu_seqlens=cu) < 2e-6


def test_bwd_matches_finite_differences_sampled_wider_head():
    """d_k = d_v = 16 over 40 tokens (more than one checkpoint segment): 25 sampled
    elements of every input."""
    rng = np.random.default_rng(9)
    c = rand_case(rng, 1, 40, 1, 16, 16)
    assert fd_max_error(c, max_elems=25, rng=rng) < 2e-6


def test_zero_state_gradients_without_initial_state():
    """No initial state: its gradient is still returned (the state entering the sequence
    is zero) and equals the finite difference around zero."""
    rng = np.random.default_rng(3)
    c = rand_case(rng, 1, 5, 1, 3, 2, s0=False)
    gr = grads(c)
    c["S0"] = np.zeros((1, 1, 3, 2), dtype=np.float32)
    for idx in np.ndindex(c["S0"].shape):
        fd = finite_difference(c, "S0", idx)
        assert abs(gr["d_initial_state"][idx] - fd) < 2e-6


# ------------------------------------------------------------- invariants ----

def test_euler_identity_values_and_initial_state():
    """o and S_T are linear in (v, S0) for fixed q, k, g, beta, so
    L = <dv, v> + <dS0, S0> exactly (up to rounding)."""
    rng = np.random.default_rng(21)
    c = rand_case(rng, 2, 64, 2, 16, 12)
    gr = grads(c)
    lhs = loss(c)
    rhs = float(np.sum(gr["dv"] * c["v"]) + np.sum(gr["d_initial_state"] * c["S0"]))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_euler_identity_queries():
    """o_t is linear in q_t and the final state does not depend on q:
    sum <dO, o> = <dq, q>."""
    rng = np.random.default_rng(22)
    c = rand_case(rng, 1, 50, 3, 8, 8, dsf=False)
    gr = grads(c)
    lhs = loss(c)
    rhs = float(np.sum(gr["dq"] * c["q"]))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_zero_beta_closed_form():
    """beta == 0: S_t = Diag(e^{G_t}) S0 with G = cumsum(g), o_t = scale S_t^T q_t.  Then
    dq_t = scale e^{G_t} * (S0 dO_t), dS0 = sum_t e^{G_t} * (scale q_t dO_t^T) + e^{G_T} * dS_T,
    dG_t = e^{G_t} * q_t * scale (S0 dO_t) (+ e^{G_T} * rowsum(S0 .* dS_T) at t = T),
    dg_s = sum_{t >= s} dG_t, and dk = dv = 0."""
    rng = np.random.default_rng(4)
    T, dk, dv, scale = 12, 5, 4, 0.8
    c = rand_case(rng, 1, T, 1, dk, dv)
    c["beta"][:] = 0.0
    gr = grads(c, scale=scale)
    S0 = c["S0"][0, 0].astype(np.float64)
    dsf = c["dsf"][0, 0].astype(np.float64)
    G = np.cumsum(c["g"][0, :, 0].astype(np.float64), axis=0)
    q = c["q"][0, :, 0].astype(np.float64)
    do = c["do"][0, :, 0].astype(np.float64)
    eG = np.exp(G)
    sdo = do @ S0.T                                  # [T, dk]: (S0 dO_t)
    dq = scale * eG * sdo
    dS0 = (eG * q).T @ (scale * do) + eG[-1][:, None] * dsf
    dG = eG * q * scale * sdo
    dG[-1] += eG[-1] * np.sum(S0 * dsf, axis=1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    np.testing.assert_allclose(gr["dq"][0, :, 0], dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gr["d_initial_state"][0, 0], dS0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gr["dg"][0, :, 0], dg, rtol=0, atol=1e-12)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)


def test_split_run_passes_state_gradient():
    """Gradients of one run over [0, T) equal two runs: [T1, T) started from the state the
    first part ends in, then [0, T1) with the second part's initial-state gradient as its
    final-state gradient."""
    rng = np.random.default_rng(8)
    T, T1 = 30, 13
    c = rand_case(rng, 1, T, 2, 6, 5)
    full = grads(c)
    part = lambda x, s: None if x is None else x[:, s]
    first = {key: part(c[key], slice(0, T1)) for key in ("q", "k", "v", "g", "beta", "do")}
    second = {key: part(c[key], slice(T1, T)) for key in ("q", "k", "v", "g", "beta", "do")}
    _, mid = oracle.fwd(first["q"], first["k"], first["v"], first["g"], first["beta"], initial_state=c["S0"])
    second.update(S0=mid.astype(np.float32), dsf=c["dsf"])
    g2 = grads(second)
    # the middle state was rounded to float32 for the second run: compare at that level
    first.update(S0=c["S0"], dsf=g2["d_initial_state"].astype(np.float32))
    g1 = grads(first)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        joined = np.concatenate([g1[key], g2[key]], axis=1)
        np.testing.assert_allclose(joined, full[key], rtol=0, atol=2e-5 * max(1.0, np.abs(full[key]).max()))
    np.testing.assert_allclose(g1["d_initial_state"], full["d_initial_state"], rtol=0,
                               atol=2e-5 * max(1.0, np.abs(full["d_initial_state"]).max()))


def test_packed_sequences_equal_separate_runs():
    rng = np.random.default_rng(12)
    lens = [7, 1, 0, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    c = rand_case(rng, 1, T, 2, 4, 6)
    c["S0"] = (0.5 * rng.standard_normal((len(lens), 2, 4, 6))).astype(np.float32)
    c["dsf"] = (0.5 * rng.standard_normal((len(lens), 2, 4, 6))).astype(np.float32)
    packed = grads(c, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s = slice(cu[n], cu[n + 1])
        sep = {key: c[key][:, s] for key in ("q", "k", "v", "g", "beta", "do")}
        sep.update(S0=c["S0"][n:n + 1], dsf=c["dsf"][n:n + 1])
        gs = grads(sep)
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_array_equal(packed[key][:, s], gs[key])
        np.testing.assert_array_equal(packed["d_initial_state"][n], gs["d_initial_state"][0])
        if L == 0:
            np.testing.assert_array_equal(gs["d_initial_state"][0], c["dsf"][n].astype(np.float64))


def test_head_subset_and_bf16_bits():
    torch = pytest.importorskip("torch")
    import kda_inputs
    rng = np.random.default_rng(13)
    c = rand_case(rng, 1, 10, 3, 8, 8)
    to_bits = lambda x: kda_inputs.to_numpy_io(torch.from_numpy(x).to(torch.bfloat16))
    from_bits = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    cb = dict(c)
    for key in ("q", "k", "v", "do"):
        cb[key] = to_bits(c[key])
    cf = dict(c)
    for key in ("q", "k", "v", "do"):
        cf[key] = from_bits(cb[key])
    gb, gf = grads(cb), grads(cf)
    for key in gb:
        np.testing.assert_array_equal(gb[key], gf[key])
    sub = grads(cf, heads=[2, 0])
    for key in ("dq", "dk", "dv", "dg"):
        np.testing.assert_array_equal(sub[key], gf[key][:, :, [2, 0]])
    np.testing.assert_array_equal(sub["d_initial_state"], gf["d_initial_state"][:, [2, 0]])


# ------------------------------------------------------- planted mistakes ----

def _bwd_pin_failures(lib_path):
    failed = []
    rng = np.random.default_rng(31)
    c = rand_case(rng, 1, 5, 1, 3, 3, unit_k=False)
    if fd_max_error(c, lib_path=lib_path) >= 2e-6:
        failed.append("finite differences")
    c = rand_case(rng, 1, 20, 1, 6, 4)
    gr = grads(c, lib_path)
    lhs = loss(c, lib_path)
    if abs(lhs - float(np.sum(gr["dv"] * c["v"]) + np.sum(gr["d_initial_state"] * c["S0"]))) > 1e-10 * max(1, abs(lhs)):
        failed.append("euler")
    return failed


@pytest.mark.parametrize("mutant", [11, 12, 13, 14, 15])
def test_planted_backward_mistakes_are_caught(tmp_path, mutant):
    path = str(tmp_path / f"libkda_oracle_m{mutant}.so")
    oracle.build(path, mutant=mutant)
    assert _bwd_pin_failures(path), f"planted backward mistake {mutant} was not caught"


def test_unmutated_backward_passes_the_same_checks():
    assert _bwd_pin_failures(oracle.LIB_PATH) == []


@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_chunkwise_backward_equals_recurrent_backward(chunk):
    """The chunkwise reverse pass (oracle/chunkwise.py, written from the chunk equations)
    reaches the token-serial gradients, including a partial last chunk."""
    from oracle import chunkwise
    rng = np.random.default_rng(40 + chunk)
    c = rand_case(rng, 1, 70, 1, 8, 6)
    ref = grads(c, scale=0.9)
    f = lambda x: x[0, :, 0].astype(np.float64)
    got = chunkwise.bwd_one(f(c["q"]), f(c["k"]), f(c["v"]), f(c["g"]), f(c["beta"]), c["S0"][0, 0], f(c["do"]),
                            c["dsf"][0, 0], chunk, scale=0.9)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        np.testing.assert_allclose(got[key], ref[key][0, :, 0], rtol=0, atol=1e-10)
    np.testing.assert_allclose(got["d_initial_state"], ref["d_initial_state"][0, 0], rtol=0, atol=1e-10)
