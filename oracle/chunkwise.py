"""Chunkwise KDA in numpy fp64 -- an independent second form of the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

It follows the Kimi Linear summary page, "Chunkwise parallel algorithm" section:
the sequence is cut into fixed-length chunks and each chunk's final state is the
next chunk's initial state; the chunk's rank-1 updates are packed with a WY
representation built from one UT transform, whose lower-triangular inverse is
computed row by row by forward substitution and then reused (no second
inversion); the output merges the inter-chunk recurrent part with the
intra-chunk parallel part.  The "less compute than general DPLR" section adds
that both DPLR vectors are tied to the key, so only two C x C chunk matrices
exist: one from (k, k) and one from (q, k).

Per chunk with positions r = 1..C, in-chunk cumulative log-gate G_r = sum_{i<=r} g_i
(per channel), and initial state S (d_k x d_v):

    Kt = k * exp(G)        Qt = q * exp(G)        Kh = k * exp(-G)
    Kb = k * exp(G_C - G)
    A  = Diag(beta) strictly_lower(Kt Kh^T)                 (C x C, from k and k)
    T  = (I + A)^{-1} Diag(beta)                            (UT transform)
    W  = T Kt,   U = T V                                    (WY factors)
    D  = U - W S                                            (delta-rule corrections)
    P  = lower_incl_diag(Qt Kh^T)                           (C x C, from q and k)
    O  = scale (Qt S + P D)
    S <- Diag(exp(G_C)) S + Kb^T D

Derivation: unrolling the token recurrence inside a chunk gives
S_r = Diag(e^{G_r}) S + sum_{i<=r} Diag(e^{G_r - G_i}) k_i d_i^T with
d_r = beta_r (v_r - (Diag(e^{g_r}) S_{r-1})^T k_r); collecting the d_r gives
(I + A) D = Diag(beta)(V - Kt S).

``anchor="subchunk"`` evaluates exp(G_r - G_i) inside A and P as a product of
factors taken relative to 16-token sub-chunk boundaries (every factor of an
off-diagonal block is <= 1), the way a finite-precision kernel has to; in fp64
both forms agree to rounding.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def forward_substitution_inverse(M: np.ndarray) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix, row by row: row r of X = M^{-1} is
    e_r - sum_{m<r} M[r, m] X[m, :] (Gaussian-elimination forward substitution)."""
    n = M.shape[0]
    X = np.zeros_like(M)
    for r in range(n):
        row = np.zeros(n)
        row[r] = 1.0
        for m in range(r):
            row -= M[r, m] * X[m]
        X[r] = row
    return X


def _gate_products(G: np.ndarray, anchor: str, sub: int) -> np.ndarray:
    """E[r, i, c] = exp(G[r, c] - G[i, c]) for i <= r (zero above the diagonal)."""
    C = G.shape[0]
    E = np.zeros((C, C, G.shape[1]))
    if anchor == "none":
        for r in range(C):
            for i in range(r + 1):
                E[r, i] = np.exp(G[r]) * np.exp(-G[i])
        return E
    if anchor != "subchunk":
        raise ValueError(anchor)
    # boundary values b_R = G at the last position before sub-chunk R (b_0 = 0)
    nsub = (C + sub - 1) // sub
    b = np.zeros((nsub + 1, G.shape[1]))
    for R in range(nsub):
        b[R + 1] = G[min((R + 1) * sub, C) - 1]
    for r in range(C):
        R = r // sub
        for i in range(r + 1):
            I = i // sub
            if I == R:  # same sub-chunk: relative to the sub-chunk start
                E[r, i] = np.exp(G[r] - b[R]) * np.exp(b[R] - G[i])
            else:  # earlier sub-chunk: three factors, each <= 1
                E[r, i] = np.exp(G[r] - b[R]) * np.exp(b[R] - b[I + 1]) * np.exp(b[I + 1] - G[i])
    return E


def chunk_step(q, k, v, g, beta, S, scale: float = 1.0, anchor: str = "none", sub: int = 16):
    """One chunk: q, k, g [C, dk]; v [C, dv]; beta [C]; S [dk, dv] (all fp64).
    Returns (O [C, dv], S_next [dk, dv])."""
    C = q.shape[0]
    G = np.cumsum(g, axis=0)
    Kt, Qt = k * np.exp(G), q * np.exp(G)
    Kb = k * np.exp(G[-1] - G)
    if anchor == "none":
        Kh = k * np.exp(-G)
        KK, QK = Kt @ Kh.T, Qt @ Kh.T
    else:
        E = _gate_products(G, anchor, sub)
        KK = np.einsum("rc,ic,ric->ri", k, k, E)
        QK = np.einsum("rc,ic,ric->ri", q, k, E)
    A = beta[:, None] * np.tril(KK, -1)
    X = forward_substitution_inverse(np.eye(C) + A)
    Tm = X * beta[None, :]  # T = (I + A)^{-1} Diag(beta)
    W, U = Tm @ Kt, Tm @ v
    D = U - W @ S
    P = np.tril(QK)
    O = scale * (Qt @ S + P @ D)
    S_next = np.exp(G[-1])[:, None] * S + Kb.T @ D
    return O, S_next


def fwd_one(q, k, v, g, beta, S0: Optional[np.ndarray], chunk: int, scale: float = 1.0, anchor: str = "none",
            sub: int = 16):
    """One (sequence, head): q, k, g [T, dk]; v [T, dv]; beta [T].  Returns (O [T, dv], S_T)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        O[sl], S = chunk_step(q[sl], k[sl], v[sl], g[sl], beta[sl], S, scale, anchor, sub)
    return O, S


def bwd_one(q, k, v, g, beta, S0: Optional[np.ndarray], d_out, d_final: Optional[np.ndarray], chunk: int,
            scale: float = 1.0):
    """Gradients of ``fwd_one`` for L = sum(d_out * O) + sum(d_final * S_T), chunk by chunk
    (fp64; q, k, g, d... [T, d]).  Returns dict(dq, dk, dv, dg, dbeta, d_initial_state).

    Reverse-mode through the chunk equations above.  With X = (I + A)^{-1} and per chunk
    S (its initial state) and dS (the gradient of the state it hands on):
        dD = scale P^T dO + Kb dS             dU = X^T dD        dY = beta * dU  (= dv)
        dS <- Diag(exp(G_C)) dS + scale Qt^T dO - Kt^T dY        (gradient of S)
    and, inside the chunk, with E[r, i, c] = exp(G_rc - G_ic):
        dP = scale lower_incl(dO D^T)         dA = -strictly_lower(dU D^T)   dL = beta * dA
        dq_r  = scale e^{G_r} (S dO_r) + sum_i dP_ri k_i E_ri
        dk_r  = -beta_r e^{G_r} (S dU_r) + sum_i dL_ri k_i E_ri           (through Kt)
              + sum_r' (dP_r'r q_r' + dL_r'r k_r') E_r'r                  (through Kh)
              + e^{G_C - G_r} (dS D_r)                                    (through Kb)
        dG    = q dq + k (dk through Kt) - k (dk through Kh) - k (dk through Kb),
                plus sum_i k_i (dk_i through Kb) + e^{G_C} rowsum(dS .* S) at the last row
        dg    = reverse cumulative sum of dG over the chunk
        dbeta = rowsum(dU .* (V - Kt S)) + rowsum(dA .* strictly_lower(Kt Kh^T))
    """
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    chunks = [slice(c0, min(c0 + chunk, T)) for c0 in range(0, T, chunk)]
    saved = []
    for sl in chunks:  # forward sweep: keep each chunk's operands and initial state
        G = np.cumsum(g[sl], axis=0)
        Kt, Qt, Kh, Kb = k[sl] * np.exp(G), q[sl] * np.exp(G), k[sl] * np.exp(-G), k[sl] * np.exp(G[-1] - G)
        Lm = np.tril(Kt @ Kh.T, -1)
        X = forward_substitution_inverse(np.eye(sl.stop - sl.start) + beta[sl][:, None] * Lm)
        Y = v[sl] - Kt @ S
        D = X @ (beta[sl][:, None] * Y)
        saved.append(dict(G=G, Kt=Kt, Qt=Qt, Kh=Kh, Kb=Kb, L=Lm, X=X, P=np.tril(Qt @ Kh.T), Y=Y, D=D, S=S.copy()))
        S = np.exp(G[-1])[:, None] * S + Kb.T @ D
    out = {"dq": np.zeros((T, dk)), "dk": np.zeros((T, dk)), "dv": np.zeros((T, dv)), "dg": np.zeros((T, dk)),
           "dbeta": np.zeros(T)}
    dS = np.zeros((dk, dv)) if d_final is None else np.array(d_final, dtype=np.float64)
    for sl, o in reversed(list(zip(chunks, saved))):
        b, do, G = beta[sl], d_out[sl], o["G"]
        dD = scale * o["P"].T @ do + o["Kb"] @ dS
        dU = o["X"].T @ dD
        dY = b[:, None] * dU
        E = np.exp(G[:, None, :] - G[None, :, :])
        dP = scale * np.tril(do @ o["D"].T)
        dA = -np.tril(dU @ o["D"].T, -1)
        dL = b[:, None] * dA
        Sc = o["S"]
        dq = scale * np.exp(G) * (do @ Sc.T) + np.einsum("ri,ic,ric->rc", dP, k[sl], E)
        dk_t = -b[:, None] * np.exp(G) * (dU @ Sc.T) + np.einsum("ri,ic,ric->rc", dL, k[sl], E)
        dk_h = np.einsum("ri,rc,ric->ic", dP, q[sl], E) + np.einsum("ri,rc,ric->ic", dL, k[sl], E)
        dk_b = np.exp(G[-1] - G) * (o["D"] @ dS.T)
        dG = q[sl] * dq + k[sl] * (dk_t - dk_h - dk_b)
        dG[-1] += np.sum(k[sl] * dk_b, axis=0) + np.exp(G[-1]) * np.sum(dS * Sc, axis=1)
        out["dq"][sl], out["dk"][sl], out["dv"][sl] = dq, dk_t + dk_h + dk_b, dY
        out["dg"][sl] = np.cumsum(dG[::-1], axis=0)[::-1]
        out["dbeta"][sl] = np.sum(dU * o["Y"], axis=1) + np.sum(dA * o["L"], axis=1)
        dS = np.exp(G[-1])[:, None] * dS + scale * o["Qt"].T @ do - o["Kt"].T @ dY
    out["d_initial_state"] = dS
    return out


def dplr_chunk_step(q, k, v, a, b, g, S, scale: float = 1.0):
    """One chunk of the general DPLR recurrence S_i = (Diag(e^{g_i}) + a_i b_i^T) S_{i-1} + k_i v_i^T
    (fp64; q, k, a, b, g [C, dk]; v [C, dv]; S [dk, dv]).  Returns (O [C, dv], S_next).

    Unrolling the chunk from its initial state S with G = cumsum(g):
        S_r = Diag(e^{G_r}) S + sum_{i<=r} Diag(e^{G_r - G_i}) (a_i u_i + k_i v_i),  u_i = b_i^T S_{i-1}.
    With Bt_r = b_r e^{G_{r-1}} (G_{-1} = 0), Qt = q e^{G}, Ah = a e^{-G}, Kh = k e^{-G},
    Ab = a e^{G_C - G}, Kb = k e^{G_C - G}, the four chunk matrices are
        M_ba = strictly_lower(Bt Ah^T)    M_bk = strictly_lower(Bt Kh^T)
        M_qa = lower_incl(Qt Ah^T)        M_qk = lower_incl(Qt Kh^T)
    and
        U  = (I - M_ba)^{-1} (Bt S + M_bk V)           (the low-rank read-outs u_i)
        O  = scale (Qt S + M_qa U + M_qk V)
        S' = Diag(e^{G_C}) S + Ab^T U + Kb^T V
    KDA ties a = -beta k, b = e^{g} k and writes with beta k, so M_ba and M_bk (and M_qa and
    M_qk) collapse into one matrix each ("Less compute than general DPLR" section)."""
    C = q.shape[0]
    G = np.cumsum(g, axis=0)
    Gp = np.vstack([np.zeros((1, G.shape[1])), G[:-1]])
    Bt, Qt = b * np.exp(Gp), q * np.exp(G)
    Ah, Kh = a * np.exp(-G), k * np.exp(-G)
    Ab, Kb = a * np.exp(G[-1] - G), k * np.exp(G[-1] - G)
    Mba, Mbk = np.tril(Bt @ Ah.T, -1), np.tril(Bt @ Kh.T, -1)
    Mqa, Mqk = np.tril(Qt @ Ah.T), np.tril(Qt @ Kh.T)
    Xinv = forward_substitution_inverse(np.eye(C) - Mba)
    U = Xinv @ (Bt @ S + Mbk @ v)
    O = scale * (Qt @ S + Mqa @ U + Mqk @ v)
    S_next = np.exp(G[-1])[:, None] * S + Ab.T @ U + Kb.T @ v
    return O, S_next


def dplr_fwd_one(q, k, v, a, b, g, S0: Optional[np.ndarray], chunk: int, scale: float = 1.0):
    """One (sequence, head) of the general DPLR recurrence, chunk by chunk."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        O[sl], S = dplr_chunk_step(q[sl], k[sl], v[sl], a[sl], b[sl], g[sl], S, scale)
    return O, S
