"""Prologue oracle: short convolution and Swish on q, k, v, L2 normalisation of q and k, and the
gate and beta activations (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module.  It shares no code with the HIP library.

Follows the Kimi Linear summary page, section "Kimi Linear model composition": every head's
query, key and value pass a short convolution and Swish; query and key get an L2
normalisation (for eigenvalue stability); the per-channel decay gate uses a GDN / Mamba-like
decay function.  The page gives no sizes or formulas; the readings implemented here:

* short convolution: causal and depthwise over time, one filter of W taps per (head, channel),
  c_t = sum_{i<W} w[i] x_{t-W+1+i}; the W-1 inputs before a sequence's first token are zero,
  or come from a carried-in convolution state (the raw inputs that preceded the sequence);
* Swish(x) = x sigmoid(x);
* L2 normalisation over the head dimension: x / sqrt(sum x^2 + eps);
* g = -softplus(g_raw) = -log(1 + exp(g_raw)) (log-domain decay in (-inf, 0)), beta = sigmoid(beta_raw).
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .epilogue import as_f64


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _conv(x: np.ndarray, w: np.ndarray, pad: np.ndarray, mutant: int) -> Tuple[np.ndarray, np.ndarray]:
    """x [L, H, d], w [H, d, W], pad [W-1, H, d]: causal depthwise convolution, and the last W-1
    inputs (the state handed to the next segment)."""
    W = w.shape[-1]
    L = x.shape[0]
    xp = np.concatenate([pad, x], axis=0)  # [L + W - 1, H, d]
    taps = w[..., ::-1] if mutant == 1 else w
    c = np.zeros(x.shape, dtype=np.float64)
    for i in range(W):
        c += taps[None, :, :, i] * xp[i:i + L]
    return c, xp[L:L + W - 1]


def prologue(q_raw, k_raw, v_raw, wq, wk, wv, g_raw, beta_raw, seq_bounds: Sequence[Tuple[int, int]], *,
             conv_state: Optional[np.ndarray] = None, eps: float = 1e-6, _mutant: int = 0):
    """Raw projections -> the operator's inputs.

    q_raw, k_raw [tokens, H, d_k], v_raw [tokens, H, d_v] (fp32, or uint16 bf16 bit patterns);
    wq, wk [H, d_k, W], wv [H, d_v, W] fp32; g_raw [tokens, H, d_k] and beta_raw [tokens, H] fp32;
    seq_bounds: (start, length) per sequence; conv_state [N, W-1, H, 2 d_k + d_v] (q | k | v raw
    inputs before each sequence, same encoding as the raw inputs) or None for zeros.

    Returns q, k, v, g, beta (float64) and the state after each sequence [N, W-1, H, 2 d_k + d_v].

    ``_mutant`` plants a known mistake (tests only): 1 = anti-causal taps, 2 = no Swish,
    3 = no L2 normalisation, 4 = g = +softplus, 5 = carried-in state ignored."""
    xs = [as_f64(a) for a in (q_raw, k_raw, v_raw)]
    ws = [np.asarray(a, dtype=np.float64) for a in (wq, wk, wv)]
    dk, dv = xs[0].shape[-1], xs[2].shape[-1]
    H, W = ws[0].shape[0], ws[0].shape[-1]
    outs = [np.zeros(x.shape, dtype=np.float64) for x in xs]
    N = len(seq_bounds)
    state_out = np.zeros((N, W - 1, H, 2 * dk + dv), dtype=np.float64)
    st = None if conv_state is None else as_f64(conv_state)
    cols = [(0, dk), (dk, 2 * dk), (2 * dk, 2 * dk + dv)]
    for n, (s, L) in enumerate(seq_bounds):
        for j in range(3):
            a, b = cols[j]
            pad = np.zeros((W - 1, H, b - a)) if (st is None or _mutant == 5) else st[n, :, :, a:b]
            c, last = _conv(xs[j][s:s + L], ws[j], pad, _mutant)
            y = c if _mutant == 2 else c * _sigmoid(c)
            if j < 2 and _mutant != 3:
                y = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps)
            outs[j][s:s + L] = y
            state_out[n, :, :, a:b] = last
    gr = np.asarray(g_raw, dtype=np.float64)
    g = _softplus(gr) if _mutant == 4 else -_softplus(gr)
    beta = _sigmoid(np.asarray(beta_raw, dtype=np.float64))
    return outs[0], outs[1], outs[2], g, beta, state_out
