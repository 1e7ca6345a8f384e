"""Output-epilogue oracle: per-head RMSNorm followed by the data-dependent output gate (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module.  It shares no code with the HIP library.

Follows the Kimi Linear summary page, section "Kimi Linear model composition": before the
output projection, every head's output passes a per-head RMSNorm and a data-dependent output
gate (itself a low-rank projection of the layer input, computed outside this operator).  The
page gives no formula; the reading implemented here, for each (token, head) row of d_v values
o, with the gate pre-activation z of the same shape and a weight w [d_v] shared by the heads:

    out = o / sqrt(mean(o * o) + eps) * w * sigmoid(z),    sigmoid(z) = 1 / (1 + exp(-z))
"""
from __future__ import annotations

import numpy as np


def as_f64(x: np.ndarray) -> np.ndarray:
    """fp32 arrays as they are; uint16 arrays are bf16 bit patterns (upper half of an fp32)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def norm_gate(o: np.ndarray, gate: np.ndarray, weight: np.ndarray, eps: float, _mutant: int = 0) -> np.ndarray:
    """RMSNorm over the last axis (one head's d_v values) times weight times sigmoid(gate).

    ``_mutant`` plants a known mistake (tests only): 1 = sum instead of mean, 2 = eps left
    out, 3 = swish instead of sigmoid, 4 = statistics over the head axis as well."""
    o, z, w = as_f64(o), as_f64(gate), as_f64(weight)
    if _mutant == 1:
        ms = np.sum(o * o, axis=-1, keepdims=True)
    elif _mutant == 4:
        ms = np.mean(o * o, axis=(-2, -1), keepdims=True)
    else:
        ms = np.mean(o * o, axis=-1, keepdims=True)
    denom = np.sqrt(ms if _mutant == 2 else ms + eps)
    gate_act = 1.0 / (1.0 + np.exp(-z))
    if _mutant == 3:
        gate_act = z * gate_act
    return o / denom * w * gate_act
