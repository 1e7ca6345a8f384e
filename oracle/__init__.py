"""KDA oracle: plain, slow, obviously correct CPU reference (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library (``gated_delta_rule_45_amd``) and never imports it.

Two independent implementations live here:

* ``fwd`` / ``decode``: the token-by-token recurrence in C (``kda_oracle.c``),
  threaded over (sequence, head) units; the definition of the operator.
* ``bwd``: its gradients for a loss linear in the outputs and the final state, by the
  chain rule through the same recurrence, token by token in reverse (``kda_oracle.c``).
* ``dplr_fwd``: the general diagonal-plus-low-rank recurrence KDA specialises ("Less
  compute than general DPLR" section), token by token (``kda_oracle.c``); the comparator.
* ``chunkwise.py``: the chunkwise form (WY/UT transform, forward-substitution
  inverse, inter-chunk state passing) in numpy fp64, used to pin that the chunk
  algebra reaches the recurrence exactly.

Both follow the Kimi Linear summary page: "Kimi Delta Attention: fine-grained
memory control" (per-channel gate, delta-rule DPLR transition) and "Chunkwise
parallel algorithm" (chunks, WY representation, UT transform, row-by-row
forward substitution, inter-chunk recurrence plus intra-chunk output).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")


def build(out_path: str = LIB_PATH, mutant: int = 0, quiet: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math).  ``mutant`` plants a known mistake
    (tests only) so the pins can be shown to catch it."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", f"-DKDA_ORACLE_MUTANT={mutant}",
           _SRC, "-o", out_path + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out_path + ".tmp", out_path)
    return out_path


_libs = {}


def _load(path: str = LIB_PATH):
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path == LIB_PATH:
            build()
        else:
            raise FileNotFoundError(path)
    lib = ctypes.CDLL(path)
    f = lib.kda_oracle_fwd
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int64, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                  P, P, P, P, P, P, ctypes.c_int, P, P, P, ctypes.c_int]
    b = lib.kda_oracle_bwd
    b.restype = ctypes.c_int
    b.argtypes = [ctypes.c_int64, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                  P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int]
    d = lib.kda_oracle_dplr_fwd
    d.restype = ctypes.c_int
    d.argtypes = [ctypes.c_int64, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                  P, P, P, P, P, P, P, P, P, ctypes.c_int]
    _libs[path] = lib
    return lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _io_kind(*arrs) -> int:
    kinds = {a.dtype for a in arrs}
    if kinds == {np.dtype(np.float32)}:
        return 0
    if kinds == {np.dtype(np.uint16)}:
        return 1
    raise TypeError(f"q, k, v must all be float32 or all uint16 (bf16 bits); got {kinds}")


def fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray, *,
        initial_state: Optional[np.ndarray] = None, cu_seqlens: Optional[np.ndarray] = None,
        scale: float = 1.0, heads: Optional[Sequence[int]] = None, threads: Optional[int] = None,
        lib_path: str = LIB_PATH):
    """Token-by-token KDA in fp64.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] -- float32, or uint16 holding bf16 bits.
    g: [B, T, H, dk] float32 natural-log gate (alpha = exp(g)); beta: [B, T, H] float32.
    initial_state: [N, H, dk, dv] float32 or None (zeros).  cu_seqlens: int [N+1] with
    B == 1 (packed variable-length batch), else N == B.  ``heads`` restricts the work to
    a subset of heads (outputs then carry only those heads, in the given order).

    Returns (o [B, T, nsel, dv] float64, final_state [N, nsel, dk, dv] float64).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_kind(q, k, v)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    assert k.shape == q.shape and v.shape[:3] == q.shape[:3] and g.shape == q.shape
    assert beta.shape == (B, T, H)
    if cu_seqlens is not None:
        assert B == 1, "packed batches use B == 1"
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        starts = np.ascontiguousarray(cu[:-1])
        lens = np.ascontiguousarray(cu[1:] - cu[:-1])
        assert cu[0] == 0 and cu[-1] == T and np.all(lens >= 0)
    else:
        starts = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    N = len(starts)
    sel = np.arange(H, dtype=np.int32) if heads is None else np.asarray(heads, dtype=np.int32)
    assert sel.ndim == 1 and len(sel) > 0 and np.all((sel >= 0) & (sel < H))
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float32)
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, len(sel), dv), dtype=np.float64)
    fin = np.zeros((N, len(sel), dk, dv), dtype=np.float64)
    lib = _load(lib_path)
    rc = lib.kda_oracle_fwd(N, _ptr(starts), _ptr(lens), H, dk, dv, io, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(g), _ptr(beta), _ptr(s0), len(sel), _ptr(sel), _ptr(o), _ptr(fin),
                            threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    return o, fin


def decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray, state: np.ndarray, *,
           scale: float = 1.0, heads: Optional[Sequence[int]] = None, threads: Optional[int] = None,
           lib_path: str = LIB_PATH):
    """One decode step per sequence: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    state [N, H, dk, dv] float32.  Returns (o [N, nsel, dv], new_state [N, nsel, dk, dv]),
    both float64.  This is one iteration of the recurrence applied to the given state."""
    N, H, dk = q.shape
    o, fin = fwd(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], initial_state=state, scale=scale,
                 heads=heads, threads=threads, lib_path=lib_path)
    return o[:, 0], fin


def _seq_layout(B, T, cu_seqlens):
    if cu_seqlens is not None:
        assert B == 1, "packed batches use B == 1"
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        starts = np.ascontiguousarray(cu[:-1])
        lens = np.ascontiguousarray(cu[1:] - cu[:-1])
        assert cu[0] == 0 and cu[-1] == T and np.all(lens >= 0)
    else:
        starts = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    return starts, lens


def bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray, d_out: np.ndarray, *,
        initial_state: Optional[np.ndarray] = None, d_final_state: Optional[np.ndarray] = None,
        cu_seqlens: Optional[np.ndarray] = None, scale: float = 1.0, heads: Optional[Sequence[int]] = None,
        threads: Optional[int] = None, lib_path: str = LIB_PATH):
    """Gradients of the token-by-token KDA, in fp64.

    The loss is L = sum(d_out * o) + sum(d_final_state * final_state): ``d_out`` has v's
    shape and dtype (float32, or uint16 bf16 bits), ``d_final_state`` is [N, H, dk, dv]
    float32 or None (zero).  Other arguments as ``fwd``.

    Returns a dict of float64 arrays over the selected heads: dq, dk, dg [B, T, nsel, dk];
    dv [B, T, nsel, dv]; dbeta [B, T, nsel]; d_initial_state [N, nsel, dk, dv].
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_kind(q, k, v, d_out)
    q, k, v, d_out = (np.ascontiguousarray(x) for x in (q, k, v, d_out))
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    assert k.shape == q.shape and v.shape[:3] == q.shape[:3] and g.shape == q.shape and d_out.shape == v.shape
    assert beta.shape == (B, T, H)
    starts, lens = _seq_layout(B, T, cu_seqlens)
    N = len(starts)
    sel = np.arange(H, dtype=np.int32) if heads is None else np.asarray(heads, dtype=np.int32)
    assert sel.ndim == 1 and len(sel) > 0 and np.all((sel >= 0) & (sel < H))
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float32)
    dsf = None if d_final_state is None else np.ascontiguousarray(d_final_state, dtype=np.float32)
    for x in (s0, dsf):
        assert x is None or x.shape == (N, H, dk, dv)
    ns = len(sel)
    out = {"dq": np.zeros((B, T, ns, dk)), "dk": np.zeros((B, T, ns, dk)), "dv": np.zeros((B, T, ns, dv)),
           "dg": np.zeros((B, T, ns, dk)), "dbeta": np.zeros((B, T, ns)),
           "d_initial_state": np.zeros((N, ns, dk, dv))}
    lib = _load(lib_path)
    rc = lib.kda_oracle_bwd(N, _ptr(starts), _ptr(lens), H, dk, dv, io, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(g), _ptr(beta), _ptr(s0), _ptr(d_out), _ptr(dsf), ns, _ptr(sel),
                            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                            _ptr(out["d_initial_state"]), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed with code {rc}")
    return out


def dplr_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, a: np.ndarray, b: np.ndarray, g: np.ndarray, *,
             initial_state: Optional[np.ndarray] = None, cu_seqlens: Optional[np.ndarray] = None,
             scale: float = 1.0, threads: Optional[int] = None, lib_path: str = LIB_PATH):
    """General DPLR recurrence in fp64: S_t = (Diag(exp g_t) + a_t b_t^T) S_{t-1} + k_t v_t^T,
    o_t = scale S_t^T q_t.  q, k, a, b: [B, T, H, dk]; v: [B, T, H, dv] (all float32, or all
    uint16 bf16 bits); g: [B, T, H, dk] float32.  Returns (o [B, T, H, dv], final [N, H, dk, dv])."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_kind(q, k, v, a, b)
    q, k, v, a, b = (np.ascontiguousarray(x) for x in (q, k, v, a, b))
    g = np.ascontiguousarray(g, dtype=np.float32)
    assert k.shape == q.shape == a.shape == b.shape == g.shape and v.shape[:3] == q.shape[:3]
    starts, lens = _seq_layout(B, T, cu_seqlens)
    N = len(starts)
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float32)
    assert s0 is None or s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    rc = _load(lib_path).kda_oracle_dplr_fwd(N, _ptr(starts), _ptr(lens), H, dk, dv, io, float(scale), _ptr(q),
                                             _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g), _ptr(s0), _ptr(o),
                                             _ptr(fin), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_dplr_fwd failed with code {rc}")
    return o, fin
