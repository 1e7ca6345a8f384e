"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libkda.so`` (C ABI in ``include/kda.h``).  It only checks
and marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory and the stream; nothing here computes
KDA itself, and there is no fallback: if the library is missing or the call fails,
an exception is raised.

Entry points (same names as the C ABI):

* ``chunk_fwd``     -- chunkwise prefill (q, k, v, g, beta, optional initial state,
                       optional cu_seqlens -> out, final state)
* ``recurrent_fwd`` -- token-by-token reference mode on the GPU (same arguments)
* ``decode_step``   -- one token per sequence, state updated in place
* ``query``         -- launch configuration, algorithmic flops/bytes, device info
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_fwd_prologue", "chunk_fwd_noalloc", "noalloc_scratch_bytes", "chunk_bwd", "dplr_chunk_fwd", "recurrent_fwd", "decode_step", "decode_step_gated", "prologue", "norm_gate", "query", "tune", "KdaError",
           "LIB_PATH", "library"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_QUERY_DEVICE = 1
KDA_ALGO_AUTO, KDA_ALGO_FUSED, KDA_ALGO_TWO_PASS = 0, 1, 2
_ALGOS = {"auto": KDA_ALGO_AUTO, "fused": KDA_ALGO_FUSED, "two_pass": KDA_ALGO_TWO_PASS}


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("chunk_size", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dv_tile", ctypes.c_int32), ("algo", ctypes.c_int)]


class PrologueProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


class QueryResult(ctypes.Structure):
    _fields_ = [("version", ctypes.c_int32), ("supported", ctypes.c_int32), ("algo", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t),
                ("chunk_size", ctypes.c_int32), ("dv_tile", ctypes.c_int32), ("threads_per_block", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("grid_blocks", ctypes.c_int64), ("flops", ctypes.c_double),
                ("hbm_bytes", ctypes.c_double), ("device_ok", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("arch", ctypes.c_char * 64), ("peak_bf16_tflops", ctypes.c_double),
                ("peak_hbm_gbps", ctypes.c_double), ("tuned_ms", ctypes.c_double)]


_lib = None
_P = ctypes.c_void_p


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]
    lib.kda_recurrent_fwd.restype = ctypes.c_int
    lib.kda_recurrent_fwd.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.kda_tune.restype = ctypes.c_int
    lib.kda_tune.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P,
                             ctypes.POINTER(QueryResult)]
    lib.kda_prologue.restype = ctypes.c_int
    lib.kda_prologue.argtypes = [ctypes.POINTER(PrologueProblem)] + [_P] * 17
    lib.kda_chunk_fwd_prologue.restype = ctypes.c_int
    lib.kda_chunk_fwd_prologue.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_float] + [_P] * 14 + \
        [ctypes.c_size_t, _P]
    lib.kda_decode_step_gated.restype = ctypes.c_int
    lib.kda_decode_step_gated.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_float, _P, _P]
    lib.kda_norm_gate.restype = ctypes.c_int
    lib.kda_norm_gate.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P]
    lib.kda_dplr_chunk_fwd.restype = ctypes.c_int
    lib.kda_dplr_chunk_fwd.argtypes = [ctypes.POINTER(Problem)] + [_P] * 12
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(Problem)] + [_P] * 17 + [ctypes.c_size_t, _P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(Problem)] + [_P] * 11
    lib.kda_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_chunk_bwd_workspace.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_query.restype = ctypes.c_int
    lib.kda_query.argtypes = [ctypes.POINTER(Problem), ctypes.c_uint32, ctypes.POINTER(QueryResult)]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != KDA_OK:
        lib = library()
        raise KdaError(status, f"{lib.kda_status_string(status).decode()}: {lib.kda_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _keep_for_stream(t: Optional[torch.Tensor], device: torch.device, stream) -> None:
    """A scratch tensor allocated here (on the current stream) and dropped on return: tell the
    caching allocator that the launch stream still uses it, so the block is not handed to a new
    allocation before the kernels queued on that stream have finished with it."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return KDA_BF16
    if dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be torch.bfloat16 or torch.float32, got {dtype}")


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _algo_code(algo) -> int:
    if isinstance(algo, str):
        if algo not in _ALGOS:
            raise ValueError(f"algo must be one of {sorted(_ALGOS)}")
        return _ALGOS[algo]
    return int(algo)


def _problem_from(q, v, cu_seqlens, chunk_size, scale, dv_tile, algo=0) -> Tuple[Problem, int]:
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("a packed batch (cu_seqlens) needs B == 1")
        n = cu_seqlens.numel() - 1
    else:
        n = B
    p = Problem(batch=B, seq_len=T, num_heads=H, head_dim_k=dk, head_dim_v=dv,
                num_seqs=n if cu_seqlens is not None else 0, io_dtype=_io_code(q.dtype), chunk_size=chunk_size,
                scale=scale, dv_tile=dv_tile, algo=_algo_code(algo))
    return p, n


def workspace_bytes(p: Problem) -> int:
    """Workspace the two-pass algorithm needs for problem p (0 if it would not be used)."""
    r = QueryResult()
    st = library().kda_query(ctypes.byref(p), 0, ctypes.byref(r))
    _check(st)
    return int(r.workspace_bytes)


def _fwd(entry: str, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, chunk_size, scale, dv_tile, out,
         final_state, output_final_state, stream, algo=0, workspace=None):
    dev = q.device
    p, n = _problem_from(q, v, cu_seqlens, chunk_size, scale, dv_tile, algo if entry in ("chunk", "tune") else 0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", q.dtype, (B, T, H, dk), dev)
    _need(k, "k", q.dtype, (B, T, H, dk), dev)
    _need(v, "v", q.dtype, (B, T, H, dv), dev)
    _need(g, "g", torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, dk, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), dev)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
        if host_cu.numel() != n + 1:
            raise ValueError("cu_seqlens_host has the wrong length")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (n, H, dk, dv), dev)
    lib = library()
    common = [ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
              None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr()), _ptr(out), _ptr(final_state)]
    if entry == "tune":
        if workspace is None and p.algo != KDA_ALGO_FUSED:  # room for the largest two-pass candidate
            need = 0
            for c in ((p.chunk_size,) if p.chunk_size else (16, 32, 64)):
                q2 = Problem(**{f: getattr(p, f) for f, _ in Problem._fields_})
                q2.chunk_size, q2.algo, q2.dv_tile = c, KDA_ALGO_TWO_PASS, 32
                r = QueryResult()
                if lib.kda_query(ctypes.byref(q2), 0, ctypes.byref(r)) == KDA_OK:
                    need = max(need, r.workspace_bytes)
            workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
        ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
        res = QueryResult()
        st = lib.kda_tune(*common, ws_ptr, ws_len, _stream_handle(dev, stream), ctypes.byref(res))
        _check(st)  # kda_tune synchronises the stream before it returns
        d = {name: getattr(res, name) for name, _ in QueryResult._fields_}
        d["arch"] = res.arch.decode()
        return d, out, final_state
    if entry == "chunk":
        own_ws = None
        if workspace is None and p.algo != KDA_ALGO_FUSED:
            need = workspace_bytes(p)
            workspace = own_ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
        ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = lib.kda_chunk_fwd(*common, ws_ptr, ws_len, _stream_handle(dev, stream))
        _keep_for_stream(own_ws, dev, stream)
    else:
        st = lib.kda_recurrent_fwd(*common, _stream_handle(dev, stream))
    _check(st)
    return out, final_state


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
              cu_seqlens_host=None, chunk_size: int = 0, scale: float = 1.0, dv_tile: int = 0,
              algo="auto", workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, output_final_state: bool = True, stream=None,
              gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
              norm_eps: float = 1e-6):
    """Chunkwise KDA forward.  q, k: [B, T, H, d_k]; v: [B, T, H, d_v] (bf16 or fp32);
    g: [B, T, H, d_k] fp32 log-gate; beta: [B, T, H] fp32; initial_state: [N, H, d_k, d_v]
    fp32 or None; cu_seqlens: int32 [N+1] (B == 1) or None.  algo: "auto", "fused" or
    "two_pass"; workspace: uint8 device tensor for the two-pass algorithm (allocated here
    when None and needed).  With gate (shape and dtype of out) and norm_weight (fp32 [d_v]),
    the output epilogue (kda_norm_gate) is applied to out in place on the same stream.
    Returns (out, final_state)."""
    out, fin = _fwd("chunk", q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, chunk_size, scale, dv_tile,
                    out, final_state, output_final_state, stream, algo=algo, workspace=workspace)
    if gate is not None or norm_weight is not None:
        norm_gate(out, gate, norm_weight, eps=norm_eps, out=out, stream=stream)
    return out, fin


def chunk_fwd_prologue(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor, conv_q: torch.Tensor,
                       conv_k: torch.Tensor, conv_v: torch.Tensor, g_raw: torch.Tensor, beta_raw: torch.Tensor,
                       initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                       cu_seqlens_host=None, norm_eps: float = 1e-6, chunk_size: int = 0, scale: float = 1.0,
                       dv_tile: int = 0, workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       final_state: Optional[torch.Tensor] = None, output_final_state: bool = True, stream=None):
    """Chunkwise forward on the raw projections with the prologue fused into the two-pass kernels
    (kda_chunk_fwd_prologue): the inputs are those of prologue() (zero convolution state), the
    result that of chunk_fwd on prologue()'s outputs.  Returns (out, final_state)."""
    dev = q_raw.device
    p, n = _problem_from(q_raw, v_raw, cu_seqlens, chunk_size, scale, dv_tile, KDA_ALGO_TWO_PASS)
    B, T, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    W = conv_q.shape[-1]
    dt = q_raw.dtype
    for t, name, tdt, shape in ((q_raw, "q_raw", dt, (B, T, H, dk)), (k_raw, "k_raw", dt, (B, T, H, dk)),
                                (v_raw, "v_raw", dt, (B, T, H, dv)), (g_raw, "g_raw", torch.float32, (B, T, H, dk)),
                                (beta_raw, "beta_raw", torch.float32, (B, T, H)),
                                (conv_q, "conv_q", torch.float32, (H, dk, W)), (conv_k, "conv_k", torch.float32, (H, dk, W)),
                                (conv_v, "conv_v", torch.float32, (H, dv, W))):
        _need(t, name, tdt, shape, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, dk, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), dev)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
        if host_cu.numel() != n + 1:
            raise ValueError("cu_seqlens_host has the wrong length")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(out, "out", dt, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (n, H, dk, dv), dev)
    own_ws = None
    if workspace is None:
        need = workspace_bytes(p)
        workspace = own_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = library().kda_chunk_fwd_prologue(
        ctypes.byref(p), W, norm_eps, _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v),
        _ptr(g_raw), _ptr(beta_raw), _ptr(initial_state), _ptr(cu_seqlens),
        None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr()), _ptr(out), _ptr(final_state),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), _stream_handle(dev, stream))
    _keep_for_stream(own_ws, dev, stream)
    _check(st)
    return out, final_state


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                      initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                      cu_seqlens_host=None, chunk_size: int = 0, scale: float = 1.0, dv_tile: int = 0,
                      out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                      output_final_state: bool = True, stream=None):
    """chunk_fwd (two-pass) with the library's fixed scratch array instead of a workspace
    (kda_chunk_fwd_noalloc): the library allocates nothing.  Pass `out` and `final_state` to
    allocate nothing here either.  Returns (out, final_state)."""
    dev = q.device
    p, n = _problem_from(q, v, cu_seqlens, chunk_size, scale, dv_tile, KDA_ALGO_TWO_PASS)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for t, name, dt, shape in ((q, "q", q.dtype, (B, T, H, dk)), (k, "k", q.dtype, (B, T, H, dk)),
                               (v, "v", q.dtype, (B, T, H, dv)), (g, "g", torch.float32, (B, T, H, dk)),
                               (beta, "beta", torch.float32, (B, T, H))):
        _need(t, name, dt, shape, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, dk, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), dev)
    host_cu = None if cu_seqlens_host is None else torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (n, H, dk, dv), dev)
    st = library().kda_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(initial_state), _ptr(cu_seqlens),
                                         None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr()),
                                         _ptr(out), _ptr(final_state), _stream_handle(dev, stream))
    _check(st)
    return out, final_state


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-device scratch array chunk_fwd_noalloc uses."""
    return int(library().kda_noalloc_scratch_bytes())


def bwd_workspace_bytes(p: Problem) -> int:
    """Workspace kda_chunk_bwd needs for problem p."""
    n = ctypes.c_size_t(0)
    _check(library().kda_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              d_out: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              d_final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
              cu_seqlens_host=None, chunk_size: int = 0, scale: float = 1.0, need_d_initial_state: bool = True,
              workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None, stream=None) -> dict:
    """Gradients of chunk_fwd for L = sum(d_out * out) + sum(d_final_state * final_state).
    Arguments as chunk_fwd; d_out has out's shape and dtype, d_final_state is [N, H, d_k, d_v]
    fp32 or None.  Returns dict(dq, dk, dv (io dtype), dg, dbeta, d_initial_state (fp32 or None));
    `out` (a dict returned by an earlier call of the same shape) is written in place."""
    dev = q.device
    p, n = _problem_from(q, v, cu_seqlens, chunk_size, scale, 0, 0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", q.dtype, (B, T, H, dk), dev)
    _need(k, "k", q.dtype, (B, T, H, dk), dev)
    _need(v, "v", q.dtype, (B, T, H, dv), dev)
    _need(g, "g", torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(d_out, "d_out", q.dtype, (B, T, H, dv), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, dk, dv), dev)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", torch.float32, (n, H, dk, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), dev)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
        if host_cu.numel() != n + 1:
            raise ValueError("cu_seqlens_host has the wrong length")
    if out is None:
        out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
               "dg": torch.empty((B, T, H, dk), dtype=torch.float32, device=dev),
               "dbeta": torch.empty((B, T, H), dtype=torch.float32, device=dev),
               "d_initial_state": torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
               if need_d_initial_state else None}
    else:
        for key, dt, shape in (("dq", q.dtype, (B, T, H, dk)), ("dk", q.dtype, (B, T, H, dk)),
                               ("dv", q.dtype, (B, T, H, dv)), ("dg", torch.float32, (B, T, H, dk)),
                               ("dbeta", torch.float32, (B, T, H))):
            _need(out[key], key, dt, shape, dev)
        if out.get("d_initial_state") is not None:
            _need(out["d_initial_state"], "d_initial_state", torch.float32, (n, H, dk, dv), dev)
    own_ws = None
    if workspace is None:
        workspace = own_ws = torch.empty(bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
    lib = library()
    st = lib.kda_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr()),
                           _ptr(d_out), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                           _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["d_initial_state"]),
                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream_handle(dev, stream))
    _keep_for_stream(own_ws, dev, stream)
    _check(st)
    return out


def dplr_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                   g: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, *, cu_seqlens_host=None, chunk_size: int = 0,
                   scale: float = 1.0, dv_tile: int = 0, out: Optional[torch.Tensor] = None,
                   final_state: Optional[torch.Tensor] = None, output_final_state: bool = True, stream=None):
    """General-DPLR comparator: S_t = (Diag(exp g_t) + a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t.
    q, k, a, b: [B, T, H, d_k]; v: [B, T, H, d_v] (same dtype); g fp32 [B, T, H, d_k].
    Returns (out, final_state)."""
    dev = q.device
    p, n = _problem_from(q, v, cu_seqlens, chunk_size, scale, dv_tile, 0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for t, name in ((q, "q"), (k, "k"), (a, "a"), (b, "b")):
        _need(t, name, q.dtype, (B, T, H, dk), dev)
    _need(v, "v", q.dtype, (B, T, H, dv), dev)
    _need(g, "g", torch.float32, (B, T, H, dk), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, dk, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), dev)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    st = library().kda_dplr_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g),
                                      _ptr(initial_state), _ptr(cu_seqlens),
                                      None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr()), _ptr(out),
                                      _ptr(final_state), _stream_handle(dev, stream))
    _check(st)
    return out, final_state


def tune(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
         initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
         cu_seqlens_host=None, chunk_size: int = 0, scale: float = 1.0, dv_tile: int = 0, algo="auto",
         workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
         final_state: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Time every supported chunk_fwd configuration on these tensors (fields given here stay
    fixed) and return the fastest as a query dict with 'tuned_ms'.  out / final_state are
    overwritten; initial_state must not be final_state."""
    cfg, _, _ = _fwd("tune", q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, chunk_size, scale,
                     dv_tile, out, final_state, True, stream, algo=algo, workspace=workspace)
    return cfg


def recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                  initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                  cu_seqlens_host=None, scale: float = 1.0, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, output_final_state: bool = True, stream=None):
    """Token-by-token KDA on the GPU (reference mode); same arguments as chunk_fwd."""
    return _fwd("recurrent", q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, 0, scale, 0, out,
                final_state, output_final_state, stream)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                state: torch.Tensor, *, scale: float = 1.0, out: Optional[torch.Tensor] = None, stream=None,
                gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                norm_eps: float = 1e-6):
    """One decode token per sequence.  q, k, g: [N, H, d_k]; v: [N, H, d_v]; beta: [N, H];
    state: [N, H, d_k, d_v] fp32 (updated in place).  With gate [N, H, d_v] and norm_weight
    [d_v] the output epilogue (RMSNorm, gate) is fused into the same kernel
    (kda_decode_step_gated) and out holds the gated output.  Returns out [N, H, d_v]."""
    if gate is not None or norm_weight is not None:
        return decode_step_gated(q, k, v, g, beta, state, gate, norm_weight, eps=norm_eps, scale=scale, out=out,
                                 stream=stream)
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", q.dtype, (N, H, dk), dev)
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(g, "g", torch.float32, (N, H, dk), dev)
    _need(beta, "beta", torch.float32, (N, H), dev)
    _need(state, "state", torch.float32, (N, H, dk, dv), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (N, H, dv), dev)
    st = library().kda_decode_step(N, H, dk, dv, _io_code(q.dtype), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(state), _ptr(out), _stream_handle(dev, stream))
    _check(st)
    return out


def decode_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                      state: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor, *, eps: float = 1e-6,
                      scale: float = 1.0, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode step with RMSNorm and the output gate in the same kernel: out = norm(o) * weight *
    sigmoid(gate) for o = scale S^T q of each (sequence, head).  Shapes as decode_step, plus gate
    [N, H, d_v] (io dtype) and weight [d_v] fp32.  Returns out [N, H, d_v]."""
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    if gate is None or weight is None:
        raise ValueError("decode_step_gated needs gate and weight")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", q.dtype, (N, H, dk), dev)
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(g, "g", torch.float32, (N, H, dk), dev)
    _need(beta, "beta", torch.float32, (N, H), dev)
    _need(state, "state", torch.float32, (N, H, dk, dv), dev)
    _need(gate, "gate", q.dtype, (N, H, dv), dev)
    _need(weight, "weight", torch.float32, (dv,), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (N, H, dv), dev)
    st = library().kda_decode_step_gated(N, H, dk, dv, _io_code(q.dtype), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(beta), _ptr(state), _ptr(gate), _ptr(weight), eps, _ptr(out),
                                         _stream_handle(dev, stream))
    _check(st)
    return out


def prologue(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor, conv_q: torch.Tensor,
             conv_k: torch.Tensor, conv_v: torch.Tensor, g_raw: torch.Tensor, beta_raw: torch.Tensor,
             cu_seqlens: Optional[torch.Tensor] = None, *, conv_state: Optional[torch.Tensor] = None,
             output_conv_state: bool = False, norm_eps: float = 1e-6, stream=None):
    """Raw projections -> (q, k, v, g, beta[, conv_state_out]).  q_raw, k_raw: [B, T, H, d_k];
    v_raw: [B, T, H, d_v] (bf16 or fp32); conv_*: fp32 [H, d, W] filter taps; g_raw: fp32
    [B, T, H, d_k]; beta_raw: fp32 [B, T, H]; cu_seqlens: int32 [N+1] (B == 1) or None;
    conv_state: [N, W-1, H, 2 d_k + d_v] raw inputs preceding each sequence, or None (zeros)."""
    dev = q_raw.device
    if q_raw.dim() != 4:
        raise ValueError("q_raw must be [B, T, H, d_k]")
    B, T, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    W = conv_q.shape[-1]
    dt = q_raw.dtype
    _need(k_raw, "k_raw", dt, (B, T, H, dk), dev)
    _need(v_raw, "v_raw", dt, (B, T, H, dv), dev)
    _need(conv_q, "conv_q", torch.float32, (H, dk, W), dev)
    _need(conv_k, "conv_k", torch.float32, (H, dk, W), dev)
    _need(conv_v, "conv_v", torch.float32, (H, dv, W), dev)
    _need(g_raw, "g_raw", torch.float32, (B, T, H, dk), dev)
    _need(beta_raw, "beta_raw", torch.float32, (B, T, H), dev)
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    else:
        N = B
    if conv_state is not None:
        _need(conv_state, "conv_state", dt, (N, W - 1, H, 2 * dk + dv), dev)
    st_out = torch.empty((N, W - 1, H, 2 * dk + dv), dtype=dt, device=dev) if output_conv_state else None
    q, k, v = torch.empty_like(q_raw), torch.empty_like(k_raw), torch.empty_like(v_raw)
    g = torch.empty_like(g_raw)
    beta = torch.empty_like(beta_raw)
    p = PrologueProblem(batch=B, seq_len=T, num_seqs=N if cu_seqlens is not None else 0, num_heads=H, head_dim_k=dk,
                        head_dim_v=dv, conv_width=W, io_dtype=_io_code(dt), norm_eps=norm_eps)
    st = library().kda_prologue(ctypes.byref(p), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(conv_q), _ptr(conv_k),
                                _ptr(conv_v), _ptr(g_raw), _ptr(beta_raw), _ptr(cu_seqlens), _ptr(conv_state),
                                _ptr(st_out), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _stream_handle(dev, stream))
    _check(st)
    return (q, k, v, g, beta, st_out) if output_conv_state else (q, k, v, g, beta)


def norm_gate(o: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor, *, eps: float = 1e-6,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Output epilogue over the last axis (one head's d values): o / sqrt(mean(o^2) + eps)
    * weight * sigmoid(gate).  o, gate: same shape and dtype (bf16 or fp32), contiguous;
    weight: fp32 [d].  out may be o (in place).  Returns out."""
    if gate is None or weight is None:
        raise ValueError("the output epilogue needs both gate and norm weight")
    dev = o.device
    d = o.shape[-1]
    _need(gate, "gate", o.dtype, tuple(o.shape), dev)
    _need(weight, "weight", torch.float32, (d,), dev)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    if out is None:
        out = torch.empty_like(o)
    _need(out, "out", o.dtype, tuple(o.shape), dev)
    rows = o.numel() // d if d else 0
    st = library().kda_norm_gate(rows, d, _io_code(o.dtype), eps, _ptr(o), _ptr(gate), _ptr(weight), _ptr(out),
                                 _stream_handle(dev, stream))
    _check(st)
    return out


def query(batch: int, seq_len: int, num_heads: int, head_dim_k: int, head_dim_v: int, io: str = "bf16", *,
          num_seqs: int = 0, chunk_size: int = 0, dv_tile: int = 0, scale: float = 1.0, algo="auto",
          device: bool = False) -> dict:
    """Launch configuration and algorithmic work of chunk_fwd for a problem (num_seqs > 0:
    packed batch with seq_len total tokens)."""
    p = Problem(batch=batch, seq_len=seq_len, num_heads=num_heads, head_dim_k=head_dim_k, head_dim_v=head_dim_v,
                num_seqs=num_seqs, io_dtype=KDA_BF16 if io == "bf16" else KDA_F32, chunk_size=chunk_size, scale=scale,
                dv_tile=dv_tile, algo=_algo_code(algo))
    r = QueryResult()
    st = library().kda_query(ctypes.byref(p), KDA_QUERY_DEVICE if device else 0, ctypes.byref(r))
    if st not in (KDA_OK, KDA_ERR_UNSUPPORTED):
        _check(st)
    d = {name: getattr(r, name) for name, _ in QueryResult._fields_}
    d["arch"] = r.arch.decode()
    d["status"] = st
    return d
