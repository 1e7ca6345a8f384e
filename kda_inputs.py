"""Seeded synthetic inputs for Kimi Delta Attention (KDA) workloads.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and shapes them into the input
distributions of the workloads; it holds none of the KDA recurrence or chunk
arithmetic.

Workloads (head dimension 128 follows the Kimi Linear paper summary,
"Kimi Linear model composition" section, where key and value head dimension is
128 in every experiment; the 4K / 128K context lengths follow the evaluation
section; the decode batch stands in for the 1M-token decode measurement,
whose cost per token does not depend on context length):

  tiny_fp32     B=1  T=256     H=2  d=64   fp32 io, chunk 16, zero initial state
  prefill       B=4  T=4096    H=16 d=128  bf16 io, chunk 64, S0 ~ 0.02*N(0,1)
  long_prefill  B=1  T=131072  H=32 d=128  bf16 io, chunk 64, g=-softplus(N(-2,1))
  decode        256 sequences x 1 token, H=32, d=128, state ~ 0.02*N(0,1)
  varlen        64 sequences, lengths U[1, 8192], packed with cu_seqlens, H=32

Recipe (one torch CPU generator seeded with the workload's seed; draw order
[lengths], q, k, v, g_raw, beta_raw, S0):
  q, k = randn, then divided by their L2 norm over d_k (per token and head)
  v    = randn
  g    = -softplus(randn + mu)          (natural-log per-channel gate, mu = 0 or -2)
  beta = sigmoid(randn)                 (one scalar per token and head)
  S0   = 0.02 * randn                   ([num_seqs, H, d_k, d_v], fp32)
q, k, v are then rounded to the io dtype (bf16 round-to-nearest-even); g, beta
and the state stay fp32.  The same bits feed the oracle and the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    io: str  # "f32" or "bf16"
    chunk: int
    seed: int
    g_mu: float = 0.0
    s0_std: Optional[float] = 0.02  # None: zero initial state
    varlen_seqs: int = 0  # >0: packed variable-length batch with this many sequences
    varlen_max: int = 0
    decode: bool = False  # one token per sequence, state updated in place


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, T=256, H=2, dk=64, dv=64, io="f32", chunk=16, seed=0,
                          s0_std=None),
    "prefill": Workload("prefill", B=4, T=4096, H=16, dk=128, dv=128, io="bf16", chunk=64, seed=1),
    "long_prefill": Workload("long_prefill", B=1, T=131072, H=32, dk=128, dv=128, io="bf16", chunk=64,
                             seed=2, g_mu=-2.0),
    "decode": Workload("decode", B=256, T=1, H=32, dk=128, dv=128, io="bf16", chunk=64, seed=3,
                       decode=True),
    "varlen": Workload("varlen", B=1, T=0, H=32, dk=128, dv=128, io="bf16", chunk=64, seed=4,
                       varlen_seqs=64, varlen_max=8192),
}


@dataclass
class Inputs:
    """One batch of KDA inputs on the CPU (torch tensors).

    q, k: [B, T, H, dk] (io dtype); v: [B, T, H, dv] (io dtype); g: [B, T, H, dk] fp32;
    beta: [B, T, H] fp32; s0: [N, H, dk, dv] fp32 or None; cu_seqlens: int32 [N+1] or None
    (then B == 1 and T is the packed token count).  For decode workloads T == 1 and
    N == B.
    """
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    s0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    io: str
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        if self.cu_seqlens is not None:
            return int(self.cu_seqlens.numel()) - 1
        return int(self.q.shape[0])

    def seq_bounds(self):
        """(start, length) of every sequence in the flattened [B*T] token axis."""
        if self.cu_seqlens is not None:
            cu = self.cu_seqlens.tolist()
            return [(cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]
        B, T = self.q.shape[0], self.q.shape[1]
        return [(b * T, T) for b in range(B)]


def _io_dtype(io: str) -> torch.dtype:
    if io == "f32":
        return torch.float32
    if io == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown io dtype {io!r}")


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, io: str, seed: int, *,
                g_mu: float = 0.0, s0_std: Optional[float] = 0.02,
                lengths: Optional[list] = None, num_seqs: Optional[int] = None,
                gen: Optional[torch.Generator] = None) -> Inputs:
    """Draw one batch following the recipe in the module docstring.

    With ``lengths`` (a list of sequence lengths) the batch is packed: B must be 1 and
    T is ignored (it becomes sum(lengths)); cu_seqlens is returned.
    """
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(seed)
    cu = None
    if lengths is not None:
        assert B == 1
        T = int(sum(lengths))
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    n = len(lengths) if lengths is not None else (num_seqs if num_seqs is not None else B)
    dt = _io_dtype(io)
    q = _unit_rows(torch.randn(B, T, H, dk, generator=gen)).to(dt)
    k = _unit_rows(torch.randn(B, T, H, dk, generator=gen)).to(dt)
    v = torch.randn(B, T, H, dv, generator=gen).to(dt)
    g = -torch.nn.functional.softplus(torch.randn(B, T, H, dk, generator=gen) + g_mu)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen))
    s0 = None
    if s0_std is not None:
        s0 = s0_std * torch.randn(n, H, dk, dv, generator=gen)
    return Inputs(q=q, k=k, v=v, g=g.contiguous(), beta=beta.contiguous(), s0=s0, cu_seqlens=cu,
                  io=io, meta=dict(seed=seed, g_mu=g_mu, s0_std=s0_std))


def varlen_lengths(num_seqs: int, max_len: int, gen: torch.Generator) -> list:
    """Sequence lengths uniform in [1, max_len]: the first draw of the workload's generator."""
    return torch.randint(1, max_len + 1, (num_seqs,), generator=gen).tolist()


def workload_inputs(name: str, *, seed: Optional[int] = None) -> Inputs:
    """Inputs of one named workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    s = w.seed if seed is None else seed
    if w.varlen_seqs:
        gen = torch.Generator("cpu").manual_seed(s)
        lengths = varlen_lengths(w.varlen_seqs, w.varlen_max, gen)
        inp = make_inputs(1, 0, w.H, w.dk, w.dv, w.io, s, g_mu=w.g_mu, s0_std=w.s0_std,
                          lengths=lengths, gen=gen)
        inp.meta["lengths"] = lengths
        return inp
    if w.decode:
        # decode: [N, 1, H, d] inputs, state [N, H, dk, dv]
        return make_inputs(w.B, 1, w.H, w.dk, w.dv, w.io, s, g_mu=w.g_mu, s0_std=w.s0_std)
    return make_inputs(w.B, w.T, w.H, w.dk, w.dv, w.io, s, g_mu=w.g_mu, s0_std=w.s0_std)


def workload_inputs_on(name: str, device, *, seed: Optional[int] = None) -> Inputs:
    """One named workload drawn on `device` by a generator of that device: the recipe, shapes and
    draw order of ``workload_inputs`` (a packed workload's lengths still come from the CPU
    generator, so they are the same lengths), but different random values.  Used to time the
    full-size workloads without drawing several GB on the host."""
    w = WORKLOADS[name]
    s = w.seed if seed is None else seed
    lengths = None
    if w.varlen_seqs:
        lengths = varlen_lengths(w.varlen_seqs, w.varlen_max, torch.Generator("cpu").manual_seed(s))
    gen = torch.Generator(device).manual_seed(s)
    B, T = (1, int(sum(lengths))) if lengths is not None else (w.B, 1 if w.decode else w.T)
    n = len(lengths) if lengths is not None else B
    dt = _io_dtype(w.io)
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=device)
    q = _unit_rows(rn(B, T, w.H, w.dk)).to(dt)
    k = _unit_rows(rn(B, T, w.H, w.dk)).to(dt)
    v = rn(B, T, w.H, w.dv).to(dt)
    g = rn(B, T, w.H, w.dk).add_(w.g_mu)
    g = -torch.nn.functional.softplus(g)
    beta = torch.sigmoid(rn(B, T, w.H))
    s0 = None if w.s0_std is None else w.s0_std * rn(n, w.H, w.dk, w.dv)
    cu = None
    if lengths is not None:
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(device)
    inp = Inputs(q=q, k=k, v=v, g=g.contiguous(), beta=beta.contiguous(), s0=s0, cu_seqlens=cu, io=w.io,
                 meta=dict(seed=s, g_mu=w.g_mu, s0_std=w.s0_std, device=str(device)))
    if lengths is not None:
        inp.meta["lengths"] = lengths
    return inp


def plant_strong_decay(inp: Inputs) -> Inputs:
    """Stress gates for decay inside a chunk far beyond the workloads' (the workloads' strongest
    16-token decay is about e^-40): in every head, channel 5 takes log-gate -100 at token 37,
    channel 9 takes -20 per token over tokens 70..109, channel 11 takes -7 per token throughout
    (e^-112 per 16 tokens), channel 13 takes -4 per token throughout (e^-64 per 16 tokens) and
    channel 2 takes -60 at every 16th token.  Tokens past the sequence are skipped; g is
    changed in place (the layout is the token-major [B, T, H, d_k] of every workload)."""
    g = inp.g
    T = g.shape[1]
    g[:, 37:38, :, 5] = -100.0
    g[:, 70:110, :, 9] = -20.0
    g[:, :, :, 11] = -7.0
    g[:, :, :, 13] = -4.0
    g[:, 7:T:16, :, 2] = -60.0
    inp.meta["strong_decay"] = True
    return inp


def to_numpy_io(x: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy: fp32 stays float32, bf16 becomes its raw uint16 bit pattern."""
    x = x.contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(f"unsupported dtype {x.dtype}")


def epilogue_inputs(shape, io: str, seed: int, *, gate_std: float = 2.0):
    """Inputs of the output epilogue for rows of shape[-1] values: o ~ N(0, 1), the gate
    pre-activation z ~ N(0, gate_std^2) (cast to the io dtype), norm weight w = 1 + 0.1 N(0, 1)
    in fp32.  Synthetic stand-ins for a trained layer's output, gate projection and weight."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = _io_dtype(io)
    o = torch.randn(*shape, generator=gen, dtype=torch.float32).to(dt)
    z = (gate_std * torch.randn(*shape, generator=gen, dtype=torch.float32)).to(dt)
    w = 1.0 + 0.1 * torch.randn(shape[-1], generator=gen, dtype=torch.float32)
    return o, z, w


def prologue_inputs(B: int, T: int, H: int, dk: int, dv: int, W: int, io: str, seed: int, *,
                    lengths: Optional[list] = None, g_mu: float = 0.0, with_state: bool = False):
    """Raw projections for the prologue.  Draw order: q_raw, k_raw, v_raw ~ N(0, 1) (cast to the
    io dtype), filter taps for q, k, v ~ N(0, 0.5^2) [H, d, W], g_raw ~ N(g_mu, 1), beta_raw ~
    N(0, 1), then (with_state) the carried-in convolution state ~ N(0, 1) in the io dtype.
    With `lengths` the tokens are one packed row (B == 1) and cu_seqlens is returned."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = _io_dtype(io)
    rn = lambda *s: torch.randn(*s, generator=gen, dtype=torch.float32)
    Tt = sum(lengths) if lengths is not None else T
    shape = (1, Tt, H) if lengths is not None else (B, T, H)
    q, k = rn(*shape, dk).to(dt), rn(*shape, dk).to(dt)
    v = rn(*shape, dv).to(dt)
    wq, wk, wv = 0.5 * rn(H, dk, W), 0.5 * rn(H, dk, W), 0.5 * rn(H, dv, W)
    g = rn(*shape, dk) + g_mu
    b = rn(*shape)
    N = len(lengths) if lengths is not None else B
    st = rn(N, W - 1, H, 2 * dk + dv).to(dt) if with_state else None
    cu = None
    if lengths is not None:
        cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    return dict(q_raw=q, k_raw=k, v_raw=v, conv_q=wq, conv_k=wk, conv_v=wv, g_raw=g, beta_raw=b, conv_state=st,
                cu_seqlens=cu)


def grad_inputs(inp: Inputs, seed: int, *, dsf_std: Optional[float] = 0.1):
    """Upstream gradients for the backward: d_out ~ N(0, 1) with out's shape, cast to the io
    dtype, then (dsf_std not None) the final-state gradient ~ N(0, dsf_std^2) [N, H, dk, dv]
    fp32.  Synthetic stand-ins for what the next layer sends back in training."""
    gen = torch.Generator("cpu").manual_seed(seed)
    B, T, H, _ = inp.q.shape
    dv = inp.v.shape[-1]
    d_out = torch.randn(B, T, H, dv, generator=gen).to(inp.q.dtype)
    dsf = None
    if dsf_std is not None:
        dsf = dsf_std * torch.randn(inp.num_seqs, H, inp.q.shape[-1], dv, generator=gen)
    return d_out, dsf


def dplr_inputs(inp: Inputs, seed: int):
    """Low-rank vectors and write key for the general-DPLR comparator on the tensors of `inp`.
    Draws, in order: a removal direction kappa = randn / |randn| over d_k (independent of the
    write key), lam, sig ~ U[0.5, 1] per (token, head, channel).  Returns
    a = -beta * lam * kappa, b = sig * kappa and the write key beta * k (cast to the io dtype).
    The transition's rank-1 part has b . a in [-beta, 0], so Diag(e^g) + a b^T stays
    contractive; with kappa = k, lam = 1 and sig = e^{g} the vectors would be KDA's."""
    gen = torch.Generator("cpu").manual_seed(seed)
    k = inp.k.float()
    kappa = _unit_rows(torch.randn(k.shape, generator=gen))
    lam = 0.5 + 0.5 * torch.rand(k.shape, generator=gen)
    sig = 0.5 + 0.5 * torch.rand(k.shape, generator=gen)
    beta = inp.beta[..., None]
    dt = inp.q.dtype
    return (-beta * lam * kappa).to(dt), (sig * kappa).to(dt), (beta * k).to(dt)
