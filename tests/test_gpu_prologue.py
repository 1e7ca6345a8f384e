"""GPU parity of the prologue (kda_prologue: short convolution + Swish, q/k L2 normalisation,
gate and beta activations) against the fp64 oracle (oracle/prologue.py), through the C ABI.

Tolerances (per element, written here):
  q, k, v  bf16: |gpu - oracle| <= 4e-3 |oracle| + 1e-6 max|oracle|  (one bf16 rounding, 2^-9,
                 plus fp32 arithmetic);  fp32: 2e-5 |oracle| + 1e-7 max|oracle|
  g, beta  fp32: |gpu - oracle| <= 2e-6 |oracle| + 1e-7
  state out: exactly the raw inputs it carries (bit for bit)
Splitting a sequence and carrying the state must reproduce the unsplit run bit for bit.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from oracle import prologue as P
import gated_delta_rule_45_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def bound_check(name, got, ref, rel, floor):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape and np.all(np.isfinite(g)), name
    excess = np.abs(g - ref) - (rel * np.abs(ref) + floor * (np.abs(ref).max() if ref.size else 0.0))
    say(f"  {name}: max_abs={np.abs(g - ref).max() if g.size else 0:.3e} worst excess={excess.max() if g.size else 0:.3e}")
    assert g.size == 0 or excess.max() <= 0, f"{name}: {int((excess > 0).sum())} elements outside the bound"


def run(inp, io, W, eps=EPS):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    return kda.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_q"], d["conv_k"], d["conv_v"], d["g_raw"],
                        d["beta_raw"], d["cu_seqlens"], conv_state=d["conv_state"], output_conv_state=True,
                        norm_eps=eps)


def reference(inp, bounds, eps=EPS):
    flat = lambda x: ki.to_numpy_io(x.reshape(-1, *x.shape[2:]))
    st = None if inp["conv_state"] is None else ki.to_numpy_io(inp["conv_state"])
    return P.prologue(flat(inp["q_raw"]), flat(inp["k_raw"]), flat(inp["v_raw"]), inp["conv_q"].numpy(),
                      inp["conv_k"].numpy(), inp["conv_v"].numpy(), inp["g_raw"].reshape(-1, *inp["g_raw"].shape[2:]).numpy(),
                      inp["beta_raw"].reshape(-1, inp["beta_raw"].shape[-1]).numpy(), bounds, conv_state=st, eps=eps)


def check_all(inp, io, W, bounds):
    got = run(inp, io, W)
    ref = reference(inp, bounds)
    rel, floor = (4e-3, 1e-6) if io == "bf16" else (2e-5, 1e-7)
    for i, name in enumerate(("q", "k", "v")):
        bound_check(name, got[i].reshape(-1, *got[i].shape[2:]), ref[i], rel, floor)
    bound_check("g", got[3].reshape(-1, *got[3].shape[2:]), ref[3], 2e-6, 1e-7)
    bound_check("beta", got[4].reshape(-1, got[4].shape[-1]), ref[4], 2e-6, 1e-7)
    st = got[5].float().cpu().double().numpy()
    assert np.array_equal(st, ref[5]), "state out differs from the raw inputs it should carry"
    return got


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_prologue_batch(io, W):
    say(f"prologue batch io={io} W={W} B=2 T=100 H=3 d_k=128 d_v=64")
    inp = ki.prologue_inputs(2, 100, 3, 128, 64, W, io, seed=W, with_state=W > 1)
    check_all(inp, io, W, [(0, 100), (100, 100)])


@pytest.mark.parametrize("W", [2, 4])
def test_prologue_packed_with_short_and_empty_sequences(W):
    lengths = [0, 1, 2, 5, 70, 3, 0, 33]
    say(f"prologue packed W={W} lengths={lengths}")
    inp = ki.prologue_inputs(1, 0, 2, 64, 128, W, "bf16", seed=10 + W, lengths=lengths, with_state=True)
    bounds = [(int(inp["cu_seqlens"][n]), lengths[n]) for n in range(len(lengths))]
    check_all(inp, "bf16", W, bounds)


def test_prologue_without_state_matches_zero_state():
    inp = ki.prologue_inputs(1, 0, 2, 128, 128, 4, "bf16", seed=21, lengths=[3, 40], with_state=True)
    inp0 = dict(inp)
    inp0["conv_state"] = None
    a = run(inp0, "bf16", 4)
    inp["conv_state"] = torch.zeros_like(inp["conv_state"])
    b = run(inp, "bf16", 4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_split_sequence_continues_bit_for_bit():
    # one call over 64 tokens equals 40 tokens, then 1 token at a time (decoding), then the rest
    inp = ki.prologue_inputs(1, 64, 2, 128, 128, 4, "bf16", seed=22, with_state=True)
    full = run(inp, "bf16", 4)
    pieces, st = [], inp["conv_state"]
    for a, b in ((0, 40), (40, 41), (41, 42), (42, 64)):
        part = {k: (v if v is None or k.startswith("conv_") and k != "conv_state" else v) for k, v in inp.items()}
        for k in ("q_raw", "k_raw", "v_raw", "g_raw", "beta_raw"):
            part[k] = inp[k][:, a:b].contiguous()
        part["conv_state"] = st
        out = run(part, "bf16", 4)
        pieces.append(out)
        st = out[5].cpu()
    for i in range(5):
        assert torch.equal(torch.cat([p[i] for p in pieces], dim=1), full[i]), i
    assert torch.equal(st.to(DEV), full[5])


def test_prologue_full_prefill_shape():
    say("prologue full prefill shape B=4 T=4096 H=16 d=128 W=4")
    inp = ki.prologue_inputs(4, 4096, 16, 128, 128, 4, "bf16", seed=23)
    check_all(inp, "bf16", 4, [(n * 4096, 4096) for n in range(4)])


@pytest.mark.parametrize("algo", ["fused", "two_pass"])
def test_prologue_then_chunk_fwd(algo):
    say(f"prologue -> chunk_fwd algo={algo} B=2 T=200 H=2 d=128")
    inp = ki.prologue_inputs(2, 200, 2, 128, 128, 4, "bf16", seed=24)
    q, k, v, g, b, _ = run(inp, "bf16", 4)
    s0 = 0.02 * torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(25))
    out, fin = kda.chunk_fwd(q, k, v, g, b, s0.to(DEV), algo=algo)
    # oracle: the prologue oracle's outputs, rounded to bf16 as the kernel stores them, into the
    # recurrence oracle
    rq, rk, rv, rg, rb, _ = reference(inp, [(0, 200), (200, 200)])
    bf = lambda x: ki.to_numpy_io(torch.from_numpy(x.reshape(2, 200, 2, 128)).float().to(torch.bfloat16))
    o_ref, s_ref = oracle.fwd(bf(rq), bf(rk), bf(rv), rg.reshape(2, 200, 2, 128).astype(np.float32),
                              rb.reshape(2, 200, 2).astype(np.float32), initial_state=s0.numpy())
    rel = np.abs(out.double().cpu().numpy() - o_ref).max() / np.abs(o_ref).max()
    srel = np.abs(fin.double().cpu().numpy() - s_ref).max() / np.abs(s_ref).max()
    say(f"  out max_rel={rel:.3e} state max_rel={srel:.3e}")
    assert rel <= 2e-2 and srel <= 2e-2


# ------------------------------------------------ prologue fused into the forward ----
TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def fused_reference(inp, bounds, B, T, eps=EPS, s0=None, cu=None):
    """Composed oracles: the prologue oracle (fp64), then the forward oracle on its outputs."""
    q, k, v, g, b, _ = reference(inp, bounds, eps)
    H, dk, dv = q.shape[1], q.shape[2], v.shape[2]
    f32 = lambda x, d: np.ascontiguousarray(x.reshape(B, T, H, d), dtype=np.float32)
    return oracle.fwd(f32(q, dk), f32(k, dk), f32(v, dv), f32(g, dk), np.ascontiguousarray(b.reshape(B, T, H), np.float32),
                      initial_state=None if s0 is None else s0.numpy(), cu_seqlens=None if cu is None else cu.numpy())


def compare_fused(name, got, ref, io):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape and np.all(np.isfinite(g)), name
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    say(f"  {name}: max_abs={err:.3e} max_rel={err / scale if scale else err:.3e}")
    if io == "f32":
        assert err <= TOL_F32_ABS, name
    else:
        assert err <= TOL_BF16_REL * scale, name


def run_fused(inp, s0=None, chunk=0, dv_tile=0, eps=EPS):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    return kda.chunk_fwd_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_q"], d["conv_k"], d["conv_v"], d["g_raw"],
                                  d["beta_raw"], None if s0 is None else s0.to(DEV), d["cu_seqlens"], norm_eps=eps,
                                  chunk_size=chunk, dv_tile=dv_tile)


@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64), ("f32", 64, 64)])
@pytest.mark.parametrize("W", [1, 3, 4])
@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_chunk_fwd_prologue_batch(io, dk, dv, W, chunk):
    """kda_chunk_fwd_prologue (convolution, Swish, L2 norm, gate and beta activations inside the
    two-pass kernels) against the prologue oracle followed by the forward oracle; T = 203 ends in a
    partial chunk at every chunk size and crosses sub-chunk and chunk boundaries with the
    convolution window."""
    B, T, H = 2, 203, 3
    say(f"fused prologue io={io} d_k={dk} d_v={dv} W={W} chunk={chunk}")
    inp = ki.prologue_inputs(B, T, H, dk, dv, W, io, seed=100 + W + dk + chunk)
    s0 = 0.1 * torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(7))
    r = kda.query(B, T, H, dk, dv, io, chunk_size=chunk, algo="two_pass")
    if not r["supported"]:
        pytest.skip(f"two-pass has no variant for {io} d_k={dk} chunk={chunk}")
    out, fin = run_fused(inp, s0=s0, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, f_ref = fused_reference(inp, [(0, T), (T, T)], B, T, s0=s0)
    compare_fused("out", out, o_ref, io)
    compare_fused("final_state", fin, f_ref, io)


@pytest.mark.parametrize("chunk,dv_tile", [(0, 0), (32, 32), (64, 16), (64, 64)])
def test_chunk_fwd_prologue_packed(chunk, dv_tile):
    """Packed batch with empty, one- and two-token sequences (the convolution window restarts at
    every sequence start, also inside a chunk slot's first rows) and the scan tilings."""
    lengths = [0, 1, 2, 5, 70, 3, 0, 133, 64]
    inp = ki.prologue_inputs(1, 0, 2, 128, 128, 4, "bf16", seed=31 + chunk + dv_tile, lengths=lengths)
    T = sum(lengths)
    bounds = [(int(inp["cu_seqlens"][n]), lengths[n]) for n in range(len(lengths))]
    say(f"fused prologue packed lengths={lengths} chunk={chunk} dv_tile={dv_tile}")
    out, fin = run_fused(inp, chunk=chunk, dv_tile=dv_tile)
    torch.cuda.synchronize()
    o_ref, f_ref = fused_reference(inp, bounds, 1, T, cu=inp["cu_seqlens"])
    compare_fused("out", out, o_ref, "bf16")
    compare_fused("final_state", fin, f_ref, "bf16")


def test_chunk_fwd_prologue_matches_the_composition_on_the_gpu():
    """The fused path against kda_prologue followed by kda_chunk_fwd (two-pass) on the same raw
    inputs (the composition rounds q, k, v to bf16 between the calls; both within the bar of the
    composed oracles), at 2 x 1,024 tokens x 8 heads, d = 128."""
    B, T, H = 2, 1024, 8
    inp = ki.prologue_inputs(B, T, H, 128, 128, 4, "bf16", seed=55)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    out_f, fin_f = run_fused(inp)
    q, k, v, g, b = kda.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_q"], d["conv_k"], d["conv_v"], d["g_raw"],
                                 d["beta_raw"], norm_eps=EPS)
    out_c, fin_c = kda.chunk_fwd(q, k, v, g, b, algo="two_pass")
    torch.cuda.synchronize()
    o_ref, f_ref = fused_reference(inp, [(n * T, T) for n in range(B)], B, T)
    compare_fused("fused out", out_f, o_ref, "bf16")
    compare_fused("fused final_state", fin_f, f_ref, "bf16")
    compare_fused("composed out", out_c, o_ref, "bf16")
    compare_fused("composed final_state", fin_c, f_ref, "bf16")


def test_chunk_fwd_prologue_strong_decay():
    """g_raw of 100 on one token and 20 over 40 tokens (g ~ -100 and -20 per token): the fused
    prep's diagonal blocks switch to the split levels from registers; finite and within the bar."""
    B, T, H = 1, 203, 2
    inp = ki.prologue_inputs(B, T, H, 128, 128, 4, "bf16", seed=61)
    inp["g_raw"][0, 37, :, 5] = 100.0
    inp["g_raw"][0, 70:110, :, 9] = 20.0
    out, fin = run_fused(inp, chunk=64)
    torch.cuda.synchronize()
    o_ref, f_ref = fused_reference(inp, [(0, T)], B, T)
    compare_fused("out", out, o_ref, "bf16")
    compare_fused("final_state", fin, f_ref, "bf16")
