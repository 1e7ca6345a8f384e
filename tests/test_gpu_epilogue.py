"""GPU parity of the output epilogue (kda_norm_gate: per-head RMSNorm and output gate) against
the fp64 oracle (oracle/epilogue.py), through the C ABI.

Tolerances (per element, written here):
  bf16 out: |gpu - oracle| <= 4e-3 |oracle| + 1e-12 max|oracle|  (one bf16 rounding, unit
            roundoff 2^-8, plus fp32 arithmetic)
  fp32 out: |gpu - oracle| <= 2e-5 |oracle| + 1e-9 max|oracle|
Composed with the forward pass and the decode step: the library's result equals the epilogue
oracle applied to the forward's own output (bound above), and end to end each row is held to
the bound propagated from the forward tolerance (see check_composed).
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from oracle import epilogue
import gated_delta_rule_45_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def check_elementwise(name, got, ref, io):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape and np.all(np.isfinite(g)), name
    rel, floor = (4e-3, 1e-12) if io == "bf16" else (2e-5, 1e-9)
    bound = rel * np.abs(ref) + floor * np.abs(ref).max()
    excess = np.abs(g - ref) - bound
    say(f"  {name}: max_abs={np.abs(g - ref).max():.3e} worst excess over bound={excess.max():.3e}")
    assert excess.max() <= 0, f"{name}: {int((excess > 0).sum())} elements outside the bound"


def oracle_norm_gate(o, z, w, eps=EPS):
    return epilogue.norm_gate(ki.to_numpy_io(o.cpu()), ki.to_numpy_io(z.cpu()), w.cpu().numpy(), eps)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [1, 17, 1000])
def test_norm_gate_rows(io, d, rows):
    say(f"norm_gate io={io} d={d} rows={rows}")
    o, z, w = ki.epilogue_inputs((rows, d), io, seed=rows + d)
    z[0, :4] = torch.tensor([30.0, -30.0, 0.0, 80.0]).to(z.dtype)  # saturated and neutral gates
    got = kda.norm_gate(o.to(DEV), z.to(DEV), w.to(DEV), eps=EPS)
    check_elementwise("out", got, oracle_norm_gate(o, z, w), io)


def test_norm_gate_full_prefill_output_in_place():
    # the prefill workload's output shape: B*T*H = 262,144 rows of 128 bf16 values, in place
    shape = (4, 4096, 16, 128)
    say(f"norm_gate in place {shape}")
    o, z, w = ki.epilogue_inputs(shape, "bf16", seed=41)
    od = o.to(DEV)
    ret = kda.norm_gate(od, z.to(DEV), w.to(DEV), eps=EPS, out=od)
    assert ret.data_ptr() == od.data_ptr()
    check_elementwise("out", od, oracle_norm_gate(o, z, w), "bf16")


def test_norm_gate_zero_rows_and_eps():
    o, z, w = ki.epilogue_inputs((64, 128), "bf16", seed=3)
    o[5] = 0
    got = kda.norm_gate(o.to(DEV), z.to(DEV), w.to(DEV), eps=0.25)
    ref = oracle_norm_gate(o, z, w, eps=0.25)
    assert torch.all(got[5] == 0)
    check_elementwise("out", got, ref, "bf16")


def check_fused_vs_plain(name, got, plain, z, w, io):
    """got = output of a kernel with the epilogue fused in, plain = the same kernel family's output
    without it (rounded to the io dtype).  The fused kernel normalises its fp32 o, plain carries
    the rounding of o to the io dtype into the epilogue: two roundings in all (bf16: 2 x 2^-8
    relative, 8e-3), and each element may also differ by the fp32 noise of o (summation order,
    1e-5 of the row's largest |o|) carried through the normalisation: 1e-5 max|o| / rms(o)
    |w sigmoid(z)|."""
    o = epilogue.as_f64(ki.to_numpy_io(plain.cpu()))
    ref = oracle_norm_gate(plain, z, w)
    zf, wf = epilogue.as_f64(ki.to_numpy_io(z.cpu())), w.double().cpu().numpy()
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS)
    noise = 1e-5 * np.abs(o).max(axis=-1, keepdims=True) / rms * np.abs(wf / (1.0 + np.exp(-zf)))
    rel, floor = (8e-3, 1e-12) if io == "bf16" else (2e-5, 1e-9)
    bound = rel * np.abs(ref) + floor * np.abs(ref).max() + noise
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape and np.all(np.isfinite(g)), name
    excess = np.abs(g - ref) - bound
    say(f"  {name}: max_abs={np.abs(g - ref).max():.3e} worst excess over bound={excess.max():.3e}")
    assert excess.max() <= 0, f"{name}: {int((excess > 0).sum())} elements outside the bound"


def check_composed(name, got, plain, o_ref, z, w, fused=False):
    """got = epilogue applied by the library after the forward; plain = the forward's own output
    without it; o_ref = the oracle's forward output (fp64).

    1. got equals the epilogue oracle applied to plain (per-element bound of this file; with
       fused, the bound of check_fused_vs_plain).
    2. End to end, each row is held to the bound propagated from the forward tolerance
       tau = 2e-2 max|o_ref|: the RMS normalisation n(o) = o / rms(o) has a derivative of norm
       at most 1 / rms(o), so |out - out_ref| <= 2 tau / rms(o_ref row) |w sigmoid(z)|
       + 4e-3 |out_ref| (the factor 2 covers second-order terms and eps)."""
    if fused:
        check_fused_vs_plain(name + " vs epilogue(plain)", got, plain, z, w, "bf16")
    else:
        check_elementwise(name + " vs epilogue(plain)", got, oracle_norm_gate(plain, z, w), "bf16")
    zf, wf = epilogue.as_f64(ki.to_numpy_io(z)), w.double().numpy()
    ref = epilogue.norm_gate(o_ref, ki.to_numpy_io(z), w.numpy(), EPS)
    tau = 2e-2 * np.abs(o_ref).max()
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    bound = 2 * tau / rms * np.abs(wf / (1.0 + np.exp(-zf))) + 4e-3 * np.abs(ref)
    err = np.abs(got.double().cpu().numpy() - ref)
    say(f"  {name} end to end: max_abs={err.max():.3e} max err/bound={(err / bound).max():.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("algo", ["fused", "two_pass"])
def test_chunk_fwd_with_epilogue(algo):
    inp = ki.make_inputs(2, 300, 3, 128, 128, "bf16", seed=12)
    say(f"chunk_fwd + epilogue algo={algo} B=2 T=300 H=3 d=128")
    _, z, w = ki.epilogue_inputs((2, 300, 3, 128), "bf16", seed=13)
    d = {k: x.to(DEV) for k, x in dict(q=inp.q, k=inp.k, v=inp.v, g=inp.g, beta=inp.beta, s0=inp.s0).items()}
    plain, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], algo=algo)
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], algo=algo, gate=z.to(DEV),
                             norm_weight=w.to(DEV), norm_eps=EPS)
    a = [ki.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
    o_ref, s_ref = oracle.fwd(*a, inp.g.numpy(), inp.beta.numpy(), initial_state=inp.s0.numpy())
    check_composed("out", out, plain.cpu(), o_ref, z, w)
    srel = np.abs(fin.double().cpu().numpy() - s_ref).max() / np.abs(s_ref).max()
    assert srel <= 2e-2


def test_decode_step_with_epilogue():
    """decode_step with gate and norm_weight runs the fused kernel (kda_decode_step_gated)."""
    inp = ki.workload_inputs("decode")
    say("decode_step + epilogue (fused), decode workload (256 seqs x 32 heads)")
    sq = lambda x: x[:, 0].contiguous()
    q, k, v, g, b = (sq(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    _, z, w = ki.epilogue_inputs(tuple(v.shape), "bf16", seed=14)
    args = [x.to(DEV) for x in (q, k, v, g, b)]
    plain = kda.decode_step(*args, inp.s0.to(DEV))
    out = kda.decode_step(*args, inp.s0.to(DEV), gate=z.to(DEV), norm_weight=w.to(DEV), norm_eps=EPS)
    o_ref, _ = oracle.decode(*(ki.to_numpy_io(x) for x in (q, k, v)), g.numpy(), b.numpy(), inp.s0.numpy())
    check_composed("out", out, plain.cpu(), o_ref, z, w, fused=True)


def check_decode_gated(name, got, o_ref, z, w, tau, rel):
    """End-to-end bound of the fused decode epilogue against the composed oracles: the decode
    tolerance tau on o, propagated through the RMS normalisation as in check_composed, plus the
    output rounding rel |out_ref|."""
    zf, wf = epilogue.as_f64(ki.to_numpy_io(z)), w.double().numpy()
    ref = epilogue.norm_gate(o_ref, ki.to_numpy_io(z), w.numpy(), EPS)
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    bound = 2 * tau / rms * np.abs(wf / (1.0 + np.exp(-zf))) + rel * np.abs(ref) + 1e-12
    g = got.double().cpu().numpy()
    assert np.all(np.isfinite(g)), name
    err = np.abs(g - ref)
    say(f"  {name}: max_abs={err.max():.3e} max err/bound={(err / bound).max():.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_decode_step_gated_dims(io, dk, dv):
    """kda_decode_step_gated (one workgroup per sequence and head, norm and gate in the same
    kernel) against the decode oracle followed by the epilogue oracle; the state against the
    decode oracle's state; and against the two-kernel composition on the GPU."""
    N, H = 37, 3
    say(f"decode_step_gated io={io} N={N} H={H} dk={dk} dv={dv}")
    inp = ki.make_inputs(N, 1, H, dk, dv, io, seed=dk + 3 * dv + (io == "f32"))
    sq = lambda x: x[:, 0].contiguous()
    q, k, v, g, b = (sq(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    _, z, w = ki.epilogue_inputs((N, H, dv), io, seed=dk + dv)
    z[0, 0, :4] = torch.tensor([30.0, -30.0, 0.0, 80.0]).to(z.dtype)  # saturated and neutral gates
    args = [x.to(DEV) for x in (q, k, v, g, b)]
    state = inp.s0.to(DEV).clone()
    out = kda.decode_step_gated(*args, state, z.to(DEV), w.to(DEV), eps=EPS)
    state2 = inp.s0.to(DEV).clone()
    plain = kda.decode_step(*args, state2)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(*(ki.to_numpy_io(x) for x in (q, k, v)), g.numpy(), b.numpy(), inp.s0.numpy())
    if io == "bf16":
        tau, rel = 2e-2 * np.abs(o_ref).max(), 4e-3
        srel = np.abs(state.double().cpu().numpy() - s_ref).max() / np.abs(s_ref).max()
        assert srel <= 2e-2
    else:
        tau, rel = 1e-4, 2e-5
        assert np.abs(state.double().cpu().numpy() - s_ref).max() <= 1e-4
    check_decode_gated("out vs oracles", out, o_ref, z, w, tau, rel)
    # the same state update as the plain decode step, up to the summation order of S'^T k
    ds = (state - state2).abs().max().item()
    say(f"  state vs decode_step: max_abs={ds:.3e}")
    assert ds <= 1e-5 * state2.abs().max().item()
    check_fused_vs_plain("out vs epilogue(decode_step)", out, plain, z, w, io)


def test_decode_step_gated_zero_output_row():
    """q = 0 for one (sequence, head): o = 0 there and the gated output is exactly 0 (eps > 0)."""
    N, H, d = 4, 2, 128
    inp = ki.make_inputs(N, 1, H, d, d, "bf16", seed=77)
    sq = lambda x: x[:, 0].contiguous()
    q, k, v, g, b = (sq(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    q[1, 1] = 0
    _, z, w = ki.epilogue_inputs((N, H, d), "bf16", seed=78)
    out = kda.decode_step_gated(*(x.to(DEV) for x in (q, k, v, g, b)), inp.s0.to(DEV).clone(), z.to(DEV), w.to(DEV),
                                eps=0.25)
    assert torch.all(out[1, 1] == 0)
    o_ref, _ = oracle.decode(*(ki.to_numpy_io(x) for x in (q, k, v)), g.numpy(), b.numpy(), inp.s0.numpy())
    ref = epilogue.norm_gate(o_ref, ki.to_numpy_io(z), w.numpy(), 0.25)
    err = np.abs(out.double().cpu().numpy() - ref).max() / np.abs(ref).max()
    say(f"  zero row: max rel err {err:.3e}")
    assert err <= 2e-2
