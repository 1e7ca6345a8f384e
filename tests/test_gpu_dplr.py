"""GPU parity of the general-DPLR comparator (kda_dplr_chunk_fwd through the C ABI) against
the fp64 oracle (oracle.dplr_fwd, pinned in test_dplr_pins.py).  Tolerances as the KDA
forward: fp32 io max|gpu - oracle| <= 1e-4; bf16 io max|gpu - oracle| / max|oracle| <= 2e-2,
output and final state separately."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
import gated_delta_rule_45_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def compare(name, got, ref, io):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape and np.all(np.isfinite(g)), name
    err = float(np.abs(g - ref).max())
    rel = err / max(float(np.abs(ref).max()), 1e-300)
    say(f"  {name}: max_abs={err:.3e} max_rel={rel:.3e}")
    if io == "f32":
        assert err <= 1e-4, f"{name}: {err:.3e}"
    else:
        assert rel <= 2e-2, f"{name}: {rel:.3e}"


def check(inp, *, chunk=64, dv_tile=32, scale=1.0, label=""):
    say(f"[{label}] io={inp.io} shape={tuple(inp.q.shape)} seqs={inp.num_seqs} chunk={chunk} dv_tile={dv_tile}")
    a, b, kw = ki.dplr_inputs(inp, 9)
    dev = lambda x: None if x is None else x.to(DEV)
    out, fin = kda.dplr_chunk_fwd(dev(inp.q), dev(kw), dev(inp.v), dev(a), dev(b), dev(inp.g), dev(inp.s0),
                                  dev(inp.cu_seqlens), chunk_size=chunk, dv_tile=dv_tile, scale=scale)
    torch.cuda.synchronize()
    n = ki.to_numpy_io
    o_ref, f_ref = oracle.dplr_fwd(n(inp.q), n(kw), n(inp.v), n(a), n(b), inp.g.numpy(),
                                   initial_state=None if inp.s0 is None else inp.s0.numpy(),
                                   cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(), scale=scale)
    compare(f"{label} out", out, o_ref, inp.io)
    compare(f"{label} final_state", fin, f_ref, inp.io)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_dplr_fp32(chunk):
    check(ki.make_inputs(2, 50, 2, 64, 64, "f32", seed=41, s0_std=0.5), chunk=chunk, scale=0.7, label=f"fp32 c{chunk}")


@pytest.mark.parametrize("chunk,dv_tile", [(16, 32), (32, 32), (64, 32), (64, 64)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_dplr_bf16(chunk, dv_tile, dk, dv):
    check(ki.make_inputs(2, 200, 2, dk, dv, "bf16", seed=42 + dk, s0_std=0.1), chunk=chunk, dv_tile=dv_tile,
          label=f"bf16 dk{dk} dv{dv} c{chunk}")


def test_dplr_packed_sequences():
    check(ki.make_inputs(1, 0, 2, 128, 128, "bf16", seed=43, lengths=[1, 70, 0, 129, 16]), label="packed")


def test_dplr_key_tied_case_equals_kda():
    """a = -beta k, b = e^g k and write key beta k make the DPLR kernel compute KDA: its output
    matches the KDA oracle (and so KDA's own kernel) to the bf16 bar."""
    inp = ki.make_inputs(2, 300, 2, 128, 128, "bf16", seed=44)
    k32 = inp.k.float()
    a = (-inp.beta[..., None] * k32).to(torch.bfloat16)
    b = (torch.exp(inp.g) * k32).to(torch.bfloat16)
    kw = (inp.beta[..., None] * k32).to(torch.bfloat16)
    dev = lambda x: x.to(DEV)
    out, fin = kda.dplr_chunk_fwd(dev(inp.q), dev(kw), dev(inp.v), dev(a), dev(b), dev(inp.g), dev(inp.s0))
    torch.cuda.synchronize()
    n = ki.to_numpy_io
    o_ref, f_ref = oracle.fwd(n(inp.q), n(inp.k), n(inp.v), inp.g.numpy(), inp.beta.numpy(),
                              initial_state=inp.s0.numpy())
    compare("tied out", out, o_ref, "bf16")
    compare("tied final_state", fin, f_ref, "bf16")


def test_dplr_prefill_full_size():
    check(ki.workload_inputs("prefill"), label="prefill")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_dplr_repeatable(chunk):
    """Two calls on the same inputs give bit-identical outputs and final states."""
    inp = ki.make_inputs(2, 150, 2, 128, 128, "bf16", seed=37, s0_std=0.1)
    a, b, kw = ki.dplr_inputs(inp, 9)
    dev = lambda x: None if x is None else x.to(DEV)
    args = (dev(inp.q), dev(kw), dev(inp.v), dev(a), dev(b), dev(inp.g), dev(inp.s0), None)
    o1, f1 = kda.dplr_chunk_fwd(*args, chunk_size=chunk, dv_tile=32)
    o2, f2 = kda.dplr_chunk_fwd(*args, chunk_size=chunk, dv_tile=32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("io,dk,chunk", [("bf16", 128, 64), ("bf16", 128, 16), ("bf16", 64, 32), ("f32", 64, 64)])
def test_dplr_strong_decay_inside_a_chunk(io, dk, chunk):
    """The comparator under the stress gates of kda_inputs.plant_strong_decay: finite outputs and
    final states within the bars."""
    inp = ki.plant_strong_decay(ki.make_inputs(2, 203, 2, dk, 128 if io == "bf16" else 64, io, seed=71 + chunk,
                                               s0_std=0.5))
    check(inp, chunk=chunk, label=f"strong decay {io} d{dk} c{chunk}")
