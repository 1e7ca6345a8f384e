"""GPU parity of the backward (kda_chunk_bwd through the C ABI) against the fp64 oracle's
gradients (oracle.bwd, the token recurrence differentiated by hand and pinned by finite
differences in test_backward_pins.py).

Tolerances, per output tensor (dq, dk, dv, dg, dbeta, d_initial_state), with
rel = max |gpu - oracle| / max |oracle|:
  fp32 io: rel <= 1e-4   (fp32 matrix-core operands; gradient magnitudes grow with the
                          sequence, so the bound is relative to the tensor's largest entry)
  bf16 io: rel <= 2e-2   (bf16 operands, fp32 accumulation and states; the forward's bar)
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
import gated_delta_rule_45_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def say(*a):
    print(*a, flush=True)


def oracle_grads(inp, d_out, dsf, heads=None, scale=1.0):
    a = [ki.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
    return oracle.bwd(*a, inp.g.numpy(), inp.beta.numpy(), ki.to_numpy_io(d_out),
                      initial_state=None if inp.s0 is None else inp.s0.numpy(),
                      d_final_state=None if dsf is None else dsf.numpy(),
                      cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(), scale=scale, heads=heads)


def compare(name, got, ref, io):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    rel = err / scale if scale > 0 else err
    say(f"  {name}: max_abs={err:.3e} max_rel={rel:.3e} (max|ref|={scale:.3e})")
    assert rel <= TOL[io], f"{name}: max rel error {rel:.3e} > {TOL[io]}"


def check_bwd(inp, *, chunk=0, scale=1.0, heads=None, seed=100, dsf_std=0.1, need_ds0=True, label=""):
    B, T, H, dk = inp.q.shape
    say(f"[{label}] io={inp.io} shape={tuple(inp.q.shape)} dv={inp.v.shape[-1]} seqs={inp.num_seqs} chunk={chunk} "
        f"scale={scale} heads={heads} s0={inp.s0 is not None} dsf={dsf_std}")
    d_out, dsf = ki.grad_inputs(inp, seed, dsf_std=dsf_std)
    dev = lambda x: None if x is None else x.to(DEV)
    got = kda.chunk_bwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(d_out),
                        initial_state=dev(inp.s0), d_final_state=dev(dsf), cu_seqlens=dev(inp.cu_seqlens),
                        chunk_size=chunk, scale=scale, need_d_initial_state=need_ds0)
    torch.cuda.synchronize()
    ref = oracle_grads(inp, d_out, dsf, heads=heads, scale=scale)
    for key in KEYS:
        if got[key] is None:
            assert not need_ds0
            continue
        x = got[key]
        if heads is not None:
            x = x[:, heads] if key == "d_initial_state" else x[:, :, heads]
        compare(f"{label} {key}", x, ref[key], inp.io)


def skip_unsupported(inp, chunk):
    B, T, H, dk = inp.q.shape
    p, _ = kda._problem_from(inp.q, inp.v, inp.cu_seqlens, chunk, 1.0, 0, 0)
    try:
        kda.bwd_workspace_bytes(p)
    except kda.KdaError as e:
        if e.status == kda.KDA_ERR_UNSUPPORTED:
            pytest.skip(f"backward has no compiled variant: {e}")
        raise


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bwd_fp32_small(chunk):
    inp = ki.make_inputs(2, 50, 2, 64, 64, "f32", seed=21, s0_std=0.5)
    check_bwd(inp, chunk=chunk, scale=0.7, label=f"fp32 d64 c{chunk}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bwd_fp32_dk128(chunk):
    inp = ki.make_inputs(1, 70, 2, 128, 128, "f32", seed=22, s0_std=0.5)
    skip_unsupported(inp, chunk)
    check_bwd(inp, chunk=chunk, label=f"fp32 d128 c{chunk}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_bwd_bf16(chunk, dk, dv):
    inp = ki.make_inputs(2, 200, 2, dk, dv, "bf16", seed=23 + dk + dv, s0_std=0.1)
    check_bwd(inp, chunk=chunk, label=f"bf16 dk{dk} dv{dv} c{chunk}")


@pytest.mark.parametrize("chunk", [16, 64])
def test_bwd_bf16_packed_sequences(chunk):
    inp = ki.make_inputs(1, 0, 3, 128, 128, "bf16", seed=31, s0_std=0.1, lengths=[1, 70, 0, 129, 64, 16])
    check_bwd(inp, chunk=chunk, label=f"packed c{chunk}")


def test_bwd_without_states():
    inp = ki.make_inputs(2, 90, 2, 128, 128, "bf16", seed=32, s0_std=None)
    check_bwd(inp, dsf_std=None, need_ds0=False, label="no states")


@pytest.mark.parametrize("case", ["beta0", "gate0", "long_memory", "strong_decay"])
def test_bwd_stress(case):
    inp = ki.make_inputs(1, 160, 2, 128, 128, "bf16", seed=33, s0_std=0.1,
                         g_mu={"long_memory": -6.0, "strong_decay": 2.0}.get(case, 0.0))
    if case == "beta0":
        inp.beta.zero_()
    if case == "gate0":
        inp.g.zero_()
    check_bwd(inp, label=case)


def test_bwd_prefill_full_size_all_heads():
    """The prefill workload (4 x 4096 tokens, 16 heads, d = 128, bf16, chunk 64): every gradient
    of every head is compared with the oracle."""
    inp = ki.workload_inputs("prefill")
    check_bwd(inp, chunk=64, label="prefill")


@pytest.mark.parametrize("dk,chunk", [(128, 64), (64, 64), (64, 32), (128, 16)])
def test_bwd_repeatable(dk, chunk):
    """Two calls on the same inputs give bit-identical gradients (no races, no atomics; a matrix-core
    result read back too early would show as run-to-run differences)."""
    inp = ki.make_inputs(2, 300, 4, dk, 128, "bf16", seed=34, s0_std=0.1)
    d_out, dsf = ki.grad_inputs(inp, 7)
    dev = lambda x: None if x is None else x.to(DEV)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(d_out))
    a = kda.chunk_bwd(*args, initial_state=dev(inp.s0), d_final_state=dev(dsf), chunk_size=chunk)
    b = kda.chunk_bwd(*args, initial_state=dev(inp.s0), d_final_state=dev(dsf), chunk_size=chunk)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bwd_fp32_packed_sequences(chunk):
    """fp32 packed batch with an empty, a single-token and a ragged sequence."""
    inp = ki.make_inputs(1, 0, 2, 64, 64, "f32", seed=35, s0_std=0.1, lengths=[33, 1, 0, 47])
    check_bwd(inp, chunk=chunk, label=f"fp32 packed c{chunk}")


def test_bwd_fp32_dk128_chunk64_packed():
    """fp32 at d_k = d_v = 128, chunk 64 (one record buffer in the reverse scan, dP^T and dL^T
    gathered from dP and dA in the gradient kernel) over a packed batch."""
    inp = ki.make_inputs(1, 0, 2, 128, 128, "f32", seed=36, s0_std=0.3, lengths=[70, 1, 0, 129, 64])
    check_bwd(inp, chunk=64, label="fp32 d128 packed c64")


def test_bwd_side_stream_workspace():
    """chunk_bwd on a side stream with the binding's own workspace gives the same gradients as on
    the current stream, with fills of the workspace's size queued on the current stream meanwhile."""
    inp = ki.make_inputs(2, 1024, 4, 128, 128, "bf16", seed=37, s0_std=0.1)
    d_out, dsf = ki.grad_inputs(inp, 8)
    dev = lambda x: None if x is None else x.to(DEV)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(d_out))
    ref = kda.chunk_bwd(*args, initial_state=dev(inp.s0), d_final_state=dev(dsf))
    torch.cuda.synchronize()
    p, _ = kda._problem_from(args[0], args[2], None, 0, 1.0, 0, 0)
    nbytes = kda.bwd_workspace_bytes(p)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = []
    for _ in range(2):
        got.append(kda.chunk_bwd(*args, initial_state=dev(inp.s0), d_final_state=dev(dsf), stream=side))
        got.append(torch.full((nbytes // 4,), float("nan"), device=DEV))
    torch.cuda.synchronize()
    for r in got[0::2]:
        for key in KEYS:
            assert torch.equal(r[key], ref[key]), key


@pytest.mark.parametrize("io,dk,chunk", [("bf16", 128, 64), ("bf16", 128, 16), ("bf16", 64, 32), ("f32", 64, 16),
                                         ("f32", 64, 32), ("f32", 128, 64), ("f32", 64, 64)])
def test_bwd_strong_decay_inside_a_chunk(io, dk, chunk):
    """Gradients under the stress gates of kda_inputs.plant_strong_decay (decay of e^-100 in one
    token, e^-112 per sub-chunk, ...): finite and within the bars."""
    inp = ki.plant_strong_decay(ki.make_inputs(2, 203, 2, dk, 128 if io == "bf16" else 64, io, seed=61 + chunk,
                                               s0_std=0.5))
    skip_unsupported(inp, chunk)
    check_bwd(inp, chunk=chunk, label=f"strong decay {io} d{dk} c{chunk}")


@pytest.mark.parametrize("chunk", [16, 64])
def test_bwd_strong_decay_every_chunk_many_per_workgroup(chunk):
    """Every chunk flagged for the split-level gradient pass (kda_inputs.plant_strong_decay decays one
    channel by e^-112 per sub-chunk throughout) and more flagged chunk-heads than the pass has
    workgroups (one per CU), so each workgroup takes several in turn (2,048 at chunk 16, 512 at 64)."""
    inp = ki.plant_strong_decay(ki.make_inputs(2, 4096, 4, 128, 128, "bf16", seed=71 + chunk, s0_std=0.5))
    skip_unsupported(inp, chunk)
    check_bwd(inp, chunk=chunk, label=f"strong decay every chunk c{chunk}")
