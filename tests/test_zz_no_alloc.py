"""kda_chunk_fwd_noalloc, through the C ABI: the two-pass forward with the library's fixed scratch
array in place of a caller's workspace gives exactly the outputs and final states of kda_chunk_fwd
with its own workspace (same kernels, same configuration), also within the oracle's bars, on two
calls in a row where the second is smaller (the array keeps the first call's contents)."""
import ctypes

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


def noalloc_call(d, inp, chunk):
    """kda_chunk_fwd_noalloc straight through ctypes (outputs allocated here, before the call)."""
    lib = kda.library()
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    p, n = kda._problem_from(d["q"], d["v"], d["cu_seqlens"], chunk, 1.0, 0, kda.KDA_ALGO_TWO_PASS)
    out = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device=DEV)
    fin = torch.empty((n, H, dk, dv), dtype=torch.float32, device=DEV)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]),
                                   P(d["initial_state"]), P(d["cu_seqlens"]), None, P(out), P(fin),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kda.KDA_OK, lib.kda_last_error().decode()
    return out, fin


def test_noalloc_matches_the_workspace_call_twice():
    cases = [
        # 4,096 tokens x 16 heads at d = 128, chunk 64: 62 MB of the 64 MiB array
        ("4096x16 c64", ki.make_inputs(1, 4096, 16, 128, 128, "bf16", seed=81), 64),
        # then a smaller packed batch with an empty and a one-token sequence, default chunk
        ("packed", ki.make_inputs(1, 0, 4, 128, 128, "bf16", seed=82, lengths=[300, 1, 0, 77]), 0),
    ]
    for label, inp, chunk in cases:
        say(f"[{label}] shape={tuple(inp.q.shape)} seqs={inp.num_seqs} chunk={chunk}")
        t = lambda x: None if x is None else x.to(DEV)
        d = dict(q=t(inp.q), k=t(inp.k), v=t(inp.v), g=t(inp.g), beta=t(inp.beta), initial_state=t(inp.s0),
                 cu_seqlens=t(inp.cu_seqlens))
        ref_o, ref_f = kda.chunk_fwd(**d, chunk_size=chunk, algo="two_pass")  # its own workspace
        out, fin = noalloc_call(d, inp, chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"{label}: outputs differ from kda_chunk_fwd"
        assert torch.equal(fin, ref_f), f"{label}: final states differ from kda_chunk_fwd"
        a = [ki.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
        o_ref, f_ref = oracle.fwd(*a, inp.g.numpy(), inp.beta.numpy(), initial_state=inp.s0.numpy(),
                                  cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.numpy())
        for name, got, ref in (("out", out, o_ref), ("final_state", fin, f_ref)):
            gg = got.double().cpu().numpy()
            rel = float(np.abs(gg - ref).max() / np.abs(ref).max())
            say(f"  {label} {name}: max_rel={rel:.3e}")
            assert np.all(np.isfinite(gg)) and rel <= 2e-2


def test_noalloc_binding_and_limit():
    """The binding's wrapper gives the same result; a problem beyond the array is refused."""
    inp = ki.make_inputs(2, 300, 4, 128, 128, "bf16", seed=83)
    t = lambda x: x.to(DEV)
    args = (t(inp.q), t(inp.k), t(inp.v), t(inp.g), t(inp.beta), t(inp.s0))
    o1, f1 = kda.chunk_fwd(*args, algo="two_pass")
    o2, f2 = kda.chunk_fwd_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert kda.noalloc_scratch_bytes() == 64 << 20
    big = ki.make_inputs(4, 4096, 16, 128, 128, "bf16", seed=84, s0_std=None)
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(t(big.q), t(big.k), t(big.v), t(big.g), t(big.beta))
    assert e.value.status == kda.KDA_ERR_WORKSPACE
