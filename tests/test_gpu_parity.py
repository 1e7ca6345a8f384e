"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (written here, checked per output tensor):
  fp32 io: max |gpu - oracle| <= 1e-4
  bf16 io: max |gpu - oracle| / max |oracle| <= 2e-2   (o and the final state separately)
The state is fp32 in both cases.  Workloads follow kda_inputs.WORKLOADS and are compared
at their full sizes, every head and every token: the oracle of a large workload runs once
(on all host threads) and its result is reused by every algorithm and chunk setting.
"""
import time

import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
import gated_delta_rule_45_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def say(*a):
    print(*a, flush=True)


def on_dev(inp):
    t = lambda x: None if x is None else x.to(DEV)
    return dict(q=t(inp.q), k=t(inp.k), v=t(inp.v), g=t(inp.g), beta=t(inp.beta), initial_state=t(inp.s0),
                cu_seqlens=t(inp.cu_seqlens))


def run_oracle(inp, heads=None, scale=1.0, s0="inp"):
    a = [ki.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
    s = inp.s0 if s0 == "inp" else s0
    return oracle.fwd(*a, inp.g.numpy(), inp.beta.numpy(), initial_state=None if s is None else s.numpy(),
                      cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(), scale=scale, heads=heads)


def _slices(got, ref, step=4096):
    """(gpu slice as float64 numpy, oracle slice) pairs along the token axis of [B, T, ...]
    tensors (whole tensors when they are small), so large workloads never need a float64 copy
    of the whole GPU output on the host."""
    if got.dim() < 2 or got.numel() <= (1 << 24):
        yield got.detach().double().cpu().numpy(), ref
        return
    for a in range(0, got.shape[1], step):
        yield got[:, a:a + step].detach().double().cpu().numpy(), ref[:, a:a + step]


def compare(name, got, ref, io):
    if not isinstance(got, torch.Tensor):
        got = torch.as_tensor(np.asarray(got, dtype=np.float64))
    assert tuple(got.shape) == ref.shape, (name, tuple(got.shape), ref.shape)
    err = scale = 0.0
    sq_diff = sq_ref = 0.0
    for g, r in _slices(got, ref):
        if not g.size:
            continue
        assert np.all(np.isfinite(g)), f"{name}: non-finite values"
        diff = g - r
        err = max(err, float(np.abs(diff).max()))
        scale = max(scale, float(np.abs(r).max()))
        sq_diff += float(np.square(diff).sum())
        sq_ref += float(np.square(r).sum())
    rel = err / scale if scale > 0 else err
    rms = float(np.sqrt(sq_diff) / max(np.sqrt(sq_ref), 1e-300))
    say(f"  {name}: max_abs={err:.3e} max_rel={rel:.3e} rms_rel={rms:.3e} (max|ref|={scale:.3e})")
    if io == "f32":
        assert err <= TOL_F32_ABS, f"{name}: max abs error {err:.3e} > {TOL_F32_ABS}"
    else:
        assert rel <= TOL_BF16_REL, f"{name}: max rel error {rel:.3e} > {TOL_BF16_REL}"


ALGOS = ["fused", "two_pass"]


def skip_unless_supported(inp, chunk_size, dv_tile, algo):
    B, T, H, dk = inp.q.shape
    r = kda.query(B, T, H, dk, inp.v.shape[-1], inp.io, num_seqs=inp.num_seqs if inp.cu_seqlens is not None else 0,
                  chunk_size=chunk_size, dv_tile=dv_tile, algo=algo)
    if r["status"] == kda.KDA_ERR_UNSUPPORTED:
        pytest.skip(f"{algo} has no compiled variant for io={inp.io} d_k={dk} chunk={chunk_size} (LDS budget)")


def check_fwd(inp, *, heads=None, chunk_size=0, dv_tile=0, scale=1.0, mode="chunk", label="", algo="auto",
              ref=None):
    say(f"[{label}] mode={mode} algo={algo} io={inp.io} shape={tuple(inp.q.shape)} v={tuple(inp.v.shape)} "
        f"seqs={inp.num_seqs} chunk={chunk_size} dv_tile={dv_tile} scale={scale} heads={heads}")
    if mode == "chunk":
        skip_unless_supported(inp, chunk_size, dv_tile, algo)
    d = on_dev(inp)
    if mode == "chunk":
        out, fin = kda.chunk_fwd(**d, chunk_size=chunk_size, dv_tile=dv_tile, scale=scale, algo=algo)
    else:
        out, fin = kda.recurrent_fwd(**d, scale=scale)
    torch.cuda.synchronize()
    del d
    o_ref, f_ref = ref if ref is not None else run_oracle(inp, heads=heads, scale=scale)
    if heads is not None:
        out = out[:, :, heads]
        fin = fin[:, heads]
    compare(f"{label} out", out, o_ref, inp.io)
    compare(f"{label} final_state", fin, f_ref, inp.io)
    return out, fin


# --------------------------------------------------------------- workloads --

@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dv_tile", [32, 64])
@pytest.mark.parametrize("algo", ALGOS)
def test_tiny_fp32_chunk(chunk, dv_tile, algo):
    check_fwd(ki.workload_inputs("tiny_fp32"), chunk_size=chunk, dv_tile=dv_tile, label="tiny_fp32", algo=algo)


def test_tiny_fp32_recurrent():
    check_fwd(ki.workload_inputs("tiny_fp32"), mode="recurrent", label="tiny_fp32")


@pytest.mark.parametrize("algo,dv_tile", [("fused", 0), ("fused", 32), ("fused", 64), ("fused", 128),
                                          ("two_pass", 0), ("two_pass", 32), ("two_pass", 64)])
def test_prefill_full(algo, dv_tile):
    check_fwd(ki.workload_inputs("prefill"), dv_tile=dv_tile, label="prefill", algo=algo)


def test_prefill_recurrent():
    check_fwd(ki.workload_inputs("prefill"), mode="recurrent", label="prefill")


_REF = {}


def workload_reference(name):
    """Inputs of a full-size workload and the oracle's outputs over all of its heads, computed
    once per session (one large workload is kept in memory at a time)."""
    if name not in _REF:
        _REF.clear()
        inp = ki.workload_inputs(name)
        say(f"[{name}] oracle over all {inp.q.shape[2]} heads, {inp.q.shape[0] * inp.q.shape[1]} tokens ...")
        t0 = time.perf_counter()
        ref = run_oracle(inp)
        say(f"[{name}] oracle done in {time.perf_counter() - t0:.1f} s")
        _REF[name] = (inp, ref)
    return _REF[name]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("chunk", [0, 64])  # the library's choice for this shape and the workload's 64
def test_long_prefill_all_heads(algo, chunk):
    inp, ref = workload_reference("long_prefill")
    check_fwd(inp, label="long_prefill", algo=algo, chunk_size=chunk, ref=ref)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("chunk,dv_tile", [(0, 0), (64, 0), (32, 32)])  # default, the workload's chunk, the other scan
def test_varlen_all_heads(algo, chunk, dv_tile):
    inp, ref = workload_reference("varlen")
    check_fwd(inp, label="varlen", algo=algo, chunk_size=chunk, dv_tile=dv_tile if algo == "two_pass" else 0,
              ref=ref)
    torch.cuda.empty_cache()


def test_decode_full():
    inp = ki.workload_inputs("decode")
    N, _, H, dk = inp.q.shape
    say(f"[decode] N={N} H={H} dk={dk}")
    state = inp.s0.to(DEV).clone()
    sq = lambda x: x[:, 0].contiguous().to(DEV)
    out = kda.decode_step(sq(inp.q), sq(inp.k), sq(inp.v), sq(inp.g), sq(inp.beta), state)
    torch.cuda.synchronize()
    a = [ki.to_numpy_io(x[:, 0].contiguous()) for x in (inp.q, inp.k, inp.v)]
    o_ref, s_ref = oracle.decode(*a, inp.g[:, 0].contiguous().numpy(), inp.beta[:, 0].contiguous().numpy(),
                                 inp.s0.numpy())
    compare("decode out", out, o_ref, "bf16")
    compare("decode state", state, s_ref, "bf16")


# -------------------------------------------------------------- edge cases --

def small(B, T, H, dk, dv, io, seed, **kw):
    return ki.make_inputs(B, T, H, dk, dv, io, seed, **kw)


@pytest.mark.parametrize("io,dk,dv,chunk", [("bf16", 128, 128, 64), ("bf16", 128, 128, 16), ("bf16", 128, 128, 32),
                                           ("bf16", 64, 128, 64), ("bf16", 128, 64, 32), ("f32", 64, 64, 64),
                                           ("f32", 128, 128, 32), ("f32", 128, 64, 16), ("f32", 128, 128, 64),
                                           ("f32", 128, 64, 64)])
@pytest.mark.parametrize("algo", ALGOS)
def test_ragged_lengths_and_dims(io, dk, dv, chunk, algo):
    # T = 203 is not a multiple of any chunk size: every sequence ends in a partial chunk
    inp = small(2, 203, 3, dk, dv, io, seed=dk + dv + chunk)
    check_fwd(inp, chunk_size=chunk, label=f"ragged-{io}-{dk}x{dv}-c{chunk}", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
def test_varlen_with_empty_and_single_token_sequences(algo):
    lens = [0, 1, 64, 65, 17, 0, 200, 63]
    inp = ki.make_inputs(1, 0, 4, 128, 128, "bf16", 21, lengths=lens)
    check_fwd(inp, label="varlen-edge", algo=algo)
    check_fwd(inp, mode="recurrent", label="varlen-edge")


def test_packed_plan_ranks_longest_first():
    """The two-pass plan of a packed batch (300 sequences: two ranking workgroups, empty ones and
    many equal chunk counts): the chunk-offset table is the prefix sum of ceil(len / C) and the
    order lists the sequences most chunks first, equal counts in batch order (integers: exact);
    the outputs, scanned in that order, still match the oracle."""
    rng = np.random.default_rng(300)
    lens = [int(x) for x in rng.integers(0, 400, size=300)]
    lens[::17] = [0] * len(lens[::17])
    lens[5::23] = [64] * len(lens[5::23])
    C = 64
    inp = ki.make_inputs(1, 0, 2, 64, 64, "bf16", 22, lengths=lens)
    T = sum(lens)
    ws_bytes = kda.query(1, T, 2, 64, 64, "bf16", num_seqs=len(lens), chunk_size=C,
                         algo="two_pass")["workspace_bytes"]
    ws = torch.full((ws_bytes,), 0xAB, dtype=torch.uint8, device=DEV)
    d = on_dev(inp)
    out, fin = kda.chunk_fwd(**d, chunk_size=C, algo="two_pass", workspace=ws)
    torch.cuda.synchronize()
    n = len(lens)
    a256 = lambda x: (x + 255) // 256 * 256
    words = ws[: a256((n + 1) * 4) + a256(n * 4)].view(torch.int32).cpu().numpy()
    nc = [(x + C - 1) // C for x in lens]
    assert words[: n + 1].tolist() == [0] + list(np.cumsum(nc))
    off = a256((n + 1) * 4) // 4  # int32 index of the order table
    assert words[off: off + n].tolist() == sorted(range(n), key=lambda i: (-nc[i], i))
    o_ref, f_ref = run_oracle(inp)
    compare("plan out", out, o_ref, "bf16")
    compare("plan final_state", fin, f_ref, "bf16")


@pytest.mark.parametrize("algo", ALGOS)
def test_no_initial_state_and_no_final_state(algo):
    inp = small(2, 150, 2, 128, 128, "bf16", 5, s0_std=None)
    check_fwd(inp, label="zero-s0", algo=algo)
    d = on_dev(inp)
    out, fin = kda.chunk_fwd(**d, output_final_state=False, algo=algo)
    torch.cuda.synchronize()
    assert fin is None
    o_ref, _ = run_oracle(inp)
    compare("no-final out", out, o_ref, "bf16")


@pytest.mark.parametrize("algo", ALGOS)
def test_in_place_state(algo):
    inp = small(2, 130, 2, 128, 128, "bf16", 6)
    d = on_dev(inp)
    st = d["initial_state"].clone()
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, final_state=st, algo=algo)
    torch.cuda.synchronize()
    o_ref, f_ref = run_oracle(inp)
    compare("inplace out", out, o_ref, "bf16")
    compare("inplace state", st, f_ref, "bf16")


def test_scale():
    check_fwd(small(1, 100, 2, 64, 64, "f32", 7), scale=0.125, label="scale")


@pytest.mark.parametrize("algo", ALGOS)
def test_zero_beta_is_pure_decay_with_state(algo):
    # beta == 0 leaves only the decayed initial state; g = -softplus(N(-3, 1)) keeps that
    # state within fp32 range over 256 tokens (with mu = 0 it decays to ~1e-85)
    inp = small(2, 256, 2, 128, 128, "bf16", 8, s0_std=1.0, g_mu=-3.0)
    inp.beta.zero_()
    check_fwd(inp, label="beta0", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
def test_unit_gate_deltanet(algo):
    inp = small(2, 256, 2, 128, 128, "bf16", 9)
    inp.g.zero_()
    check_fwd(inp, label="g0", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
def test_long_memory_gate(algo):
    inp = small(1, 1024, 2, 128, 128, "bf16", 10, g_mu=-6.0, s0_std=1.0)
    check_fwd(inp, label="long-memory", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
def test_strong_gate(algo):
    # mean per-token log-decay about -2.1: 16-token sub-chunks decay by ~e^-34
    inp = small(1, 512, 2, 128, 128, "bf16", 11, g_mu=2.0)
    check_fwd(inp, label="strong-gate", algo=algo)


def test_strong_gate_fp32():
    inp = small(1, 256, 2, 64, 64, "f32", 12, g_mu=2.0)
    check_fwd(inp, chunk_size=64, label="strong-gate-f32")


# ---------------------------------------------------------- cross-checks ----

@pytest.mark.parametrize("algo", ALGOS)
def test_chunk_equals_recurrent_on_gpu(algo):
    inp = small(2, 777, 4, 128, 128, "bf16", 13)
    d = on_dev(inp)
    o1, f1 = kda.chunk_fwd(**d, algo=algo)
    o2, f2 = kda.recurrent_fwd(**d)
    torch.cuda.synchronize()
    compare("chunk vs recurrent out", o1, o2.double().cpu().numpy(), "bf16")
    compare("chunk vs recurrent state", f1, f2.double().cpu().numpy(), "bf16")


def test_repeated_decode_equals_forward():
    inp = small(3, 40, 2, 128, 128, "bf16", 14)
    d = on_dev(inp)
    o_fwd, f_fwd = kda.chunk_fwd(**d)
    state = d["initial_state"].clone()
    outs = []
    for t in range(inp.q.shape[1]):
        sl = lambda x: x[:, t].contiguous()
        outs.append(kda.decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), state))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    o_ref, f_ref = run_oracle(inp)
    compare("decode-seq out", o_dec, o_ref, "bf16")
    compare("decode-seq state", state, f_ref, "bf16")
    compare("chunk out (same inputs)", o_fwd, o_ref, "bf16")


def test_split_invariance():
    # running [0, T1) then [T1, T) from the GPU final state equals one run
    inp = small(1, 300, 2, 128, 128, "bf16", 15)
    d = on_dev(inp)
    o, f = kda.chunk_fwd(**d)
    T1 = 137
    cut = lambda x, s: x[:, s].contiguous()
    oa, fa = kda.chunk_fwd(cut(d["q"], slice(0, T1)), cut(d["k"], slice(0, T1)), cut(d["v"], slice(0, T1)),
                           cut(d["g"], slice(0, T1)), cut(d["beta"], slice(0, T1)), d["initial_state"])
    ob, fb = kda.chunk_fwd(cut(d["q"], slice(T1, None)), cut(d["k"], slice(T1, None)), cut(d["v"], slice(T1, None)),
                           cut(d["g"], slice(T1, None)), cut(d["beta"], slice(T1, None)), fa)
    torch.cuda.synchronize()
    o_ref, f_ref = run_oracle(inp)
    compare("split out", torch.cat([oa, ob], dim=1), o_ref, "bf16")
    compare("split state", fb, f_ref, "bf16")


def test_query_on_device():
    r = kda.query(4, 4096, 16, 128, 128, "bf16", device=True)
    say(f"  device: {r['arch']} CUs={r['compute_units']}")
    assert r["device_ok"] == 1 and r["arch"].startswith("gfx950")


def test_tune_picks_a_configuration_that_matches_the_oracle():
    inp = ki.make_inputs(2, 300, 4, 128, 128, "bf16", seed=31)
    say("tune B=2 T=300 H=4 d=128 bf16")
    d = on_dev(inp)
    cfg = kda.tune(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    say(f"  chosen: chunk={cfg['chunk_size']} dv_tile={cfg['dv_tile']} algo={cfg['algo']} {cfg['tuned_ms']:.4f} ms")
    assert cfg["supported"] == 1 and cfg["tuned_ms"] > 0 and cfg["chunk_size"] in (16, 32, 64)
    algo = {kda.KDA_ALGO_FUSED: "fused", kda.KDA_ALGO_TWO_PASS: "two_pass"}[cfg["algo"]]
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                             chunk_size=cfg["chunk_size"], dv_tile=cfg["dv_tile"], algo=algo)
    o_ref, s_ref = run_oracle(inp)
    compare("o", out, o_ref, "bf16")
    compare("final_state", fin, s_ref, "bf16")


@pytest.mark.parametrize("dk,chunk", [(128, 64), (64, 64), (128, 32), (64, 16)])
@pytest.mark.parametrize("algo", ALGOS)
def test_forward_repeatable(dk, chunk, algo):
    """Two calls on the same inputs give bit-identical outputs and final states (a race or a
    matrix-core result read back too early would show as run-to-run differences)."""
    inp = ki.make_inputs(2, 300, 4, dk, 128, "bf16", seed=36, s0_std=0.1)
    t = lambda x: None if x is None else x.to(DEV)
    args = (t(inp.q), t(inp.k), t(inp.v), t(inp.g), t(inp.beta), t(inp.s0))
    o1, f1 = kda.chunk_fwd(*args, chunk_size=chunk, algo=algo)
    o2, f2 = kda.chunk_fwd(*args, chunk_size=chunk, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("io,dk,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("bf16", 128, 16), ("f32", 64, 32),
                                         ("bf16", 128, 32), ("f32", 128, 16)])
def test_scan_tilings_agree(io, dk, chunk):
    """The two-pass forward with 16-, 32- and 64-column tiles (one wave of one 16-column slice,
    two waves of one or two slices; at d_k = 128, chunk 64 also two different scan kernels: chain
    and output on separate waves with S and D handed over through LDS, against waves that do the
    whole chunk) rounds the same operands and accumulates in the same order, so all agree bit for
    bit; each is also checked against the oracle.  Packed sequences with an empty and a one-token
    sequence exercise the first and last chunk of each.  Tiles without a compiled variant for the
    shape (16 columns of bf16 at chunk 16) are left out."""
    lens = [0, 1, 77, 3 * chunk + 5, 2 * chunk]
    inp = ki.make_inputs(1, 0, 3, dk, 128, io, seed=41, s0_std=0.1, lengths=lens)
    d = on_dev(inp)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
    out = {}
    for tile in (16, 32, 64):
        if not kda.query(1, inp.q.shape[1], 3, dk, 128, io, chunk_size=chunk, dv_tile=tile, algo="two_pass",
                         num_seqs=len(lens))["supported"]:
            say(f"  tile {tile}: not compiled for {io} d_k={dk} chunk={chunk}")
            continue
        out[tile] = kda.chunk_fwd(*args, chunk_size=chunk, dv_tile=tile, algo="two_pass")
    if len(out) < 2:
        pytest.skip(f"fewer than two two-pass tilings compiled for {io} d_k={dk} chunk={chunk}")
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(inp)
    for tile in out:
        compare(f"o (tile {tile})", out[tile][0], o_ref, io)
        compare(f"final_state (tile {tile})", out[tile][1], s_ref, io)
    first = min(out)
    for tile in out:
        assert torch.equal(out[first][0], out[tile][0]), f"outputs differ between the {first}- and {tile}-column scans"
        assert torch.equal(out[first][1], out[tile][1]), \
            f"final states differ between the {first}- and {tile}-column scans"


def test_side_stream_workspace():
    """chunk_fwd launched on a side stream with the workspace allocated by the binding (on the
    current stream): allocations and fills queued on the current stream right after each call may
    not land in that workspace while the side stream's kernels still read it."""
    inp = small(4, 2048, 8, 128, 128, "bf16", 16)
    d = on_dev(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws_bytes = kda.query(4, 2048, 8, 128, 128, "bf16")["workspace_bytes"]
    assert ws_bytes > 0
    results = []
    for _ in range(3):
        out, fin = kda.chunk_fwd(**d, algo="two_pass", stream=side)
        junk = torch.full((ws_bytes // 4,), float("nan"), device=DEV)  # same size class as the workspace
        results.append((out, fin, junk))
    torch.cuda.synchronize()
    o_ref, f_ref = run_oracle(inp)
    for out, fin, _ in results:
        compare("side-stream out", out, o_ref, "bf16")
        compare("side-stream final_state", fin, f_ref, "bf16")


@pytest.mark.parametrize("io,dk,chunk", [("bf16", 128, 64), ("bf16", 128, 32), ("bf16", 128, 16), ("bf16", 64, 64),
                                         ("f32", 64, 64), ("f32", 128, 32), ("f32", 64, 16), ("f32", 128, 64)])
@pytest.mark.parametrize("algo", ALGOS)
def test_strong_decay_inside_a_chunk(io, dk, chunk, algo):
    """Channels that decay by e^-100 in one token, e^-20 per token over 40 tokens, e^-112 and
    e^-64 per 16-token sub-chunk and e^-60 every 16th token (kda_inputs.plant_strong_decay):
    outputs and final states stay finite and within the bars (the diagonal blocks of the chunk
    matrices switch to the split-level factors where a sub-chunk decays beyond 2^-96)."""
    inp = ki.plant_strong_decay(small(2, 203, 2, dk, 128, io, 51 + dk + chunk, s0_std=0.5))
    check_fwd(inp, chunk_size=chunk, label=f"strong-decay-{io}-d{dk}-c{chunk}", algo=algo)


def test_fp32_dk128_chunk64_packed():
    """fp32 at d_k = 128 with chunk 64: the two-pass scan with one record buffer (two barriers per
    chunk), over a packed batch with an empty and a one-token sequence."""
    inp = ki.make_inputs(1, 0, 3, 128, 128, "f32", 53, s0_std=0.5, lengths=[150, 1, 0, 64, 90, 200])
    check_fwd(inp, chunk_size=64, label="f32-d128-c64 packed", algo="two_pass")
    check_fwd(inp, chunk_size=64, dv_tile=32, label="f32-d128-c64 packed tile 32", algo="two_pass")


def test_strong_decay_recurrent_and_packed():
    inp = ki.plant_strong_decay(ki.make_inputs(1, 0, 3, 128, 128, "bf16", 52, s0_std=0.5,
                                               lengths=[150, 1, 0, 64, 90]))
    check_fwd(inp, mode="recurrent", label="strong-decay recurrent")
    for algo in ALGOS:
        check_fwd(inp, label="strong-decay packed", algo=algo)
