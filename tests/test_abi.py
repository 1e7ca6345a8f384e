"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/kda.h declares, and rejects invalid calls on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_45_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_decode_step", "kda_recurrent_fwd", "kda_query"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = kda.library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in kda.h but not exported by libkda.so"


def test_exported_symbols_are_c_linkage():
    # C linkage: the plain name resolves (a C++-mangled symbol would not)
    lib = ctypes.CDLL(kda.LIB_PATH)
    assert lib.kda_status_string is not None


def test_status_strings():
    lib = kda.library()
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(99) == b"KDA_ERR_UNKNOWN"


def problem(**kw):
    base = dict(batch=1, seq_len=128, num_heads=2, head_dim_k=64, head_dim_v=64, num_seqs=0, io_dtype=kda.KDA_BF16,
                chunk_size=0, scale=1.0, dv_tile=0)
    base.update(kw)
    return kda.Problem(**base)


FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: validation fails first or no launch
fake = lambda i: ctypes.c_void_p(0x100000 * (i + 1))  # distinct aligned addresses, one per argument


def call_chunk(p, q=fake(0), k=fake(1), v=fake(2), g=fake(3), beta=fake(4), s0=None, cu=None, cu_host=None,
               out=fake(5), sf=None):
    lib = kda.library()
    return lib.kda_chunk_fwd(ctypes.byref(p) if p is not None else None, q, k, v, g, beta, s0, cu, cu_host, out, sf,
                             None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(seq_len=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(batch=-2), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(head_dim_k=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(head_dim_v=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk_size=128), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk_size=24), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv_tile=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv_tile=128), kda.KDA_ERR_INVALID_ARGUMENT),  # larger than d_v = 64
    (dict(io_dtype=7), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID_ARGUMENT),
    # fp32 at d_k = 128, chunk 64 runs two-pass only (the fused kernel's LDS does not hold it):
    # without a workspace the call is refused
    (dict(io_dtype=kda.KDA_F32, head_dim_k=128, head_dim_v=128, chunk_size=64), kda.KDA_ERR_WORKSPACE),
    (dict(io_dtype=kda.KDA_F32, head_dim_k=128, head_dim_v=128, chunk_size=64, algo=kda.KDA_ALGO_FUSED),
     kda.KDA_ERR_UNSUPPORTED),
])
def test_chunk_fwd_rejects_bad_problems(kw, status):
    assert call_chunk(problem(**kw)) == status
    assert kda.library().kda_last_error() != b""


def test_chunk_fwd_rejects_null_and_misaligned_pointers():
    lib = kda.library()
    assert call_chunk(None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_chunk(problem(), q=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert b"q is NULL" in lib.kda_last_error()
    assert call_chunk(problem(), out=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_chunk(problem(), g=ctypes.c_void_p(0x10004)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert b"not 16-byte aligned" in lib.kda_last_error()
    assert call_chunk(problem(), s0=ctypes.c_void_p(0x10008)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_chunk(problem(), out=FAKE, q=FAKE) == kda.KDA_ERR_INVALID_ARGUMENT  # out aliases q
    assert b"aliases" in lib.kda_last_error()
    assert call_chunk(problem(), s0=fake(7), sf=fake(8), out=fake(7)) == kda.KDA_ERR_INVALID_ARGUMENT


def test_chunk_fwd_checks_host_cu_seqlens():
    lens = [3, 5, 0, 7]
    good = [0, 3, 8, 8, 15]
    arr = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    p = problem(seq_len=15, num_seqs=4)
    # B != 1 with cu_seqlens
    assert call_chunk(problem(batch=2, seq_len=15, num_seqs=4), cu=FAKE) == kda.KDA_ERR_INVALID_ARGUMENT
    bad_start = arr([1, 3, 8, 8, 15])
    assert call_chunk(p, cu=FAKE, cu_host=bad_start) == kda.KDA_ERR_INVALID_ARGUMENT
    decreasing = arr([0, 3, 2, 8, 15])
    assert call_chunk(p, cu=FAKE, cu_host=decreasing) == kda.KDA_ERR_INVALID_ARGUMENT
    wrong_end = arr([0, 3, 8, 8, 14])
    assert call_chunk(p, cu=FAKE, cu_host=wrong_end) == kda.KDA_ERR_INVALID_ARGUMENT
    assert b"expected seq_len" in kda.library().kda_last_error()
    # host copy without device offsets
    assert call_chunk(p, cu=None, cu_host=arr(good)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert sum(lens) == 15


def test_algo_and_workspace_validation():
    lib = kda.library()
    assert call_chunk(problem(algo=7)) == kda.KDA_ERR_INVALID_ARGUMENT
    # two-pass requested without a workspace
    assert call_chunk(problem(algo=kda.KDA_ALGO_TWO_PASS)) == kda.KDA_ERR_WORKSPACE
    assert b"workspace" in lib.kda_last_error()
    # two-pass on a 128-column tile does not exist
    p = problem(head_dim_v=128, dv_tile=128, algo=kda.KDA_ALGO_TWO_PASS)
    assert call_chunk(p) == kda.KDA_ERR_UNSUPPORTED


def test_empty_problems_launch_nothing_and_succeed():
    # zero sequences: nothing to do, no HIP call
    assert call_chunk(problem(batch=0)) == kda.KDA_OK
    assert call_chunk(problem(seq_len=0, num_seqs=0), cu=FAKE) == kda.KDA_OK


def test_decode_step_validation():
    lib = kda.library()
    f = lambda *a: lib.kda_decode_step(*a)
    args = lambda **kw: [kw.get("N", 4), kw.get("H", 2), kw.get("dk", 128), kw.get("dv", 128), kw.get("io", 1), 1.0,
                         fake(0), fake(1), fake(2), fake(3), fake(4), kw.get("state", ctypes.c_void_p(0x20000)), kw.get("out", ctypes.c_void_p(0x30000)), None]
    assert f(*args(N=-1)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(H=0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(dk=32)) == kda.KDA_ERR_UNSUPPORTED
    assert f(*args(io=3)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(state=None)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(out=ctypes.c_void_p(0x30002))) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(N=0)) == kda.KDA_OK


def test_chunk_fwd_prologue_validation():
    """Every refusal happens on the host, before any launch (no GPU needed): each call below has
    exactly one defect."""
    lib = kda.library()
    P = lambda i: ctypes.c_void_p(0x100000 * (i + 1))
    WS = ctypes.c_void_p(0x10000000)

    def call(prob=None, W=4, eps=1e-6, taps=(P(3), P(4), P(5)), out=P(9), ws=WS, ws_bytes=1 << 30):
        prob = prob or problem(seq_len=100)
        return lib.kda_chunk_fwd_prologue(ctypes.byref(prob), W, eps, P(0), P(1), P(2), *taps, P(6), P(7), None, None,
                                          None, out, None, ws, ws_bytes, None)
    assert call(prob=problem(seq_len=100, algo=kda.KDA_ALGO_FUSED)) == kda.KDA_ERR_UNSUPPORTED
    assert call(W=0) == kda.KDA_ERR_UNSUPPORTED
    assert call(W=5) == kda.KDA_ERR_UNSUPPORTED
    assert call(eps=-1.0) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(eps=float("inf")) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(taps=(P(3), None, P(5))) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "conv_k" in lib.kda_last_error().decode()
    assert call(taps=(P(3), P(4), ctypes.c_void_p(0x600002))) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(out=P(4)) == kda.KDA_ERR_INVALID_ARGUMENT  # out aliases conv_k
    assert call(out=P(0)) == kda.KDA_ERR_INVALID_ARGUMENT  # out aliases q_raw
    assert call(ws=None) == kda.KDA_ERR_WORKSPACE
    assert call(ws_bytes=1024) == kda.KDA_ERR_WORKSPACE
    assert call(prob=problem(seq_len=100, chunk_size=48)) == kda.KDA_ERR_UNSUPPORTED
    assert call(prob=problem(batch=0)) == kda.KDA_OK  # nothing to compute, nothing launched


def test_decode_step_gated_validation():
    """Every refusal happens on the host, before any launch (no GPU needed)."""
    lib = kda.library()
    f = lambda *a: lib.kda_decode_step_gated(*a)
    P = lambda i: ctypes.c_void_p(0x100000 * (i + 1))

    def args(**kw):
        return [kw.get("N", 4), kw.get("H", 2), kw.get("dk", 128), kw.get("dv", 128), kw.get("io", 1), 1.0,
                P(0), P(1), P(2), P(3), P(4), kw.get("state", P(5)), kw.get("gate", P(6)), kw.get("weight", P(7)),
                kw.get("eps", 1e-6), kw.get("out", P(8)), None]
    assert f(*args(N=-1)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(dv=96)) == kda.KDA_ERR_UNSUPPORTED
    assert f(*args(io=2)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(eps=-1.0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(eps=float("nan"))) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(gate=None)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "gate" in lib.kda_last_error().decode()
    assert f(*args(weight=ctypes.c_void_p(0x800004))) == kda.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(out=P(6))) == kda.KDA_ERR_INVALID_ARGUMENT   # out aliases gate
    assert f(*args(state=P(7))) == kda.KDA_ERR_INVALID_ARGUMENT  # state aliases weight
    assert f(*args(out=P(5))) == kda.KDA_ERR_INVALID_ARGUMENT   # out aliases state
    assert f(*args(N=0)) == kda.KDA_OK


def test_recurrent_validation():
    lib = kda.library()
    p = problem(head_dim_k=80)
    st = lib.kda_recurrent_fwd(ctypes.byref(p), fake(0), fake(1), fake(2), fake(3), fake(4), None, None, None,
                               fake(5), None, None)
    assert st == kda.KDA_ERR_UNSUPPORTED


def test_query_reports_config_and_work():
    # prefill workload: B=4, T=4096, H=16, d=128, bf16; chunk 32 by default
    assert kda.query(4, 4096, 16, 128, 128, "bf16")["chunk_size"] == 32
    r = kda.query(4, 4096, 16, 128, 128, "bf16", chunk_size=64)
    assert r["status"] == kda.KDA_OK and r["supported"] == 1
    assert r["algo"] == kda.KDA_ALGO_TWO_PASS and r["chunk_size"] == 64
    # plan (chunk-offset table and longest-first order, 256 B each) + one record per chunk-head:
    # K~, Q~, K-^T (16 KB each),
    # the lower 16x32 tiles of T and of P (5 KB each: the two diagonal tiles of even row tiles
    # keep only their left 16 columns), Gamma (512 B), rounded up to whole KB
    rec = 3 * 16384 + 2 * 5120 + 512
    rec = (rec + 1023) // 1024 * 1024
    assert r["workspace_bytes"] == 2 * 256 + 4 * 64 * 16 * rec
    assert r["grid_blocks"] == 4 * 16 * (128 // r["dv_tile"])
    rf = kda.query(4, 4096, 16, 128, 128, "bf16", chunk_size=64, algo="fused")
    assert rf["algo"] == kda.KDA_ALGO_FUSED and rf["workspace_bytes"] == 0
    assert rf["grid_blocks"] == 4 * 16 * (128 // rf["dv_tile"])
    ht = 4 * 4096 * 16
    assert r["flops"] == pytest.approx(ht * (2 * 64 * 256 + 64 * 64 / 3 + 6 * 128 * 128))
    assert r["hbm_bytes"] == pytest.approx(ht * 1540 + 2 * 4 * 128 * 128 * 64)
    assert 0 < rf["lds_bytes"] <= 160 * 1024
    # the two-pass scan at this shape: 2 chain + 2 output + 4 copy waves; two double-buffered
    # records and V tiles [64][32] bf16, then the parity-alternating S (8 bf16 fragments per lane)
    # and D (4 fragments per lane) slots of the two chain waves
    assert r["threads_per_block"] == 64 * 8
    assert r["lds_bytes"] == 2 * rec + 2 * 64 * 32 * 2 + 2 * 2 * 64 * (64 + 32)
    assert r["peak_hbm_gbps"] == 8000.0 and r["peak_bf16_tflops"] == 2500.0
    # unsupported variant is reported, not raised
    r = kda.query(1, 64, 1, 128, 128, "f32", chunk_size=64, algo="fused")
    assert r["status"] == kda.KDA_ERR_UNSUPPORTED and r["supported"] == 0
    # fp32, d_k = 128, chunk 64: two-pass with one record buffer (the 117 KB fp32 record does not
    # fit twice): record + V tile [64][32] fp32, 2 compute + 4 copy waves
    r = kda.query(1, 64, 1, 128, 128, "f32", chunk_size=64, dv_tile=32)
    assert r["status"] == kda.KDA_OK and r["algo"] == kda.KDA_ALGO_TWO_PASS
    rec32 = (3 * 32768 + 2 * 10240 + 512 + 1023) // 1024 * 1024
    assert rec32 == 119808 and r["lds_bytes"] == rec32 + 64 * 32 * 4 and r["threads_per_block"] == 64 * 6
    # one (sequence, head): too few 32-column workgroups to fill the GPU, so by default 16-column
    # tiles (one compute wave and the four copy waves)
    r = kda.query(1, 64, 1, 128, 128, "f32", chunk_size=64)
    assert r["dv_tile"] == 16 and r["lds_bytes"] == rec32 + 64 * 16 * 4 and r["threads_per_block"] == 64 * 5
    # packed batch: num_seqs > 0, seq_len = total tokens
    r = kda.query(1, 1000, 32, 128, 128, "bf16", num_seqs=64)
    assert r["grid_blocks"] == 64 * 32 * (128 // r["dv_tile"])


def call_norm_gate(rows=8, d=128, io=kda.KDA_BF16, eps=1e-6, o=fake(0), gate=fake(1), weight=fake(2), out=fake(3)):
    return kda.library().kda_norm_gate(rows, d, io, eps, o, gate, weight, out, None)


def test_norm_gate_validation():
    lib = kda.library()
    assert call_norm_gate(rows=0) == kda.KDA_OK  # nothing to do, nothing launched
    assert call_norm_gate(rows=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_norm_gate(d=96) == kda.KDA_ERR_UNSUPPORTED
    assert call_norm_gate(io=7) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_norm_gate(eps=-1.0) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_norm_gate(eps=float("nan")) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_norm_gate(gate=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert b"gate" in lib.kda_last_error()
    assert call_norm_gate(out=ctypes.c_void_p(0x100008)) == kda.KDA_ERR_INVALID_ARGUMENT  # misaligned
    assert call_norm_gate(out=fake(1)) == kda.KDA_ERR_INVALID_ARGUMENT  # out aliases gate
    assert b"alias" in lib.kda_last_error()


def prologue_problem(**kw):
    base = dict(batch=2, seq_len=16, num_seqs=0, num_heads=2, head_dim_k=64, head_dim_v=64, conv_width=4,
                io_dtype=kda.KDA_BF16, norm_eps=1e-6)
    base.update(kw)
    return kda.PrologueProblem(**base)


def call_prologue(p, ptrs=None, **over):
    a = [fake(i) for i in range(17)]  # q_raw k_raw v_raw conv_q conv_k conv_v g_raw beta_raw cu st st_out q k v g beta
    a[8], a[9], a[10] = None, None, None
    for i, v in over.items():
        a[int(i[1:])] = v
    return kda.library().kda_prologue(ctypes.byref(p) if p is not None else None, *a, None)


def test_prologue_validation():
    lib = kda.library()
    assert call_prologue(None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_prologue(prologue_problem(conv_width=5)) == kda.KDA_ERR_UNSUPPORTED
    assert call_prologue(prologue_problem(conv_width=0)) == kda.KDA_ERR_UNSUPPORTED
    assert call_prologue(prologue_problem(head_dim_k=96)) == kda.KDA_ERR_UNSUPPORTED
    assert call_prologue(prologue_problem(norm_eps=-1.0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_prologue(prologue_problem(num_seqs=3)) == kda.KDA_ERR_INVALID_ARGUMENT  # batch != 1
    assert call_prologue(prologue_problem(batch=1, num_seqs=3)) == kda.KDA_ERR_INVALID_ARGUMENT  # no cu_seqlens
    assert b"cu_seqlens" in lib.kda_last_error()
    assert call_prologue(prologue_problem(), a11=fake(0)) == kda.KDA_ERR_INVALID_ARGUMENT  # q aliases q_raw
    assert b"alias" in lib.kda_last_error()
    assert call_prologue(prologue_problem(), a9=fake(20), a10=fake(20)) == kda.KDA_ERR_INVALID_ARGUMENT  # state in place
    assert call_prologue(prologue_problem(), a0=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_prologue(prologue_problem(), a6=ctypes.c_void_p(0x100004)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_prologue(prologue_problem(seq_len=0)) == kda.KDA_OK  # no tokens, no state out: nothing to do


def test_tune_validation():
    lib = kda.library()
    res = kda.QueryResult()
    p = problem()
    args = [fake(i) for i in range(5)]
    # no result struct
    assert lib.kda_tune(ctypes.byref(p), *args, None, None, None, fake(5), None, None, 0, None, None) == \
        kda.KDA_ERR_INVALID_ARGUMENT
    # initial state aliasing the final state
    assert lib.kda_tune(ctypes.byref(p), *args, fake(6), None, None, fake(5), fake(6), None, 0, None,
                        ctypes.byref(res)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert b"alias" in lib.kda_last_error()
    # invalid problem is reported before any launch
    bad = problem(head_dim_k=96)
    assert lib.kda_tune(ctypes.byref(bad), *args, None, None, None, fake(5), None, None, 0, None,
                        ctypes.byref(res)) == kda.KDA_ERR_UNSUPPORTED


def _bwd_problem(**kw):
    base = dict(batch=2, seq_len=100, num_heads=2, head_dim_k=128, head_dim_v=128, num_seqs=0,
                io_dtype=kda.KDA_BF16, chunk_size=64, scale=1.0, dv_tile=0, algo=0)
    base.update(kw)
    return kda.Problem(**base)


def test_bwd_workspace_query():
    lib = kda.library()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace(ctypes.byref(_bwd_problem()), ctypes.byref(n)) == kda.KDA_OK
    # plan + two-pass records (60,416 B per chunk and head at bf16, d_k = 128, chunk 64), then chunk
    # states and their gradients, D and dU tiles (all bf16, the operand type), in 256-byte sections
    a256 = lambda x: (x + 255) // 256 * 256
    rec = (3 * 16384 + 2 * 5120 + 512 + 1023) // 1024 * 1024  # whole KB: 60,416
    # reverse-scan records as the scan keeps them in LDS (rows padded by 16 B): M [64][136] and
    # N [64][72], Q~^T and (beta K~)^T [128][72] (bf16), e^{G_C} and beta (fp32): 64,256 B,
    # rounded up to whole KB
    brec = (64 * 136 * 2 + 64 * 72 * 2 + 2 * 128 * 72 * 2 + 512 + 256 + 1023) // 1024 * 1024
    # and one int32 flag per chunk and head (strong decay inside the chunk), in a 256-byte section
    slots = 2 * 2  # 2 sequences x ceil(100 / 64)
    assert n.value == a256(2 * 256 + slots * 2 * rec) + 2 * slots * 2 * 128 * 128 * 2 + 2 * slots * 2 * 64 * 128 * 2 + \
        a256(slots * 2 * brec) + a256(slots * 2 * 4)
    # a packed batch reserves one partial chunk per sequence
    assert lib.kda_chunk_bwd_workspace(ctypes.byref(_bwd_problem(batch=1, seq_len=300, num_seqs=5)),
                                       ctypes.byref(n)) == kda.KDA_OK
    slots = 5 + 5
    assert n.value == a256(2 * 256 + slots * 2 * rec) + 2 * slots * 2 * 128 * 128 * 2 + 2 * slots * 2 * 64 * 128 * 2 + \
        a256(slots * 2 * brec) + a256(slots * 2 * 4)
    assert lib.kda_chunk_bwd_workspace(ctypes.byref(_bwd_problem(chunk_size=48)), ctypes.byref(n)) == \
        kda.KDA_ERR_UNSUPPORTED
    assert n.value == 0
    assert lib.kda_chunk_bwd_workspace(ctypes.byref(_bwd_problem()), None) == kda.KDA_ERR_INVALID_ARGUMENT


def test_bwd_validation():
    lib = kda.library()
    p = _bwd_problem()
    P = lambda a: ctypes.c_void_p(a)
    good = [P(0x10000 * (i + 1)) for i in range(16)]
    ws_ok = 1 << 30

    def call(ptrs, ws=P(0x100000), ws_bytes=ws_ok, prob=p):
        return lib.kda_chunk_bwd(ctypes.byref(prob), *ptrs, ws, ws_bytes, None)

    # q k v g beta s0 cu cu_host d_out d_sf dq dk dv dg dbeta ds0
    ptrs = good[:6] + [None, None] + good[8:16]
    for i, name in [(0, "q"), (8, "d_out"), (10, "dq"), (11, "dk"), (12, "dv"), (13, "dg"), (14, "dbeta")]:
        bad = list(ptrs)
        bad[i] = None
        assert call(bad) == kda.KDA_ERR_INVALID_ARGUMENT, name
        assert name in lib.kda_last_error().decode()
    bad = list(ptrs)
    bad[13] = P(0x10008)  # dg misaligned
    assert call(bad) == kda.KDA_ERR_INVALID_ARGUMENT
    bad = list(ptrs)
    bad[11] = ptrs[1]  # dk aliases k
    assert call(bad) == kda.KDA_ERR_INVALID_ARGUMENT
    bad = list(ptrs)
    bad[15] = ptrs[10]  # d_initial_state aliases dq
    assert call(bad) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(ptrs, ws=None) == kda.KDA_ERR_WORKSPACE
    assert call(ptrs, ws_bytes=1000) == kda.KDA_ERR_WORKSPACE
    assert call(ptrs, ws=P(0x100010)) == kda.KDA_ERR_WORKSPACE  # misaligned
    assert call(ptrs, prob=_bwd_problem(head_dim_k=96)) == kda.KDA_ERR_UNSUPPORTED
    assert call(ptrs, prob=_bwd_problem(chunk_size=128)) == kda.KDA_ERR_UNSUPPORTED
    # fp32 at chunk 64 with d = 128 is supported (one record buffer in the reverse scan, dP^T and
    # dL^T gathered in the gradient kernel): its workspace is reported, and a call with a smaller
    # one is refused before anything is launched
    n = ctypes.c_size_t(0)
    p32 = _bwd_problem(io_dtype=kda.KDA_F32)
    assert lib.kda_chunk_bwd_workspace(ctypes.byref(p32), ctypes.byref(n)) == kda.KDA_OK and n.value > 0
    assert call(ptrs, prob=p32, ws_bytes=n.value - 256) == kda.KDA_ERR_WORKSPACE
    # empty batch: nothing to do
    assert call(ptrs, prob=_bwd_problem(batch=0)) == kda.KDA_OK


def test_dplr_validation():
    lib = kda.library()
    P = lambda a: ctypes.c_void_p(a)
    ptrs = [P(0x10000 * (i + 1)) for i in range(6)] + [None, None, None, P(0x90000), None]
    # q k v a b g s0 cu cu_host out sf
    call = lambda prob, pp: lib.kda_dplr_chunk_fwd(ctypes.byref(prob), *pp, None)
    assert call(_bwd_problem(chunk_size=48), ptrs) == kda.KDA_ERR_UNSUPPORTED
    assert call(_bwd_problem(dv_tile=128), ptrs) == kda.KDA_ERR_UNSUPPORTED
    for i, name in [(3, "a"), (4, "b")]:
        bad = list(ptrs)
        bad[i] = None
        assert call(_bwd_problem(), bad) == kda.KDA_ERR_INVALID_ARGUMENT
        assert name in lib.kda_last_error().decode()
    bad = list(ptrs)
    bad[9] = ptrs[3]  # out aliases a
    assert call(_bwd_problem(), bad) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(_bwd_problem(batch=0), ptrs) == kda.KDA_OK


def test_noalloc_refuses_problems_beyond_its_array_on_the_host():
    """kda_chunk_fwd_noalloc validates and sizes the problem before touching the device: NULL problem
    and a workspace beyond its fixed 64 MiB array are refused with a message (no GPU needed)."""
    lib = kda.library()
    assert lib.kda_noalloc_scratch_bytes() == 64 << 20
    P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(6)]  # distinct aligned addresses, never read
    assert lib.kda_chunk_fwd_noalloc(None, *P[:5], None, None, None, P[5], None, None) == \
        kda.KDA_ERR_INVALID_ARGUMENT
    p = kda.Problem(batch=4, seq_len=4096, num_heads=16, head_dim_k=128, head_dim_v=128, num_seqs=0,
                    io_dtype=kda.KDA_BF16, chunk_size=64, scale=1.0, dv_tile=0, algo=0)
    # the arguments are checked first (here: out aliases q), then the size
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(p), *P[:5], None, None, None, P[0], None, None) == \
        kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(p), *P[:5], None, None, None, P[5], None, None) == \
        kda.KDA_ERR_WORKSPACE
    msg = lib.kda_last_error().decode()
    assert "247464448" in msg and str(64 << 20) in msg  # 512 B of plan + 4 x 64 x 16 records of 60,416 B
    p.chunk_size = 48
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(p), *P[:5], None, None, None, P[5], None, None) == \
        kda.KDA_ERR_UNSUPPORTED
    # an empty problem computes nothing and needs no device
    p.chunk_size, p.batch = 64, 0
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None,
                                     None) == kda.KDA_OK
