"""Host-side checks of the C ABI (no GPU needed): exports, workspace planning, validation codes.

Every call here fails validation (or is a pure host query) before anything is enqueued, so it
runs on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

from dependent_positional_attention_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "path_attn.h")

OK, INVALID, UNSUPPORTED = native.PATH_OK, native.PATH_ERR_INVALID_ARG, native.PATH_ERR_UNSUPPORTED
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:path_status|int|const char\*|size_t)\s+(path_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    return native.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(L, n), f"{n} declared in path_attn.h but not exported"
    assert set(names) == set(native.EXPORTS)


def test_version_and_strings(L):
    assert L.path_abi_version() == 9
    for s in range(5):
        assert L.path_status_string(s)
    assert L.path_status_string(99) == b"unknown status"


def ws_bytes(L, *args):
    n = ctypes.c_size_t(0)
    st = L.path_attn_fwd_workspace_bytes(*args, ctypes.byref(n))
    return st, n.value


def test_workspace_planning(L):
    st, n = ws_bytes(L, 8, 24, 4096, 64, 64, BF16, 0)
    assert st == OK and n > 8 * 24 * 4096 * 64 * 2 * 3
    st, n0 = ws_bytes(L, 1, 1, 0, 16, 16, F32, 0)
    assert st == OK
    assert ws_bytes(L, 1, 1, 64, 48, 16, F32, 0)[0] == UNSUPPORTED  # head dim not built
    assert ws_bytes(L, 1, 1, 64, 16, 24, F32, 0)[0] == UNSUPPORTED  # chunk not built
    assert ws_bytes(L, 1, 1, 64, 16, 16, 7, 0)[0] == UNSUPPORTED  # dtype
    assert ws_bytes(L, -1, 1, 64, 16, 16, F32, 0)[0] == INVALID
    assert ws_bytes(L, 1, 1, 64, 16, 16, F32, 5)[0] == INVALID  # transport
    lay = native.WsLayout()
    assert L.path_attn_workspace_layout(2, 3, 100, 16, 16, F32, 0, ctypes.byref(lay)) == OK
    assert lay.num_chunks == 7 and lay.layout_id == 0 and lay.off_p_lo == -1 and lay.off_qtilde_lo == -1
    offs = [lay.off_qtilde, lay.off_ktilde, lay.off_p, lay.off_s, lay.off_fox_local, lay.off_fox_total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and lay.total_bytes >= offs[-1]
    assert lay.num_sub_chunks == 7 and lay.off_ktilde_c2 == lay.off_p_c2 == lay.off_p_c2_lo == -1


@pytest.mark.parametrize("chunk,groups", [(128, 2), (256, 1)])
def test_workspace_planning_grouped_chunks(L, chunk, groups):
    """Chunks of 128 / 256 on the matrix-core path: 64-token sub-chunks plus carried keys for every
    sub-chunk and the products of whole chunks."""
    for transport in (0, 1):
        lay = native.WsLayout()
        assert L.path_attn_workspace_layout(2, 3, 300, 64, chunk, BF16, transport, ctypes.byref(lay)) == OK
        assert lay.layout_id == 2 and lay.num_chunks == -(-300 // chunk) and lay.num_sub_chunks == 5
        assert lay.off_ktilde_c2 >= 0 and lay.off_p_c2 >= 0 and (lay.off_p_c2_lo >= 0) == (transport == 1)
        sizes = {lay.off_ktilde_c2: 6 * 5 * 64 * 64 * 2, lay.off_p_c2: 6 * groups * 64 * 64 * 2}
        for o, n in sizes.items():
            assert o % 256 == 0 and o + n <= lay.total_bytes
        st, n1 = ws_bytes(L, 2, 3, 300, 64, chunk, BF16, transport)
        assert st == OK and n1 == lay.total_bytes
    assert ws_bytes(L, 1, 1, 300, 64, chunk, F32, 0)[0] == UNSUPPORTED  # fp32 has no grouped chunks
    assert ws_bytes(L, 1, 1, 300, 32, chunk, BF16, 0)[0] == UNSUPPORTED
    assert ws_bytes(L, 1, 1, 300, 64, 512, BF16, 0)[0] == UNSUPPORTED


def test_packed_in_chunk_logits_region(L):
    """The matrix-core layouts keep the in-chunk logits S as a packed lower triangle of 4-float groups:
    sum over rows a = 0..63 of (floor(a/4) + 1) groups = 544 groups = 2176 floats per 64-token chunk
    (the vector path keeps the full C x C square)."""
    groups = sum(a // 4 + 1 for a in range(64))
    assert groups == 544
    for chunk in (64, 128):
        lay = native.WsLayout()
        assert L.path_attn_workspace_layout(2, 3, 300, 64, chunk, BF16, 0, ctypes.byref(lay)) == OK
        M = lay.num_sub_chunks
        assert lay.off_fox_local - lay.off_s == -(-(6 * M * groups * 16) // 256) * 256
    assert L.path_attn_workspace_layout(2, 3, 100, 16, 16, F32, 0, ctypes.byref(lay)) == OK
    assert lay.off_fox_local - lay.off_s == -(-(6 * 7 * 16 * 16 * 4) // 256) * 256


def test_chunk_zero_selects_the_fastest_chunk(L):
    """chunk 0 plans exactly what the measured table picks: chunk 256 on the matrix-core path beyond 4096
    tokens, chunk 64 up to 4096 tokens and on the vector path."""
    for args, chunk, dtype in (((2, 3, 5000, 64), 256, BF16), ((2, 3, 1000, 64), 64, BF16), ((1, 2, 100, 16), 64, F32)):
        for transport in (0, 1):
            a, b = native.WsLayout(), native.WsLayout()
            assert L.path_attn_workspace_layout(*args, 0, dtype, transport, ctypes.byref(a)) == OK
            assert L.path_attn_workspace_layout(*args, chunk, dtype, transport, ctypes.byref(b)) == OK
            assert bytes(a) == bytes(b)
    assert ws_bytes(L, 1, 1, 64, 64, -1, BF16, 0)[0] == INVALID


def fwd(L, q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=None, B=1, H=1, Lq=64, d=16,
        chunk=16, scale=0.25, dtype=F32, transport=0, ws=FAKE, ws_n=1 << 30):
    return L.path_attn_fwd(q, k, v, w, beta, logf, out, lse, B, H, Lq, d, chunk, scale, dtype, transport, ws, ws_n,
                           None)


def test_fwd_validation(L):
    assert fwd(L, q=None) == INVALID
    assert fwd(L, out=None) == INVALID
    assert fwd(L, ws=None) == INVALID
    assert fwd(L, beta=None) == INVALID
    assert fwd(L, ws_n=100) == INVALID  # workspace too small
    assert fwd(L, d=48) == UNSUPPORTED
    assert fwd(L, chunk=8) == UNSUPPORTED
    assert fwd(L, dtype=3) == UNSUPPORTED
    assert fwd(L, q=MISALIGNED) == UNSUPPORTED
    assert fwd(L, lse=MISALIGNED) == UNSUPPORTED
    assert fwd(L, B=-1) == INVALID
    # empty problems are valid and enqueue nothing, even with null tensors
    assert fwd(L, Lq=0, q=None, k=None, out=None, ws=None) == OK
    assert fwd(L, B=0, q=None, ws=None) == OK


def dec(L, kc=FAKE, vc=FAKE, fc=None, cap=128, t=10, tb=None, q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, f=None,
        out=FAKE, lse=None, B=1, H=1, d=64, scale=0.125, dtype=BF16, splits=0, ws=FAKE, ws_n=1 << 20):
    return L.path_decode_step(kc, vc, fc, cap, t, tb, q, k, v, w, beta, f, out, lse, B, H, d, scale, dtype, splits, ws,
                              ws_n, None)


def test_decode_validation(L):
    assert dec(L, t=128) == INVALID  # t >= capacity
    assert dec(L, t=-1) == INVALID
    assert dec(L, kc=None) == INVALID
    assert dec(L, w=None) == INVALID
    assert dec(L, d=48) == UNSUPPORTED
    assert dec(L, dtype=9) == UNSUPPORTED
    assert dec(L, vc=MISALIGNED) == UNSUPPORTED
    assert dec(L, ws_n=16) == INVALID
    assert dec(L, splits=-2) == INVALID
    assert dec(L, fc=FAKE) == INVALID  # FoX slot biases without the gate
    assert dec(L, f=FAKE) == INVALID  # gate without slot biases
    assert dec(L, fc=MISALIGNED, f=FAKE) == UNSUPPORTED
    assert dec(L, tb=MISALIGNED) == UNSUPPORTED
    assert dec(L, B=0, kc=None) == OK
    n = ctypes.c_size_t(0)
    assert L.path_decode_workspace_bytes(32, 24, 64, 65536 + 128, 0, ctypes.byref(n)) == OK
    assert n.value == 32 * 24 * 65 * 66 * 4
    assert L.path_decode_workspace_bytes(1, 1, 48, 100, 0, ctypes.byref(n)) == UNSUPPORTED


def handoff(L, v=FAKE, lf=None, ws=FAKE, ws_n=1 << 40, kc=FAKE, vc=FAKE, fc=None, cap=4096, B=1, H=2, Lq=4096, d=64,
            chunk=64, dtype=BF16, transport=0):
    return L.path_attn_cache_from_prefill(v, lf, ws, ws_n, kc, vc, fc, cap, B, H, Lq, d, chunk, dtype, transport,
                                          None)


def test_cache_handoff_validation(L):
    assert handoff(L, cap=4095) == INVALID  # capacity below the prompt length
    assert handoff(L, v=None) == INVALID
    assert handoff(L, kc=None) == INVALID
    assert handoff(L, ws=None) == INVALID
    assert handoff(L, ws_n=1024) == INVALID  # workspace smaller than the prefill plan
    assert handoff(L, vc=MISALIGNED) == UNSUPPORTED
    assert handoff(L, d=48) == UNSUPPORTED
    assert handoff(L, chunk=8) == UNSUPPORTED
    assert handoff(L, transport=5) == INVALID
    assert handoff(L, B=-1) == INVALID
    assert handoff(L, lf=FAKE) == INVALID  # FoX gates without a slot-bias output
    assert handoff(L, fc=FAKE) == INVALID
    assert handoff(L, lf=FAKE, fc=MISALIGNED) == UNSUPPORTED
    # an empty prompt or batch is valid and enqueues nothing
    assert handoff(L, Lq=0, v=None, ws=None, kc=None, vc=None) == OK
    assert handoff(L, H=0, v=None) == OK


def deferred(L, kc=FAKE, vc=FAKE, fc=None, cap=128, t=10, t_cur=8, period=4, state=FAKE, state_n=1 << 20, q=FAKE,
             k=FAKE, v=FAKE, w=FAKE, beta=FAKE, f=None, out=FAKE, lse=None, B=1, H=1, d=64, dtype=BF16, splits=0,
             ws=FAKE, ws_n=1 << 20):
    return L.path_decode_step_deferred(kc, vc, fc, cap, t, t_cur, period, state, state_n, q, k, v, w, beta, f, out, lse,
                                       B, H, d, 0.125, dtype, splits, ws, ws_n, None)


def test_deferred_decode_validation(L):
    assert deferred(L, period=0) == INVALID
    assert deferred(L, period=17) == INVALID
    assert deferred(L, t_cur=11) == INVALID  # t_cur > t
    assert deferred(L, t_cur=6, period=4) == INVALID  # 4 waiting steps exceed the period
    assert deferred(L, t=128) == INVALID
    assert deferred(L, state=None) == INVALID
    assert deferred(L, state_n=64) == INVALID
    assert deferred(L, fc=FAKE) == INVALID
    assert deferred(L, state=MISALIGNED) == UNSUPPORTED
    assert deferred(L, d=48) == UNSUPPORTED
    assert deferred(L, B=0, kc=None) == OK
    n = ctypes.c_size_t(0)
    assert L.path_decode_deferred_state_bytes(32, 24, 64, ctypes.byref(n)) == OK
    assert n.value == 32 * 24 * 16 * 66 * 4


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        native.path_attn_fwd(x, x, x, x, torch.zeros(1, 1, 4))


def bwd_call(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE,
             dv=FAKE, dw=FAKE, dbeta=FAKE, dlogf=None, B=1, H=2, Lq=100, d=16, chunk=16, scale=0.25, dt=F32, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.path_attn_bwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"], a["out"], a["lse"], a["dout"],
                           a["dq"], a["dk"], a["dv"], a["dw"], a["dbeta"], a["dlogf"], a["B"], a["H"], a["Lq"],
                           a["d"], a["chunk"], ctypes.c_float(a["scale"]), a["dt"], a["ws"], a["ws_bytes"],
                           a["stream"])


def test_bwd_workspace_planning(L):
    n = ctypes.c_size_t(0)
    assert L.path_attn_bwd_workspace_bytes(8, 24, 4096, 64, 64, BF16, ctypes.byref(n)) == OK
    # states and their gradients of one band of query chunks at a time (bf16 for a bf16 input): 64 chunks
    # in bands of 4 ceil(sqrt(64)) = 32, the largest band (chunks 32 .. 63) holding 32 + ... + 63 pairs
    pairs = sum(range(32, 64))
    assert n.value >= 2 * 8 * 24 * pairs * 64 * 64 * 2
    assert n.value < 2 * 8 * 24 * pairs * 64 * 64 * 2 + (2 << 30)
    nf = ctypes.c_size_t(0)
    assert L.path_attn_bwd_workspace_bytes(8, 24, 4096, 64, 64, F32, ctypes.byref(nf)) == OK
    # an fp32 input: fp32 states, qtilde and ktilde [BH, L, 64], P [BH, 64 chunks, 64, 64] and the full
    # square of in-chunk logits (a bf16 input keeps 544 4-float groups per chunk), and no stored A^{-1}
    # per chunk (64 x 64 fp32 for each of the 64 chunks)
    BH, chunks = 8 * 24, 64
    assert nf.value - n.value == (2 * BH * pairs * 64 * 64 * 2 + 2 * BH * 4096 * 64 * 2 + BH * chunks * 64 * 64 * 2
                                  + BH * chunks * (64 * 64 - 544 * 4) * 4 - BH * chunks * 64 * 64 * 4)
    n0 = ctypes.c_size_t(0)
    assert L.path_attn_bwd_workspace_bytes(8, 24, 4096, 64, 0, BF16, ctypes.byref(n0)) == OK
    assert n0.value == n.value  # chunk 0 = 64
    assert L.path_attn_bwd_workspace_bytes(1, 1, 64, 64, 128, BF16, ctypes.byref(n)) == UNSUPPORTED
    assert L.path_attn_bwd_workspace_bytes(1, 1, 64, 48, 64, F32, ctypes.byref(n)) == UNSUPPORTED
    assert L.path_attn_bwd_workspace_bytes(1, 1, 64, 64, 64, 9, ctypes.byref(n)) == UNSUPPORTED
    assert L.path_attn_bwd_workspace_bytes(1, -1, 64, 64, 64, F32, ctypes.byref(n)) == INVALID
    assert L.path_attn_bwd_workspace_bytes(1, 1, 64, 64, 64, F32, None) == INVALID
    assert L.path_attn_bwd_workspace_bytes(1, 1, 64, 16, 16, F32, ctypes.byref(n)) == OK  # one chunk... of 4
    assert L.path_attn_bwd_workspace_bytes(1, 1, 16, 16, 16, F32, ctypes.byref(n)) == OK and n.value > 0


def test_bwd_workspace_grows_as_l_sqrt_l(L):
    """The backward keeps per-pair states for one band of about sqrt(M) query chunks at a time, so its
    workspace grows as L^1.5 (a factor 8 per factor 4 in L), not as L^2 (a factor 16)."""
    def size(Lq, B=1, H=1):
        n = ctypes.c_size_t(0)
        assert L.path_attn_bwd_workspace_bytes(B, H, Lq, 64, 64, BF16, ctypes.byref(n)) == OK
        return n.value
    for Lq in (4096, 16384):
        assert size(4 * Lq) <= 8.5 * size(Lq), Lq
    assert size(32768, 1, 24) < 18e9  # long-context shape: 24 heads of 32768 tokens


def test_bwd_validation(L):
    assert bwd_call(L, q=None) == INVALID
    assert bwd_call(L, lse=None) == INVALID  # the backward needs the forward's lse
    assert bwd_call(L, dbeta=None) == INVALID
    assert bwd_call(L, logf=FAKE) == INVALID  # dlog_forget missing
    assert bwd_call(L, dlogf=FAKE) == INVALID  # dlog_forget without log_forget
    assert bwd_call(L, ws_bytes=16) == INVALID
    assert bwd_call(L, dq=MISALIGNED) == UNSUPPORTED
    assert bwd_call(L, d=48) == UNSUPPORTED
    assert bwd_call(L, chunk=128) == UNSUPPORTED
    assert bwd_call(L, dt=3) == UNSUPPORTED
    assert bwd_call(L, Lq=-1) == INVALID
    assert bwd_call(L, Lq=0, q=None) == OK  # empty: nothing to do
    assert bwd_call(L, B=0) == OK


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N with N > 1 exits (status 2) with a message, before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "ONE MI355X" in r.stderr and "not supported" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("L,layout_id", [(64, 1), (4096, 1), (4097, 2), (8192, 2), (32768, 2)])
def test_automatic_chunk_table(L, layout_id):
    """chunk = 0 on the matrix-core path (bf16, d = 64): 64-token chunks (layout 1) up to 4096 tokens,
    256-token chunks (layout 2, four sub-chunks per chunk) beyond, as measured fastest; the vector path
    (fp32) takes 64."""
    lay = native.WsLayout()
    lib = native.lib()
    assert lib.path_attn_workspace_layout(1, 2, L, 64, 0, BF16, 0, ctypes.byref(lay)) == OK
    assert lay.layout_id == layout_id
    if layout_id == 2:
        assert lay.num_chunks == -(-L // 256) and lay.num_sub_chunks == -(-L // 64)
    assert lib.path_attn_workspace_layout(1, 2, L, 64, 0, F32, 0, ctypes.byref(lay)) == OK
    assert lay.layout_id == 0 and lay.num_chunks == -(-L // 64)
