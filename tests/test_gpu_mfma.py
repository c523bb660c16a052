"""Parity of the matrix-core prefill path (bf16 inputs, fp32 accumulation, head dim 64, chunk 64)
against the fp64 oracle: per-chunk intermediates, end-to-end outputs at small shapes spanning several
tiles and a ragged tail, and sampled rows at the full 760M-class / PaTH-FoX / long-context shapes."""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import assert_parity, errors, fwd_inputs_dev, host, TOL

pytestmark = pytest.mark.gpu

C, D = 64, 64
LOG2E = 1.4426950408889634


def perm_src():
    """Original column held by each stored slot (slot 8g+j of a 32-block holds 16(j/4)+4g+(j%4))."""
    idx = np.zeros(64, dtype=np.int64)
    for p in range(64):
        blk, p32 = divmod(p, 32)
        g, j = divmod(p32, 8)
        idx[p] = 32 * blk + 16 * (j // 4) + 4 * g + (j % 4)
    return idx


PERM = perm_src()


def unpermute_cols(x):
    out = np.empty_like(x)
    out[..., PERM] = x
    return out


def run(x, transport="bf16", chunk=C, keep_ws=False):
    t = fwd_inputs_dev(x)
    B, H, L, d = x.q.shape
    n = native.path_attn_fwd_workspace_bytes(B, H, L, d, chunk, torch.bfloat16, transport)
    ws = torch.zeros(max(n, 16), device="cuda", dtype=torch.uint8)
    out, lse = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale,
                                    chunk=chunk, transport=transport, workspace=ws)
    torch.cuda.synchronize()
    if keep_ws:
        return host(out), host(lse), ws
    return host(out), host(lse)


S_CHUNK = 2176  # floats of one chunk's packed in-chunk logits (matrix-core layouts)


def unpack_s(flat, BH, M):
    """The packed lower-triangle S of the matrix-core layouts as [BH, M, C, C] (zeros where nothing is
    stored): row a of a chunk holds columns 0 .. 4 floor(a/4) + 3 from float 4 (a + 2u(u-1) + uv),
    u = floor(a/4), v = a mod 4."""
    flat = np.asarray(flat).reshape(BH, M, S_CHUNK)
    out = np.zeros((BH, M, C, C))
    for a in range(C):
        u, v = divmod(a, 4)
        start, n = 4 * (a + 2 * u * (u - 1) + u * v), 4 * (u + 1)
        out[:, :, a, :n] = flat[:, :, start:start + n]
    return out


def ws_view(ws, off, count, dtype):
    b = ws[off:off + count * (2 if dtype == torch.bfloat16 else 4)]
    return b.view(dtype).float().cpu().numpy().astype(np.float64)


def test_layout_is_matrix_core():
    lay = native.path_attn_workspace_layout(1, 1, 128, D, C, torch.bfloat16, "bf16x3")
    assert lay.layout_id == 1 and lay.off_qtilde_lo >= 0 and lay.off_p_lo >= 0


def _worst(got, want, bound):
    """Largest |got - want| / bound over the elements (<= 1 passes)."""
    return float(np.max(np.abs(np.asarray(got) - np.asarray(want)) / bound))


@pytest.mark.parametrize("transport", ["bf16", "bf16x3"])
@pytest.mark.parametrize("recipe", ["stress_qk", "beta2", "lm"])
def test_chunk_intermediates(recipe, transport):
    """qtilde, ktilde, P and the in-chunk logits S of every chunk against the oracle's by-definition terms
    (the workspace holds qtilde and S multiplied by scale * log2(e)), element by element.  Bounds:
    a value stored in bf16 is within half an ulp of the value the kernel formed, i.e. within the bf16
    unit roundoff 2^-8 relative, and the formed value is within 2^-14 of the largest entry (fp32
    accumulation of products whose non-input operand is carried as bf16 hi + lo, lo*lo dropped); with
    bf16x3 transport qtilde and P are stored as hi + lo and keep that 2^-14.  S is stored in fp32: its
    error is that of fp32 sums of 64 products (2^-18 |q_a| |k_b|) and of the hi + lo products with lo*lo
    dropped (2^-16 relative per product), bounded by 2^-14 |q_a| |k_b| in logit units."""
    B, H, L = 1, 2, 150
    x = synth.make_fwd_inputs(B, H, L, D, recipe=recipe, dtype="bf16", seed=11)
    print(f"[case] intermediates recipe={recipe} transport={transport}", flush=True)
    _, _, ws = run(x, transport, keep_ws=True)
    x3 = transport == "bf16x3"
    lay = native.path_attn_workspace_layout(B, H, L, D, C, torch.bfloat16, transport)
    M = lay.num_chunks
    Lp = M * C
    qt = ws_view(ws, lay.off_qtilde, B * H * Lp * D, torch.bfloat16)
    ph = ws_view(ws, lay.off_p, B * H * M * D * D, torch.bfloat16)
    if x3:
        qt = qt + ws_view(ws, lay.off_qtilde_lo, B * H * Lp * D, torch.bfloat16)
        ph = ph + ws_view(ws, lay.off_p_lo, B * H * M * D * D, torch.bfloat16)
    else:
        assert lay.off_qtilde_lo < 0 and lay.off_p_lo < 0
    qt = unpermute_cols(qt.reshape(B * H, Lp, D))
    P = unpermute_cols(ph.reshape(B * H, M, D, D))
    kt = unpermute_cols(ws_view(ws, lay.off_ktilde, B * H * Lp * D, torch.bfloat16).reshape(B * H, Lp, D))
    S = unpack_s(ws_view(ws, lay.off_s, B * H * M * S_CHUNK, torch.float32), B * H, M)
    store = 0.0 if x3 else 2.0 ** -8  # relative rounding of the stored qtilde and P (bf16 unit roundoff)
    worst = dict(q=0.0, k=0.0, p=0.0, s=0.0)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for c in range(M):
            rows = slice(c * C, min((c + 1) * C, L))
            n = rows.stop - rows.start
            q, k, w = (getattr(x, a)[b, h, rows].astype(np.float64) for a in ("q", "k", "w"))
            beta = x.beta[b, h, rows].astype(np.float64)
            rq, rk, rs = oracle.chunk_terms(q, k, w, beta)
            u = x.scale * LOG2E
            rq, rs = rq * u, rs * u
            worst["q"] = max(worst["q"], _worst(qt[bh, c * C:c * C + n], rq,
                                                store * np.abs(rq) + 2.0 ** -14 * np.abs(rq).max()))
            worst["k"] = max(worst["k"], _worst(kt[bh, c * C:c * C + n], rk,
                                                2.0 ** -8 * np.abs(rk) + 2.0 ** -14 * np.abs(rk).max()))
            # the padded tail of a ragged chunk holds identity transitions
            rp = oracle.householder_product(w, beta)
            worst["p"] = max(worst["p"], _worst(P[bh, c], rp, store * np.abs(rp) + 2e-5))
            nq = np.linalg.norm(q, axis=1)
            nk = np.linalg.norm(k, axis=1)
            sb = 2.0 ** -14 * np.outer(nq, nk) * u + 1e-30
            worst["s"] = max(worst["s"], _worst(np.tril(S[bh, c, :n, :n]), np.tril(rs), sb))
    print(f"[intermediates] {recipe} {transport}: worst error / bound " +
          ", ".join(f"{k} {v:.3f}" for k, v in worst.items()), flush=True)
    for key, v in worst.items():
        assert v <= 1.0, f"{key}: error {v:.3f} x its bound"


CASES = [
    (2, 3, 64, "lm", "bf16"), (2, 3, 100, "stress_qk", "bf16"), (1, 2, 256, "beta2", "bf16"),
    (1, 2, 700, "beta02", "bf16"), (2, 2, 1000, "stress_qk", "bf16x3"), (1, 3, 1, "lm", "bf16"),
    (1, 2, 65, "fox", "bf16"), (2, 2, 777, "fox", "bf16x3"), (1, 2, 513, "stress_qk_beta2", "bf16x3"),
    (1, 1, 300, "beta0", "bf16"),
]


@pytest.mark.parametrize("B,H,L,recipe,transport", CASES)
def test_small_shapes(B, H, L, recipe, transport):
    x = synth.make_fwd_inputs(B, H, L, D, recipe=recipe, dtype="bf16", seed=L)
    print(f"[case] mfma B={B} H={H} L={L} recipe={recipe} transport={transport}", flush=True)
    go, gl = run(x, transport)
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale)
    assert_parity(go, ro, "bf16", "out")
    assert_parity(gl, rl, "bf16", "lse")


CASES_128 = [
    (1, 2, 128, "lm", "bf16"), (2, 2, 300, "stress_qk", "bf16"), (1, 3, 64, "lm", "bf16"),
    (1, 2, 700, "fox", "bf16x3"), (1, 3, 1000, "beta2", "bf16"), (1, 2, 513, "stress_qk_beta2", "bf16x3"),
    (2, 2, 900, "fox", "bf16"),
]


@pytest.mark.parametrize("chunk", [128, 256])
@pytest.mark.parametrize("B,H,L,recipe,transport", CASES_128)
def test_small_shapes_grouped_chunks(B, H, L, recipe, transport, chunk):
    """128- and 256-token chunks: the scan moves queries once per chunk (keys carried to the chunk top)."""
    x = synth.make_fwd_inputs(B, H, L, D, recipe=recipe, dtype="bf16", seed=L + 1)
    print(f"[case] mfma chunk {chunk} B={B} H={H} L={L} recipe={recipe} transport={transport}", flush=True)
    go, gl = run(x, transport, chunk=chunk)
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale)
    assert_parity(go, ro, "bf16", "out")
    assert_parity(gl, rl, "bf16", "lse")


@pytest.mark.parametrize("L,expect", [(777, 64), (4096, 64), (4097, 256), (32768, 256)])
def test_chunk_zero_follows_the_measured_table(L, expect):
    """The automatic chunk on the matrix-core path is the one the chunk sweep measured fastest: 64 up to
    4096 tokens (the 760M-class length included), 256 beyond (the long-context length 32768 included):
    bit-identical outputs to that chunk."""
    x = synth.make_fwd_inputs(1, 2 if L <= 4096 else 1, L, D, recipe="fox", dtype="bf16", seed=6)
    print(f"[case] chunk 0 at L={L} (expect {expect})", flush=True)
    a_out, a_lse = run(x, "bf16", chunk=0)
    b_out, b_lse = run(x, "bf16", chunk=expect)
    assert np.array_equal(a_out, b_out) and np.array_equal(a_lse, b_lse)


@pytest.mark.parametrize("transport,chunk", [("bf16", 128), ("bf16x3", 128), ("bf16", 256), ("bf16x3", 256)])
def test_grouped_chunk_terms(transport, chunk):
    """P over each whole chunk and every sub-chunk's keys carried to its chunk's top, against the oracle's
    explicit products / by-definition keys over the chunk's tokens."""
    G = chunk // 64
    B, H, L = 1, 2, 576  # 9 sub-chunks: whole chunks of 128 (4) or 256 (2) and a ragged rest
    x = synth.make_fwd_inputs(B, H, L, D, recipe="beta2", dtype="bf16", seed=3)
    _, _, ws = run(x, transport, chunk=chunk, keep_ws=True)
    lay = native.path_attn_workspace_layout(B, H, L, D, chunk, torch.bfloat16, transport)
    M = lay.num_sub_chunks
    MG = M // G
    assert lay.layout_id == 2 and M == 9
    ph = ws_view(ws, lay.off_p_c2, B * H * MG * D * D, torch.bfloat16).reshape(B * H, MG, D, D)
    if transport == "bf16x3":
        ph = ph + ws_view(ws, lay.off_p_c2_lo, B * H * MG * D * D, torch.bfloat16).reshape(B * H, MG, D, D)
    PG = unpermute_cols(ph)
    KC = unpermute_cols(ws_view(ws, lay.off_ktilde_c2, B * H * M * 64 * D, torch.bfloat16).reshape(B * H, M, 64, D))
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for c in range(MG):
            rows = slice(chunk * c, chunk * c + chunk)
            q, k, w = (getattr(x, a)[b, h, rows].astype(np.float64) for a in ("q", "k", "w"))
            beta = x.beta[b, h, rows].astype(np.float64)
            rp = oracle.householder_product(w, beta)
            ma, _ = errors(PG[bh, c], rp)
            assert ma <= (2e-5 if transport == "bf16x3" else 2e-2), f"P over {chunk} tokens, chunk {c}: {ma:.2e}"
            _, rk, _ = oracle.chunk_terms(q, k, w, beta)  # keys carried to the end of the chunk's tokens
            for j in range(G - 1):  # every sub-chunk but the top one
                want = rk[64 * j:64 * j + 64]
                got = KC[bh, G * c + j]
                assert errors(got, want)[0] <= 2 ** -6 * max(1.0, np.abs(want).max()), f"carried keys {c}/{j}"


@pytest.mark.parametrize("transport,fox", [("bf16", False), ("bf16x3", True)])
def test_prep_then_scan_equals_fwd(transport, fox):
    """path_attn_prep followed by path_attn_scan is bit-identical to path_attn_fwd."""
    x = synth.make_fwd_inputs(2, 2, 333, D, recipe="fox" if fox else "lm", dtype="bf16", seed=8)
    t = fwd_inputs_dev(x)
    n = native.path_attn_fwd_workspace_bytes(2, 2, 333, D, C, torch.bfloat16, transport)
    ws = torch.zeros(n, device="cuda", dtype=torch.uint8)
    o1, l1 = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale, chunk=C,
                                  transport=transport, workspace=ws)
    ws2 = torch.zeros(n, device="cuda", dtype=torch.uint8)
    native.path_attn_prep(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale, chunk=C,
                          transport=transport, workspace=ws2)
    o2, l2 = native.path_attn_scan(t["v"], t["logf"], chunk=C, transport=transport, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_negative_control_plain_attention_fails():
    x = synth.make_fwd_inputs(1, 2, 512, D, recipe="stress_qk", dtype="bf16", seed=4)
    ro, _ = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, scale=x.scale)
    plain = synth.FwdInputs(**{**x.__dict__, "beta": np.zeros_like(x.beta)})
    go, _ = run(plain)
    ma, rel = errors(go, ro)
    assert ma > TOL["bf16"]["max_abs"] and rel > TOL["bf16"]["rel_l2"]


def sampled_rows(L, seed=0):
    rng = np.random.default_rng(seed)
    blocks = [np.arange(0, 64), np.arange(L - 64, L)]
    for s in rng.choice(np.arange(1, L // 64 - 1), size=4, replace=False):
        blocks.append(np.arange(64 * s, 64 * s + 64))
    return np.unique(np.concatenate(blocks))


@pytest.mark.parametrize("B,H,L,recipe,transport,chunk", [
    (8, 24, 4096, "lm", "bf16", C),         # 760M-class layer
    (8, 24, 4096, "fox", "bf16", C),        # PaTH-FoX at the same shape
    (8, 24, 4096, "stress_qk", "bf16", C),  # S1 at full shape
    (1, 24, 32768, "lm", "bf16", C),        # long-context extrapolation shape, the benchmarked transport
    (1, 24, 32768, "lm", "bf16", 128),      # ... and its 128-token chunks
    (1, 24, 32768, "lm", "bf16x3", C),
    (1, 24, 32768, "stress_qk_beta2", "bf16x3", C),  # S1+S2: norm-preserving long-range transport
    (1, 24, 32768, "lm", "bf16x3", 128),    # long context, 128-token chunks
    (1, 24, 32768, "stress_qk_beta2", "bf16x3", 128),
    (8, 24, 4096, "stress_qk", "bf16", 128),
    (8, 24, 4096, "lm", "bf16", 256),       # 256-token chunks
    (1, 24, 32768, "stress_qk_beta2", "bf16x3", 256),
])
def test_full_size_sampled_rows(B, H, L, recipe, transport, chunk):
    print(f"[case] full B={B} H={H} L={L} recipe={recipe} transport={transport} chunk={chunk}", flush=True)
    x = synth.make_fwd_inputs(B, H, L, D, recipe=recipe, dtype="bf16", seed=0)
    go, gl = run(x, transport, chunk=chunk)
    rows = sampled_rows(L)
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale, rows=rows)
    assert_parity(go[:, :, rows], ro, "bf16", "out")
    assert_parity(gl[:, :, rows], rl, "bf16", "lse")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))


def test_long_context_transport_precision():
    """Norm-preserving transport over 512 chunks (S1 + S2 at L = 32768, sampled rows): bf16x3 meets the
    bf16 tolerance; plain bf16 transport re-rounds the running queries at each of the 511 chunk steps
    (a random walk of 2^-9 relative per step), so its error is recorded and must not beat bf16x3's."""
    B, H, L = 1, 24, 32768
    x = synth.make_fwd_inputs(B, H, L, D, recipe="stress_qk_beta2", dtype="bf16", seed=0)
    rows = sampled_rows(L)
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, scale=x.scale, rows=rows)
    res, outs = {}, {}
    for transport in ("bf16x3", "bf16"):
        print(f"[case] long-context transport precision, transport={transport}", flush=True)
        go, gl = run(x, transport)
        outs[transport] = go[:, :, rows], gl[:, :, rows]
        res[transport] = errors(outs[transport][0], ro), errors(outs[transport][1], rl)
        print(f"[long] transport {transport}: out max_abs {res[transport][0][0]:.3e} rel_l2 {res[transport][0][1]:.3e};"
              f" lse max_abs {res[transport][1][0]:.3e} rel_l2 {res[transport][1][1]:.3e}", flush=True)
    assert_parity(outs["bf16x3"][0], ro, "bf16", "out (bf16x3)")
    assert_parity(outs["bf16x3"][1], rl, "bf16", "lse (bf16x3)")
    assert res["bf16x3"][0][1] <= res["bf16"][0][1], "bf16x3 transport must not be less accurate than bf16"
