"""Pins for the fp64 oracle: each one ties it to the pages or to mathematics, not to itself.

Citations are to the PaTH summary (gist.science/ko/paper/2505.16381, "summary" below)
and the lecture notes on PaTH (brianyu43.github.io/gpumode/lecture_074.html, "notes").

P0  golden      hand-worked 3-token example (tests/golden/hand_example_d2.json)
P1  beta = 0    every H is I: plain causal softmax attention (textbook numpy)
P2  brute force explicit d x d products H_{j+1}...H_i on tiny inputs (summary, section 2)
P3  invariants  beta = 2 with unit w keeps norms (notes, "idea": H is orthogonal); 0<beta<2 never grows them
P4  UT identity H_0...H_{n-1} = I - W^T T^{-1} W, on sub-ranges and n > d (summary, section 3)
P5  beta = 2    absolute form: logits = (A_j k_j).(A_i q_i) with A_i = H_0...H_i (notes, "idea")
P6  det         det(H_0...H_{n-1}) = prod_s (1 - beta_s |w_s|^2)
P7  chunked     boundary-adjusted rows + right-to-left chunk scan reproduce the oracle (summary, section 3)
P8  special     row 0, constant values, f = 0, closed-form FoX bias with beta = 0
P9  decode      in-place key updates (summary, section 3 "inference") == prefill rows; PaTH-FoX decode
                (per-slot forget bias grown in place) == FoX prefill rows and the beta = 0 closed form
P10 mutations   plausible mistakes planted in a copy of the oracle make the pins fail
P11 cache       key cache after a prompt (summary, section 3 "inference"): explicit products,
                last-row logits, the decode recurrence, norms under beta = 2
P12 backward    gradients of every input (q, k, v, w, beta, f) against central finite differences of
                the pinned forward, against torch autograd through explicit d x d products, and for
                beta = 0 against the gradient of plain causal attention; planted mistakes are caught
"""
import ctypes
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest

from dependent_positional_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- numpy references

def H(w, beta):
    w = np.asarray(w, dtype=np.float64)
    return np.eye(len(w)) - beta * np.outer(w, w)


def brute_logits(q, k, w, beta, scale, logf=None):
    """z[i, j] = scale * k_j^T H_{j+1} ... H_i q_i (+ sum_{s=j+1..i} f_s), -inf above the diagonal."""
    L, d = q.shape
    z = np.full((L, L), -np.inf)
    for j in range(L):
        M = np.eye(d)
        bias = 0.0
        for i in range(j, L):
            if i > j:
                M = M @ H(w[i], beta[i])
                if logf is not None:
                    bias += logf[i]
            z[i, j] = scale * (k[j] @ M @ q[i]) + bias
    return z


def softmax_attend(z, v):
    m = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    return (p / l) @ v, (m + np.log(l))[:, 0]


def plain_causal_attention(q, k, v, scale, bias=None):
    L = q.shape[0]
    z = scale * (q @ k.T)
    if bias is not None:
        z = z + bias
    z[np.triu_indices(L, 1)] = -np.inf
    return softmax_attend(z, v)


def rand_problem(L, d, seed, beta_mode="sigmoid", fox=False, unit=True):
    r = np.random.default_rng(seed)
    q, k, v = r.standard_normal((3, L, d))
    w = r.standard_normal((L, d))
    if unit:
        w /= np.linalg.norm(w, axis=1, keepdims=True)
    if beta_mode == "sigmoid":
        beta = 2.0 / (1.0 + np.exp(-1.5 * r.standard_normal(L)))
    elif beta_mode == "two":
        beta = np.full(L, 2.0)
    elif beta_mode == "zero":
        beta = np.zeros(L)
    else:
        raise ValueError(beta_mode)
    logf = -np.log1p(np.exp(-(3.0 + r.standard_normal(L)))) if fox else None
    return q, k, v, w, beta, logf


def assert_close(a, b, tol, what=""):
    err = np.max(np.abs(np.asarray(a) - np.asarray(b)))
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- P0

def test_p0_golden_hand_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_example_d2.json")))
    q, k, v, w = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "w"))
    beta, logf = np.array(g["beta"]), np.array(g["logf"])
    for fox, key in ((None, "logits"), (logf, "logits_fox")):
        for i in range(3):
            z = oracle_lib.row_logits(q[i], k, w, beta, i, logf=fox, scale=g["scale"])
            assert_close(z, g[key][i], 1e-14, f"{key} row {i}")
        out, lse = oracle_lib.fwd(q, k, v, w, beta, logf=fox, scale=g["scale"])
        for i in range(3):
            zi = np.array(g[key][i])
            p = np.exp(zi - zi.max())
            assert_close(out[i], (p / p.sum()) @ v[: i + 1], 1e-14, f"{key} out row {i}")
            assert_close(lse[i], zi.max() + np.log(p.sum()), 1e-14, f"{key} lse row {i}")


# ----------------------------------------------------------------------------- P1

@pytest.mark.parametrize("L,d,scale", [(1, 4, 1.0), (37, 8, 0.3), (64, 16, 0.25)])
def test_p1_beta_zero_is_plain_causal_attention(oracle_lib, L, d, scale):
    q, k, v, w, _, _ = rand_problem(L, d, seed=L)
    out, lse = oracle_lib.fwd(q, k, v, w, np.zeros(L), scale=scale)
    ro, rl = plain_causal_attention(q, k, v, scale)
    assert_close(out, ro, 1e-12, "out")
    assert_close(lse, rl, 1e-12, "lse")


def test_p1_synth_beta0_recipe(oracle_lib):
    x = synth.make_fwd_inputs(2, 2, 33, 16, recipe="beta0", dtype="bf16", seed=3)
    out, lse = oracle_lib.fwd(x.q, x.k, x.v, x.w, x.beta, scale=x.scale)
    for b in range(2):
        for h in range(2):
            ro, rl = plain_causal_attention(*(t[b, h].astype(np.float64) for t in (x.q, x.k, x.v)), x.scale)
            assert_close(out[b, h], ro, 1e-12)
            assert_close(lse[b, h], rl, 1e-12)


# ----------------------------------------------------------------------------- P2

@pytest.mark.parametrize("L,d,fox,beta_mode", [(12, 5, False, "sigmoid"), (12, 5, True, "sigmoid"),
                                               (64, 16, False, "sigmoid"), (20, 3, True, "two")])
def test_p2_bruteforce_products(oracle_lib, L, d, fox, beta_mode):
    q, k, v, w, beta, logf = rand_problem(L, d, seed=100 + L + d, beta_mode=beta_mode, fox=fox)
    # deliberately non-unit w as well: the oracle uses w as given
    w = w * (1.0 + 0.1 * np.random.default_rng(7).standard_normal((L, 1)))
    scale = 0.37
    z = brute_logits(q, k, w, beta, scale, logf)
    for i in range(L):
        zi = oracle_lib.row_logits(q[i], k, w, beta, i, logf=logf, scale=scale)
        assert_close(zi, z[i, : i + 1], 1e-11, f"row {i}")
    out, lse = oracle_lib.fwd(q, k, v, w, beta, logf=logf, scale=scale)
    ro, rl = softmax_attend(z, v)
    assert_close(out, ro, 1e-12, "out")
    assert_close(lse, rl, 1e-11, "lse")


def test_p2_config1_shape_bruteforce(oracle_lib):
    """The tiny fp32 workload (B=H=1, L=64, d=16) against explicit products."""
    x = synth.make_fwd_inputs(1, 1, 64, 16, recipe="tiny", dtype="f32", seed=0)
    q, k, v, w = (t[0, 0].astype(np.float64) for t in (x.q, x.k, x.v, x.w))
    beta = x.beta[0, 0].astype(np.float64)
    for scale in (0.25, 1.0):
        z = brute_logits(q, k, w, beta, scale)
        out, lse = oracle_lib.fwd(x.q, x.k, x.v, x.w, x.beta, scale=scale)
        ro, rl = softmax_attend(z, v)
        assert_close(out[0, 0], ro, 1e-11)
        assert_close(lse[0, 0], rl, 1e-11)


def test_p2_transport_matches_explicit_product(oracle_lib):
    L, d = 30, 7
    _, _, _, w, beta, _ = rand_problem(L, d, seed=5)
    x = np.random.default_rng(9).standard_normal(d)
    for lo, hi in [(0, 29), (3, 17), (10, 10), (12, 11)]:
        M = np.eye(d)
        for s in range(lo, hi + 1):
            M = M @ H(w[s], beta[s])
        assert_close(oracle_lib.transport(x, w, beta, lo, hi), M @ x, 1e-12, f"[{lo},{hi}]")


# ----------------------------------------------------------------------------- P3

def test_p3_norms(oracle_lib):
    L, d = 200, 16
    _, _, _, w, _, _ = rand_problem(L, d, seed=11)
    x = np.random.default_rng(1).standard_normal(d)
    n0 = np.linalg.norm(x)
    two = np.full(L, 2.0)
    for hi in (0, 10, 199):
        assert abs(np.linalg.norm(oracle_lib.transport(x, w, two, 0, hi)) - n0) <= 1e-12 * n0
    beta = np.random.default_rng(2).uniform(0.0, 2.0, L)
    prev = n0
    for lo in range(L - 1, -1, -1):  # growing product H_lo ... H_{L-1}
        n = np.linalg.norm(oracle_lib.transport(x, w, beta, lo, L - 1))
        assert n <= prev * (1 + 1e-13)
        prev = n


# ----------------------------------------------------------------------------- P4

def _np_tinv(W, beta):
    """T^{-1} with T = diag(1/beta) + strict_upper(W W^T), solved by numpy (beta > 0 here)."""
    n = W.shape[0]
    T = np.triu(W @ W.T, 1) + np.diag(1.0 / beta)
    return np.linalg.solve(T, np.eye(n))


@pytest.mark.parametrize("n,d", [(16, 16), (64, 64), (128, 64), (5, 9)])
def test_p4_ut_identity(oracle_lib, n, d):
    _, _, _, W, beta, _ = rand_problem(n, d, seed=n * 7 + d)
    tinv = oracle_lib.ut_tinv(W, beta)
    assert np.allclose(np.tril(tinv, -1), 0.0)
    P = np.eye(d)
    for s in range(n):
        P = P @ H(W[s], beta[s])
    assert_close(np.eye(d) - W.T @ tinv @ W, P, 1e-12, "UT identity")
    assert_close(oracle_lib.householder_product(W, beta), P, 1e-12, "explicit product")
    assert_close(tinv, _np_tinv(W, beta), 1e-9 * max(1.0, np.abs(tinv).max()), "vs numpy solve")
    # every contiguous sub-range uses the matching principal block of T^{-1}
    for a, b in [(0, n - 1), (1, n // 2), (n // 3, n - 1), (2, 2)]:
        Pab = np.eye(d)
        for s in range(a, b + 1):
            Pab = Pab @ H(W[s], beta[s])
        Wab = W[a:b + 1]
        assert_close(np.eye(d) - Wab.T @ tinv[a:b + 1, a:b + 1] @ Wab, Pab, 1e-12, f"sub-range {a}..{b}")


def test_p4_ut_handles_beta_zero_and_two(oracle_lib):
    n, d = 32, 16
    _, _, _, W, _, _ = rand_problem(n, d, seed=4)
    beta = np.where(np.arange(n) % 3 == 0, 0.0, 2.0)
    tinv = oracle_lib.ut_tinv(W, beta)
    P = np.eye(d)
    for s in range(n):
        P = P @ H(W[s], beta[s])
    assert_close(np.eye(d) - W.T @ tinv @ W, P, 1e-12)


# ----------------------------------------------------------------------------- P5

@pytest.mark.parametrize("fox", [False, True])
def test_p5_beta_two_absolute_form(oracle_lib, fox):
    L, d = 48, 8
    q, k, v, w, beta, logf = rand_problem(L, d, seed=21, beta_mode="two", fox=fox)
    A = np.eye(d)
    qa, ka = np.zeros_like(q), np.zeros_like(k)
    for i in range(L):
        A = A @ H(w[i], 2.0)
        qa[i], ka[i] = A @ q[i], A @ k[i]
    bias = None
    if fox:
        F = np.cumsum(logf)
        bias = F[:, None] - F[None, :]
    ro, rl = plain_causal_attention(qa, ka, v, 0.5, bias)
    out, lse = oracle_lib.fwd(q, k, v, w, beta, logf=logf, scale=0.5)
    assert_close(out, ro, 1e-11)
    assert_close(lse, rl, 1e-11)


# ----------------------------------------------------------------------------- P6

def test_p6_determinant(oracle_lib):
    n, d = 24, 12
    _, _, _, W, beta, _ = rand_problem(n, d, seed=8)
    W = W * np.random.default_rng(3).uniform(0.5, 1.2, (n, 1))  # non-unit rows
    P = oracle_lib.householder_product(W, beta)
    want = np.prod(1.0 - beta * np.sum(W * W, axis=1))
    assert abs(np.linalg.det(P) - want) <= 1e-10 * max(1.0, abs(want))
    tinv = oracle_lib.ut_tinv(W, beta)
    assert abs(np.linalg.det(np.eye(d) - W.T @ tinv @ W) - want) <= 1e-10 * max(1.0, abs(want))


# ----------------------------------------------------------------------------- P7

def chunked_forward(q, k, v, w, beta, scale, C, logf=None):
    """Blockwise PaTH forward written from the summary, section 3, in numpy.

    Per chunk: T^{-1} (numpy solve), boundary-adjusted rows
      Qt = Q - (T^{-1} (W Q^T * [t<=a]))^T W,  Kt = K - ((K W^T * [s>b]) T^{-1}) W,
      P_c = I - W^T T^{-1} W,  S_intra^T = K Q^T - ((K W^T * [s>b]) T^{-1}) (W Q^T * [t<=a]);
    then, per query chunk m, a right-to-left scan over key chunks n < m with the
    running queries Q_run <- Q_run P_n^T.  A ragged last chunk is padded with
    beta = 0 tokens (identity transitions) whose keys are never attended.
    """
    L, d = q.shape
    M = -(-L // C)
    Lp = M * C
    pad = lambda x: np.concatenate([x, np.zeros((Lp - L,) + x.shape[1:])]) if Lp > L else x
    q, k, v, w, beta = map(pad, (q, k, v, w, beta))
    F = np.cumsum(pad(logf)) if logf is not None else np.zeros(Lp)
    le = np.triu(np.ones((C, C)))  # [t <= a] as (t, a)
    gt = np.triu(np.ones((C, C)), 1)  # [s > b] as (b, s)
    Qt, Kt, Pc, Sin = [], [], [], []
    for c in range(M):
        sl = slice(c * C, (c + 1) * C)
        Wc, Qc, Kc, bc = w[sl], q[sl], k[sl], beta[sl]
        A = np.eye(C) + bc[:, None] * np.triu(Wc @ Wc.T, 1)
        Ti = np.linalg.solve(A, np.diag(bc))
        X = Ti @ ((Wc @ Qc.T) * le)
        Y = ((Kc @ Wc.T) * gt) @ Ti
        Qt.append(Qc - X.T @ Wc)
        Kt.append(Kc - Y @ Wc)
        Pc.append(np.eye(d) - Wc.T @ Ti @ Wc)
        Sin.append((Kc @ Qc.T - Y @ ((Wc @ Qc.T) * le)).T)  # [a, b]
    out = np.zeros((L, d))
    lse = np.zeros(L)
    for m in range(M):
        rows = np.arange(m * C, (m + 1) * C)
        z = np.full((C, Lp), -np.inf)
        diag = scale * Sin[m] + (F[rows][:, None] - F[rows][None, :])
        z[:, m * C:(m + 1) * C] = np.where(np.tril(np.ones((C, C))) > 0, diag, -np.inf)
        Qrun = Qt[m].copy()
        for n in range(m - 1, -1, -1):
            cols = np.arange(n * C, (n + 1) * C)
            z[:, cols] = scale * Qrun @ Kt[n].T + (F[rows][:, None] - F[cols][None, :])
            Qrun = Qrun @ Pc[n].T
        o, l = softmax_attend(z, v)
        for a, i in enumerate(rows):
            if i < L:
                out[i], lse[i] = o[a], l[a]
    return out, lse, (Qt, Kt, Pc, Sin)


@pytest.mark.parametrize("L,d,C,fox", [(64, 16, 16, False), (50, 8, 8, True), (37, 6, 16, False),
                                       (96, 16, 32, True), (40, 4, 8, False)])
def test_p7_chunked_scheme_matches_oracle(oracle_lib, L, d, C, fox):
    q, k, v, w, beta, logf = rand_problem(L, d, seed=L * 3 + C, fox=fox)
    scale = 0.4
    ro, rl, _ = chunked_forward(q, k, v, w, beta, scale, C, logf)
    out, lse = oracle_lib.fwd(q, k, v, w, beta, logf=logf, scale=scale)
    assert_close(out, ro, 1e-11, "out")
    assert_close(lse, rl, 1e-11, "lse")


def test_p7_chunk_terms_definition_vs_ut(oracle_lib):
    C, d = 16, 8
    q, k, v, w, beta, _ = rand_problem(C, d, seed=77)
    _, _, (Qt, Kt, Pc, Sin) = chunked_forward(q, k, v, w, beta, 1.0, C)
    qt, kt, s = oracle_lib.chunk_terms(q, k, w, beta)
    assert_close(qt, Qt[0], 1e-12, "qtilde")
    assert_close(kt, Kt[0], 1e-12, "ktilde")
    assert_close(np.tril(s), np.tril(Sin[0]), 1e-12, "sintra")
    assert_close(oracle_lib.householder_product(w, beta), Pc[0], 1e-12, "P_c")


# ----------------------------------------------------------------------------- P8

def test_p8_special_cases(oracle_lib):
    L, d = 40, 8
    q, k, v, w, beta, logf = rand_problem(L, d, seed=31, fox=True)
    out, lse = oracle_lib.fwd(q, k, v, w, beta, scale=0.7)
    assert_close(out[0], v[0], 1e-15, "row 0 output")
    assert_close(lse[0], 0.7 * q[0] @ k[0], 1e-14, "row 0 lse")
    c = np.random.default_rng(0).standard_normal(d)
    oc, _ = oracle_lib.fwd(q, k, np.tile(c, (L, 1)), w, beta, scale=0.7)
    assert_close(oc, np.tile(c, (L, 1)), 1e-13, "constant values")
    o0, l0 = oracle_lib.fwd(q, k, v, w, beta, logf=np.zeros(L), scale=0.7)
    assert_close(o0, out, 0.0, "f = 0 is plain PaTH")
    assert_close(l0, lse, 0.0)
    F = np.cumsum(logf)
    ro, rl = plain_causal_attention(q, k, v, 0.7, F[:, None] - F[None, :])
    of, lf = oracle_lib.fwd(q, k, v, w, np.zeros(L), logf=logf, scale=0.7)
    assert_close(of, ro, 1e-12, "beta = 0 with FoX")
    assert_close(lf, rl, 1e-12)


def test_p8_sampled_rows_equal_full(oracle_lib):
    x = synth.make_fwd_inputs(2, 3, 70, 16, recipe="fox", dtype="bf16", seed=5)
    out, lse = oracle_lib.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale)
    rows = [0, 13, 64, 69]
    so, sl = oracle_lib.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale, rows=rows)
    assert_close(so, out[:, :, rows], 0.0)
    assert_close(sl, lse[:, :, rows], 0.0)


# ----------------------------------------------------------------------------- P9

def test_p9_decode_from_empty_equals_prefill(oracle_lib):
    BH, S, d = 3, 33, 8
    r = np.random.default_rng(12)
    q, k, v, w = r.standard_normal((4, S, BH, d))
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = r.uniform(0, 2, (S, BH))
    kc, vc = np.zeros((BH, S, d)), np.zeros((BH, S, d))
    out, lse = oracle_lib.decode(kc, vc, 0, q, k, v, w, beta, scale=0.6)
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 1))
    po, pl = oracle_lib.fwd(tr(q), tr(k), tr(v), tr(w), tr(beta), scale=0.6)
    assert_close(tr(out), po, 1e-12, "out")
    assert_close(tr(lse), pl, 1e-12, "lse")
    # the cache holds k_j <- H_{S-1} ... H_{j+1} k_j (explicit products)
    for bh in range(BH):
        for j in range(S):
            M = np.eye(d)
            for s in range(S - 1, j, -1):
                M = M @ H(w[s, bh], beta[s, bh])
            assert_close(kc[bh, j], M @ k[j, bh], 1e-12, f"cache key {j}")


def test_p9_fox_decode_from_empty_equals_prefill(oracle_lib):
    """PaTH-FoX decode (per-slot forget bias grown in place) == the FoX prefill definition, row by row."""
    BH, S, d = 3, 29, 6
    r = np.random.default_rng(17)
    q, k, v, w = r.standard_normal((4, S, BH, d))
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = r.uniform(0, 2, (S, BH))
    f = -np.log1p(np.exp(-(1.0 + r.standard_normal((S, BH)))))
    kc, vc, fc = np.zeros((BH, S, d)), np.zeros((BH, S, d)), np.zeros((BH, S))
    out, lse = oracle_lib.decode(kc, vc, 0, q, k, v, w, beta, scale=0.4, fcache=fc, logf=f)
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 1))
    po, pl = oracle_lib.fwd(tr(q), tr(k), tr(v), tr(w), tr(beta), logf=tr(f), scale=0.4)
    assert_close(tr(out), po, 1e-12, "out")
    assert_close(tr(lse), pl, 1e-12, "lse")
    # the slot biases are the suffix sums of the gates after each slot
    for bh in range(BH):
        want = np.array([f[j + 1:, bh].sum() for j in range(S)])
        assert_close(fc[bh], want, 1e-12, "slot bias")
        assert_close(oracle_lib.cache_bias(f[:, bh]), want, 1e-12, "cache_bias")


def test_p9_fox_bias_beta_zero_closed_form(oracle_lib):
    """beta = 0 and constant gate f: logits are scale q.k_j + (t - j) f (ALiBi-like closed form)."""
    BH, S, d, fval = 1, 12, 4, -0.3
    r = np.random.default_rng(3)
    q, k, v, w = r.standard_normal((4, S, BH, d))
    kc, vc, fc = np.zeros((BH, S, d)), np.zeros((BH, S, d)), np.zeros((BH, S))
    out, lse = oracle_lib.decode(kc, vc, 0, q, k, v, w, np.zeros((S, BH)), scale=1.0, fcache=fc,
                                 logf=np.full((S, BH), fval))
    for t in range(S):
        z = k[:t + 1, 0] @ q[t, 0] + fval * (t - np.arange(t + 1))
        p = np.exp(z - z.max())
        assert_close(out[t, 0], (p / p.sum()) @ v[:t + 1, 0], 1e-12, "out")
        assert_close(lse[t, 0], z.max() + np.log(p.sum()), 1e-12, "lse")


def test_p9_decode_with_initial_cache(oracle_lib):
    BH, T0, S, d = 2, 20, 5, 8
    r = np.random.default_rng(13)
    cache_k, cache_v = r.standard_normal((2, BH, T0 + S, d))
    q, k, v, w = r.standard_normal((4, S, BH, d))
    beta = r.uniform(0, 2, (S, BH))
    kc, vc = cache_k.copy(), cache_v.copy()
    out, lse = oracle_lib.decode(kc, vc, T0, q, k, v, w, beta, scale=0.5)
    for bh in range(BH):
        keys = list(cache_k[bh, :T0])
        vals = list(cache_v[bh, :T0])
        for s in range(S):
            Hs = H(w[s, bh], beta[s, bh])
            keys = [Hs @ kk for kk in keys] + [k[s, bh]]
            vals.append(v[s, bh])
            z = 0.5 * np.array(keys) @ q[s, bh]
            p = np.exp(z - z.max())
            assert_close(out[s, bh], (p / p.sum()) @ np.array(vals), 1e-12)
            assert_close(lse[s, bh], z.max() + np.log(p.sum()), 1e-12)


# ----------------------------------------------------------------------------- P10

MUTATIONS = {
    # sign of the rank-one term flipped
    "sign": ("r[t] -= c * w[t];", "r[t] += c * w[t];"),
    # H_j applied before key j is scored (product would start at s = j)
    "order": ("    z[j] = scale * dot(K + j * d, r, d) + bias;\n    apply_h(r, W + j * d, beta[j], d);",
              "    apply_h(r, W + j * d, beta[j], d);\n    z[j] = scale * dot(K + j * d, r, d) + bias;"),
    # FoX bias includes f_j itself
    "fox_index": ("    if (logf) bias += logf[j];\n  }\n}",
                  "  }\n}"),
    # scale dropped
    "scale": ("z[j] = scale * dot(K + j * d, r, d) + bias;", "z[j] = dot(K + j * d, r, d) + bias;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_p10_planted_mistakes_are_caught(oracle_lib, name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle_lib.__file__), "path_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation site for {name} not found"
    if name == "fox_index":
        # drop the accumulation after scoring and add it before, so f_j enters key j's bias
        src = src.replace(old, new).replace(
            "  for (int64_t j = i; j >= 0; --j) {\n    z[j] =",
            "  for (int64_t j = i; j >= 0; --j) {\n    if (logf) bias += logf[j];\n    z[j] =")
    else:
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tdir:
        c = os.path.join(tdir, "m.c")
        so = os.path.join(tdir, "m.so")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, c, "-lm"],
                       check=True)
        real = oracle_lib.lib()
        mutated = ctypes.CDLL(so)
        for f in ("path_oracle_fwd", "path_oracle_row_logits"):
            getattr(mutated, f).argtypes = getattr(real, f).argtypes
            getattr(mutated, f).restype = ctypes.c_int
        monkeypatch.setattr(oracle_lib, "_lib", mutated)
        failures = 0
        for pin in (lambda: test_p2_bruteforce_products(oracle_lib, 12, 5, True, "sigmoid"),
                    lambda: test_p1_beta_zero_is_plain_causal_attention(oracle_lib, 37, 8, 0.3),
                    lambda: test_p0_golden_hand_example(oracle_lib)):
            try:
                pin()
            except AssertionError:
                failures += 1
        assert failures >= 1, f"mutation {name} slipped through every pin"


# ----------------------------------------------------------------------------- P11

def _explicit_cache(k, w, beta):
    """slot j = H_{L-1} ... H_{j+1} k_j from explicit d x d matrices."""
    L, d = k.shape
    out = np.zeros_like(k)
    for j in range(L):
        M = np.eye(d)
        for s in range(L - 1, j, -1):
            M = M @ H(w[s], beta[s])
        out[j] = M @ k[j]
    return out


@pytest.mark.parametrize("L,d,beta_mode", [(1, 4, "sigmoid"), (9, 5, "sigmoid"), (17, 8, "two"), (6, 3, "zero")])
def test_p11_cache_keys_explicit_products(oracle_lib, L, d, beta_mode):
    q, k, v, w, beta, _ = rand_problem(L, d, 40 + L, beta_mode=beta_mode)
    got = oracle_lib.cache_keys(k, w, beta)
    assert_close(got, _explicit_cache(k, w, beta), 1e-12, "cache keys")
    if beta_mode == "zero":
        assert_close(got, k, 0.0, "beta = 0 keeps the keys")
    if beta_mode == "two":  # reflections keep norms
        assert_close(np.linalg.norm(got, axis=1), np.linalg.norm(k, axis=1), 1e-12, "norms")
    # a row range equals the matching slice of the full cache
    if L > 2:
        assert_close(oracle_lib.cache_keys(k, w, beta, rows=(1, L - 1)), got[1:L - 1], 0.0, "row range")


def test_p11_cache_keys_give_last_row_logits(oracle_lib):
    L, d, scale = 23, 6, 0.7
    q, k, v, w, beta, _ = rand_problem(L, d, 77)
    cache = oracle_lib.cache_keys(k, w, beta)
    z = brute_logits(q, k, w, beta, scale)
    # the query at position L-1 scores the cache exactly as the definition does
    assert_close(scale * cache @ q[L - 1], z[L - 1], 1e-12, "last-row logits")
    # and so does any other query placed at position L-1
    r = np.random.default_rng(5).standard_normal((4, d))
    for qq in r:
        q2 = q.copy()
        q2[L - 1] = qq
        assert_close(scale * cache @ qq, brute_logits(q2, k, w, beta, scale)[L - 1], 1e-12, "probe query")


def test_p11_cache_keys_equal_decode_recurrence(oracle_lib):
    BH, L, d = 2, 31, 8
    r = np.random.default_rng(21)
    q, k, v, w = r.standard_normal((4, L, BH, d))
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = r.uniform(0, 2, (L, BH))
    kc, vc = np.zeros((BH, L, d)), np.zeros((BH, L, d))
    oracle_lib.decode(kc, vc, 0, q, k, v, w, beta, scale=0.5)
    for bh in range(BH):
        assert_close(oracle_lib.cache_keys(k[:, bh], w[:, bh], beta[:, bh]), kc[bh], 1e-12, f"head {bh}")


CACHE_MUTATIONS = {
    # H_j itself applied to key j
    "includes_own": ("for (int64_t s = j + 1; s < L; ++s) apply_h(r,", "for (int64_t s = j; s < L; ++s) apply_h(r,"),
    # newest transition applied first
    "reversed": ("for (int64_t s = j + 1; s < L; ++s) apply_h(r,", "for (int64_t s = L - 1; s > j; --s) apply_h(r,"),
}


@pytest.mark.parametrize("name", sorted(CACHE_MUTATIONS))
def test_p11_planted_cache_mistakes_are_caught(oracle_lib, name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle_lib.__file__), "path_oracle.c")).read()
    old, new = CACHE_MUTATIONS[name]
    assert old in src, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tdir:
        c, so = os.path.join(tdir, "m.c"), os.path.join(tdir, "m.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, c, "-lm"],
                       check=True)
        mutated = ctypes.CDLL(so)
        mutated.path_oracle_cache_keys.argtypes = oracle_lib.lib().path_oracle_cache_keys.argtypes
        mutated.path_oracle_cache_keys.restype = ctypes.c_int
        monkeypatch.setattr(oracle_lib, "_lib", mutated)
        with pytest.raises(AssertionError):
            test_p11_cache_keys_explicit_products(oracle_lib, 9, 5, "sigmoid")


FOX_DECODE_MUTATIONS = {
    # the new slot starts with its own gate
    "own_gate": ("        Fc[t] = 0.0;", "        Fc[t] = J->fs[tok];"),
    # the bias is subtracted
    "bias_sign": ("+ (Fc ? Fc[j] : 0.0);", "- (Fc ? Fc[j] : 0.0);"),
}


@pytest.mark.parametrize("name", sorted(FOX_DECODE_MUTATIONS))
def test_p9_planted_fox_decode_mistakes_are_caught(oracle_lib, name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle_lib.__file__), "path_oracle.c")).read()
    old, new = FOX_DECODE_MUTATIONS[name]
    assert old in src, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tdir:
        c, so = os.path.join(tdir, "m.c"), os.path.join(tdir, "m.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, c, "-lm"],
                       check=True)
        real = oracle_lib.lib()
        mutated = ctypes.CDLL(so)
        for f in ("path_oracle_decode", "path_oracle_fwd", "path_oracle_cache_bias"):
            getattr(mutated, f).argtypes = getattr(real, f).argtypes
            getattr(mutated, f).restype = ctypes.c_int
        monkeypatch.setattr(oracle_lib, "_lib", mutated)
        with pytest.raises(AssertionError):
            test_p9_fox_bias_beta_zero_closed_form(oracle_lib)


# ----------------------------------------------------------------------------- P12

def _fd_grads(oracle_lib, q, k, v, w, beta, logf, dout, scale, h=1e-6):
    """Central differences of sum(dout * out) for every input coordinate (tiny problems only)."""
    args = [q, k, v, w, beta] + ([logf] if logf is not None else [])

    def loss(a):
        out, _ = oracle_lib.fwd(*a[:5], logf=a[5] if len(a) > 5 else None, scale=scale, nthreads=1)
        return float((out * dout).sum())

    grads = []
    for ai in range(len(args)):
        g = np.zeros_like(args[ai])
        for idx in np.ndindex(args[ai].shape):
            a = [x.copy() for x in args]
            a[ai][idx] += h
            lp = loss(a)
            a[ai][idx] -= 2 * h
            g[idx] = (lp - loss(a)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("L,d,beta_mode,fox", [(1, 3, "sigmoid", True), (7, 3, "sigmoid", True),
                                               (12, 5, "sigmoid", False), (9, 4, "two", True),
                                               (8, 3, "zero", True)])
def test_p12_backward_matches_finite_differences(oracle_lib, L, d, beta_mode, fox):
    q, k, v, w, beta, logf = rand_problem(L, d, 300 + L, beta_mode=beta_mode, fox=fox)
    dout = np.random.default_rng(301 + L).standard_normal((L, d))
    got = oracle_lib.bwd(q, k, v, w, beta, dout, logf=logf, scale=0.6, nthreads=1)
    want = _fd_grads(oracle_lib, q, k, v, w, beta, logf, dout, 0.6)
    names = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")
    for name, g, fd in zip(names, got, want):
        assert_close(g, fd, 2e-8 * max(1.0, np.abs(fd).max()), name)
    if not fox:
        assert got[5] is None


def _torch_explicit_grads(q, k, v, w, beta, logf, dout, scale):
    """torch autograd through the definition built from explicit d x d matrices."""
    import torch
    t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tw, tb = map(t, (q, k, v, w, beta))
    tf = t(logf) if logf is not None else None
    L, d = q.shape
    eye = torch.eye(d, dtype=torch.float64)
    rows = []
    for i in range(L):
        zi = []
        M = eye
        bias = torch.zeros((), dtype=torch.float64)
        for j in range(i, -1, -1):  # M = H_{j+1} ... H_i
            zi.append(scale * (tk[j] @ (M @ tq[i])) + bias)
            M = (eye - tb[j] * torch.outer(tw[j], tw[j])) @ M
            if tf is not None:
                bias = bias + tf[j]
        z = torch.stack(zi[::-1])
        rows.append(torch.softmax(z, 0) @ tv[: i + 1])
    out = torch.stack(rows)
    (out * torch.tensor(dout)).sum().backward()
    gs = [x.grad.numpy() for x in (tq, tk, tv, tw, tb)]
    return gs + [tf.grad.numpy() if tf is not None else None]


@pytest.mark.parametrize("L,d,fox", [(6, 4, True), (10, 3, False)])
def test_p12_backward_matches_autograd_of_explicit_products(oracle_lib, L, d, fox):
    q, k, v, w, beta, logf = rand_problem(L, d, 320 + L, fox=fox, unit=False)  # raw w: no norm assumed
    dout = np.random.default_rng(321).standard_normal((L, d))
    got = oracle_lib.bwd(q, k, v, w, beta, dout, logf=logf, scale=0.45, nthreads=1)
    want = _torch_explicit_grads(q, k, v, w, beta, logf, dout, 0.45)
    for name, g, a in zip(("dq", "dk", "dv", "dw", "dbeta", "dlogf"), got, want):
        if a is None:
            assert g is None
        else:
            assert_close(g, a, 1e-11 * max(1.0, np.abs(a).max()), name)


def test_p12_beta_zero_is_plain_attention_gradient(oracle_lib):
    import torch
    L, d, scale = 29, 8, 0.35
    q, k, v, w, beta, _ = rand_problem(L, d, 340, beta_mode="zero")
    dout = np.random.default_rng(341).standard_normal((L, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    z = scale * tq @ tk.T
    z = z.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    z.retain_grad()
    (torch.softmax(z, 1) @ tv * torch.tensor(dout)).sum().backward()
    dq, dk, dv, dw, dbeta, _ = oracle_lib.bwd(q, k, v, w, beta, dout, scale=scale)
    for name, g, a in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
        assert_close(g, a.numpy(), 1e-12, name)
    assert np.all(dw == 0.0), "with beta = 0 the output does not depend on w"
    # at beta = 0, d z_ij / d beta_s = -scale (w_s . k_j)(w_s . q_i) for every pair j < s <= i
    dz = z.grad.numpy()
    want = np.array([-scale * sum(dz[i, j] * (w[s] @ k[j]) * (w[s] @ q[i])
                                  for i in range(s, L) for j in range(s)) for s in range(L)])
    assert_close(dbeta, want, 1e-12, "dbeta closed form")


BWD_MUTATIONS = {
    # dbeta with the wrong sign
    "dbeta_sign": ("dbeta[s] = -dot(ws, cu, d);", "dbeta[s] = dot(ws, cu, d);"),
    # dw from dH_s w_s only (the transpose term dropped)
    "dw_no_transpose": ("-beta[s] * (cu[t] + cv[t]);", "-beta[s] * (2.0 * cu[t]);"),
    # query gradient carried one transition too far (a_{j,i+1} -> a_{j,i+1} moved by H_i ... starting at i)
    "dq_index": ("const double* a = A + (j * (L + 1) + i + 1) * d;",
                 "const double* a = A + (j * (L + 1) + (i > j ? i : i + 1)) * d;"),
    # forget gradient counts the pairs j <= s instead of j < s
    "df_range": ("for (int64_t j = 0; j < s; ++j) {\n        c += dZ[i * L + j] * aw[j];\n        df += dZ[i * L + j];\n      }",
                 "for (int64_t j = 0; j < s; ++j) {\n        c += dZ[i * L + j] * aw[j];\n        df += dZ[i * L + j];\n      }\n      df += dZ[i * L + s];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_p12_planted_backward_mistakes_are_caught(oracle_lib, name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle_lib.__file__), "path_oracle.c")).read()
    old, new = BWD_MUTATIONS[name]
    assert old in src, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tdir:
        c, so = os.path.join(tdir, "m.c"), os.path.join(tdir, "m.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, c, "-lm"],
                       check=True)
        real = oracle_lib.lib()
        mutated = ctypes.CDLL(so)
        for f in ("path_oracle_bwd", "path_oracle_fwd"):
            getattr(mutated, f).argtypes = getattr(real, f).argtypes
            getattr(mutated, f).restype = ctypes.c_int
        monkeypatch.setattr(oracle_lib, "_lib", mutated)
        with pytest.raises(AssertionError):
            test_p12_backward_matches_finite_differences(oracle_lib, 7, 3, "sigmoid", True)
