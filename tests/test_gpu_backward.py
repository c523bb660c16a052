"""Parity of the backward pass (path_attn_bwd) against the fp64 oracle's gradients, element by element on
seeded inputs.  The GPU forward supplies out and lse, as in a training step; the oracle differentiates its
own exact forward.

Tolerance (per gradient tensor, relative to its largest reference entry): the fp32 path keeps fp32
throughout, so its error is fp32 rounding carried through the chunk chain; the bf16 path widens bf16
inputs, works in fp32, and rounds each gradient to bf16 once (2^-9 relative) after using the forward's
bf16-rounded output in D_i = dO_i . o_i, which moves every dz by up to p_ij |dO_i| |o_i| 2^-9.  The bf16
bound is the spec bf16 relative-L2 bound, 1e-2, applied to max-abs (relative to the largest entry)
and to rel-L2 alike.
"""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import dev, errors, fwd_inputs_dev, host

pytestmark = pytest.mark.gpu

GRAD_TOL = {"f32": 1e-5, "bf16": 1e-2}
NAMES = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")


def gpu_grads(x: synth.FwdInputs, dout: np.ndarray, chunk: int, fwd_chunk: int = 0):
    t = fwd_inputs_dev(x)
    out, lse = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale,
                                    chunk=fwd_chunk or (64 if x.dtype == "bf16" else chunk))
    g = native.path_attn_bwd(t["q"], t["k"], t["v"], t["w"], t["beta"], out, lse, dev(dout, x.dtype), t["logf"],
                             scale=x.scale, chunk=chunk)
    torch.cuda.synchronize()
    return [None if a is None else host(a) for a in g]


def check(x: synth.FwdInputs, chunk: int, what: str, seed: int = 0):
    print(f"[case] backward {what} shape={x.shape} dtype={x.dtype} recipe={x.recipe} chunk={chunk}", flush=True)
    dout = synth.make_out_grad(x.shape, dtype=x.dtype, seed=seed)
    got = gpu_grads(x, dout, chunk)
    want = oracle.bwd(x.q, x.k, x.v, x.w, x.beta, dout, logf=x.logf, scale=x.scale)
    tol = GRAD_TOL[x.dtype]
    worst = {}
    for name, g, r in zip(NAMES, got, want):
        if r is None:
            assert g is None, f"{what}: {name} returned without log_forget"
            continue
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite values"
        if float(np.max(np.abs(r))) == 0.0:
            # an exactly zero gradient (a single token: o_0 = v_0 exactly, so dz_00 = dO_0 . v_0 - D_0 is 0 in
            # exact arithmetic).  The kernels form dO . v and D = dO . o as two fp32 sums of the same d
            # products in different orders, each within d 2^-24 sum|dO_x v_x| <= d 2^-24 |dO| |v| of the exact
            # value; every gradient multiplies dz by at most two of scale q, scale k, w, beta (<= 2).
            nrm = lambda a: float(np.max(np.linalg.norm(np.asarray(a, np.float64), axis=-1)))
            e_dz = 2 * x.shape[-1] * 2.0 ** -24 * nrm(dout) * nrm(x.v)
            bound = e_dz * 2 * (1 + x.scale) * max(nrm(x.q), 1.0) * max(nrm(x.k), 1.0)
            assert np.max(np.abs(g)) <= bound, \
                f"{what} {name}: {np.max(np.abs(g)):.3e} where the gradient is 0 (bound {bound:.1e})"
            worst[name] = (0.0, 0.0)
            continue
        ma, rel = errors(g, r)
        ref = max(float(np.max(np.abs(r))), 1e-30)
        worst[name] = (ma / ref, rel)
        assert ma <= tol * ref and rel <= tol, \
            f"{what} {name}: max_abs {ma:.3e} vs max|ref| {ref:.3e} (tol {tol:.0e} of it), rel_l2 {rel:.3e}"
    print("   " + "  ".join(f"{n} {a:.1e}/{b:.1e}" for n, (a, b) in worst.items()), flush=True)
    return got, want


@pytest.mark.parametrize("d,chunk", [(16, 16), (32, 32), (64, 64), (16, 64), (64, 16), (32, 64)])
@pytest.mark.parametrize("recipe", ["tiny", "fox", "beta2"])
def test_fp32_backward_shapes(d, chunk, recipe):
    x = synth.make_fwd_inputs(1, 2, 150, d, recipe=recipe, dtype="f32", seed=d + chunk)
    check(x, chunk, f"f32 d={d} C={chunk}", seed=d)


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 65])
def test_fp32_backward_ragged(L):
    x = synth.make_fwd_inputs(1, 2, L, 16, recipe="fox", dtype="f32", seed=L)
    check(x, 16, f"ragged L={L}", seed=L)


@pytest.mark.parametrize("L,d,chunk", [(704, 16, 16), (1664, 64, 64)])
def test_fp32_backward_two_bands(L, d, chunk):
    """fp32 inputs long enough for two bands of query chunks (4 ceil(sqrt(M)) chunks each: M = 44 and 26
    chunks), so the key-side sums carry from one band to the next, on the vector kernels and on the fp32
    matrix cores; PaTH-FoX, one head."""
    x = synth.make_fwd_inputs(1, 1, L, d, recipe="fox", dtype="f32", seed=L)
    check(x, chunk, f"f32 two bands L={L} d={d} C={chunk}", seed=L + 1)


def test_beta_zero_leaves_w_without_gradient():
    """With every beta = 0 the output does not depend on w: dw must be exactly zero."""
    x = synth.make_fwd_inputs(1, 2, 130, 32, recipe="beta0", dtype="f32", seed=4)
    got, _ = check(x, 32, "beta0")
    assert np.all(got[3] == 0.0)


def test_bf16_beta_zero_leaves_w_without_gradient():
    """The matrix-core backward (bf16, d = chunk = 64) at beta = 0: the output does not depend on w, and
    every term of dw in the per-chunk gradient kernel is a product with diag(beta) = 0 (Ti = A^-1 diag(beta),
    X = Ti U, Y = R Ti, dU, dR and dN all vanish), so dw must be exactly zero, not merely small."""
    x = synth.make_fwd_inputs(1, 2, 200, 64, recipe="beta0", dtype="bf16", seed=5)
    got, _ = check(x, 64, "bf16 beta0", seed=6)
    assert np.all(got[3] == 0.0)


@pytest.mark.parametrize("recipe", ["lm", "fox", "stress_qk"])
def test_bf16_backward(recipe):
    x = synth.make_fwd_inputs(1, 2, 300, 64, recipe=recipe, dtype="bf16", seed=11)
    check(x, 64, f"bf16 {recipe}", seed=12)


def test_bf16_backward_several_heads():
    x = synth.make_fwd_inputs(2, 3, 520, 64, recipe="fox", dtype="bf16", seed=21)
    check(x, 64, "bf16 B=2 H=3", seed=22)


def test_full_size_backward_sampled_heads_equal_single_head_runs():
    """The backward at the benchmark's size (B=8, H=24, L=4096, bf16, PaTH-FoX) in its launch configuration.
    The fp64 oracle's backward needs minutes per head at this length, so the full-size run is tied to the
    oracle-checked kernels through a property that holds at any size: (batch, head) slices are independent
    and the kernels are deterministic, so every sampled head's gradients equal, bit for bit, those of the
    same head run on its own (B = H = 1, a different grid)."""
    B, H, L, d = 8, 24, 4096, 64
    print(f"[case] full-size backward B={B} H={H} L={L} d={d} bf16 fox", flush=True)
    x = synth.make_fwd_inputs(B, H, L, d, recipe="fox", dtype="bf16", seed=31)
    dout = synth.make_out_grad(x.shape, dtype="bf16", seed=32)
    t = fwd_inputs_dev(x)
    out, lse = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale, chunk=64)
    do = dev(dout, "bf16")
    full = native.path_attn_bwd(t["q"], t["k"], t["v"], t["w"], t["beta"], out, lse, do, t["logf"], scale=x.scale,
                                chunk=64)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (7, 23), (3, 17)]:
        sl = lambda a: a[b:b + 1, h:h + 1].contiguous()
        one = native.path_attn_bwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["w"]), sl(t["beta"]), sl(out), sl(lse),
                                   sl(do), sl(t["logf"]), scale=x.scale, chunk=64)
        torch.cuda.synchronize()
        for name, gf, g1 in zip(NAMES, full, one):
            assert torch.equal(sl(gf), g1), f"head ({b}, {h}) {name}: full-size run differs from the single-head run"
            assert torch.isfinite(g1.float()).all()


def test_bf16_backward_long_chain():
    """A 32-chunk chain (L = 2048, one head, PaTH-FoX, beta spread over (0, 2)) against the oracle: the
    states and their gradients pass through up to 31 chunk transitions, which bounds how the bf16
    rounding of the per-pair states accumulates along the chain."""
    x = synth.make_fwd_inputs(1, 1, 2048, 64, recipe="fox", dtype="bf16", seed=41)
    check(x, 64, "bf16 L=2048", seed=42)


def test_bf16_backward_two_bands_ragged():
    """The matrix-core backward over two bands of query chunks (L = 1637: 26 chunks in bands of 24) with a
    ragged last chunk (37 tokens), two heads, PaTH-FoX: the band boundary, the key-side sums carried
    across it and the clamped rows of the last chunk together."""
    x = synth.make_fwd_inputs(1, 2, 1637, 64, recipe="fox", dtype="bf16", seed=51)
    check(x, 64, "bf16 two bands ragged L=1637", seed=52)


@pytest.mark.parametrize("L", [1, 40, 64, 65, 129])
def test_bf16_backward_short_and_ragged(L):
    """The matrix-core backward (d = chunk = 64) at its edges: one partial chunk (no chunk pairs at all),
    exactly one chunk, one token past it, and two chunks plus one token; PaTH-FoX, two heads."""
    x = synth.make_fwd_inputs(1, 2, L, 64, recipe="fox", dtype="bf16", seed=100 + L)
    check(x, 64, f"bf16 L={L}", seed=200 + L)
