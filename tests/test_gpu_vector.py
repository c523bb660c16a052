"""Parity of the vector-ALU prefill path (fp32, and bf16 at shapes outside the matrix-core kernels)
against the fp64 oracle, element by element on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import assert_parity, errors, fwd_inputs_dev, host, TOL

pytestmark = pytest.mark.gpu


def run(x: synth.FwdInputs, chunk: int, transport="bf16"):
    t = fwd_inputs_dev(x)
    out, lse = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"], scale=x.scale,
                                    chunk=chunk, transport=transport)
    torch.cuda.synchronize()
    return host(out), host(lse)


def check(x: synth.FwdInputs, chunk: int, what: str):
    print(f"[case] {what} shape={x.shape} dtype={x.dtype} recipe={x.recipe} chunk={chunk}", flush=True)
    go, gl = run(x, chunk)
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale)
    assert_parity(go, ro, x.dtype, what + " out")
    assert_parity(gl, rl, x.dtype, what + " lse")


@pytest.mark.parametrize("scale", [0.25, 1.0])
def test_tiny_fp32_workload(scale):
    """B=1, H=1, L=64, d=16, chunk 16, fp32, seed 0 (both the 1/sqrt(d) scale and the literal scale 1)."""
    x = synth.make_fwd_inputs(1, 1, 64, 16, recipe="tiny", dtype="f32", seed=0, scale=scale)
    check(x, 16, f"tiny scale={scale}")


@pytest.mark.parametrize("d,chunk", [(16, 16), (16, 64), (32, 32), (64, 16), (64, 64), (32, 64)])
@pytest.mark.parametrize("recipe", ["tiny", "fox", "beta2"])
def test_fp32_shapes(d, chunk, recipe):
    x = synth.make_fwd_inputs(2, 3, 150, d, recipe=recipe, dtype="f32", seed=d + chunk)
    check(x, chunk, f"f32 d={d} C={chunk}")


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 63, 65])
def test_ragged_lengths(L):
    x = synth.make_fwd_inputs(1, 2, L, 16, recipe="fox", dtype="f32", seed=L)
    check(x, 16, f"ragged L={L}")


@pytest.mark.parametrize("d,chunk", [(16, 16), (32, 32), (64, 32)])
def test_bf16_vector_shapes(d, chunk):
    x = synth.make_fwd_inputs(2, 2, 200, d, recipe="stress_qk", dtype="bf16", seed=3)
    check(x, chunk, f"bf16 vector d={d} C={chunk}")


def test_chunk_invariance_fp32():
    x = synth.make_fwd_inputs(1, 2, 256, 32, recipe="stress_qk_beta2", dtype="f32", seed=9)
    a, la = run(x, 16)
    b, lb = run(x, 64)
    ma, rel = errors(a, b)
    assert ma <= 1e-5 and rel <= 1e-5


def test_empty_sequence_is_a_noop():
    x = synth.make_fwd_inputs(1, 1, 0, 16, recipe="tiny", dtype="f32")
    go, gl = run(x, 16)
    assert go.shape == (1, 1, 0, 16) and gl.shape == (1, 1, 0)


def test_negative_control_plain_attention_fails():
    """beta = 0 on the GPU (plain causal attention) must NOT pass against the oracle on stressed inputs:
    the parity bar is able to tell PaTH from ordinary attention."""
    x = synth.make_fwd_inputs(1, 2, 128, 32, recipe="stress_qk", dtype="f32", seed=1)
    ro, _ = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, scale=x.scale)
    plain = synth.FwdInputs(**{**x.__dict__, "beta": np.zeros_like(x.beta)})
    go, _ = run(plain, 32)
    ma, rel = errors(go, ro)
    assert ma > TOL["bf16"]["max_abs"] and rel > TOL["bf16"]["rel_l2"]
