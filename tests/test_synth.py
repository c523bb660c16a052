"""The seeded input generator: determinism, distributions, rounding."""
import numpy as np
import pytest
import torch

from dependent_positional_attention_amd import synth


def test_same_seed_same_bits():
    a = synth.make_fwd_inputs(2, 3, 50, 16, recipe="fox", seed=4)
    b = synth.make_fwd_inputs(2, 3, 50, 16, recipe="fox", seed=4)
    for n in ("q", "k", "v", "w", "beta", "logf"):
        assert np.array_equal(getattr(a, n).view(np.uint32), getattr(b, n).view(np.uint32)), n
    c = synth.make_fwd_inputs(2, 3, 50, 16, recipe="fox", seed=5)
    assert not np.array_equal(a.q, c.q)


def test_streams_are_independent_of_other_tensors():
    a = synth.make_fwd_inputs(1, 1, 32, 16, recipe="lm", seed=0)
    b = synth.make_fwd_inputs(1, 1, 32, 16, recipe="stress_qk", seed=0)
    assert np.array_equal(a.v, b.v) and np.array_equal(a.w, b.w) and np.array_equal(a.beta, b.beta)


def test_bf16_rounding_matches_torch_rne():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000) * 10.0 ** r.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-40]])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_distributions():
    x = synth.make_fwd_inputs(4, 4, 1024, 64, recipe="fox", dtype="bf16", seed=0)
    assert abs(x.q.std() - 1 / 8) < 2e-3 and abs(x.q.mean()) < 2e-3
    nrm = np.linalg.norm(x.w.astype(np.float64), axis=-1)
    assert np.all(np.abs(nrm - 1.0) < 2e-2)  # bf16 rounding of a unit vector
    assert x.beta.dtype == np.float32 and np.all((x.beta > 0) & (x.beta < 2))
    assert x.beta.min() < 0.05 and x.beta.max() > 1.95  # N(0, 1.5) logits reach both ends
    assert np.all(x.logf < 0) and abs(x.logf.mean() - (-0.07)) < 0.02
    t = synth.make_fwd_inputs(1, 1, 64, 16, recipe="tiny", dtype="f32", seed=0)
    assert abs(t.q.std() - 1.0) < 0.1
    f32 = synth.make_fwd_inputs(1, 1, 64, 16, recipe="tiny", dtype="f32", seed=0)
    assert np.allclose(np.linalg.norm(f32.w.astype(np.float64), axis=-1), 1.0, atol=1e-6)


@pytest.mark.parametrize("recipe,vals", [("beta2", {2.0}), ("beta0", {0.0}), ("beta02", {0.0, 2.0})])
def test_beta_recipes(recipe, vals):
    x = synth.make_fwd_inputs(1, 2, 300, 16, recipe=recipe, seed=1)
    assert set(np.unique(x.beta).tolist()) == vals


def test_decode_inputs():
    s = synth.make_decode_steps(4, 2, 3, 64, seed=0)
    assert s.q.shape == (4, 2, 3, 64) and s.beta.shape == (4, 2, 3)
    kc, vc = synth.make_decode_cache(2, 3, 100, 64, seed=0)
    assert kc.shape == (2, 3, 100, 64) and not np.array_equal(kc, vc)
