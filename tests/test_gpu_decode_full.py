"""Parity of decode at the full decode workload: batch 32, 24 heads, d = 64, a bf16 cache of 65536
tokens, in the launch configuration the benchmark times (automatic key split), for the in-place step
and for the deferred-update step (period 16).  The fp64 oracle recomputes sampled (batch, head) pairs
over their whole cache; every step's outputs and the updated cache slots of those pairs are checked.

The cache is drawn on the device from a seeded generator (N(0,1)/sqrt(d), rounded to bf16), as the
benchmark fills it; the oracle reads the sampled pairs' slots back before the first step.
"""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import assert_parity, dev, dev_f32, host
from tests.test_gpu_decode import check_cache, run_deferred

pytestmark = pytest.mark.gpu

B, H, D, T0 = 32, 24, 64, 65536
PAIRS = [(0, 0), (31, 23), (7, 11), (16, 5), (25, 19)]


def fill_cache(cap: int, seed: int):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    kc = torch.zeros((B, H, cap, D), device="cuda", dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for b in range(B):
        kc[b, :, :T0] = (torch.randn((H, T0, D), device="cuda", generator=gen) / np.sqrt(D)).to(torch.bfloat16)
        vc[b, :, :T0] = (torch.randn((H, T0, D), device="cuda", generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    return kc, vc


def sampled(kc, vc, cap):
    ok = np.zeros((len(PAIRS), cap, D))
    ov = np.zeros((len(PAIRS), cap, D))
    for i, (b, h) in enumerate(PAIRS):
        ok[i, :T0] = host(kc[b, h, :T0])
        ov[i, :T0] = host(vc[b, h, :T0])
    return ok, ov


def pick(x):
    """[S, B, H, ...] step inputs -> [S, pairs, ...]."""
    return np.ascontiguousarray(np.stack([x[:, b, h] for b, h in PAIRS], axis=1))


def test_full_size_in_place_decode_sampled():
    S = 3
    cap = T0 + S
    print(f"[case] full-size decode B={B} H={H} d={D} T0={T0} steps={S} pairs={PAIRS}", flush=True)
    kc, vc = fill_cache(cap, seed=1234)
    ok, ov = sampled(kc, vc, cap)
    st = synth.make_decode_steps(S, B, H, D, dtype="bf16", seed=3)
    outs, lses = [], []
    for s in range(S):
        o, l = native.path_decode_step(kc, vc, T0 + s, dev(st.q[s], "bf16"), dev(st.k[s], "bf16"),
                                       dev(st.v[s], "bf16"), dev(st.w[s], "bf16"), dev_f32(st.beta[s]),
                                       scale=st.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    go, gl = np.stack(outs), np.stack(lses)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    ro, rl = oracle.decode(ok, ov, T0, pick(st.q), pick(st.k), pick(st.v), pick(st.w), pick(st.beta), st.scale)
    assert_parity(pick(go), ro, "bf16", "out")
    assert_parity(pick(gl), rl, "bf16", "lse")
    for i, (b, h) in enumerate(PAIRS):
        check_cache(host(kc[b, h, :T0 + S]), ok[i, :T0 + S], "bf16", S)
        assert torch.equal(vc[b, h, T0:T0 + S].cpu(), dev(pick(st.v)[:, i], "bf16").cpu())


def test_full_size_deferred_decode_sampled():
    P = 16
    S = P + 1
    cap = T0 + S
    print(f"[case] full-size deferred decode B={B} H={H} d={D} T0={T0} period={P} steps={S} pairs={PAIRS}",
          flush=True)
    kc, vc = fill_cache(cap, seed=4321)
    ok, ov = sampled(kc, vc, cap)
    st = synth.make_decode_steps(S, B, H, D, dtype="bf16", seed=5)
    go, gl, t_cur = run_deferred(kc, vc, None, T0, st, P)
    assert t_cur == T0 + P  # one update, after the 16th step
    ok2, ov2 = ok.copy(), ov.copy()  # the oracle updates its cache in place
    ro, rl = oracle.decode(ok, ov, T0, pick(st.q), pick(st.k), pick(st.v), pick(st.w), pick(st.beta), st.scale)
    assert_parity(pick(go), ro, "bf16", "out")
    assert_parity(pick(gl), rl, "bf16", "lse")
    # slots 0 .. t_cur - 1 are current after the update: the oracle's cache after P steps
    oracle.decode(ok2, ov2, T0, pick(st.q)[:P], pick(st.k)[:P], pick(st.v)[:P], pick(st.w)[:P],
                  pick(st.beta)[:P], st.scale)
    for i, (b, h) in enumerate(PAIRS):
        check_cache(host(kc[b, h, :t_cur]), ok2[i, :t_cur], "bf16", P)
