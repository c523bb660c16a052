"""Parity of the decode step (in-place key update + split-key attention) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import assert_parity, dev, dev_f32, errors, host

pytestmark = pytest.mark.gpu


def check_cache(got, want, dtype, steps):
    """The cache is stored state, re-rounded to the storage dtype at every step (the in-place update
    rule itself), while the oracle keeps it in fp64.  Each rounding moves an element by at most half
    an ulp (2^-8 relative for bf16) and the transitions never grow a key's norm, so after `steps`
    steps a bf16 cache is within (steps + 1) half-ulps of the largest element.  An fp32 cache is held
    to the fp32 output tolerance."""
    bound = (steps + 1) * 2.0 ** -8 * np.max(np.abs(want)) if dtype == "bf16" else 1e-5
    ma, rel = errors(got, want)
    assert ma <= bound, f"cache max_abs {ma:.3e} > derived bound {bound:.3e}"
    assert rel <= (1e-2 if dtype == "bf16" else 1e-5), f"cache rel_l2 {rel:.3e}"


def run_steps(kc, vc, t0, steps: synth.DecodeStepInputs, splits=0):
    outs, lses = [], []
    S = steps.q.shape[0]
    for s in range(S):
        o, l = native.path_decode_step(kc, vc, t0 + s, dev(steps.q[s], steps.dtype), dev(steps.k[s], steps.dtype),
                                       dev(steps.v[s], steps.dtype), dev(steps.w[s], steps.dtype),
                                       dev_f32(steps.beta[s]), scale=steps.scale, splits=splits)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    return np.stack(outs), np.stack(lses)


def oracle_steps(cache_k, cache_v, t0, cap, steps):
    B, H, _, d = cache_k.shape
    BH = B * H
    kc = np.zeros((BH, cap, d))
    vc = np.zeros((BH, cap, d))
    kc[:, :t0] = cache_k.reshape(BH, -1, d)[:, :t0]
    vc[:, :t0] = cache_v.reshape(BH, -1, d)[:, :t0]
    S = steps.q.shape[0]
    sh = lambda x: x.reshape(S, BH, -1) if x.ndim == 4 else x.reshape(S, BH)
    out, lse = oracle.decode(kc, vc, t0, sh(steps.q), sh(steps.k), sh(steps.v), sh(steps.w), sh(steps.beta),
                             steps.scale)
    return out.reshape(S, B, H, d), lse.reshape(S, B, H), kc.reshape(B, H, cap, d)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 16), ("bf16", 128), ("f32", 64), ("bf16", 16),
                                     ("f32", 128), ("bf16", 32)])
def test_decode_with_cache(dtype, d):
    B, H, T0, S = 2, 3, 700, 6
    cap = T0 + S + 5
    print(f"[case] decode dtype={dtype} d={d} T0={T0} steps={S}", flush=True)
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype=dtype, seed=d)
    steps = synth.make_decode_steps(S, B, H, d, dtype=dtype, seed=d)
    kc = torch.zeros((B, H, cap, d), device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    vc = torch.zeros_like(kc)
    kc[:, :, :T0] = dev(ck, dtype)
    vc[:, :, :T0] = dev(cv, dtype)
    go, gl = run_steps(kc, vc, T0, steps)
    ro, rl, rk = oracle_steps(ck, cv, T0, cap, steps)
    assert_parity(go, ro, dtype, "out")
    assert_parity(gl, rl, dtype, "lse")
    check_cache(host(kc)[:, :, :T0 + S], rk[:, :, :T0 + S], dtype, S)
    assert np.all(host(kc)[:, :, T0 + S:] == 0)  # slots past t untouched


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_from_empty_equals_prefill(dtype):
    """Decoding S tokens from an empty cache reproduces prefill rows 0..S-1 (oracle prefill)."""
    B, H, S, d = 1, 4, 40, 64
    steps = synth.make_decode_steps(S, B, H, d, dtype=dtype, seed=2)
    kc = torch.zeros((B, H, S, d), device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    vc = torch.zeros_like(kc)
    go, gl = run_steps(kc, vc, 0, steps)
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))  # [S,B,H,...] -> [B,H,S,...]
    ro, rl = oracle.fwd(tr(steps.q), tr(steps.k), tr(steps.v), tr(steps.w), tr(steps.beta), scale=steps.scale)
    assert_parity(tr(go), ro, dtype, "out")
    assert_parity(tr(gl), rl, dtype, "lse")


def test_split_count_does_not_change_the_cache():
    """Splits own disjoint key ranges: the updated cache is bit-identical for any split count."""
    B, H, T0, d = 2, 2, 3000, 64
    ck, cv = synth.make_decode_cache(B, H, T0 + 1, d, dtype="bf16", seed=5)
    steps = synth.make_decode_steps(1, B, H, d, dtype="bf16", seed=5)
    res = []
    for splits in (1, 3, 0, 64):
        kc, vc = dev(ck, "bf16"), dev(cv, "bf16")
        o, _ = run_steps(kc, vc, T0, steps, splits=splits)
        res.append((kc.view(torch.int16).cpu().numpy(), o))
    for kbits, o in res[1:]:
        assert np.array_equal(kbits, res[0][0])
        ma, rel = errors(o, res[0][1])
        assert ma <= 1e-3 and rel <= 1e-3


def initial_slot_bias(B, H, T0, cap, seed):
    """PaTH-FoX slot biases of a T0-token cache: suffix sums of gates drawn like the prompts' (fp32 values)."""
    g = synth.logsigmoid(np.random.default_rng(seed).normal(3.0, 1.0, (B, H, T0)))
    suf = np.zeros((B, H, cap), dtype=np.float32)
    rev = np.cumsum(g[:, :, ::-1], axis=-1)[:, :, ::-1]  # sum_{s>=j}
    suf[:, :, :T0 - 1] = rev[:, :, 1:]
    return suf


def fox_gates(S, B, H, seed):
    return synth.logsigmoid(np.random.default_rng(seed + 1).normal(3.0, 1.0, (S, B, H))).astype(np.float32)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 32), ("bf16", 128)])
def test_fox_decode_with_cache(dtype, d):
    """PaTH-FoX decode: slot biases grow in place by each new gate; outputs and the bias state vs the oracle."""
    B, H, T0, S = 2, 3, 900, 4
    cap = T0 + S + 3
    print(f"[case] fox decode dtype={dtype} d={d} T0={T0} steps={S}", flush=True)
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype=dtype, seed=d + 1)
    steps = synth.make_decode_steps(S, B, H, d, dtype=dtype, seed=d + 1)
    fc0 = initial_slot_bias(B, H, T0, cap, seed=d)
    gates = fox_gates(S, B, H, seed=d)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((B, H, cap, d), device="cuda", dtype=td)
    vc = torch.zeros_like(kc)
    kc[:, :, :T0] = dev(ck, dtype)
    vc[:, :, :T0] = dev(cv, dtype)
    fc = dev_f32(fc0)
    outs, lses = [], []
    for s in range(S):
        o, l = native.path_decode_step(kc, vc, T0 + s, dev(steps.q[s], dtype), dev(steps.k[s], dtype),
                                       dev(steps.v[s], dtype), dev(steps.w[s], dtype), dev_f32(steps.beta[s]),
                                       dev_f32(gates[s]), fcache=fc, scale=steps.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    BH = B * H
    okc, ovc = np.zeros((BH, cap, d)), np.zeros((BH, cap, d))
    okc[:, :T0] = ck.reshape(BH, T0, d)
    ovc[:, :T0] = cv.reshape(BH, T0, d)
    ofc = fc0.reshape(BH, cap).astype(np.float64)
    sh = lambda x: x.reshape(S, BH, -1) if x.ndim == 4 else x.reshape(S, BH)
    ro, rl = oracle.decode(okc, ovc, T0, sh(steps.q), sh(steps.k), sh(steps.v), sh(steps.w), sh(steps.beta),
                           steps.scale, fcache=ofc, logf=sh(gates))
    assert_parity(np.stack(outs), ro.reshape(S, B, H, d), dtype, "out")
    assert_parity(np.stack(lses), rl.reshape(S, B, H), dtype, "lse")
    # fp32 slot biases: one rounding per added gate
    want = ofc.reshape(B, H, cap)[:, :, :T0 + S]
    got = host(fc)[:, :, :T0 + S]
    bound = (S + 1) * 2.0 ** -24 * np.max(np.abs(want)) + 1e-7
    assert np.max(np.abs(got - want)) <= bound, f"slot bias error {np.max(np.abs(got - want)):.3e} > {bound:.3e}"
    assert np.all(host(fc)[:, :, T0 + S:] == 0)


@pytest.mark.parametrize("fox", [False, True])
def test_ragged_batch(fox):
    """Per-sequence token counts: each sequence matches the oracle run on its own cache; an out-of-range count
    gives NaN for that sequence and leaves its slots untouched."""
    B, H, d, S = 4, 2, 64, 2
    counts = np.array([1500, 37, 0, -1], dtype=np.int32)  # the last one is invalid
    t_bound = 1500
    cap = t_bound + S + 1
    print(f"[case] ragged decode fox={fox} counts={counts.tolist()}", flush=True)
    ck, cv = synth.make_decode_cache(B, H, cap, d, dtype="bf16", seed=11)
    steps = synth.make_decode_steps(S, B, H, d, dtype="bf16", seed=11)
    gates = fox_gates(S, B, H, seed=11) if fox else None
    # each sequence's slot biases as of its own count (suffix sums of its prompt gates)
    fc0 = np.zeros((B, H, cap), dtype=np.float32)
    if fox:
        g = synth.logsigmoid(np.random.default_rng(12).normal(3.0, 1.0, (B, H, cap)))
        for b, tb0 in enumerate(counts):
            if tb0 > 1:
                rev = np.cumsum(g[b, :, :tb0][:, ::-1], axis=-1)[:, ::-1]
                fc0[b, :, :tb0 - 1] = rev[:, 1:]
    kc, vc = dev(ck, "bf16"), dev(cv, "bf16")
    fc = dev_f32(fc0) if fox else None
    kc_before = kc.clone()
    outs, lses = [], []
    for s in range(S):
        tb = torch.from_numpy(np.where(counts >= 0, counts + s, counts).astype(np.int32)).cuda()
        o, l = native.path_decode_step(kc, vc, t_bound + s, dev(steps.q[s], "bf16"), dev(steps.k[s], "bf16"),
                                       dev(steps.v[s], "bf16"), dev(steps.w[s], "bf16"), dev_f32(steps.beta[s]),
                                       dev_f32(gates[s]) if fox else None, fcache=fc, t_batch=tb, scale=steps.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    go, gl = np.stack(outs), np.stack(lses)
    for b, tb0 in enumerate(counts):
        if tb0 < 0:
            assert np.all(np.isnan(go[:, b])) and np.all(np.isnan(gl[:, b]))
            assert torch.equal(kc[b], kc_before[b]), "an invalid sequence's slots were touched"
            if fox:
                assert np.array_equal(host(fc)[b], fc0[b].astype(np.float64))
            continue
        okc, ovc = np.zeros((H, cap, d)), np.zeros((H, cap, d))
        okc[:, :tb0] = ck[b, :, :tb0]
        ovc[:, :tb0] = cv[b, :, :tb0]
        sl = lambda x: np.ascontiguousarray(x[:, b])
        kw = dict(fcache=fc0[b].astype(np.float64), logf=sl(gates)) if fox else {}
        ro, rl = oracle.decode(okc, ovc, int(tb0), sl(steps.q), sl(steps.k), sl(steps.v), sl(steps.w),
                               sl(steps.beta), steps.scale, **kw)
        assert_parity(go[:, b], ro, "bf16", f"out seq {b}")
        assert_parity(gl[:, b], rl, "bf16", f"lse seq {b}")
        # slots past this sequence's own count are untouched
        assert torch.equal(kc[b, :, tb0 + S:], kc_before[b, :, tb0 + S:])


def run_deferred(kc, vc, fc, t0, steps, period, gates=None, force_at=None):
    """Decode with deferred key updates from a current cache at t0; returns outputs, lse and the final t_cur."""
    B, H, cap, d = kc.shape
    dtype = steps.dtype
    state = torch.zeros(native.path_decode_deferred_state_bytes(B, H, d) // 4, device="cuda", dtype=torch.float32)
    outs, lses = [], []
    t_cur = t0
    for s in range(steps.q.shape[0]):
        t = t0 + s
        per = (t - t_cur + 1) if (force_at is not None and s == force_at) else period
        o, l, t_cur = native.path_decode_step_deferred(
            kc, vc, t, t_cur, dev(steps.q[s], dtype), dev(steps.k[s], dtype), dev(steps.v[s], dtype),
            dev(steps.w[s], dtype), dev_f32(steps.beta[s]), dev_f32(gates[s]) if gates is not None else None,
            period=per, state=state, fcache=fc, scale=steps.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    return np.stack(outs), np.stack(lses), t_cur


@pytest.mark.parametrize("dtype,d,fox,period", [("bf16", 64, False, 8), ("bf16", 64, True, 16), ("f32", 32, True, 4),
                                                ("bf16", 128, False, 3), ("bf16", 16, False, 1), ("f32", 64, False, 5)])
def test_deferred_decode_matches_oracle(dtype, d, fox, period):
    """Deferred key updates give the in-place rule's outputs at every step; after an updating step the slots
    equal the oracle's cache."""
    B, H, T0 = 2, 3, 600
    S = 2 * period + 3
    cap = T0 + S + 2
    print(f"[case] deferred decode dtype={dtype} d={d} fox={fox} period={period} steps={S}", flush=True)
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype=dtype, seed=d + period)
    steps = synth.make_decode_steps(S, B, H, d, dtype=dtype, seed=d + period)
    gates = fox_gates(S, B, H, seed=period) if fox else None
    fc0 = initial_slot_bias(B, H, T0, cap, seed=period) if fox else None
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((B, H, cap, d), device="cuda", dtype=td)
    vc = torch.zeros_like(kc)
    kc[:, :, :T0] = dev(ck, dtype)
    vc[:, :, :T0] = dev(cv, dtype)
    fc = dev_f32(fc0) if fox else None
    go, gl, t_cur = run_deferred(kc, vc, fc, T0, steps, period, gates)
    BH = B * H
    okc, ovc = np.zeros((BH, cap, d)), np.zeros((BH, cap, d))
    okc[:, :T0] = ck.reshape(BH, T0, d)
    ovc[:, :T0] = cv.reshape(BH, T0, d)
    sh = lambda x: x.reshape(S, BH, -1) if x.ndim == 4 else x.reshape(S, BH)
    kw = dict(fcache=fc0.reshape(BH, cap).astype(np.float64), logf=sh(gates)) if fox else {}
    ro, rl = oracle.decode(okc, ovc, T0, sh(steps.q), sh(steps.k), sh(steps.v), sh(steps.w), sh(steps.beta),
                           steps.scale, **kw)
    assert_parity(go, ro.reshape(S, B, H, d), dtype, "out")
    assert_parity(gl, rl.reshape(S, B, H), dtype, "lse")
    # the last updating step left slots 0 .. t_cur - 1 current; the oracle's cache after that step
    assert t_cur > T0
    n_upd = t_cur - T0
    okc2, ovc2 = np.zeros((BH, cap, d)), np.zeros((BH, cap, d))
    okc2[:, :T0] = ck.reshape(BH, T0, d)
    ovc2[:, :T0] = cv.reshape(BH, T0, d)
    kw2 = dict(fcache=fc0.reshape(BH, cap).astype(np.float64), logf=sh(gates)[:n_upd]) if fox else {}
    oracle.decode(okc2, ovc2, T0, sh(steps.q)[:n_upd], sh(steps.k)[:n_upd], sh(steps.v)[:n_upd],
                  sh(steps.w)[:n_upd], sh(steps.beta)[:n_upd], steps.scale, **kw2)
    check_cache(host(kc)[:, :, :t_cur], okc2.reshape(B, H, cap, d)[:, :, :t_cur], dtype, n_upd)
    if fox:
        want = kw2["fcache"].reshape(B, H, cap)[:, :, :t_cur]
        got = host(fc)[:, :, :t_cur]
        bound = (n_upd + 1) * 2.0 ** -24 * np.max(np.abs(want)) + 1e-6
        assert np.max(np.abs(got - want)) <= bound


@pytest.mark.parametrize("fox", [False, True])
def test_deferred_period_one_is_the_in_place_step(fox):
    """period 1 updates the keys at every step: outputs and caches bit-identical to path_decode_step."""
    B, H, T0, S, d = 2, 2, 900, 4, 64
    cap = T0 + S
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype="bf16", seed=31)
    steps = synth.make_decode_steps(S, B, H, d, dtype="bf16", seed=31)
    gates = fox_gates(S, B, H, seed=31) if fox else None
    fc0 = initial_slot_bias(B, H, T0, cap, seed=31) if fox else None
    caches = []
    for deferred in (False, True):
        kc = torch.zeros((B, H, cap, d), device="cuda", dtype=torch.bfloat16)
        vc = torch.zeros_like(kc)
        kc[:, :, :T0] = dev(ck, "bf16")
        vc[:, :, :T0] = dev(cv, "bf16")
        fc = dev_f32(fc0) if fox else None
        if deferred:
            go, gl, _ = run_deferred(kc, vc, fc, T0, steps, 1, gates)
        else:
            outs, lses = [], []
            for s in range(S):
                o, l = native.path_decode_step(kc, vc, T0 + s, dev(steps.q[s], "bf16"), dev(steps.k[s], "bf16"),
                                               dev(steps.v[s], "bf16"), dev(steps.w[s], "bf16"),
                                               dev_f32(steps.beta[s]), dev_f32(gates[s]) if fox else None,
                                               fcache=fc, scale=steps.scale)
                outs.append(host(o))
                lses.append(host(l))
            go, gl = np.stack(outs), np.stack(lses)
        torch.cuda.synchronize()
        caches.append((go, gl, kc.view(torch.int16).cpu().numpy(), host(fc) if fox else None))
    a, b = caches
    assert np.array_equal(a[2], b[2]), "key caches differ"
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "outputs differ"
    if fox:
        assert np.array_equal(a[3], b[3])


def test_deferred_forced_update():
    """An update forced mid-period (period = t - t_cur + 1) leaves the cache current, like the oracle's."""
    B, H, T0, S, d, period = 1, 2, 300, 9, 64, 8
    cap = T0 + S
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype="bf16", seed=41)
    steps = synth.make_decode_steps(S, B, H, d, dtype="bf16", seed=41)
    kc = torch.zeros((B, H, cap, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :, :T0] = dev(ck, "bf16")
    vc[:, :, :T0] = dev(cv, "bf16")
    go, gl, t_cur = run_deferred(kc, vc, None, T0, steps, period, force_at=4)
    assert t_cur == T0 + 5
    BH = B * H
    okc, ovc = np.zeros((BH, cap, d)), np.zeros((BH, cap, d))
    okc[:, :T0] = ck.reshape(BH, T0, d)
    ovc[:, :T0] = cv.reshape(BH, T0, d)
    sh = lambda x: x.reshape(S, BH, -1) if x.ndim == 4 else x.reshape(S, BH)
    ro, rl = oracle.decode(okc, ovc, T0, sh(steps.q)[:5], sh(steps.k)[:5], sh(steps.v)[:5], sh(steps.w)[:5],
                           sh(steps.beta)[:5], steps.scale)
    assert_parity(go[:5], ro.reshape(5, B, H, d), "bf16", "out")
    # slots 0 .. T0 + 4 became current at the forced update (step 4); nothing updated them since
    check_cache(host(kc)[:, :, :T0 + 5], okc.reshape(B, H, cap, d)[:, :, :T0 + 5], "bf16", 5)


@pytest.mark.parametrize("dtype,period", [("bf16", 4), ("f32", 3)])
def test_deferred_decode_from_empty_equals_prefill(dtype, period):
    """Deferred decoding of S tokens from an empty cache reproduces prefill rows 0..S-1 (oracle prefill)."""
    B, H, S, d = 1, 3, 23, 64
    steps = synth.make_decode_steps(S, B, H, d, dtype=dtype, seed=7)
    kc = torch.zeros((B, H, S, d), device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    vc = torch.zeros_like(kc)
    go, gl, t_cur = run_deferred(kc, vc, None, 0, steps, period)
    assert t_cur == S - S % period
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))  # [S,B,H,...] -> [B,H,S,...]
    ro, rl = oracle.fwd(tr(steps.q), tr(steps.k), tr(steps.v), tr(steps.w), tr(steps.beta), scale=steps.scale)
    assert_parity(tr(go), ro, dtype, "out")
    assert_parity(tr(gl), rl, dtype, "lse")
