"""Parity of the prefill -> decode cache hand-off (path_attn_cache_from_prefill) against the fp64 oracle.

The oracle's cache slot j is H_{L-1} ... H_{j+1} k_j (PaTH summary, section 3, inference rule), pinned
in the oracle pins to explicit products, to the last row's logits and to the decode recurrence.  Here the
library's slots are compared with it, and a decode step taken from the handed-off cache is compared with
the oracle's prefill row at the same position.

Error bound of a slot (bf16 storage): the workspace holds ktilde rounded to bf16 (half an ulp, 2^-9
relative, per element) and the slot is rounded to bf16 once more; the chained chunk products have norm
at most 1 (every transition is a contraction for 0 <= beta <= 2 and unit w), so a slot's error in the
2-norm stays within a few 2^-9 of |k_j|.  With bf16 transport each chunk product also enters the matrix
cores rounded to bf16, which adds up to 2^-9 per chained chunk.  The fp32 path is held to 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from dependent_positional_attention_amd import native, synth
from tests.gpu_util import assert_parity, dev, dev_f32, errors, host

pytestmark = pytest.mark.gpu

SENTINEL = 7.0  # slots at and beyond L must keep it


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def prefill_cache(x, chunk, transport, cap, L=None, fox=False):
    """Prefill on the first L tokens of x, then fill caches of `cap` slots pre-set to SENTINEL
    (and, for PaTH-FoX, the slot biases)."""
    B, H, Lx, d = x.q.shape
    L = Lx if L is None else L
    cut = lambda a: np.ascontiguousarray(a[:, :, :L])
    t = {n: dev(cut(getattr(x, n)), x.dtype) for n in ("q", "k", "v", "w")}
    beta = dev_f32(cut(x.beta))
    logf = dev_f32(cut(x.logf)) if fox else None
    td = torch_dtype(x.dtype)
    nbytes = native.path_attn_fwd_workspace_bytes(B, H, L, d, chunk, td, transport)
    ws = torch.zeros(max(nbytes, 16), device="cuda", dtype=torch.uint8)
    out, lse = native.path_attn_fwd(t["q"], t["k"], t["v"], t["w"], beta, logf, scale=x.scale, chunk=chunk,
                                    transport=transport, workspace=ws)
    kc = torch.full((B, H, cap, d), SENTINEL, device="cuda", dtype=td)
    vc = torch.full_like(kc, SENTINEL)
    fc = torch.full((B, H, cap), SENTINEL, device="cuda", dtype=torch.float32) if fox else None
    native.path_attn_cache_from_prefill(t["v"], logf, workspace=ws, chunk=chunk, transport=transport, kcache=kc,
                                        vcache=vc, fcache=fc)
    torch.cuda.synchronize()
    t["fcache"] = fc
    return kc, vc, t, (out, lse)


def slot_bound(dtype, transport, L, chunk):
    if dtype == "f32":
        return 1e-5
    grain = 64 if chunk in (64, 128) else chunk
    chained = (L + grain - 1) // grain
    return (3 + (chained if transport == "bf16" else 0)) * 2.0 ** -9


def check_slots(got, want, k_in, dtype, transport, L, chunk, what="cache"):
    """got, want: [..., L, d] slots; k_in: the prompt keys (row norms bound the error)."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite slots"
    err = np.linalg.norm(got - want, axis=-1) / np.maximum(np.linalg.norm(k_in, axis=-1), 1e-30)
    bound = slot_bound(dtype, transport, L, chunk)
    assert err.max() <= bound, f"{what}: worst slot error {err.max():.3e} x |k_j| > {bound:.3e}"
    _, rel = errors(got, want)
    assert rel <= (1e-2 if dtype == "bf16" else 1e-5), f"{what}: rel_l2 {rel:.3e}"


def oracle_slots(x, L, heads=None, rows=None):
    B, H = x.q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    out = []
    for b, h in heads:
        K, W, beta = (np.ascontiguousarray(a[b, h, :L], dtype=np.float64) for a in (x.k, x.w, x.beta))
        if rows is None:
            out.append(oracle.cache_keys(K, W, beta))
        else:
            out.append(np.stack([oracle.cache_keys(K, W, beta, rows=(j, j + 1))[0] for j in rows]))
    return np.stack(out)


@pytest.mark.parametrize("dtype,d,chunk,transport,L,recipe", [
    ("bf16", 64, 64, "bf16", 300, "lm"),         # ragged tail, several chunks
    ("bf16", 64, 64, "bf16x3", 256, "lm"),
    ("bf16", 64, 64, "bf16x3", 512, "beta2"),    # norm-preserving transitions
    ("bf16", 64, 128, "bf16x3", 333, "lm"),      # 128-token chunks: the hand-off chains 64-token halves
    ("bf16", 64, 128, "bf16", 64, "lm"),         # one half-chunk
    ("bf16", 64, 64, "bf16", 1100, "lm"),        # 18 chunks: the chain cut into segments of 5, 5, 5, 3
    ("bf16", 64, 64, "bf16x3", 1100, "beta2"),   # the same, norm-preserving, bf16x3 segment products
    ("bf16", 64, 64, "bf16", 1, "lm"),           # one token: the slot is the key
    ("bf16", 32, 32, "bf16", 100, "lm"),         # vector path, bf16 storage
    ("f32", 64, 64, "bf16", 200, "lm"),          # vector path, fp32
    ("f32", 16, 16, "bf16", 77, "tiny"),
])
def test_cache_slots_match_oracle(dtype, d, chunk, transport, L, recipe):
    print(f"[case] handoff dtype={dtype} d={d} chunk={chunk} transport={transport} L={L} recipe={recipe}",
          flush=True)
    B, H = 2, 3
    x = synth.make_fwd_inputs(B, H, L, d, recipe=recipe, dtype=dtype, seed=L + d)
    cap = L + 9
    kc, vc, _, _ = prefill_cache(x, chunk, transport, cap)
    got_k, got_v = host(kc), host(vc)
    want = oracle_slots(x, L).reshape(B, H, L, d)
    check_slots(got_k[:, :, :L], want, x.k.astype(np.float64), dtype, transport, L, chunk)
    assert np.array_equal(got_v[:, :, :L], x.v.astype(np.float64)), "value slots are a copy"
    assert np.all(got_k[:, :, L:] == SENTINEL) and np.all(got_v[:, :, L:] == SENTINEL), "slots >= L touched"


@pytest.mark.parametrize("dtype,chunk,transport,L,S", [
    ("bf16", 64, "bf16", 1000, 3),
    ("bf16", 128, "bf16x3", 512, 2),
    ("f32", 64, "bf16", 130, 2),
])
def test_prefill_then_decode_matches_definition(dtype, chunk, transport, L, S):
    """Prompt of L tokens through prefill + hand-off, then S decode steps: rows L..L+S-1 of the oracle."""
    print(f"[case] prefill+decode dtype={dtype} chunk={chunk} transport={transport} L={L} S={S}", flush=True)
    B, H, d = 2, 2, 64
    x = synth.make_fwd_inputs(B, H, L + S, d, recipe="lm", dtype=dtype, seed=9)
    kc, vc, _, (pout, plse) = prefill_cache(x, chunk, transport, L + S, L=L)
    outs, lses = [], []
    for s in range(S):
        tok = lambda a: dev(np.ascontiguousarray(a[:, :, L + s]), dtype)
        o, l = native.path_decode_step(kc, vc, L + s, tok(x.q), tok(x.k), tok(x.v), tok(x.w),
                                       dev_f32(np.ascontiguousarray(x.beta[:, :, L + s])), scale=x.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    rows = list(range(L, L + S))
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, scale=x.scale, rows=rows)
    assert_parity(np.stack(outs, axis=2), ro, dtype, "decode out")
    assert_parity(np.stack(lses, axis=2), rl, dtype, "decode lse")
    # the prompt's own last row, for reference
    po, pl = oracle.fwd(x.q[:, :, :L], x.k[:, :, :L], x.v[:, :, :L], x.w[:, :, :L], x.beta[:, :, :L],
                        scale=x.scale, rows=[L - 1])
    assert_parity(host(pout)[:, :, L - 1:L], po, dtype, "prefill last row")


def sampled_slots(L, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 63, 64, 65, 127, 128, L // 2 - 1, L // 2, L - 65, L - 64, L - 2, L - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, L, size=18)]))


@pytest.mark.parametrize("B,H,L,chunk,transport,recipe", [
    (8, 24, 4096, 64, "bf16", "lm"),           # 760M-class layer, as the prefill bench runs it
    (1, 24, 32768, 128, "bf16x3", "lm"),       # long context, 128-token chunks
    (1, 24, 32768, 64, "bf16x3", "stress_qk_beta2"),
])
def test_full_size_handoff_sampled(B, H, L, chunk, transport, recipe):
    """Sampled slots of sampled heads at the full shapes, and one decode step at t = L from the cache."""
    print(f"[case] full handoff B={B} H={H} L={L} chunk={chunk} transport={transport} recipe={recipe}", flush=True)
    d = 64
    x = synth.make_fwd_inputs(B, H, L + 1, d, recipe=recipe, dtype="bf16", seed=1)
    kc, vc, t, _ = prefill_cache(x, chunk, transport, L + 1, L=L)
    # the value cache is an exact copy of the prompt's values
    assert torch.equal(vc[:, :, :L], t["v"])
    heads = [(0, 0), (B - 1, H - 1), (B // 2, 11)]
    rows = sampled_slots(L)
    got = np.stack([host(kc[b, h, rows]) for b, h in heads])
    want = oracle_slots(x, L, heads=heads, rows=rows)
    kin = np.stack([x.k[b, h, rows] for b, h in heads]).astype(np.float64)
    check_slots(got, want, kin, "bf16", transport, L, chunk, "sampled slots")
    # one decode step at t = L: the oracle's prefill row L on L + 1 tokens
    tok = lambda a: dev(np.ascontiguousarray(a[:, :, L]), "bf16")
    o, l = native.path_decode_step(kc, vc, L, tok(x.q), tok(x.k), tok(x.v), tok(x.w),
                                   dev_f32(np.ascontiguousarray(x.beta[:, :, L])), scale=x.scale)
    go, gl = host(o), host(l)
    for b, h in heads:
        sl = lambda a: a[b:b + 1, h:h + 1]
        ro, rl = oracle.fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.w), sl(x.beta), scale=x.scale, rows=[L])
        assert_parity(go[b, h], ro[0, 0, 0], "bf16", f"decode out head {(b, h)}")
        assert_parity(gl[b, h], rl[0, 0, 0], "bf16", f"decode lse head {(b, h)}")


@pytest.mark.parametrize("dtype,chunk,transport,L,S", [
    ("bf16", 64, "bf16", 700, 3),
    ("bf16", 128, "bf16x3", 4096, 2),
    ("f32", 32, "bf16", 150, 2),
])
def test_fox_prefill_then_decode(dtype, chunk, transport, L, S):
    """PaTH-FoX prompt: slot biases are the suffix sums of the prompt's gates, and FoX decode from the handed-off
    cache gives the oracle's FoX prefill rows L..L+S-1."""
    print(f"[case] fox prefill+decode dtype={dtype} chunk={chunk} transport={transport} L={L} S={S}", flush=True)
    B, H = 2, 2
    d = 64 if dtype == "bf16" else 32
    x = synth.make_fwd_inputs(B, H, L + S, d, recipe="fox", dtype=dtype, seed=21)
    kc, vc, t, _ = prefill_cache(x, chunk, transport, L + S, L=L, fox=True)
    fc = t["fcache"]
    got = host(fc)
    for b in range(B):
        for h in range(H):
            want = oracle.cache_bias(x.logf[b, h, :L])
            bound = 1e-5 * np.sum(np.abs(x.logf[b, h, :L])) + 1e-7
            err = np.max(np.abs(got[b, h, :L] - want))
            assert err <= bound, f"slot bias head {(b, h)}: {err:.3e} > {bound:.3e}"
    assert np.all(got[:, :, L:] == SENTINEL)
    outs, lses = [], []
    for s in range(S):
        tok = lambda a: dev(np.ascontiguousarray(a[:, :, L + s]), dtype)
        o, l = native.path_decode_step(kc, vc, L + s, tok(x.q), tok(x.k), tok(x.v), tok(x.w),
                                       dev_f32(np.ascontiguousarray(x.beta[:, :, L + s])),
                                       dev_f32(np.ascontiguousarray(x.logf[:, :, L + s])), fcache=fc, scale=x.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf, scale=x.scale, rows=list(range(L, L + S)))
    assert_parity(np.stack(outs, axis=2), ro, dtype, "fox decode out")
    assert_parity(np.stack(lses, axis=2), rl, dtype, "fox decode lse")


@pytest.mark.parametrize("fox,period", [(False, 4), (True, 3)])
def test_prefill_then_deferred_decode(fox, period):
    """Prompt through prefill + hand-off, then decode with deferred key updates: rows L..L+S-1 of the oracle."""
    B, H, d, L, S = 2, 2, 64, 640, 9
    print(f"[case] prefill+deferred decode fox={fox} period={period} L={L} S={S}", flush=True)
    x = synth.make_fwd_inputs(B, H, L + S, d, recipe="fox" if fox else "lm", dtype="bf16", seed=13)
    kc, vc, t, _ = prefill_cache(x, 64, "bf16", L + S, L=L, fox=fox)
    fc = t["fcache"]
    state = torch.zeros(native.path_decode_deferred_state_bytes(B, H, d) // 4, device="cuda", dtype=torch.float32)
    outs, lses, t_cur = [], [], L
    for s in range(S):
        tok = lambda a: dev(np.ascontiguousarray(a[:, :, L + s]), "bf16")
        f = dev_f32(np.ascontiguousarray(x.logf[:, :, L + s])) if fox else None
        o, l, t_cur = native.path_decode_step_deferred(
            kc, vc, L + s, t_cur, tok(x.q), tok(x.k), tok(x.v), tok(x.w),
            dev_f32(np.ascontiguousarray(x.beta[:, :, L + s])), f, period=period, state=state, fcache=fc,
            scale=x.scale)
        outs.append(host(o))
        lses.append(host(l))
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(x.q, x.k, x.v, x.w, x.beta, logf=x.logf if fox else None, scale=x.scale,
                        rows=list(range(L, L + S)))
    assert_parity(np.stack(outs, axis=2), ro, "bf16", "deferred decode out")
    assert_parity(np.stack(lses, axis=2), rl, "bf16", "deferred decode lse")
