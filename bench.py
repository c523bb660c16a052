#!/usr/bin/env python3
"""PaTH attention benchmark on one MI355X.

Prefill workload (the line's `value`): the 760M-class layer, B=8, H=24, L=4096,
d=64, chunk 64, bf16 inputs with fp32 accumulation, synthetic seeded inputs
(q,k,v ~ N(0,1)/sqrt(d), unit Gaussian w, beta = 2*sigmoid(N(0,1.5))).  One
step = one path_attn_fwd call (per-chunk prep + attention scan) over inputs
already resident in HBM; value = B*L / step time, in tokens/s.

Also reported on the same JSON line:
  roofline      the whole path_attn_fwd call (per-chunk prep + attention scan),
                timed with HIP events on the stream it runs on: algorithmic flops
                per call (4 d L(L+1)/2 B H for QK^T and PV over the causal pairs,
                plus 2 C d^2 (M-1)(M-2)/2 B H for the chunk-to-chunk query
                transport) over the measured call time, against the bf16 MFMA
                peak.  The scan kernel alone, and the attention flops alone, are
                detail fields.
  cpu_baseline  the fp64 CPU oracle timed on this host over a bounded sample of
                the same workload (whole heads), scaled to tokens/s.
  decode        batch 32, H=24, d=64, 65536 cached tokens, 128 steps timed back
                to back: HBM bytes the step must move (cached keys read and
                written back, cached values read) over the measured time.
  fox_prefill   the PaTH-FoX prefill at the same shape (adds log-forget gates): step and scan.
  chunk_sweep   the same prefill step at chunk 64, 128 and 256 (chunks above 64 are grouped
                64-token sub-chunks; the scan moves its queries once per chunk).
  cache_handoff the prefill workspace turned into a decode cache (path_attn_cache_from_prefill)
                at the prefill shape: time and HBM bytes it must move.
  long_context  B=1, H=24, L=32768: whole prefill step at chunk 64, 128 and
                256 (transport once per chunk), tokens/s and the fraction of
                bf16 peak for each chunk size's own flop count; with the chunk
                sweep at L=4096 this is the table chunk = 0 follows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk/CU, dense
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="prefill warm-up runs at least this long (and at least --warmup steps)")
    ap.add_argument("--transport", default="bf16", choices=["bf16", "bf16x3"])
    ap.add_argument("--fox", action="store_true", help="PaTH-FoX prefill (log-forget gates) instead of PaTH")
    ap.add_argument("--L", type=int, default=4096)
    ap.add_argument("--B", type=int, default=8)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--decode-cache", type=int, default=65536)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 32K-token prefill at chunk 64 and 128")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the chunk 64 / 128 / 256 comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (a known-size reference for HBM counters)")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_B8_H24_L4096_d64_hbm_counters.md")
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_B32_H24_T65536_d64_hbm_counters.md")


def kernel_digest(*sources):
    """Digest of kernel sources (ties HBM counter readings to the code they measured)."""
    import hashlib
    h = hashlib.sha256()
    for f in sources + ("common.h", "tiles.h"):
        with open(os.path.join(ROOT, "dependent_positional_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path, kernel, source):
    """HBM bytes per launch (read + written) of `kernel` from a committed rocprofv3 counter summary,
    or None when there is none or the kernel source has changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    digest = kernel_digest(source)
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic ") and f"kernel={kernel} " in line:
                kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t and not t.startswith("kernel="))
                if kv.get("source_digest") == digest:
                    return float(kv["read_bytes"]) + float(kv["write_bytes"])
    return None


def prefill_flops(B, H, L, d, C):
    M = -(-L // C)
    return 4.0 * d * (L * (L + 1) / 2) * B * H + 2.0 * C * d * d * ((M - 1) * (M - 2) / 2) * B * H


def warm_up(fn, steps, seconds):
    """Run fn at least `steps` times and for at least `seconds` (synchronising every 10 calls so that the
    time is the GPU's): the clock of an idle GPU takes ~20 ms of work to settle."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < steps or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed(fn, n):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_prefill(args):
    import torch
    from dependent_positional_attention_amd import native, synth

    B, H, L, d, C = args.B, 24, args.L, 64, 64
    recipe = "fox" if args.fox else "lm"
    log(f"[bench] generating prefill inputs B={B} H={H} L={L} d={d} recipe={recipe}")
    x = synth.make_fwd_inputs(B, H, L, d, recipe=recipe, dtype="bf16", seed=0)

    def dev_bf16(a):
        return torch.from_numpy(synth.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()

    q, k, v, w = (dev_bf16(getattr(x, n)) for n in ("q", "k", "v", "w"))
    beta = torch.from_numpy(x.beta).cuda()
    logf = torch.from_numpy(x.logf).cuda() if x.logf is not None else None
    nbytes = native.path_attn_fwd_workspace_bytes(B, H, L, d, C, torch.bfloat16, args.transport)
    ws = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), device="cuda", dtype=torch.float32)

    def step():
        native.path_attn_fwd(q, k, v, w, beta, logf, scale=x.scale, chunk=C, transport=args.transport, out=out,
                             lse=lse, workspace=ws)

    def prep():
        native.path_attn_prep(q, k, v, w, beta, logf, scale=x.scale, chunk=C, transport=args.transport,
                              workspace=ws)

    def scan():
        native.path_attn_scan(v, logf, chunk=C, transport=args.transport, workspace=ws, out=out,
                              lse=lse)

    # at least W warm-up steps, and at least --min-warmup-s seconds of them: on a freshly started GPU the
    # clock settles over the first ~20 steps (~20 ms), which a short warm-up would leave in the timed region
    n_warm = warm_up(step, args.warmup, args.min_warmup_s)
    log(f"[bench] prefill warmup done ({n_warm} steps); timing {args.steps} steps")
    t0 = time.perf_counter()
    ms_step = timed(step, args.steps)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # the dominant kernel alone (scan), and the prep alone, same stream, same workspace
    prep()
    ms_prep = timed(prep, args.steps)
    ms_scan = timed(scan, args.steps)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite output"
    F = prefill_flops(B, H, L, d, C)
    tflops = F / (ms_scan * 1e-3) / 1e12
    step_tf = F / (ms_step * 1e-3) / 1e12
    log(f"[bench] prefill: step {ms_step:.3f} ms (wall {wall_ms:.3f}) = {step_tf:.1f} TFLOP/s = "
        f"{step_tf / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 peak (whole call); prep alone {ms_prep:.3f} ms, "
        f"scan alone {ms_scan:.3f} ms = {tflops / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 peak")
    res = dict(B=B, H=H, L=L, d=d, C=C, recipe=recipe, warmup_steps_run=n_warm, ms_step=ms_step, wall_ms=wall_ms,
               ms_prep=ms_prep,
               ms_scan=ms_scan, flops=F, scan_tflops=tflops, tokens_per_s=B * L / (ms_step * 1e-3))
    return res, x, dict(q=q, k=k, v=v, w=w, beta=beta, logf=logf, scale=x.scale, ws=ws, out=out, lse=lse)


def backward_flops(B, H, L, d, C):
    """Algorithmic flops of the backward: the five attention products (logits, dO V^T, dV, dK, dQ:
    2.5x the forward's two) and, per chunk pair crossed, three d x d transports (the kept state, its
    gradient, and the reduction into dP)."""
    M = -(-L // C)
    return 2.5 * 4.0 * d * (L * (L + 1) / 2) * B * H + 3 * 2.0 * C * d * d * ((M - 1) * (M - 2) / 2) * B * H


def bench_backward(args, res, ctx):
    """Gradients of the prefill just timed (same inputs, its out and lse), for a Gaussian upstream gradient."""
    import torch
    from dependent_positional_attention_amd import native, synth

    q, k, v, w, beta, logf, scale, out, lse = (ctx[n] for n in ("q", "k", "v", "w", "beta", "logf", "scale", "out",
                                                                  "lse"))
    B, H, L, d = q.shape
    C = 64
    dout = torch.from_numpy(synth.bf16_bits(synth.make_out_grad((B, H, L, d), dtype="bf16", seed=0)).view("int16")
                            ).view(torch.bfloat16).cuda()
    nbytes = native.path_attn_bwd_workspace_bytes(B, H, L, d, C, torch.bfloat16)
    ws = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
             torch.empty((B, H, L), device="cuda", dtype=torch.float32),
             None if logf is None else torch.empty((B, H, L), device="cuda", dtype=torch.float32))

    def run():
        native.path_attn_bwd(q, k, v, w, beta, out, lse, dout, logf, scale=scale, chunk=C, workspace=ws, grads=grads)

    # warm up as the prefill does (the clock settles over the first runs): at least 3 calls and 0.3 s
    t0, runs = time.perf_counter(), 0
    while runs < 3 or time.perf_counter() - t0 < 0.3:
        run()
        torch.cuda.synchronize()
        runs += 1
    n = 5
    ms = timed(run, n)
    for g in grads:
        if g is not None:
            assert torch.isfinite(g.float()).all(), "non-finite gradient"
    F = backward_flops(B, H, L, d, C)
    tf = F / (ms * 1e-3) / 1e12
    x3_peak = MFMA_BF16_PEAK_TFLOPS / 3  # fp32-accurate products as three bf16 products (hi.hi + hi.lo + lo.hi)
    log(f"[bench] backward: {ms:.2f} ms, {B * L / (ms * 1e-3) / 1e6:.3f} M tokens/s, {tf:.2f} TFLOP/s = "
        f"{tf / MFMA_BF16_PEAK_TFLOPS:.3f} of the dense bf16 peak, {tf / x3_peak:.3f} of the bf16x3 peak "
        f"(workspace {nbytes / 2**30:.1f} GiB)")
    del ws
    return {"workload": f"PaTH backward, B={B}, H={H}, L={L}, d={d}, chunk {C}, bf16 in/out, fp32 accumulation",
            "ms": ms, "steps": n, "tokens_per_s": B * L / (ms * 1e-3), "flops": F, "tflops": tf, "bound": "mfma",
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
            "bf16x3_peak": x3_peak, "frac_of_bf16x3_peak": tf / x3_peak,
            "note": "the products run on the bf16 matrix cores (bf16 operands exact, p and dz rounded to bf16 "
                    "once, other fp32 operands split into hi+lo), so peak = dense bf16 peak; bf16x3_peak = bf16 peak / 3 (an fp32-accurate "
                    "product as three bf16 products)",
            "workspace_bytes": nbytes}


def bench_handoff(args, res, ctx):
    """Prefill -> decode cache hand-off from the prefill workspace just timed (same shape and chunk)."""
    import torch
    from dependent_positional_attention_amd import native

    B, H, L, d, C = res["B"], res["H"], res["L"], res["d"], res["C"]
    v, ws = ctx["v"], ctx["ws"]
    kc = torch.empty((B, H, L, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.empty_like(kc)

    def run():
        native.path_attn_cache_from_prefill(v, workspace=ws, chunk=C, transport=args.transport, kcache=kc,
                                            vcache=vc)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ms = timed(run, args.steps)
    assert torch.isfinite(kc.float()).all(), "non-finite cache"
    # bytes the hand-off must move: ktilde, the chunk products (hi, + lo for bf16x3) and the values read,
    # both caches written
    M = -(-L // 64)
    p_parts = 2 if args.transport == "bf16x3" else 1
    nbytes = B * H * (L * d * 2 + M * d * d * 2 * p_parts + L * d * 2 + 2 * L * d * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] cache hand-off: {ms * 1e3:.1f} us, {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of HBM peak "
        f"({M} chained 64-token chunks per head)")
    return {"workload": f"prefill -> decode cache hand-off, B={B}, H={H}, L={L}, d={d}, chunk {C}, bf16",
            "ms": ms, "bytes": nbytes, "achieved_gbs": gbs, "peak_gbs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
            "chained_steps_per_head": M}


def bench_fox(args, ctx):
    """PaTH-FoX prefill at the same shape (the same q, k, v, w, beta plus log-forget gates
    logsigmoid(N(3, 1))): whole step and the scan alone, interleaved round by round with the plain
    PaTH step on the same inputs (median of 3 rounds of 10 steps each) so that both see the same clock."""
    import numpy as np
    import torch
    from dependent_positional_attention_amd import native, synth

    q, k, v, w, beta, scale, ws = (ctx[n] for n in ("q", "k", "v", "w", "beta", "scale", "ws"))
    B, H, L, d = q.shape
    C = 64
    logf = torch.from_numpy(synth.logsigmoid(synth._normal(0, "logf", (B, H, L), 1.0, 3.0)).astype(np.float32)).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), device="cuda", dtype=torch.float32)

    def step(f):
        native.path_attn_fwd(q, k, v, w, beta, f, scale=scale, chunk=C, transport=args.transport, out=out,
                             lse=lse, workspace=ws)

    def scan(f):
        native.path_attn_scan(v, f, chunk=C, transport=args.transport, workspace=ws, out=out, lse=lse)

    warm_up(lambda: step(logf), 10, args.min_warmup_s)
    t = {"fox": [], "plain": [], "fox_scan": [], "plain_scan": []}
    for _ in range(3):
        t["fox"].append(timed(lambda: step(logf), 10))
        t["plain"].append(timed(lambda: step(None), 10))
        t["fox_scan"].append(timed(lambda: scan(logf), 10))
        t["plain_scan"].append(timed(lambda: scan(None), 10))
    med = {key: sorted(v_)[1] for key, v_ in t.items()}
    step(logf)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite FoX output"
    ms, ms_scan = med["fox"], med["fox_scan"]
    F = prefill_flops(B, H, L, d, C)
    tf = F / (ms_scan * 1e-3) / 1e12
    log(f"[bench] PaTH-FoX prefill: step {ms:.3f} ms, {B * L / (ms * 1e-3) / 1e6:.2f} M tokens/s "
        f"({ms / med['plain']:.3f}x the plain step's {med['plain']:.3f} ms, interleaved); scan {ms_scan:.3f} ms "
        f"= {tf / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 peak ({ms_scan / med['plain_scan']:.3f}x the plain scan)")
    return {"workload": f"PaTH-FoX prefill forward, B={B}, H={H}, L={L}, d={d}, chunk {C}, bf16, "
                        f"transport {args.transport}; median of 3 rounds of 10 steps, interleaved with the plain step",
            "ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3),
            "scan_ms": ms_scan, "scan_tflops": tf, "scan_frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS,
            "plain_ms_per_step_interleaved": med["plain"], "ratio_to_plain": ms / med["plain"],
            "plain_scan_ms_interleaved": med["plain_scan"], "scan_ratio_to_plain": ms_scan / med["plain_scan"]}


def bench_chunks(args, ctx):
    """Whole prefill step at chunk 64, 128 and 256 on the same inputs, interleaved round by round so
    that clock drift treats every chunk size alike."""
    import torch
    from dependent_positional_attention_amd import native

    q, k, v, w, beta, logf, scale = (ctx[n] for n in ("q", "k", "v", "w", "beta", "logf", "scale"))
    B, H, L, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), device="cuda", dtype=torch.float32)
    chunks = (64, 128, 256)
    wss = {C: torch.empty(native.path_attn_fwd_workspace_bytes(B, H, L, d, C, torch.bfloat16, args.transport),
                          device="cuda", dtype=torch.uint8) for C in chunks}
    steps = {C: (lambda C=C: native.path_attn_fwd(q, k, v, w, beta, logf, scale=scale, chunk=C,
                                                  transport=args.transport, out=out, lse=lse, workspace=wss[C]))
             for C in chunks}
    times = {C: [] for C in chunks}
    for C in chunks:
        warm_up(steps[C], 2, args.min_warmup_s / 3)
    for _ in range(4):
        for C in chunks:
            times[C].append(timed(steps[C], 5))
    res = {}
    for C in chunks:
        ms = sorted(times[C])[len(times[C]) // 2]
        res[f"chunk{C}"] = {"ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3)}
        log(f"[bench] chunk sweep: chunk {C}: {ms:.3f} ms per step, {B * L / (ms * 1e-3) / 1e6:.2f} M tokens/s")
    return {"workload": f"PaTH prefill step at B={B}, H={H}, L={L}, d={d}, bf16, transport {args.transport}; "
                        "median of 4 interleaved rounds of 5 steps", "auto_chunk": auto_chunk(B, H, L, d), **res}


def bench_cpu(x, args):
    import numpy as np
    import oracle

    B, H, L, d = x.q.shape
    cores = oracle.host_threads()
    # calibrate on 2 heads, then size the sample to about args.cpu_seconds
    heads = [(0, 0), (0, 1)]

    def run(hs):
        sel = lambda a: np.stack([a[b, h] for b, h in hs])
        t0 = time.perf_counter()
        oracle.fwd(sel(x.q), sel(x.k), sel(x.v), sel(x.w), sel(x.beta),
                   logf=None if x.logf is None else sel(x.logf), scale=x.scale, nthreads=cores)
        return time.perf_counter() - t0

    t = run(heads)
    per_head = t / len(heads)
    n = int(max(1, min(B * H, args.cpu_seconds / max(per_head, 1e-3))))
    hs = [divmod(i, H) for i in range(n)]
    t = run(hs)
    scale = (B * H) / n
    tok_s = B * L / (t * scale)
    # one head on one thread (the oracle's serial cost)
    t0 = time.perf_counter()
    oracle.fwd(x.q[0, :1], x.k[0, :1], x.v[0, :1], x.w[0, :1], x.beta[0, :1],
               logf=None if x.logf is None else x.logf[0, :1], scale=x.scale, nthreads=1)
    t1 = time.perf_counter() - t0
    model = cpu_model()
    log(f"[bench] cpu oracle: {n} of {B * H} heads (all {L} rows each) in {t:.2f} s on {cores} threads "
        f"-> {tok_s:.1f} tokens/s for the full workload; one head on one thread {t1:.2f} s ({model})")
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {B * H} (batch, head) slices, every one of the {L} query rows, fp64; "
                      f"time scaled by {scale:.2f} to the full B={B}, H={H} workload",
            "seconds": t, "cpu_model": model, "single_thread_one_head_s": t1}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def auto_chunk(B, H, L, d):
    """The chunk path_attn_fwd uses for chunk = 0 (from the workspace layout it plans)."""
    import torch
    from dependent_positional_attention_amd import native
    lay = native.path_attn_workspace_layout(B, H, L, d, 0, torch.bfloat16, "bf16")
    return 64 if lay.layout_id == 1 else -(-L // lay.num_chunks)


def bench_long(args):
    """Long-context prefill (B=1, H=24, L=32768, d=64, bf16): whole step at chunk 64, 128 and 256, interleaved
    round by round (median of 3 rounds of 3 steps), each against its own flop count."""
    import torch
    from dependent_positional_attention_amd import native, synth

    B, H, L, d = 1, 24, 32768, 64
    log(f"[bench] long context: generating inputs B={B} H={H} L={L} d={d}")
    x = synth.make_fwd_inputs(B, H, L, d, recipe="lm", dtype="bf16", seed=0)

    def dev_bf16(a):
        return torch.from_numpy(synth.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()

    q, k, v, w = (dev_bf16(getattr(x, n)) for n in ("q", "k", "v", "w"))
    beta = torch.from_numpy(x.beta).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), device="cuda", dtype=torch.float32)
    chunks = (64, 128, 256)
    wss = {C: torch.empty(native.path_attn_fwd_workspace_bytes(B, H, L, d, C, torch.bfloat16, args.transport),
                          device="cuda", dtype=torch.uint8) for C in chunks}
    steps = {C: (lambda C=C: native.path_attn_fwd(q, k, v, w, beta, None, scale=x.scale, chunk=C,
                                                  transport=args.transport, out=out, lse=lse, workspace=wss[C]))
             for C in chunks}
    for C in chunks:
        warm_up(steps[C], 2, args.min_warmup_s / 3)
    times = {C: [] for C in chunks}
    for _ in range(3):
        for C in chunks:
            times[C].append(timed(steps[C], 3))
    res = {}
    for C in chunks:
        ms = sorted(times[C])[len(times[C]) // 2]
        F = prefill_flops(B, H, L, d, C)
        tf = F / (ms * 1e-3) / 1e12
        log(f"[bench] long context chunk {C}: step {ms:.3f} ms, {B * L / (ms * 1e-3) / 1e6:.2f} M tokens/s, "
            f"{tf:.1f} TFLOP/s = {tf / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 peak (whole step, own flop count)")
        res[f"chunk{C}"] = {"ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3), "flops": F, "tflops": tf,
                            "frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS}
    # prompt -> decode hand-off from the chunk-64 workspace (its last step above left the per-chunk terms)
    steps[64]()
    kc = torch.empty((B, H, L, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    hand = lambda: native.path_attn_cache_from_prefill(v, None, workspace=wss[64], capacity=L, chunk=64,
                                                       transport=args.transport, kcache=kc, vcache=vc)
    hand()
    torch.cuda.synchronize()
    ms_h = timed(hand, 10)
    nbytes = B * H * (L // 64) * 40 * 1024  # ktilde, P, V read and the K, V slots written, per 64-token chunk
    gbs = nbytes / (ms_h * 1e-3) / 1e9
    log(f"[bench] long context hand-off: {ms_h * 1e3:.1f} us, {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of HBM peak "
        f"(each head's {L // 64}-chunk chain cut into segments)")
    res["cache_handoff"] = {"ms": ms_h, "bytes": nbytes, "achieved_gbs": gbs, "peak_gbs": HBM_PEAK_GBS,
                            "frac": gbs / HBM_PEAK_GBS}
    del wss, kc, vc
    return {"workload": "PaTH prefill, long context: B=1, H=24, L=32768, d=64, bf16, transport " + args.transport
                        + "; median of 3 interleaved rounds of 3 steps",
            "transport": args.transport, "auto_chunk": auto_chunk(B, H, L, d), **res}


def bench_decode(args):
    import numpy as np
    import torch
    from dependent_positional_attention_amd import native, synth

    Bd, H, d = 32, 24, 64
    T0, S = args.decode_cache, args.decode_steps
    W = 3
    cap = T0 + 2 * S  # room for the deferred-update steps that follow the timed in-place ones
    log(f"[bench] decode: batch {Bd}, H {H}, d {d}, cache {T0}, {S} steps; filling the cache on the GPU")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    kc = torch.empty((Bd, H, cap, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    for b in range(Bd):  # N(0,1)/sqrt(d) drawn on the device, one batch row at a time
        kc[b] = (torch.randn((H, cap, d), device="cuda", generator=gen) / math.sqrt(d)).to(torch.bfloat16)
        vc[b] = (torch.randn((H, cap, d), device="cuda", generator=gen) / math.sqrt(d)).to(torch.bfloat16)
    st = synth.make_decode_steps(S + W, Bd, H, d, dtype="bf16", seed=0)

    def dev_bf16(a):
        return torch.from_numpy(synth.bf16_bits(a).view("int16")).view(torch.bfloat16).cuda()

    qs, ks, vs, wsd = (dev_bf16(getattr(st, n)) for n in ("q", "k", "v", "w"))
    betas = torch.from_numpy(st.beta).cuda()
    out = torch.empty((Bd, H, d), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((Bd, H), device="cuda", dtype=torch.float32)
    wsb = torch.empty(native.path_decode_workspace_bytes(Bd, H, d, cap), device="cuda", dtype=torch.uint8)

    def step(i, t):
        native.path_decode_step(kc, vc, t, qs[i], ks[i], vs[i], wsd[i], betas[i], scale=st.scale, out=out, lse=lse,
                                workspace=wsb)

    for i in range(W):
        step(i, T0 - W + i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(S):
        step(W + i, T0 + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    # bytes the step must move: cached keys read + written back, cached values read (t keys each),
    # plus the new token's q, k, v, w read and its k, v written
    nbytes = sum(Bd * H * (3 * (T0 + i) * d * 2 + 6 * d * 2) for i in range(S))
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode: {S} steps in {ms:.2f} ms ({ms / S:.3f} ms/step), {gbs:.0f} GB/s "
        f"= {gbs / HBM_PEAK_GBS:.3f} of HBM peak")
    # the same steps with the key updates deferred (period 16), continuing from the cache just left
    P = 16
    state = torch.zeros(native.path_decode_deferred_state_bytes(Bd, H, d) // 4, device="cuda", dtype=torch.float32)
    t_cur = T0 + S
    tdef = T0 + S
    ndef = min(S, cap - tdef)
    dbytes, ms_def = 0, float("nan")
    if ndef >= P:
        ndef -= ndef % P
        e0.record()
        for i in range(ndef):
            t = tdef + i
            _, _, t_cur = native.path_decode_step_deferred(kc, vc, t, t_cur, qs[i % (S + W)], ks[i % (S + W)],
                                                           vs[i % (S + W)], wsd[i % (S + W)], betas[i % (S + W)],
                                                           period=P, state=state, scale=st.scale, out=out, lse=lse,
                                                           workspace=wsb)
        e1.record()
        torch.cuda.synchronize()
        ms_def = e0.elapsed_time(e1)
        dbytes = sum(Bd * H * (((3 if (i + 1) % P == 0 else 2) * (tdef + i)) * d * 2 + 6 * d * 2) for i in range(ndef))
        log(f"[bench] decode, key updates deferred (period {P}): {ndef} steps in {ms_def:.2f} ms "
            f"({ms_def / ndef:.3f} ms/step, {ms / S / (ms_def / ndef):.2f}x the in-place step), "
            f"{dbytes / (ms_def * 1e-3) / 1e9:.0f} GB/s")
    deferred = None if not ndef >= P else {
        "period": P, "steps": ndef, "ms_per_step": ms_def / ndef, "speedup_vs_in_place": (ms / S) / (ms_def / ndef),
        "achieved_gbs": dbytes / (ms_def * 1e-3) / 1e9,
        "note": "keys brought up to date every 16 steps; between updates the query is moved instead (same outputs)"}
    return {"metric": "PaTH decode step HBM GB/s at 64K cache", "value": gbs, "unit": "GB/s",
            "ms_per_step": ms / S, "steps": S, "deferred_updates": deferred,
            "config": {"workload": "decode batch 32 x 24 heads, d=64, bf16 cache of 65536 tokens growing by 1/step",
                       "batch": Bd, "heads": H, "d": d, "cache_tokens": T0},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(DECODE_COUNTERS, "decode_update_attend_kernel", "decode.hip"),
                         "traffic_unit": "bytes per update+attend launch",
                         "kernel": "decode update+attend and combine, whole step"}}


def measure_peaks(args):
    """Ceilings measured on this GPU, beside the published ones: a large bf16 GEMM through the vendor
    library (hipBLASLt via torch.mm; dense, contiguous operands) for the matrix cores, and a plain 2 GiB
    device copy for HBM (bytes read + written over time).  The kernels' fractions are also reported
    against these."""
    import torch
    n = 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    a = torch.randn((n, n), device="cuda", dtype=torch.float32, generator=gen).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.float32, generator=gen).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.mm(a, b, out=c)
    ms_mm = timed(lambda: torch.mm(a, b, out=c), 20)
    gemm = 2.0 * n ** 3 / (ms_mm * 1e-3) / 1e12
    del a, b, c
    nbytes = 2 << 30
    src = torch.ones(nbytes, device="cuda", dtype=torch.uint8)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms_cp = timed(lambda: dst.copy_(src), 10)
    copy = 2.0 * nbytes / (ms_cp * 1e-3) / 1e9
    del src, dst
    log(f"[bench] measured ceilings: bf16 GEMM {n}^3 {gemm:.0f} TFLOP/s ({gemm / MFMA_BF16_PEAK_TFLOPS:.3f} of the "
        f"published peak), 2 GiB device copy {copy:.0f} GB/s ({copy / HBM_PEAK_GBS:.3f})")
    return {"bf16_gemm_tflops": gemm, "gemm": f"torch.mm bf16 {n}x{n}x{n} (hipBLASLt)", "copy_gbs": copy,
            "copy": "2 GiB device-to-device copy, read + write bytes"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures PaTH attention on ONE MI355X: this library has no multi-GPU path, so "
              "--gpus N with N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done (3 dispatches)")
        del src, dst
    res, x, ctx = bench_prefill(args)
    handoff = bench_handoff(args, res, ctx)
    sweep = None if args.no_sweep else bench_chunks(args, ctx)
    fox = None if (args.no_sweep or args.fox) else bench_fox(args, ctx)
    bwd = None if args.no_backward else bench_backward(args, res, ctx)
    del ctx
    cpu = None if args.no_cpu else bench_cpu(x, args)
    dec = None if args.no_decode else bench_decode(args)
    long_ctx = None if args.no_long else bench_long(args)
    peaks = measure_peaks(args)
    F = res["flops"]
    achieved = F / (res["ms_step"] * 1e-3) / 1e12
    scan_tf = F / (res["ms_scan"] * 1e-3) / 1e12
    B_, H_, L_, d_ = res["B"], res["H"], res["L"], res["d"]
    attn_flops = 4.0 * d_ * (L_ * (L_ + 1) / 2) * B_ * H_
    ktag = "<{},{},1,2,4>".format("true" if args.fox else "false", "true" if args.transport == "bf16x3" else "false")
    ptag = "<{}>".format("true" if args.transport == "bf16x3" else "false")
    t_scan = measured_traffic(PREFILL_COUNTERS, "mfma_attn_kernel" + ktag, "mfma_path.hip")
    t_prep = measured_traffic(PREFILL_COUNTERS, "mfma_prep_kernel" + ptag, "mfma_path.hip")
    line = {
        "metric": "PaTH fwd tokens/s + MFMA TFLOPS% at L=4096; decode GB/s% at 64K cache",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"PaTH{'-FoX' if args.fox else ''} prefill forward, 760M-class layer",
                   "B": res["B"], "H": res["H"], "L": res["L"], "d": res["d"], "chunk": res["C"],
                   "transport": args.transport, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None if t_scan is None or t_prep is None else t_scan + t_prep,
                     "traffic_unit": "HBM bytes per path_attn_fwd call (prep + scan kernels)",
                     "kernel": "path_attn_fwd = mfma_prep_kernel + mfma_attn_kernel",
                     "launch_ms": res["ms_step"], "flops_per_launch": F,
                     "frac_of_measured_gemm": achieved / peaks["bf16_gemm_tflops"],
                     "attention_flops_per_launch": attn_flops,
                     "attention_only_frac": attn_flops / (res["ms_step"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "scan_only": {"kernel": "mfma_attn_kernel", "launch_ms": res["ms_scan"], "achieved": scan_tf,
                                   "frac": scan_tf / MFMA_BF16_PEAK_TFLOPS, "traffic": t_scan},
                     "prep_only": {"kernel": "mfma_prep_kernel", "launch_ms": res["ms_prep"], "traffic": t_prep}},
        "prefill_detail": {"ms_prep": res["ms_prep"], "ms_scan": res["ms_scan"], "wall_ms_per_step": res["wall_ms"],
                           "warmup_steps_run": res["warmup_steps_run"],
                           "step_tflops": F / (res["ms_step"] * 1e-3) / 1e12,
                           "step_frac_of_peak": F / (res["ms_step"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "decode": dec,
        "cache_handoff": handoff,
        "chunk_sweep": sweep,
        "fox_prefill": fox,
        "backward": bwd,
        "long_context": long_ctx,
        "measured_ceilings": peaks,
    }
    if dec is not None:
        dec["roofline"]["frac_of_measured_copy"] = dec["value"] / peaks["copy_gbs"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
