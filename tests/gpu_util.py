"""Helpers for GPU parity tests: host<->device conversion and the error metrics."""
from __future__ import annotations

import numpy as np
import torch

from dependent_positional_attention_amd import synth

TOL = {
    # bf16 storage, fp32 accumulation: max-abs and relative L2, on outputs and lse
    "bf16": dict(max_abs=2e-3, rel_l2=1e-2),
    # fp32 throughout
    "f32": dict(max_abs=1e-5, rel_l2=1e-5),
}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy array holding exact stored values -> device tensor of the storage dtype."""
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30)) if diff.size else 0.0
    return max_abs, rel


def assert_parity(got, want, dtype: str, what: str = ""):
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    ma, rel = errors(got, want)
    assert ma <= tol["max_abs"] and rel <= tol["rel_l2"], \
        f"{what}: max_abs {ma:.3e} (tol {tol['max_abs']:.0e}), rel_l2 {rel:.3e} (tol {tol['rel_l2']:.0e})"
    return ma, rel


def fwd_inputs_dev(x: synth.FwdInputs):
    t = {n: dev(getattr(x, n), x.dtype) for n in ("q", "k", "v", "w")}
    t["beta"] = dev_f32(x.beta)
    t["logf"] = dev_f32(x.logf) if x.logf is not None else None
    return t
