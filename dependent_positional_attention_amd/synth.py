"""Seeded synthetic inputs for PaTH attention.

This module is shared by the CPU oracle tests and the GPU path.  It holds none
of the method's arithmetic: it draws Gaussian tensors, L2-normalises the
transition directions w, squashes the beta logits through 2*sigmoid (the range
(0, 2) stated in the PaTH summary, section 2 "core mechanism"), draws the
PaTH-FoX log-forget gates through logsigmoid, and rounds every tensor to the
dtype the kernels store.  What PaTH does with these tensors lives elsewhere.

Every tensor is drawn in float64 from its own PCG64 stream, keyed by
``(seed, stream id)``, and then rounded (round-to-nearest-even) to bf16 or
fp32.  The returned numpy arrays are float32 and hold exactly the values the
GPU consumes, so the oracle can widen them to float64 without any further
rounding.

Recipes (shapes and distributions of the workloads the pages motivate):

* ``tiny``      B=1,H=1,L=64,d=16 fp32; q,k,v ~ N(0,1); beta = 2*sigmoid(N(0,1)).
* ``lm``        the 760M-class layer: q,k,v ~ N(0,1)/sqrt(d); beta = 2*sigmoid(N(0,1.5)).
* ``fox``       ``lm`` plus f = logsigmoid(N(3,1)) per token.
* ``stress_qk`` (S1) q,k ~ N(0,1) instead of N(0,1)/sqrt(d).
* ``beta2``     (S2) beta == 2 exactly (pure reflections).
* ``beta02``    (S3) beta drawn from {0, 2}.
* ``beta0``     beta == 0 (every transition is the identity).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# One stream id per tensor so that changing one tensor's shape never changes another's values.
STREAM_IDS = {
    "q": 1, "k": 2, "v": 3, "w": 4, "beta": 5, "logf": 6,
    "dec_q": 11, "dec_k": 12, "dec_v": 13, "dec_w": 14, "dec_beta": 15,
    "cache_k": 21, "cache_v": 22,
    "dout": 31,
}


def rng(seed: int, name: str) -> np.random.Generator:
    """PCG64 stream for tensor ``name`` under ``seed``."""
    return np.random.Generator(np.random.PCG64([int(seed), STREAM_IDS[name]]))


# ----------------------------------------------------------------------------- rounding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even) and return the raw uint16 bit patterns.

    float64 input is first rounded to float32 (RNE); the float32 -> bf16 step then
    adds 0x7FFF plus the lowest kept bit before truncating, which is RNE on the
    16 dropped bits.  NaN stays NaN.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype; returns float32 holding the exact stored values."""
    if dtype == "bf16":
        return bf16_from_bits(bf16_bits(x))
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------- draws

def _normal(seed, name, shape, std=1.0, mean=0.0):
    g = rng(seed, name).standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        g *= std
    if mean != 0.0:
        g += mean
    return g


def unit_rows(g: np.ndarray) -> np.ndarray:
    """Normalise the last axis of a Gaussian draw to unit L2 norm (float64)."""
    n = np.sqrt(np.sum(g * g, axis=-1, keepdims=True))
    return g / n


def sigmoid2(z: np.ndarray) -> np.ndarray:
    """2*sigmoid(z), evaluated stably in float64."""
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 2.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = 2.0 * ez / (1.0 + ez)
    return out


def logsigmoid(z: np.ndarray) -> np.ndarray:
    """log(sigmoid(z)) = -log1p(exp(-z)), stable for both signs (float64)."""
    return np.where(z >= 0, -np.log1p(np.exp(-np.abs(z))), z - np.log1p(np.exp(-np.abs(z))))


@dataclasses.dataclass
class FwdInputs:
    """Prefill inputs, [B,H,L,d] for q/k/v/w and [B,H,L] for beta/logf (float32 holding stored values)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray
    beta: np.ndarray
    logf: Optional[np.ndarray]
    dtype: str
    scale: float
    recipe: str
    seed: int

    @property
    def shape(self):
        return self.q.shape


RECIPES = ("tiny", "lm", "fox", "stress_qk", "beta2", "beta02", "beta0", "stress_qk_beta2")


def make_fwd_inputs(B: int, H: int, L: int, d: int, *, recipe: str = "lm", dtype: str = "bf16",
                    seed: int = 0, scale: Optional[float] = None, fox: Optional[bool] = None) -> FwdInputs:
    """Draw one prefill problem.

    ``recipe`` picks the distributions (see module docstring).  ``fox`` forces the
    log-forget tensor on or off (default: on only for the ``fox`` recipe).
    ``scale`` defaults to 1/sqrt(d).
    """
    if recipe not in RECIPES:
        raise ValueError(f"unknown recipe {recipe!r}")
    shape = (B, H, L, d)
    tok = (B, H, L)
    if recipe == "tiny":
        qk_std, v_std, beta_std = 1.0, 1.0, 1.0
    else:
        qk_std, v_std, beta_std = 1.0 / math.sqrt(d), 1.0 / math.sqrt(d), 1.5
    if recipe in ("stress_qk", "stress_qk_beta2"):
        qk_std = 1.0
    q = round_to(_normal(seed, "q", shape, qk_std), dtype)
    k = round_to(_normal(seed, "k", shape, qk_std), dtype)
    v = round_to(_normal(seed, "v", shape, v_std), dtype)
    w = round_to(unit_rows(_normal(seed, "w", shape)), dtype)
    if recipe in ("beta2", "stress_qk_beta2"):
        beta64 = np.full(tok, 2.0)
    elif recipe == "beta0":
        beta64 = np.zeros(tok)
    elif recipe == "beta02":
        beta64 = 2.0 * rng(seed, "beta").integers(0, 2, size=tok).astype(np.float64)
    else:
        beta64 = sigmoid2(_normal(seed, "beta", tok, beta_std))
    beta = beta64.astype(np.float32)
    use_fox = (recipe == "fox") if fox is None else fox
    logf = logsigmoid(_normal(seed, "logf", tok, 1.0, 3.0)).astype(np.float32) if use_fox else None
    return FwdInputs(q=q, k=k, v=v, w=w, beta=beta, logf=logf, dtype=dtype,
                     scale=(1.0 / math.sqrt(d)) if scale is None else float(scale),
                     recipe=recipe, seed=seed)


def make_out_grad(shape, *, dtype: str = "bf16", seed: int = 0, std: float = 1.0) -> np.ndarray:
    """Upstream gradient of the prefill output for backward tests: Gaussian, stored values of ``dtype``."""
    return round_to(_normal(seed, "dout", tuple(shape), std), dtype)


@dataclasses.dataclass
class DecodeStepInputs:
    """Per-step decode inputs: q/k/v/w [S,B,H,d], beta [S,B,H] (float32 holding stored values)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray
    beta: np.ndarray
    dtype: str
    scale: float
    seed: int


def make_decode_steps(steps: int, B: int, H: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                      qkv_std: Optional[float] = None, scale: Optional[float] = None) -> DecodeStepInputs:
    """Draw ``steps`` decode tokens: q,k,v ~ N(0,1)/sqrt(d), w unit Gaussian, beta = 2*sigmoid(N(0,1))."""
    shape = (steps, B, H, d)
    std = 1.0 / math.sqrt(d) if qkv_std is None else qkv_std
    return DecodeStepInputs(
        q=round_to(_normal(seed, "dec_q", shape, std), dtype),
        k=round_to(_normal(seed, "dec_k", shape, std), dtype),
        v=round_to(_normal(seed, "dec_v", shape, std), dtype),
        w=round_to(unit_rows(_normal(seed, "dec_w", shape)), dtype),
        beta=sigmoid2(_normal(seed, "dec_beta", (steps, B, H))).astype(np.float32),
        dtype=dtype, scale=(1.0 / math.sqrt(d)) if scale is None else float(scale), seed=seed)


def make_decode_cache(B: int, H: int, T: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                      std: Optional[float] = None):
    """Initial cache contents for T tokens, [B,H,T,d] each for K and V, N(0,1)/sqrt(d).

    The cached keys stand for an already-transported state; they are plain Gaussian
    draws.  Host-side draw: use it for sizes that fit host memory comfortably.
    """
    s = 1.0 / math.sqrt(d) if std is None else std
    return (round_to(_normal(seed, "cache_k", (B, H, T, d), s), dtype),
            round_to(_normal(seed, "cache_v", (B, H, T, d), s), dtype))
