"""ctypes binding of libpathattn.so -- argument marshalling only.

Every step of PaTH attention runs in the HIP kernels behind the C ABI
(include/path_attn.h); this module passes torch tensors' device pointers and
the current HIP stream through, allocating outputs and workspace with torch
when the caller does not pass them.  There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch  # imported first so the HIP runtime torch ships is the one in the process

_HERE = os.path.dirname(os.path.abspath(__file__))
# PATHATTN_LIB points the binding at another build of the same library (A/B comparisons).
LIB_PATH = os.environ.get("PATHATTN_LIB") or os.path.join(_HERE, "libpathattn.so")

PATH_OK, PATH_ERR_INVALID_ARG, PATH_ERR_UNSUPPORTED, PATH_ERR_HIP, PATH_ERR_SCRATCH = 0, 1, 2, 3, 4
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
TRANSPORT = {"bf16": 0, "bf16x3": 1}

_lib = None


class PathAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().path_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")


class WsLayout(ctypes.Structure):
    _fields_ = [("layout_id", ctypes.c_int), ("num_chunks", ctypes.c_int64), ("off_qtilde", ctypes.c_int64),
                ("off_qtilde_lo", ctypes.c_int64), ("off_ktilde", ctypes.c_int64), ("off_p", ctypes.c_int64),
                ("off_p_lo", ctypes.c_int64), ("off_s", ctypes.c_int64), ("off_fox_local", ctypes.c_int64),
                ("off_fox_total", ctypes.c_int64), ("total_bytes", ctypes.c_int64),
                ("num_sub_chunks", ctypes.c_int64), ("off_ktilde_c2", ctypes.c_int64), ("off_p_c2", ctypes.c_int64),
                ("off_p_c2_lo", ctypes.c_int64)]


EXPORTS = ("path_abi_version", "path_status_string", "path_attn_fwd_workspace_bytes", "path_attn_fwd",
           "path_attn_prep", "path_attn_scan", "path_attn_workspace_layout", "path_decode_workspace_bytes",
           "path_decode_step", "path_attn_cache_from_prefill", "path_decode_deferred_state_bytes",
           "path_decode_step_deferred", "path_attn_bwd_workspace_bytes", "path_attn_bwd", "path_decode_step_noalloc",
           "path_decode_noalloc_scratch_bytes")


def lib():
    """Load libpathattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python -m dependent_positional_attention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.path_abi_version.argtypes, L.path_abi_version.restype = [], i32
        L.path_status_string.argtypes, L.path_status_string.restype = [i32], ctypes.c_char_p
        L.path_attn_fwd_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.path_attn_workspace_layout.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(WsLayout)]
        L.path_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, i32, vp, sz,
                                    vp]
        L.path_attn_prep.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, i32, vp, sz, vp]
        L.path_attn_scan.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, vp, sz, vp]
        L.path_decode_workspace_bytes.argtypes = [i64, i64, i32, i64, i32, ctypes.POINTER(sz)]
        L.path_decode_step.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, f32,
                                       i32, i32, vp, sz, vp]
        L.path_attn_cache_from_prefill.argtypes = [vp, vp, vp, sz, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, i32,
                                                   vp]
        L.path_decode_deferred_state_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(sz)]
        L.path_decode_step_deferred.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, sz, vp, vp, vp, vp, vp, vp, vp,
                                                vp, i64, i64, i32, f32, i32, i32, vp, sz, vp]
        L.path_decode_step_noalloc.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32,
                                               f32, i32, i32, vp]
        L.path_decode_noalloc_scratch_bytes.argtypes, L.path_decode_noalloc_scratch_bytes.restype = [], sz
        L.path_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(sz)]
        L.path_attn_bwd.argtypes = [vp] * 15 + [i64, i64, i64, i32, i32, f32, i32, vp, sz, vp]
        for f in ("path_attn_fwd_workspace_bytes", "path_attn_workspace_layout", "path_attn_fwd", "path_attn_prep",
                  "path_attn_scan", "path_decode_workspace_bytes", "path_decode_step", "path_attn_cache_from_prefill",
                  "path_decode_deferred_state_bytes", "path_decode_step_deferred", "path_attn_bwd_workspace_bytes",
                  "path_attn_bwd", "path_decode_step_noalloc"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != PATH_OK:
        raise PathAttnError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def path_attn_fwd_workspace_bytes(B, H, L, d, chunk, dtype: torch.dtype, transport: str = "bf16") -> int:
    n = ctypes.c_size_t(0)
    _check("path_attn_fwd_workspace_bytes",
           lib().path_attn_fwd_workspace_bytes(B, H, L, d, chunk, DTYPE[dtype], TRANSPORT[transport],
                                               ctypes.byref(n)))
    return n.value


def path_attn_workspace_layout(B, H, L, d, chunk, dtype: torch.dtype, transport: str = "bf16") -> WsLayout:
    lay = WsLayout()
    _check("path_attn_workspace_layout",
           lib().path_attn_workspace_layout(B, H, L, d, chunk, DTYPE[dtype], TRANSPORT[transport],
                                            ctypes.byref(lay)))
    return lay


def path_attn_fwd(q, k, v, w, beta, log_forget=None, *, scale: Optional[float] = None, chunk: int = 64,
                  transport: str = "bf16", out=None, lse=None, workspace=None, stream=None,
                  want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """PaTH / PaTH-FoX prefill forward.  q,k,v,w: [B,H,L,d]; beta, log_forget: [B,H,L] fp32."""
    _require(q, "q")
    B, H, L, d = q.shape
    for name, t in (("k", k), ("v", v), ("w", w)):
        _require(t, name, q.dtype, q.shape)
    _require(beta, "beta", torch.float32, (B, H, L))
    if log_forget is not None:
        _require(log_forget, "log_forget", torch.float32, (B, H, L))
    if q.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", q.dtype, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, H, L))
    nbytes = path_attn_fwd_workspace_bytes(B, H, L, d, chunk, q.dtype, transport)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), device=q.device, dtype=torch.uint8)
    _require(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("path_attn_fwd", lib().path_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(log_forget), _ptr(out), _ptr(lse), B, H, L, d, chunk,
        float(scale), DTYPE[q.dtype], TRANSPORT[transport], _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def path_attn_prep(q, k, v, w, beta, log_forget=None, *, scale: Optional[float] = None, chunk: int = 64,
                   transport: str = "bf16", workspace, stream=None) -> torch.Tensor:
    """Per-chunk terms only (first phase of path_attn_fwd), written into `workspace`; the logit
    scale is folded into the stored queries and in-chunk logits."""
    _require(q, "q")
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t in (("k", k), ("v", v), ("w", w)):
        _require(t, name, q.dtype, q.shape)
    _require(beta, "beta", torch.float32, (B, H, L))
    if log_forget is not None:
        _require(log_forget, "log_forget", torch.float32, (B, H, L))
    _require(workspace, "workspace")
    _check("path_attn_prep", lib().path_attn_prep(
        _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(log_forget), B, H, L, d, chunk, float(scale),
        DTYPE[q.dtype], TRANSPORT[transport], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return workspace


def path_attn_scan(v, log_forget=None, *, chunk: int = 64, transport: str = "bf16", workspace, out=None, lse=None,
                   stream=None, want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention scan from a workspace filled by path_attn_prep with the same arguments."""
    _require(v, "v")
    B, H, L, d = v.shape
    if out is None:
        out = torch.empty_like(v)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), device=v.device, dtype=torch.float32)
    _require(workspace, "workspace")
    _check("path_attn_scan", lib().path_attn_scan(
        _ptr(v), _ptr(log_forget), _ptr(out), _ptr(lse), B, H, L, d, chunk, DTYPE[v.dtype], TRANSPORT[transport],
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def path_attn_cache_from_prefill(v, log_forget=None, *, workspace, capacity: Optional[int] = None, chunk: int = 64,
                                 transport: str = "bf16", kcache=None, vcache=None, fcache=None,
                                 stream=None):
    """Decode caches [B,H,capacity,d] after a prompt, from a workspace filled by path_attn_prep /
    path_attn_fwd with the same arguments.  v: the prompt's values [B,H,L,d].  With the prompt's
    log_forget [B,H,L] (PaTH-FoX) the slot biases fcache [B,H,capacity] fp32 are filled too.
    Returns (kcache, vcache, fcache) (fcache None for plain PaTH)."""
    _require(v, "v")
    B, H, L, d = v.shape
    if kcache is None:
        cap = L if capacity is None else int(capacity)
        kcache = torch.empty((B, H, cap, d), device=v.device, dtype=v.dtype)
    _require(kcache, "kcache", v.dtype)
    B2, H2, cap, d2 = kcache.shape
    if (B2, H2, d2) != (B, H, d):
        raise ValueError(f"kcache shape {tuple(kcache.shape)} does not match v {tuple(v.shape)}")
    if vcache is None:
        vcache = torch.empty_like(kcache)
    _require(vcache, "vcache", v.dtype, kcache.shape)
    if log_forget is not None:
        _require(log_forget, "log_forget", torch.float32, (B, H, L))
        if fcache is None:
            fcache = torch.empty((B, H, cap), device=v.device, dtype=torch.float32)
        _require(fcache, "fcache", torch.float32, (B, H, cap))
    elif fcache is not None:
        raise ValueError("fcache is filled from log_forget: pass both or neither")
    _require(workspace, "workspace")
    _check("path_attn_cache_from_prefill", lib().path_attn_cache_from_prefill(
        _ptr(v), _ptr(log_forget), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(kcache),
        _ptr(vcache), _ptr(fcache), cap, B, H, L, d, chunk, DTYPE[v.dtype], TRANSPORT[transport], _stream(stream)))
    return kcache, vcache, fcache


def path_decode_workspace_bytes(B, H, d, capacity, splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check("path_decode_workspace_bytes", lib().path_decode_workspace_bytes(B, H, d, capacity, splits,
                                                                           ctypes.byref(n)))
    return n.value


def path_decode_step(kcache, vcache, t: int, q_t, k_t, v_t, w_t, beta_t, log_forget_t=None, *, fcache=None,
                     t_batch=None, scale: Optional[float] = None, splits: int = 0, out=None, lse=None,
                     workspace=None, stream=None, want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One decode step.  kcache, vcache: [B,H,capacity,d] (updated in place); q_t..w_t: [B,H,d]; beta_t: [B,H].

    PaTH-FoX: log_forget_t [B,H] and fcache [B,H,capacity] fp32 (slot biases, updated in place).
    Ragged batch: t_batch [B] int32 per-sequence token counts, each <= t (t sizes the key split)."""
    _require(kcache, "kcache")
    B, H, cap, d = kcache.shape
    _require(vcache, "vcache", kcache.dtype, kcache.shape)
    for name, x in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _require(x, name, kcache.dtype, (B, H, d))
    _require(beta_t, "beta_t", torch.float32, (B, H))
    if (log_forget_t is None) != (fcache is None):
        raise ValueError("PaTH-FoX decode needs both log_forget_t and fcache")
    if log_forget_t is not None:
        _require(log_forget_t, "log_forget_t", torch.float32, (B, H))
        _require(fcache, "fcache", torch.float32, (B, H, cap))
    if t_batch is not None:
        _require(t_batch, "t_batch", torch.int32, (B,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), device=kcache.device, dtype=kcache.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H), device=kcache.device, dtype=torch.float32)
    if workspace is None:
        workspace = torch.empty(max(path_decode_workspace_bytes(B, H, d, cap, splits), 16), device=kcache.device,
                                dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("path_decode_step", lib().path_decode_step(
        _ptr(kcache), _ptr(vcache), _ptr(fcache), cap, int(t), _ptr(t_batch), _ptr(q_t), _ptr(k_t), _ptr(v_t),
        _ptr(w_t), _ptr(beta_t), _ptr(log_forget_t), _ptr(out), _ptr(lse), B, H, d, float(scale),
        DTYPE[kcache.dtype], int(splits), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def path_decode_noalloc_scratch_bytes() -> int:
    return int(lib().path_decode_noalloc_scratch_bytes())


def path_decode_step_noalloc(kcache, vcache, t: int, q_t, k_t, v_t, w_t, beta_t, log_forget_t=None, *, fcache=None,
                             t_batch=None, scale: Optional[float] = None, splits: int = 0, out, lse=None,
                             stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """path_decode_step with the split partials in the library's fixed scratch array (no workspace): the
    caller passes every output buffer (out, and lse unless it is not wanted), so nothing is allocated here."""
    _require(kcache, "kcache")
    B, H, cap, d = kcache.shape
    _require(vcache, "vcache", kcache.dtype, kcache.shape)
    for name, x in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t), ("out", out)):
        _require(x, name, kcache.dtype, (B, H, d))
    _require(beta_t, "beta_t", torch.float32, (B, H))
    if (log_forget_t is None) != (fcache is None):
        raise ValueError("PaTH-FoX decode needs both log_forget_t and fcache")
    if log_forget_t is not None:
        _require(log_forget_t, "log_forget_t", torch.float32, (B, H))
        _require(fcache, "fcache", torch.float32, (B, H, cap))
    if t_batch is not None:
        _require(t_batch, "t_batch", torch.int32, (B,))
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, H))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check("path_decode_step_noalloc", lib().path_decode_step_noalloc(
        _ptr(kcache), _ptr(vcache), _ptr(fcache), cap, int(t), _ptr(t_batch), _ptr(q_t), _ptr(k_t), _ptr(v_t),
        _ptr(w_t), _ptr(beta_t), _ptr(log_forget_t), _ptr(out), _ptr(lse), B, H, d, float(scale),
        DTYPE[kcache.dtype], int(splits), _stream(stream)))
    return out, lse


def path_decode_deferred_state_bytes(B, H, d) -> int:
    n = ctypes.c_size_t(0)
    _check("path_decode_deferred_state_bytes", lib().path_decode_deferred_state_bytes(B, H, d, ctypes.byref(n)))
    return n.value


def path_decode_step_deferred(kcache, vcache, t: int, t_cur: int, q_t, k_t, v_t, w_t, beta_t, log_forget_t=None, *,
                              period: int, state, fcache=None, scale: Optional[float] = None, splits: int = 0,
                              out=None, lse=None, workspace=None, stream=None,
                              want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor], int]:
    """One decode step with deferred key updates (see path_attn.h).  Returns (out, lse, next t_cur): the keys
    are brought up to date when t - t_cur + 1 == period, after which t_cur becomes t + 1."""
    _require(kcache, "kcache")
    B, H, cap, d = kcache.shape
    _require(vcache, "vcache", kcache.dtype, kcache.shape)
    for name, x in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _require(x, name, kcache.dtype, (B, H, d))
    _require(beta_t, "beta_t", torch.float32, (B, H))
    if (log_forget_t is None) != (fcache is None):
        raise ValueError("PaTH-FoX decode needs both log_forget_t and fcache")
    if log_forget_t is not None:
        _require(log_forget_t, "log_forget_t", torch.float32, (B, H))
        _require(fcache, "fcache", torch.float32, (B, H, cap))
    _require(state, "state", torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), device=kcache.device, dtype=kcache.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H), device=kcache.device, dtype=torch.float32)
    if workspace is None:
        workspace = torch.empty(max(path_decode_workspace_bytes(B, H, d, cap, splits), 16), device=kcache.device,
                                dtype=torch.uint8)
    _check("path_decode_step_deferred", lib().path_decode_step_deferred(
        _ptr(kcache), _ptr(vcache), _ptr(fcache), cap, int(t), int(t_cur), int(period), _ptr(state),
        state.numel() * state.element_size(), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t),
        _ptr(log_forget_t), _ptr(out), _ptr(lse), B, H, d, float(scale), DTYPE[kcache.dtype], int(splits),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    nxt = t + 1 if t - t_cur + 1 == period else t_cur
    return out, lse, nxt


def path_attn_bwd_workspace_bytes(B, H, L, d, chunk, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t(0)
    _check("path_attn_bwd_workspace_bytes",
           lib().path_attn_bwd_workspace_bytes(B, H, L, d, chunk, DTYPE[dtype], ctypes.byref(n)))
    return n.value


def path_attn_bwd(q, k, v, w, beta, out, lse, dout, log_forget=None, *, scale: Optional[float] = None,
                  chunk: int = 64, workspace=None, grads=None, stream=None):
    """Gradients of path_attn_fwd for the upstream gradient dout (loss = sum(dout * out)).

    q,k,v,w,out,dout: [B,H,L,d]; beta, log_forget, lse: [B,H,L] fp32 (lse as path_attn_fwd wrote it).
    Returns (dq, dk, dv, dw, dbeta, dlog_forget); dlog_forget is None without log_forget.  ``grads`` may
    hold those six tensors preallocated (dlog_forget None without log_forget).
    """
    _require(q, "q")
    B, H, L, d = q.shape
    for name, t in (("k", k), ("v", v), ("w", w), ("out", out), ("dout", dout)):
        _require(t, name, q.dtype, q.shape)
    for name, t in (("beta", beta), ("lse", lse)):
        _require(t, name, torch.float32, (B, H, L))
    if log_forget is not None:
        _require(log_forget, "log_forget", torch.float32, (B, H, L))
    if q.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                 torch.empty((B, H, L), device=q.device, dtype=torch.float32),
                 None if log_forget is None else torch.empty((B, H, L), device=q.device, dtype=torch.float32))
    dq, dk, dv, dw, dbeta, dlogf = grads
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dw", dw)):
        _require(t, name, q.dtype, q.shape)
    _require(dbeta, "dbeta", torch.float32, (B, H, L))
    if dlogf is not None:
        _require(dlogf, "dlog_forget", torch.float32, (B, H, L))
    nbytes = path_attn_bwd_workspace_bytes(B, H, L, d, chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), device=q.device, dtype=torch.uint8)
    _require(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("path_attn_bwd", lib().path_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(log_forget), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(dbeta), _ptr(dlogf), B, H, L, d, chunk, float(scale),
        DTYPE[q.dtype], _ptr(workspace), ws_bytes, _stream(stream)))
    return dq, dk, dv, dw, dbeta, dlogf

