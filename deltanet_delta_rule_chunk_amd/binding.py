"""Thin ctypes binding of libdeltanet.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
checks tensors (device, dtype, contiguity, shape), allocates outputs and the
workspace through PyTorch's caching allocator (recorded on the launch stream
when that is not the current one), and passes raw device pointers and the HIP
stream (the current one unless ``stream=`` names another) to the C ABI.  If
the library is missing it raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdeltanet.so")

DN_OK = 0
DN_F32 = 0
DN_BF16 = 1
STATUS_NAMES = {0: "DN_OK", 1: "DN_ERR_NULL_ARG", 2: "DN_ERR_BAD_SHAPE", 3: "DN_ERR_UNSUPPORTED",
                4: "DN_ERR_MISALIGNED", 5: "DN_ERR_ALIASING", 6: "DN_ERR_WORKSPACE",
                7: "DN_ERR_HIP"}
# Every symbol include/deltanet.h declares.
EXPORTS = ("deltanet_chunk_fwd", "deltanet_chunk_fwd_workspace_bytes", "deltanet_decode_step",
           "deltanet_gated_chunk_fwd", "deltanet_gated_chunk_fwd_workspace_bytes",
           "deltanet_gated_decode_step", "deltanet_feature_prep", "deltanet_chunk_fwd_features",
           "deltanet_chunk_fwd_features_workspace_bytes", "deltanet_decode_step_features",
           "deltanet_kda_chunk_fwd", "deltanet_kda_chunk_fwd_workspace_bytes",
           "deltanet_kda_decode_step", "deltanet_chunk_bwd", "deltanet_chunk_bwd_workspace_bytes",
           "deltanet_status_string", "deltanet_last_hip_error", "deltanet_version",
           "deltanet_profile_start", "deltanet_profile_stop", "deltanet_chunk_fwd_noalloc")
PROFILE_SLOTS = ("chunk_prep", "chunk_scan", "decode", "features", "bwd_prep", "bwd_fwd_scan",
                 "bwd_scan", "bwd_cc", "bwd_qk")

_lib = None


class DeltaNetError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({detail})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m deltanet_delta_rule_chunk_amd.build`"
            " (there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.deltanet_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_chunk_fwd.restype = i
    lib.deltanet_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                               vp]
    lib.deltanet_chunk_fwd_noalloc.restype = i
    lib.deltanet_chunk_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_chunk_fwd_workspace_bytes.restype = sz
    lib.deltanet_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.deltanet_decode_step.restype = i
    lib.deltanet_gated_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                             vp, sz, vp]
    lib.deltanet_gated_chunk_fwd.restype = i
    lib.deltanet_gated_chunk_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_gated_chunk_fwd_workspace_bytes.restype = sz
    lib.deltanet_gated_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.deltanet_gated_decode_step.restype = i
    lib.deltanet_feature_prep.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.deltanet_feature_prep.restype = i
    lib.deltanet_chunk_fwd_features.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                                i, i, vp, sz, vp]
    lib.deltanet_chunk_fwd_features.restype = i
    lib.deltanet_chunk_fwd_features_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.deltanet_chunk_fwd_features_workspace_bytes.restype = sz
    lib.deltanet_decode_step_features.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.deltanet_decode_step_features.restype = i
    lib.deltanet_kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                           vp, sz, vp]
    lib.deltanet_kda_chunk_fwd.restype = i
    lib.deltanet_kda_chunk_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_kda_chunk_fwd_workspace_bytes.restype = sz
    lib.deltanet_kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.deltanet_kda_decode_step.restype = i
    lib.deltanet_chunk_bwd.argtypes = [vp] * 12 + [i] * 7 + [vp, sz, vp]
    lib.deltanet_chunk_bwd.restype = i
    lib.deltanet_chunk_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_chunk_bwd_workspace_bytes.restype = sz
    lib.deltanet_status_string.argtypes = [i]
    lib.deltanet_status_string.restype = ctypes.c_char_p
    lib.deltanet_last_hip_error.argtypes = []
    lib.deltanet_last_hip_error.restype = i
    lib.deltanet_version.argtypes = []
    lib.deltanet_version.restype = i
    lib.deltanet_profile_start.argtypes = []
    lib.deltanet_profile_start.restype = i
    lib.deltanet_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int), i]
    lib.deltanet_profile_stop.restype = i
    _lib = lib
    return lib


def _code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return DN_F32
    if dt == torch.bfloat16:
        return DN_BF16
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(lib, status: int, what: str):
    detail = lib.deltanet_status_string(status).decode()
    if status == 7:
        detail += f"; hipError {lib.deltanet_last_hip_error()}"
    raise DeltaNetError(status, what, detail)


def _stream(device: torch.device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _alloc(shape, dtype: torch.dtype, device: torch.device, stream) -> torch.Tensor:
    """A new tensor from PyTorch's caching allocator.  The allocator ties a
    block to the stream current at allocation; when the kernels run on another
    stream, the block is also recorded on that stream, so that it is not
    handed out again while those kernels may still use it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def workspace_bytes(B: int, H: int, L: int, d_k: int, d_v: int, C: int,
                    in_dtype: torch.dtype = torch.bfloat16, gated: bool = False,
                    features: bool = False) -> int:
    lib = load()
    if features:
        return int(lib.deltanet_chunk_fwd_features_workspace_bytes(B, H, L, d_k, d_v, C,
                                                                    _code(in_dtype), int(gated)))
    fn = lib.deltanet_gated_chunk_fwd_workspace_bytes if gated else lib.deltanet_chunk_fwd_workspace_bytes
    return int(fn(B, H, L, d_k, d_v, C, _code(in_dtype)))


def bwd_workspace_bytes(B: int, H: int, L: int, d_k: int, d_v: int, C: int = 64,
                        in_dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load().deltanet_chunk_bwd_workspace_bytes(B, H, L, d_k, d_v, C, _code(in_dtype)))


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              S0: Optional[torch.Tensor], dO: torch.Tensor, dS_final: Optional[torch.Tensor] = None,
              C: int = 64, *, want_dS0: bool = True, workspace: Optional[torch.Tensor] = None,
              stream=None):
    """Gradient of the chunked forward (``deltanet_chunk_bwd``).  q,k ``[B,H,L,d_k]``,
    v ``[B,H,L,d_v]`` (fp32 or bf16), beta ``[B,H,L]``, S0 ``[B,H,d_k,d_v]`` or None,
    dO ``[B,H,L,d_v]`` fp32, dS_final ``[B,H,d_k,d_v]`` fp32 or None.  Returns fp32
    ``(dq, dk, dv, dbeta, dS0)`` (dS0 None when ``want_dS0`` is False)."""
    lib = load()
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _check(q, "q", (B, H, L, d_k), device=dev)
    _check(k, "k", (B, H, L, d_k), q.dtype, dev)
    _check(v, "v", (B, H, L, d_v), q.dtype, dev)
    _check(beta, "beta", (B, H, L), torch.float32, dev)
    _check(dO, "dO", (B, H, L, d_v), torch.float32, dev)
    for t, n in ((S0, "S0"), (dS_final, "dS_final")):
        if t is not None:
            _check(t, n, (B, H, d_k, d_v), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev, stream=stream)
    dq, dk = _alloc((B, H, L, d_k), **f32), _alloc((B, H, L, d_k), **f32)
    dv, db = _alloc((B, H, L, d_v), **f32), _alloc((B, H, L), **f32)
    dS0 = _alloc((B, H, d_k, d_v), **f32) if want_dS0 else None
    need = bwd_workspace_bytes(B, H, L, d_k, d_v, C, q.dtype)
    if workspace is None and need > 0:
        workspace = _alloc(need, torch.uint8, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.deltanet_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO),
                                _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(dS0),
                                B, H, L, d_k, d_v, C, _code(q.dtype), _ptr(workspace), ws_bytes,
                                _stream(dev, stream))
    if st != DN_OK:
        _raise(lib, st, "deltanet_chunk_bwd")
    return dq, dk, dv, db, dS0


class _DeltaRule(torch.autograd.Function):
    """``chunk_fwd`` (fp32 o) with its gradient from ``chunk_bwd``.  Only the
    inputs are kept for the backward, which recomputes the forward inside the
    library.  The gradients come back in fp32; autograd casts them to the
    inputs' dtype."""

    @staticmethod
    def forward(ctx, q, k, v, beta, S0, C):
        o, S_final = chunk_fwd(q, k, v, beta, S0, C)
        ctx.save_for_backward(q, k, v, beta, S0)
        ctx.C = C
        return o, S_final

    @staticmethod
    def backward(ctx, dO, dS_final):
        q, k, v, beta, S0 = ctx.saved_tensors
        want_dS0 = S0 is not None and ctx.needs_input_grad[4]
        dq, dk, dv, db, dS0 = chunk_bwd(q, k, v, beta, S0, dO.contiguous(), dS_final.contiguous(),
                                        ctx.C, want_dS0=want_dS0)
        return dq, dk, dv, db, dS0, None


def delta_rule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
               S0: Optional[torch.Tensor] = None, C: int = 64
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable chunked delta-rule forward for training: ``(o, S_final)``
    as ``chunk_fwd`` returns them (o in fp32), with gradients for q, k, v,
    beta and S0 from ``deltanet_chunk_bwd``."""
    return _DeltaRule.apply(q, k, v, beta, S0, C)


def kda_workspace_bytes(B: int, H: int, L: int, d_k: int, d_v: int, C: int = 64,
                        in_dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load().deltanet_kda_chunk_fwd_workspace_bytes(B, H, L, d_k, d_v, C,
                                                             _code(in_dtype)))


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                  beta: torch.Tensor, S0: Optional[torch.Tensor] = None, C: int = 64, *,
                  out_dtype: torch.dtype = torch.float32, o: Optional[torch.Tensor] = None,
                  S_final: Optional[torch.Tensor] = None, want_state: bool = True,
                  workspace: Optional[torch.Tensor] = None, stream=None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked forward with per-dimension decay (``deltanet_kda_chunk_fwd``):
    ``chunk_fwd``'s arguments with alpha ``[B,H,L,d_k]`` fp32."""
    lib = load()
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _check(q, "q", (B, H, L, d_k), device=dev)
    _check(k, "k", (B, H, L, d_k), q.dtype, dev)
    _check(v, "v", (B, H, L, d_v), q.dtype, dev)
    _check(alpha, "alpha", (B, H, L, d_k), torch.float32, dev)
    _check(beta, "beta", (B, H, L), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = _alloc((B, H, L, d_v), out_dtype, dev, stream)
    _check(o, "o", (B, H, L, d_v), out_dtype, dev)
    if S_final is None and want_state:
        S_final = _alloc((B, H, d_k, d_v), torch.float32, dev, stream)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, d_k, d_v), torch.float32, dev)
    need = kda_workspace_bytes(B, H, L, d_k, d_v, C, q.dtype)
    if workspace is None and need > 0:
        workspace = _alloc(need, torch.uint8, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.deltanet_kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                                    _ptr(o), _ptr(S_final), B, H, L, d_k, d_v, C, _code(q.dtype),
                                    _code(out_dtype), _ptr(workspace), ws_bytes,
                                    _stream(dev, stream))
    if st != DN_OK:
        _raise(lib, st, "deltanet_kda_chunk_fwd")
    return o, S_final


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                    o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode step with per-dimension decay (``deltanet_kda_decode_step``):
    alpha ``[B,H,d_k]`` fp32; S updated in place; returns o = q S_new."""
    lib = load()
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _check(q, "q", (B, H, d_k), device=dev)
    _check(k, "k", (B, H, d_k), q.dtype, dev)
    _check(v, "v", (B, H, d_v), q.dtype, dev)
    _check(alpha, "alpha", (B, H, d_k), torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = _alloc((B, H, d_v), out_dtype, dev, stream)
    _check(o, "o", (B, H, d_v), out_dtype, dev)
    st = lib.deltanet_kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S),
                                      _ptr(o), B, H, d_k, d_v, _code(q.dtype), _code(out_dtype),
                                      _stream(dev, stream))
    if st != DN_OK:
        _raise(lib, st, "deltanet_kda_decode_step")
    return o


def feature_prep(q_raw: torch.Tensor, k_raw: torch.Tensor, beta_logit: torch.Tensor, *,
                 in_place: bool = False, stream=None
                 ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The layer's feature maps: ``normalise(silu(q_raw))``, ``normalise(silu(k_raw))``
    (``[B,H,L,d_k]``, same dtype as the inputs) and ``sigmoid(beta_logit)``
    (``[B,H,L]`` fp32), by ``deltanet_feature_prep``.  ``in_place`` writes the
    results over the inputs."""
    lib = load()
    B, H, L, d_k = q_raw.shape
    dev = q_raw.device
    _check(q_raw, "q_raw", (B, H, L, d_k), device=dev)
    _check(k_raw, "k_raw", (B, H, L, d_k), q_raw.dtype, dev)
    _check(beta_logit, "beta_logit", (B, H, L), torch.float32, dev)
    if in_place:
        qh, kh, b = q_raw, k_raw, beta_logit
    else:
        qh = _alloc(q_raw.shape, q_raw.dtype, dev, stream)
        kh = _alloc(k_raw.shape, k_raw.dtype, dev, stream)
        b = _alloc(beta_logit.shape, beta_logit.dtype, dev, stream)
    st = lib.deltanet_feature_prep(_ptr(q_raw), _ptr(k_raw), _ptr(beta_logit), _ptr(qh), _ptr(kh),
                                   _ptr(b), B, H, L, d_k, _code(q_raw.dtype), _stream(dev, stream))
    if st != DN_OK:
        _raise(lib, st, "deltanet_feature_prep")
    return qh, kh, b


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              S0: Optional[torch.Tensor] = None, C: int = 64, *,
              out_dtype: torch.dtype = torch.float32, o: Optional[torch.Tensor] = None,
              S_final: Optional[torch.Tensor] = None, want_state: bool = True,
              workspace: Optional[torch.Tensor] = None, stream=None,
              alpha: Optional[torch.Tensor] = None, features: bool = False
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked delta-rule forward.  q,k ``[B,H,L,d_k]``, v ``[B,H,L,d_v]`` (fp32 or
    bf16, same dtype), beta ``[B,H,L]`` fp32, S0 ``[B,H,d_k,d_v]`` fp32 or None.
    With ``alpha`` (``[B,H,L]`` fp32) the gated form runs
    (``deltanet_gated_chunk_fwd``).  With ``features`` q, k are the raw
    projections and beta the logits, mapped by the layer's feature maps first
    (``deltanet_chunk_fwd_features``).  Returns ``(o, S_final)``; S_final is
    None when ``want_state`` is False."""
    lib = load()
    B, H, L, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _check(q, "q", (B, H, L, d_k), device=dev)
    _check(k, "k", (B, H, L, d_k), q.dtype, dev)
    _check(v, "v", (B, H, L, d_v), q.dtype, dev)
    _check(beta, "beta", (B, H, L), torch.float32, dev)
    if alpha is not None:
        _check(alpha, "alpha", (B, H, L), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = _alloc((B, H, L, d_v), out_dtype, dev, stream)
    _check(o, "o", (B, H, L, d_v), out_dtype, dev)
    if S_final is None and want_state:
        S_final = _alloc((B, H, d_k, d_v), torch.float32, dev, stream)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, d_k, d_v), torch.float32, dev)
    in_code = _code(q.dtype)
    need = workspace_bytes(B, H, L, d_k, d_v, C, q.dtype, gated=alpha is not None,
                           features=features)
    if workspace is None and need > 0:
        workspace = _alloc(need, torch.uint8, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if features:
        st = lib.deltanet_chunk_fwd_features(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                             _ptr(S0), _ptr(o), _ptr(S_final), B, H, L, d_k, d_v,
                                             C, in_code, _code(out_dtype), _ptr(workspace),
                                             ws_bytes, _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_chunk_fwd_features")
    elif alpha is None:
        st = lib.deltanet_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o),
                                    _ptr(S_final), B, H, L, d_k, d_v, C, in_code,
                                    _code(out_dtype), _ptr(workspace), ws_bytes,
                                    _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_chunk_fwd")
    else:
        st = lib.deltanet_gated_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(S0), _ptr(o), _ptr(S_final), B, H, L, d_k, d_v, C,
                                          in_code, _code(out_dtype), _ptr(workspace), ws_bytes,
                                          _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_gated_chunk_fwd")
    return o, S_final


def gated_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                    beta: torch.Tensor, S0: Optional[torch.Tensor] = None, C: int = 64, **kw
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated (Gated DeltaNet) chunked forward: ``chunk_fwd`` with a per-token
    decay alpha ``[B,H,L]`` fp32 applied to the state before each write."""
    return chunk_fwd(q, k, v, beta, S0, C, alpha=alpha, **kw)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                S: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                o: Optional[torch.Tensor] = None, stream=None,
                alpha: Optional[torch.Tensor] = None, features: bool = False) -> torch.Tensor:
    """One decode step; updates S ``[B,H,d_k,d_v]`` in place and returns o
    ``[B,H,d_v]`` = q S_new.  With ``alpha`` (``[B,H]`` fp32) the gated step
    runs (``deltanet_gated_decode_step``).  With ``features`` q, k are the raw
    projections and beta the logits, mapped inside the step's kernel
    (``deltanet_decode_step_features``)."""
    lib = load()
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _check(q, "q", (B, H, d_k), device=dev)
    _check(k, "k", (B, H, d_k), q.dtype, dev)
    _check(v, "v", (B, H, d_v), q.dtype, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = _alloc((B, H, d_v), out_dtype, dev, stream)
    _check(o, "o", (B, H, d_v), out_dtype, dev)
    if alpha is not None:
        _check(alpha, "alpha", (B, H), torch.float32, dev)
    if features:
        st = lib.deltanet_decode_step_features(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                               _ptr(S), _ptr(o), B, H, d_k, d_v, _code(q.dtype),
                                               _code(out_dtype), _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_decode_step_features")
    elif alpha is None:
        st = lib.deltanet_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(o),
                                      B, H, d_k, d_v, _code(q.dtype), _code(out_dtype),
                                      _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_decode_step")
    else:
        st = lib.deltanet_gated_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                            _ptr(S), _ptr(o), B, H, d_k, d_v, _code(q.dtype),
                                            _code(out_dtype), _stream(dev, stream))
        if st != DN_OK:
            _raise(lib, st, "deltanet_gated_decode_step")
    return o


def gated_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                      beta: torch.Tensor, S: torch.Tensor, **kw) -> torch.Tensor:
    """Gated decode step: ``decode_step`` with the per-(b, h) decay alpha."""
    return decode_step(q, k, v, beta, S, alpha=alpha, **kw)


def profile_start() -> None:
    """Start bracketing this thread's kernel launches with HIP events."""
    st = load().deltanet_profile_start()
    if st != DN_OK:
        _raise(load(), st, "deltanet_profile_start")


def profile_stop() -> dict:
    """Stop, wait for the recorded events and return
    ``{slot: (total_ms, launches)}`` for the slots that launched."""
    lib = load()
    n = len(PROFILE_SLOTS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    st = lib.deltanet_profile_stop(ms, cnt, n)
    if st != DN_OK:
        _raise(lib, st, "deltanet_profile_stop")
    return {PROFILE_SLOTS[i]: (ms[i], cnt[i]) for i in range(n) if cnt[i]}
