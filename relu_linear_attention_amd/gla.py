"""ctypes binding of libgla.so (C ABI in include/gla.h).

Argument marshalling only: every step of the operator runs in the HIP
library.  The functions carry the C names and take torch tensors that live in
device memory ([B, N, H, d], contiguous, bfloat16 or float32); sizes are taken
from the tensors and the latent grid (T, Hs, Ws).  If the library has not
been built, loading raises - there is no fallback.

Operator: "SANA-Video 2.0" (arXiv 2607.21553) Section 2 Eq. (1) with the
sigmoid output gate; "SANA-Video" notes page Sections 3.2 (ReLU, RoPE after
ReLU in the numerator only) and 3.4 (block-causal carry).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgla.so")

GLA_OK, GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED, GLA_ERR_ALLOC, GLA_ERR_HIP = range(5)
GLA_BF16, GLA_F32 = 0, 1
GLA_NUM_STAGES = 6

# every symbol include/gla.h declares
EXPORTS = (
    "gla_forward", "gla_block_causal_forward", "gla_workspace_bytes", "gla_forward_ws",
    "gla_forward_noalloc", "gla_state", "gla_block_step", "gla_gated_forward", "gla_backward",
    "gla_backward_workspace_bytes", "gla_saved_state_bytes", "gla_forward_train",
    "gla_backward_saved", "gla_token_causal_forward", "gla_token_causal_workspace_bytes",
    "gla_status_string", "gla_last_error", "gla_profile_enable",
    "gla_profile_read", "gla_stage_name", "gla_uses_matrix_cores",
)

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f = ctypes.c_float


class GlaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status}): {detail}")


def load():
    """Load libgla.so (built by relu_linear_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m relu_linear_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    tensors5 = [_vp] * 5
    sizes6 = [_i64] * 6
    lib.gla_forward.argtypes = tensors5 + sizes6 + [_f, _f, ctypes.c_int, _vp]
    lib.gla_block_causal_forward.argtypes = tensors5 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp]
    lib.gla_workspace_bytes.argtypes = sizes6 + [_i64, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.gla_forward_ws.argtypes = (tensors5 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp,
                                                        ctypes.c_size_t, _vp])
    lib.gla_forward_noalloc.argtypes = tensors5 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp]
    lib.gla_state.argtypes = [_vp] * 4 + sizes6 + [_i64, _f, ctypes.c_int, _vp]
    lib.gla_block_step.argtypes = (tensors5 + [_vp, _vp] + sizes6 + [_i64, ctypes.c_int, _f, _f,
                                                                    ctypes.c_int, _vp,
                                                                    ctypes.c_size_t, _vp])
    lib.gla_gated_forward.argtypes = ([_vp] * 7 + sizes6 + [_i64, _f, _f, _f, ctypes.c_int, _vp,
                                                            ctypes.c_size_t, _vp])
    lib.gla_backward.argtypes = ([_vp] * 9 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp,
                                                        ctypes.c_size_t, _vp])
    lib.gla_backward_workspace_bytes.argtypes = sizes6 + [_i64, ctypes.c_int,
                                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.gla_saved_state_bytes.argtypes = sizes6 + [_i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.gla_forward_train.argtypes = (tensors5 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp, _vp,
                                                           ctypes.c_size_t, _vp])
    lib.gla_backward_saved.argtypes = ([_vp] * 10 + sizes6 + [_i64, _f, _f, ctypes.c_int, _vp,
                                                              ctypes.c_size_t, _vp])
    lib.gla_token_causal_forward.argtypes = (tensors5 + sizes6 + [_f, _f, ctypes.c_int, _vp,
                                                                  ctypes.c_size_t, _vp])
    lib.gla_token_causal_workspace_bytes.argtypes = sizes6 + [ctypes.c_int,
                                                              ctypes.POINTER(ctypes.c_size_t)]
    for name in ("gla_forward", "gla_block_causal_forward", "gla_workspace_bytes",
                 "gla_forward_ws", "gla_forward_noalloc", "gla_state", "gla_block_step", "gla_gated_forward",
                 "gla_backward", "gla_backward_workspace_bytes", "gla_saved_state_bytes",
                 "gla_forward_train", "gla_backward_saved", "gla_token_causal_forward",
                 "gla_token_causal_workspace_bytes", "gla_profile_enable",
                 "gla_profile_read"):
        getattr(lib, name).restype = ctypes.c_int
    lib.gla_status_string.argtypes = [ctypes.c_int]
    lib.gla_status_string.restype = ctypes.c_char_p
    lib.gla_last_error.argtypes = []
    lib.gla_last_error.restype = ctypes.c_char_p
    lib.gla_profile_enable.argtypes = [ctypes.c_int]
    lib.gla_profile_read.argtypes = [ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]
    lib.gla_stage_name.argtypes = [ctypes.c_int]
    lib.gla_stage_name.restype = ctypes.c_char_p
    lib.gla_uses_matrix_cores.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.gla_uses_matrix_cores.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gla_status_string(status).decode()


def gla_status_string(status: int) -> str:
    return status_string(status)


def gla_last_error() -> str:
    return load().gla_last_error().decode()


def _check(status: int, where: str):
    if status != GLA_OK:
        raise GlaError(status, where, gla_last_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _sizes(q, grid):
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    if N != T * Hs * Ws:
        raise ValueError(f"N={N} does not match the grid {T}x{Hs}x{Ws}")
    return B, H, T, Hs, Ws, d


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensors(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")


def gla_forward(q, k, v, g, out, grid, rope_theta=10000.0, eps=1e-6, stream=None):
    """Non-causal operator; writes out ([B, N, H, d], same dtype as q)."""
    _check_tensors(q, k, v, g, out)
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    st = load().gla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T, Hs, Ws, d,
                            rope_theta, eps, _dtype_code(q), _stream_handle(stream))
    _check(st, "gla_forward")


def gla_block_causal_forward(q, k, v, g, out, grid, frames_per_block, rope_theta=10000.0,
                             eps=1e-6, stream=None):
    """Block-causal operator with blocks of frames_per_block latent frames."""
    _check_tensors(q, k, v, g, out)
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    st = load().gla_block_causal_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T,
                                         Hs, Ws, d, frames_per_block, rope_theta, eps,
                                         _dtype_code(q), _stream_handle(stream))
    _check(st, "gla_block_causal_forward")


def gla_workspace_bytes(B, H, T, Hs, Ws, d, frames_per_block=0, dtype=GLA_BF16) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_workspace_bytes(B, H, T, Hs, Ws, d, frames_per_block, dtype, ctypes.byref(n))
    _check(st, "gla_workspace_bytes")
    return int(n.value)


def gla_forward_ws(q, k, v, g, out, grid, workspace, frames_per_block=0, rope_theta=10000.0,
                   eps=1e-6, stream=None):
    """Either operator with a caller-owned workspace (a uint8 device tensor)."""
    _check_tensors(q, k, v, g, out, workspace)
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    st = load().gla_forward_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T, Hs, Ws, d,
                               frames_per_block, rope_theta, eps, _dtype_code(q),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream_handle(stream))
    _check(st, "gla_forward_ws")


def gla_forward_noalloc(q, k, v, g, out, grid, frames_per_block=0, rope_theta=10000.0, eps=1e-6,
                        stream=None):
    """gla_forward_ws without a workspace: the library's static per-device
    scratch array serves instead, and nothing is allocated."""
    _check_tensors(q, k, v, g, out)
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    st = load().gla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T, Hs,
                                    Ws, d, frames_per_block, rope_theta, eps, _dtype_code(q),
                                    _stream_handle(stream))
    _check(st, "gla_forward_noalloc")


def gla_state(k, v, S_out, z_out, grid, frames_per_block=0, rope_theta=10000.0, stream=None):
    """Export S [B, H, nb, d, d] and z [B, H, nb, d] (float32 device tensors)."""
    _check_tensors(k, v, S_out, z_out)
    B, H, T, Hs, Ws, d = _sizes(k, grid)
    st = load().gla_state(_ptr(k), _ptr(v), _ptr(S_out), _ptr(z_out), B, H, T, Hs, Ws, d,
                          frames_per_block, rope_theta, _dtype_code(k), _stream_handle(stream))
    _check(st, "gla_state")


def gla_block_step(q, k, v, g, out, S, z, block_grid, t_offset, update=True, rope_theta=10000.0,
                   eps=1e-6, workspace=None, stream=None):
    """One streaming block-causal step: the block of block_grid = (Tb, Hs, Ws)
    latent frames at temporal position t_offset attends to itself and to
    the cache S ([B, H, d, d] float32), z ([B, H, d] float32); with update
    the cache then takes the block's sums in place.  out (with q and g) may
    be None for a cache-only update."""
    _check_tensors(*[t for t in (q, k, v, g, out, S, z, workspace) if t is not None])
    B, H, Tb, Hs, Ws, d = _sizes(k, block_grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_block_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), _ptr(S), _ptr(z),
                               B, H, Tb, Hs, Ws, d, int(t_offset), 1 if update else 0,
                               rope_theta, eps, _dtype_code(k), _ptr(workspace), ws_bytes,
                               _stream_handle(stream))
    _check(st, "gla_block_step")


def gla_gated_forward(q, k, v, g, beta, rms_weight, out, grid, frames_per_block=0,
                      rope_theta=10000.0, eps=1e-6, rms_eps=1e-6, workspace=None, stream=None):
    """The gated mixer of Eq. (1) without W_o: beta [B, N, H] (None: no write
    gate) and rms_weight [d] (None: no RMSNorm), both of q's dtype."""
    _check_tensors(*[t for t in (q, k, v, g, beta, rms_weight, out, workspace) if t is not None])
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_gated_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(rms_weight),
                                  _ptr(out), B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                                  rms_eps, _dtype_code(q), _ptr(workspace), ws_bytes,
                                  _stream_handle(stream))
    _check(st, "gla_gated_forward")


def gla_backward(q, k, v, g, dout, dq, dk, dv, dg, grid, frames_per_block=0, rope_theta=10000.0,
                 eps=1e-6, workspace=None, stream=None):
    """Gradients dq, dk, dv, dg (written in place) of sum(dout * out)."""
    _check_tensors(*[t for t in (q, k, v, g, dout, dq, dk, dv, dg, workspace) if t is not None])
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dg), B, H, T, Hs, Ws, d, frames_per_block, rope_theta,
                             eps, _dtype_code(q), _ptr(workspace), ws_bytes,
                             _stream_handle(stream))
    _check(st, "gla_backward")


def gla_backward_workspace_bytes(B, H, T, Hs, Ws, d, frames_per_block=0, dtype=GLA_BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gla_backward_workspace_bytes(B, H, T, Hs, Ws, d, frames_per_block, dtype,
                                               ctypes.byref(n)), "gla_backward_workspace_bytes")
    return n.value


def gla_saved_state_bytes(B, H, T, Hs, Ws, d, frames_per_block=0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gla_saved_state_bytes(B, H, T, Hs, Ws, d, frames_per_block, ctypes.byref(n)),
           "gla_saved_state_bytes")
    return n.value


def gla_forward_train(q, k, v, g, out, saved, grid, frames_per_block=0, rope_theta=10000.0,
                      eps=1e-6, workspace=None, stream=None):
    """Either operator, which also writes its reduced state (S, z of every
    (batch, head, block), fp32) into `saved` (a device tensor of
    gla_saved_state_bytes() bytes) for gla_backward_saved."""
    _check_tensors(*[t for t in (q, k, v, g, out, saved, workspace) if t is not None])
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T, Hs, Ws,
                                  d, frames_per_block, rope_theta, eps, _dtype_code(q),
                                  _ptr(saved), _ptr(workspace), ws_bytes, _stream_handle(stream))
    _check(st, "gla_forward_train")


def gla_backward_saved(q, k, v, g, dout, dq, dk, dv, dg, saved, grid, frames_per_block=0,
                       rope_theta=10000.0, eps=1e-6, workspace=None, stream=None):
    """gla_backward given the state a gla_forward_train call kept in `saved`
    (the state stage is not re-run)."""
    _check_tensors(*[t for t in (q, k, v, g, dout, dq, dk, dv, dg, saved, workspace)
                     if t is not None])
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_backward_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(dg), _ptr(saved), B, H, T, Hs, Ws, d,
                                   frames_per_block, rope_theta, eps, _dtype_code(q),
                                   _ptr(workspace), ws_bytes, _stream_handle(stream))
    _check(st, "gla_backward_saved")


def gla_token_causal_forward(q, k, v, g, out, grid, rope_theta=10000.0, eps=1e-6, workspace=None,
                             stream=None):
    """Token-causal form: token i attends to tokens 0..i (out written in place)."""
    _check_tensors(*[t for t in (q, k, v, g, out, workspace) if t is not None])
    B, H, T, Hs, Ws, d = _sizes(q, grid)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gla_token_causal_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, T,
                                         Hs, Ws, d, rope_theta, eps, _dtype_code(q),
                                         _ptr(workspace), ws_bytes, _stream_handle(stream))
    _check(st, "gla_token_causal_forward")


def gla_token_causal_workspace_bytes(B, H, T, Hs, Ws, d, dtype=GLA_BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gla_token_causal_workspace_bytes(B, H, T, Hs, Ws, d, dtype, ctypes.byref(n)),
           "gla_token_causal_workspace_bytes")
    return n.value


def gla_profile_enable(enable: bool = True):
    _check(load().gla_profile_enable(1 if enable else 0), "gla_profile_enable")


def gla_profile_read():
    """Returns {stage name: (launches, total_ms)} for the recorded launches."""
    lib = load()
    launches = (_i64 * GLA_NUM_STAGES)()
    ms = (ctypes.c_double * GLA_NUM_STAGES)()
    _check(lib.gla_profile_read(launches, ms), "gla_profile_read")
    return {lib.gla_stage_name(s).decode(): (int(launches[s]), float(ms[s]))
            for s in range(GLA_NUM_STAGES)}


def gla_stage_name(stage: int) -> str:
    return load().gla_stage_name(stage).decode()


def gla_uses_matrix_cores(T, Hs, Ws, d, dtype=GLA_BF16) -> int:
    return int(load().gla_uses_matrix_cores(T, Hs, Ws, d, dtype))
