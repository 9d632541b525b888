"""Oracle for the gated ReLU linear-attention token mixer (fp64, CPU).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path (the
HIP library and its binding) never imports this package.

This module compiles ``oracle.c`` with gcc into ``liboracle.so`` and wraps its
entry points with numpy marshalling:

* :func:`rope`    - 3D rotary embedding of one vector at a (t, h, w) position
* :func:`state`   - S = sum_n RoPE(phi(k_n))^T v_n and z = sum_n phi(k_n),
                    per (batch, head), inclusive per temporal block
* :func:`apply`   - out_i = (RoPE(phi(q_i)) S) / (phi(q_i).z + eps) * sigmoid(g_i)
* :func:`forward` - state followed by apply over every token
* :func:`block_step`, :func:`gated_forward`, :func:`backward`,
  :func:`token_causal` - the streaming step, the gated mixer, the gradients
  and the token-causal form

The formulas follow "SANA-Video 2.0" (arXiv 2607.21553) Section 2, Eq. (1)
(gate, +eps) and the SANA-Video notes page, Section 3.2 (ReLU feature map,
RoPE after ReLU in the numerator only) and Section 3.4 (block-causal carry);
the C source states every reading taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.ora_rope.argtypes = [_ptr, _ptr, _i64, _ptr, _dbl]
    lib.ora_rope.restype = None
    lib.ora_state.argtypes = [_ptr, _ptr] + [_i64] * 7 + [_dbl, _ptr, _ptr, _ptr]
    lib.ora_state.restype = ctypes.c_int
    lib.ora_apply.argtypes = ([_ptr] * 4 + [_i64] * 7 + [_dbl, _dbl, _ptr, _ptr, _i64, _ptr])
    lib.ora_apply.restype = ctypes.c_int
    lib.ora_forward.argtypes = [_ptr] * 4 + [_i64] * 7 + [_dbl, _dbl, _ptr, _ptr]
    lib.ora_forward.restype = ctypes.c_int
    lib.ora_block_step.argtypes = [_ptr] * 6 + [_i64] * 7 + [_dbl, _dbl, _ptr, _ptr, _ptr]
    lib.ora_block_step.restype = ctypes.c_int
    lib.ora_gated_forward.argtypes = [_ptr] * 6 + [_i64] * 7 + [_dbl, _dbl, _dbl, _ptr]
    lib.ora_gated_forward.restype = ctypes.c_int
    lib.ora_backward.argtypes = [_ptr] * 5 + [_i64] * 7 + [_dbl, _dbl] + [_ptr] * 4
    lib.ora_backward.restype = ctypes.c_int
    lib.ora_token_causal.argtypes = [_ptr] * 4 + [_i64] * 6 + [_dbl, _dbl, _ptr]
    lib.ora_token_causal.restype = ctypes.c_int
    lib.ora_num_blocks.argtypes = [_i64, _i64]
    lib.ora_num_blocks.restype = _i64
    lib.ora_num_threads.argtypes = []
    lib.ora_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _pos0(pos0):
    if pos0 is None:
        return None
    return np.ascontiguousarray(np.asarray(pos0, dtype=np.int64).reshape(3))


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def num_blocks(T: int, frames_per_block: int) -> int:
    return int(_load().ora_num_blocks(T, frames_per_block))


def num_threads() -> int:
    return int(_load().ora_num_threads())


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate one feature vector x (length d) at position pos = (t, h, w)."""
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    y = np.empty_like(x)
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(3))
    _load().ora_rope(_p(x), _p(y), x.size, _p(p), float(theta))
    return y


def state(k, v, grid, frames_per_block: int = 0, theta: float = 10000.0, pos0=None):
    """k, v: [B, N, H, d] arrays.  Returns S [B, H, nb, d, d], z [B, H, nb, d] (fp64)."""
    k, v = _f32(k), _f32(v)
    B, N, H, d = k.shape
    T, Hs, Ws = grid
    assert v.shape == k.shape and N == T * Hs * Ws
    nb = num_blocks(T, frames_per_block)
    S = np.empty((B, H, nb, d, d), dtype=np.float64)
    z = np.empty((B, H, nb, d), dtype=np.float64)
    p0 = _pos0(pos0)
    rc = _load().ora_state(_p(k), _p(v), B, H, T, Hs, Ws, d, frames_per_block, float(theta),
                           _p(p0), _p(S), _p(z))
    _check(rc, "state")
    return S, z


def apply(q, g, S, z, grid, frames_per_block: int = 0, theta: float = 10000.0,
          eps: float = 1e-6, tokens=None, pos0=None) -> np.ndarray:
    """Outputs [B, ntok, H, d] (fp64) for the given token indices (all if None)."""
    q, g = _f32(q), _f32(g)
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    S = np.ascontiguousarray(S, dtype=np.float64)
    z = np.ascontiguousarray(z, dtype=np.float64)
    if tokens is not None:
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(-1))
        ntok = tokens.size
    else:
        ntok = N
    out = np.empty((B, ntok, H, d), dtype=np.float64)
    p0 = _pos0(pos0)
    rc = _load().ora_apply(_p(q), _p(g), _p(S), _p(z), B, H, T, Hs, Ws, d, frames_per_block,
                           float(theta), float(eps), _p(p0), _p(tokens), ntok, _p(out))
    _check(rc, "apply")
    return out


def forward(q, k, v, g, grid, frames_per_block: int = 0, theta: float = 10000.0,
            eps: float = 1e-6, pos0=None) -> np.ndarray:
    """Whole operator; q, k, v, g: [B, N, H, d].  Returns out [B, N, H, d] (fp64)."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    out = np.empty((B, N, H, d), dtype=np.float64)
    p0 = _pos0(pos0)
    rc = _load().ora_forward(_p(q), _p(k), _p(v), _p(g), B, H, T, Hs, Ws, d, frames_per_block,
                             float(theta), float(eps), _p(p0), _p(out))
    _check(rc, "forward")
    return out


def block_step(q, k, v, g, S_cache, z_cache, block_grid, t_offset: int, theta: float = 10000.0,
               eps: float = 1e-6, want_out: bool = True):
    """One step of the streaming block-causal mode: a block of Tb x Hs x Ws
    tokens ([B, N_b, H, d]) whose first frame is at temporal position
    t_offset, attending to itself and to the cache (S_cache [B, H, d, d],
    z_cache [B, H, d]).  Returns (out [B, N_b, H, d] or None, S_new, z_new),
    all fp64; q and g may be None when want_out is False."""
    k, v = _f32(k), _f32(v)
    B, N, H, d = k.shape
    Tb, Hs, Ws = block_grid
    assert N == Tb * Hs * Ws and v.shape == k.shape
    S_cache = np.ascontiguousarray(S_cache, dtype=np.float64).reshape(B, H, d, d)
    z_cache = np.ascontiguousarray(z_cache, dtype=np.float64).reshape(B, H, d)
    qq = _f32(q) if want_out else None
    gg = _f32(g) if want_out else None
    out = np.empty((B, N, H, d), dtype=np.float64) if want_out else None
    S_new = np.empty((B, H, d, d), dtype=np.float64)
    z_new = np.empty((B, H, d), dtype=np.float64)
    rc = _load().ora_block_step(_p(qq), _p(k), _p(v), _p(gg), _p(S_cache), _p(z_cache), B, H, Tb,
                                Hs, Ws, d, int(t_offset), float(theta), float(eps), _p(out),
                                _p(S_new), _p(z_new))
    _check(rc, "block_step")
    return out, S_new, z_new


def gated_forward(q, k, v, g, beta, w, grid, frames_per_block: int = 0, theta: float = 10000.0,
                  eps: float = 1e-6, rms_eps: float = 1e-6) -> np.ndarray:
    """The gated mixer of Eq. (1) without W_o: beta [B, N, H] write gate (None:
    1), w [d] RMSNorm weight (None: no RMSNorm).  Returns out [B, N, H, d]."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    bt = None if beta is None else _f32(beta).reshape(B, N, H)
    ww = None if w is None else _f32(w).reshape(d)
    out = np.empty((B, N, H, d), dtype=np.float64)
    rc = _load().ora_gated_forward(_p(q), _p(k), _p(v), _p(g), _p(bt), _p(ww), B, H, T, Hs, Ws, d,
                                   frames_per_block, float(theta), float(eps), float(rms_eps),
                                   _p(out))
    _check(rc, "gated_forward")
    return out


def backward(q, k, v, g, dout, grid, frames_per_block: int = 0, theta: float = 10000.0,
             eps: float = 1e-6):
    """Gradients of sum(dout * forward(...)) with respect to q, k, v, g, each
    [B, N, H, d] fp64."""
    q, k, v, g, dout = _f32(q), _f32(k), _f32(v), _f32(g), _f32(dout)
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    outs = [np.empty((B, N, H, d), dtype=np.float64) for _ in range(4)]
    rc = _load().ora_backward(_p(q), _p(k), _p(v), _p(g), _p(dout), B, H, T, Hs, Ws, d,
                              frames_per_block, float(theta), float(eps), *[_p(o) for o in outs])
    _check(rc, "backward")
    return tuple(outs)


def token_causal(q, k, v, g, grid, theta: float = 10000.0, eps: float = 1e-6) -> np.ndarray:
    """Token-causal form: token i attends to tokens 0..i through running sums.
    q, k, v, g: [B, N, H, d].  Returns out [B, N, H, d] (fp64)."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    out = np.empty((B, N, H, d), dtype=np.float64)
    rc = _load().ora_token_causal(_p(q), _p(k), _p(v), _p(g), B, H, T, Hs, Ws, d, float(theta),
                                  float(eps), _p(out))
    _check(rc, "token_causal")
    return out
