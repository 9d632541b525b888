"""The C ABI without a GPU: the library loads, exports every symbol that
include/gla.h declares, and rejects bad arguments on the host before any HIP
call.  No compute call is made here."""
import ctypes
import os
import re

import pytest

from relu_linear_attention_amd import gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.LIB_PATH):
        from relu_linear_attention_amd import build

        build.build()
    return gla.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(gla.EXPORTS) == _declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, text in [(0, "success"), (1, "invalid argument"), (2, "unsupported configuration"),
                       (3, "workspace allocation failed"), (4, "HIP runtime error")]:
        assert gla.status_string(code) == text
    assert gla.status_string(99) == "unknown status"


FAKE = 1 << 20  # a non-null address; validation fails before anything reads it


def _fwd(lib, ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9), B=1, H=2, T=2, Hs=4, Ws=4,
         d=32, theta=10000.0, eps=1e-6, dtype=gla.GLA_BF16):
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return lib.gla_forward(*p, B, H, T, Hs, Ws, d, theta, eps, dtype, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(d=24), "d must be"),
    (dict(d=144), "d must be"),
    (dict(d=0), "d must be"),
    (dict(B=0), ">= 1"),
    (dict(T=-1), ">= 1"),
    (dict(Ws=0), ">= 1"),
    (dict(dtype=7), "dtype"),
    (dict(eps=-1.0), "eps"),
    (dict(eps=float("nan")), "eps"),
    (dict(theta=float("inf")), "rope_theta"),
    (dict(B=1 << 20, H=1 << 20, T=1 << 20, Hs=1 << 20, Ws=1), "overflow"),
    (dict(ptrs=(0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4)), "null"),
    (dict(ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 0)), "null"),
    (dict(ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 2 + 64)), "overlaps input k"),
    (dict(ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE)), "overlaps input q"),
])
def test_forward_rejects_bad_arguments(lib, kw, needle):
    assert _fwd(lib, **kw) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def test_block_causal_rejects_bad_blocks(lib):
    p = [ctypes.c_void_p(FAKE * i) for i in (1, 3, 5, 7, 9)]
    assert lib.gla_block_causal_forward(*p, 1, 2, 6, 4, 4, 32, 4, 1e4, 1e-6, 0, None) == 1
    assert "divide" in gla.gla_last_error()
    assert lib.gla_block_causal_forward(*p, 1, 2, 6, 4, 4, 32, 0, 1e4, 1e-6, 0, None) == 1
    assert ">= 1" in gla.gla_last_error()


def test_forward_ws_rejects_bad_workspace(lib):
    p = [ctypes.c_void_p(FAKE * i) for i in (1, 3, 5, 7, 9)]
    assert lib.gla_forward_ws(*p, 1, 2, 2, 4, 4, 32, 0, 1e4, 1e-6, 0, None, 1 << 20, None) == 1
    assert "workspace" in gla.gla_last_error()
    assert lib.gla_forward_ws(*p, 1, 2, 2, 4, 4, 32, 0, 1e4, 1e-6, 0, ctypes.c_void_p(FAKE + 8),
                              1 << 20, None) == 1
    assert "aligned" in gla.gla_last_error()
    assert lib.gla_forward_ws(*p, 1, 2, 6, 4, 4, 32, 4, 1e4, 1e-6, 0, ctypes.c_void_p(FAKE * 11),
                              1 << 20, None) == 1


def test_state_rejects_bad_arguments(lib):
    k, v = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE * 2)
    assert lib.gla_state(k, v, None, ctypes.c_void_p(FAKE * 3), 1, 1, 2, 2, 2, 32, 0, 1e4, 0,
                         None) == 1
    assert lib.gla_state(k, v, ctypes.c_void_p(FAKE * 3), ctypes.c_void_p(FAKE * 4), 1, 1, 2, 2, 2,
                         40, 0, 1e4, 0, None) == 1


def _step(lib, ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9), S=FAKE * 11, z=FAKE * 13,
          B=1, H=2, Tb=2, Hs=4, Ws=4, d=32, t_offset=0, update=1, ws=None, ws_bytes=0):
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    c = [ctypes.c_void_p(x) if x else None for x in (S, z)]
    w = ctypes.c_void_p(ws) if ws else None
    return lib.gla_block_step(*p, *c, B, H, Tb, Hs, Ws, d, t_offset, update, 1e4, 1e-6,
                              gla.GLA_BF16, w, ws_bytes, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(S=0), "null cache"),
    (dict(z=0), "null cache"),
    (dict(ptrs=(FAKE, 0, FAKE * 5, FAKE * 7, FAKE * 9)), "null"),
    (dict(ptrs=(0, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9)), "null"),
    (dict(ptrs=(0, FAKE * 3, FAKE * 5, 0, 0), update=0), "nothing"),
    (dict(t_offset=-1), "t_offset"),
    (dict(t_offset=(1 << 31) - 2), "t_offset"),
    (dict(S=FAKE * 11 + 2), "aligned"),
    (dict(z=FAKE * 11 + 64), "overlap"),
    (dict(S=FAKE * 3 + 128), "overlaps k"),
    (dict(z=FAKE * 9), "overlaps out"),
    (dict(d=40), "d must be"),
    (dict(ws=FAKE * 15 + 8, ws_bytes=1 << 20), "aligned"),
])
def test_block_step_rejects_bad_arguments(lib, kw, needle):
    assert _step(lib, **kw) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def _gated(lib, beta=FAKE * 11, w=FAKE * 13, rms_eps=1e-6, out=FAKE * 9, F=0):
    p = [ctypes.c_void_p(x) if x else None for x in (FAKE, FAKE * 3, FAKE * 5, FAKE * 7)]
    gb = [ctypes.c_void_p(x) if x else None for x in (beta, w, out)]
    return lib.gla_gated_forward(*p, *gb, 1, 2, 2, 4, 4, 32, F, 1e4, 1e-6, rms_eps, gla.GLA_BF16,
                                 None, 0, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(beta=FAKE * 11 + 1), "beta is misaligned"),
    (dict(w=FAKE * 13 + 1), "rms_weight is misaligned"),
    (dict(rms_eps=0.0), "rms_eps"),
    (dict(rms_eps=float("nan")), "rms_eps"),
    (dict(beta=FAKE * 9 + 64), "overlaps beta"),
    (dict(w=FAKE * 9 + 64), "overlaps rms_weight"),
    (dict(out=0), "null"),
    (dict(F=3), "divide"),
])
def test_gated_forward_rejects_bad_arguments(lib, kw, needle):
    assert _gated(lib, **kw) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def _bwd(lib, ins=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9),
         outs=(FAKE * 11, FAKE * 13, FAKE * 15, FAKE * 17), F=0, eps=1e-6, ws=None):
    p = [ctypes.c_void_p(x) if x else None for x in ins + outs]
    w = ctypes.c_void_p(ws) if ws else None
    return lib.gla_backward(*p, 1, 2, 2, 4, 4, 32, F, 1e4, eps, gla.GLA_BF16, w, 1 << 20, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(ins=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, 0)), "null tensor pointer (dout)"),
    (dict(outs=(FAKE * 11, 0, FAKE * 15, FAKE * 17)), "null tensor pointer (dk)"),
    (dict(outs=(FAKE * 11, FAKE * 13, FAKE * 15, FAKE * 9 + 64)), "dg overlaps input dout"),
    (dict(outs=(FAKE * 11, FAKE * 11 + 64, FAKE * 15, FAKE * 17)), "dq overlaps dk"),
    (dict(F=3), "divide"),
    (dict(eps=-1.0), "eps"),
    (dict(ws=FAKE * 19 + 8), "aligned"),
])
def test_backward_rejects_bad_arguments(lib, kw, needle):
    assert _bwd(lib, **kw) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def _causal(lib, ts=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9), d=32, eps=1e-6, theta=1e4,
            ws=None):
    p = [ctypes.c_void_p(x) if x else None for x in ts]
    w = ctypes.c_void_p(ws) if ws else None
    return lib.gla_token_causal_forward(*p, 1, 2, 2, 4, 4, d, theta, eps, gla.GLA_BF16, w, 1 << 20,
                                        None)


@pytest.mark.parametrize("kw,needle", [
    (dict(ts=(FAKE, 0, FAKE * 5, FAKE * 7, FAKE * 9)), "null tensor pointer"),
    (dict(ts=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 5 + 32)), "out overlaps input v"),
    (dict(d=40), "multiple of 16"),
    (dict(eps=float("nan")), "eps"),
    (dict(theta=float("inf")), "rope_theta"),
    (dict(ws=FAKE * 19 + 8), "aligned"),
])
def test_token_causal_rejects_bad_arguments(lib, kw, needle):
    assert _causal(lib, **kw) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def test_saved_state_bytes(lib):
    # one record of d*d + d floats per (batch, head, temporal block)
    assert gla.gla_saved_state_bytes(2, 3, 6, 4, 5, 64, 0) == 2 * 3 * 1 * (64 * 64 + 64) * 4
    assert gla.gla_saved_state_bytes(2, 3, 6, 4, 5, 64, 2) == 2 * 3 * 3 * (64 * 64 + 64) * 4
    n = ctypes.c_size_t(0)
    assert lib.gla_saved_state_bytes(1, 1, 3, 2, 2, 128, 2, ctypes.byref(n)) == 1
    assert "divide" in gla.gla_last_error()
    assert lib.gla_saved_state_bytes(1, 1, 3, 2, 2, 128, 0, None) == 1


def _train(lib, saved, ts=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, FAKE * 9)):
    p = [ctypes.c_void_p(x) for x in ts]
    s = ctypes.c_void_p(saved) if saved else None
    return lib.gla_forward_train(*p, 1, 2, 2, 4, 4, 32, 0, 1e4, 1e-6, gla.GLA_BF16, s, None, 0,
                                 None)


def _bwd_saved(lib, saved):
    p = [ctypes.c_void_p(FAKE * i) for i in (1, 3, 5, 7, 9, 11, 13, 15, 17)]
    s = ctypes.c_void_p(saved) if saved else None
    return lib.gla_backward_saved(*p, s, 1, 2, 2, 4, 4, 32, 0, 1e4, 1e-6, gla.GLA_BF16, None, 0,
                                  None)


@pytest.mark.parametrize("call", [_train, _bwd_saved])
@pytest.mark.parametrize("saved,needle", [
    (0, "saved must not be null"),
    (FAKE * 21 + 16, "256-byte aligned"),
    (FAKE * 3 + 256, "overlaps"),  # inside k (each fake tensor spans 4 KiB here)
])
def test_training_pair_rejects_bad_saved_state(lib, call, saved, needle):
    assert call(lib, saved) == gla.GLA_ERR_INVALID_ARG
    assert needle in gla.gla_last_error()


def test_workspace_query_rejects_bad_sizes(lib):
    n = ctypes.c_size_t(0)
    assert lib.gla_workspace_bytes(1, 1, 3, 2, 2, 128, 2, 0, ctypes.byref(n)) == 1
    assert lib.gla_workspace_bytes(1, 1, 3, 2, 2, 128, 0, 0, None) == 1


def test_kernel_family_selection(lib):
    # bf16 with d = 64 / 128 runs on the matrix cores; fp32 and other d on vector kernels
    assert gla.gla_uses_matrix_cores(21, 45, 80, 128, gla.GLA_BF16) == 1
    assert gla.gla_uses_matrix_cores(21, 45, 80, 64, gla.GLA_BF16) == 1
    assert gla.gla_uses_matrix_cores(2, 4, 4, 32, gla.GLA_BF16) == 0
    assert gla.gla_uses_matrix_cores(2, 4, 4, 128, gla.GLA_F32) == 0
    assert gla.gla_uses_matrix_cores(2, 4, 4, 112, gla.GLA_BF16) == 0
    # spatial RoPE rows that do not fit in LDS fall back to the vector kernels
    assert gla.gla_uses_matrix_cores(2, 200, 200, 128, gla.GLA_BF16) == 0
    assert gla.gla_uses_matrix_cores(2, 4, 4, 40, gla.GLA_BF16) == -1


def test_profile_read_without_records(lib):
    gla.gla_profile_enable(True)
    rec = gla.gla_profile_read()
    assert set(rec) == {"rope_table", "state_partials", "reduce_prefix", "apply", "backward",
                        "causal_apply"}
    assert all(v == (0, 0.0) for v in rec.values())
    gla.gla_profile_enable(False)


def _device_count() -> int:
    try:
        import torch

        return torch.cuda.device_count()  # does not initialise the GPU
    except Exception:
        return 0


@pytest.mark.skipif(_device_count() > 0, reason="a GPU is visible: the call would launch kernels")
def test_valid_call_without_a_device_is_a_hip_error(lib):
    # arguments that pass every host check; the first HIP call (the device
    # query) fails, which is GLA_ERR_HIP naming that call
    p = [ctypes.c_void_p(FAKE * i) for i in (1, 3, 5, 7, 9)]
    assert lib.gla_forward(*p, 1, 2, 2, 4, 4, 32, 1e4, 1e-6, 0, None) == 4
    assert "hipGetDevice" in gla.gla_last_error()
    assert gla.status_string(4) == "HIP runtime error"
