"""Failure statuses that need a device: GLA_ERR_ALLOC and GLA_ERR_UNSUPPORTED.

The tensors are fake addresses: these calls fail in planning or at the
workspace allocation, before the first enqueue (the header's contract), so
no kernel ever reads them.  A later real call on the same stream must still
work and match the oracle.
"""
import ctypes

import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

GAP = 1 << 40  # fake tensors 1 TiB apart never overlap


def _fake(n):
    return [ctypes.c_void_p(GAP * (i + 1)) for i in range(n)]


def _still_works():
    import torch

    x = host_inputs(1, 2, 4, 6, 2, 128, "bf16", seed=61)
    dev = to_device(x, "bf16")
    out = torch.empty_like(dev["q"])
    gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], out, (2, 4, 6))
    torch.cuda.synchronize()
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (2, 4, 6), 0, 1e4, 1e-6)
    assert max_rel_err(to_host_f32(out), ref) <= TOL["bf16"]


def test_workspace_allocation_failure_is_alloc_error():
    import torch

    lib = gla.load()
    # 2^22 heads of 16 tokens at d = 128: each tensor 17 GB (never touched),
    # the workspace about 0.55 TB, more than the device holds
    B, H, T, Hs, Ws, d = 1, 1 << 22, 1, 1, 16, 128
    need = gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, 0)
    total = torch.cuda.get_device_properties(0).total_memory
    print(f"case: workspace {need / 1e9:.0f} GB on a {total / 1e9:.0f} GB device", flush=True)
    assert need > total
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.gla_forward(*_fake(5), B, H, T, Hs, Ws, d, 1e4, 1e-6, gla.GLA_BF16, stream)
    assert st == 3, gla.gla_last_error()
    assert "workspace" in gla.gla_last_error()
    st = lib.gla_backward(*_fake(9), B, H, T, Hs, Ws, d, 0, 1e4, 1e-6, gla.GLA_BF16, None, 0,
                          stream)
    assert st == 3, gla.gla_last_error()
    torch.cuda.synchronize()
    _still_works()


def test_oversized_grid_is_unsupported():
    import torch

    lib = gla.load()
    # 2^31 (batch, head) units: more workgroups than one launch can address
    B, H, T, Hs, Ws, d = 1, 1 << 31, 1, 1, 1, 16
    print("case: 2^31 heads of one token", flush=True)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.gla_forward(*_fake(5), B, H, T, Hs, Ws, d, 1e4, 1e-6, gla.GLA_BF16, stream)
    assert st == 2, gla.gla_last_error()
    assert "units" in gla.gla_last_error()
    torch.cuda.synchronize()
    _still_works()
