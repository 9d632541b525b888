"""gla_forward_noalloc: the entry point that allocates nothing (its kernels
use the library's static per-device scratch array) against gla_forward_ws,
which runs the same kernels on a caller workspace.  Two calls in a row, the
second on a smaller input, each bitwise equal to gla_forward_ws and within
the operator's tolerance of the fp64 oracle; a call whose workspace exceeds
the scratch array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = pytest.mark.gpu

CASES = [
    # (B, T, Hs, Ws, H, d, dtype, frames_per_block): the first call is the larger one
    (1, 6, 20, 24, 4, 128, "bf16", 0),
    (1, 2, 5, 7, 2, 128, "bf16", 0),
]


@pytest.fixture(scope="module")
def dev():
    if not have_gpu():
        pytest.skip("no GPU")
    import torch

    torch.cuda.set_device(0)
    return torch


def _run_pair(torch, gla, case, seed):
    from relu_linear_attention_amd.inputs import host_inputs

    B, T, Hs, Ws, H, d, dtype, F = case
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=seed)
    t = to_device(x, dtype)
    out_na = torch.full_like(t["q"], float("nan"))
    out_ws = torch.full_like(t["q"], float("nan"))
    code = gla.GLA_BF16 if dtype == "bf16" else gla.GLA_F32
    ws = torch.empty(gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, F, code), dtype=torch.uint8,
                     device="cuda")
    gla.gla_forward_noalloc(t["q"], t["k"], t["v"], t["g"], out_na, (T, Hs, Ws), F)
    gla.gla_forward_ws(t["q"], t["k"], t["v"], t["g"], out_ws, (T, Hs, Ws), ws, F)
    torch.cuda.synchronize()
    return x, out_na, out_ws


@pytest.mark.parametrize("order", ["large_then_small", "causal_then_plain"])
def test_noalloc_matches_forward_ws_twice(dev, order):
    torch = dev
    from relu_linear_attention_amd import gla

    cases = CASES if order == "large_then_small" else [
        (1, 6, 8, 10, 4, 128, "bf16", 2),  # block-causal, three blocks
        (2, 2, 3, 5, 3, 64, "bf16", 0),
    ]
    for i, case in enumerate(cases):
        B, T, Hs, Ws, H, d, dtype, F = case
        print(f"noalloc call {i}: case {case}", flush=True)
        x, out_na, out_ws = _run_pair(torch, gla, case, seed=10 + i)
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), case
        ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), F)
        err = max_rel_err(to_host_f32(out_na), ref)
        assert err <= TOL[dtype], (case, err)


def test_noalloc_refuses_oversized_call(dev):
    from relu_linear_attention_amd import gla

    lib = gla.load()
    # 512 heads of a 32-token grid: the workspace (partials, states and the
    # bf16 parts of S for 512 units) exceeds the 64 MiB scratch array.  The
    # pointers are never dereferenced: the call is refused on the host.
    n = ctypes.c_size_t(0)
    assert lib.gla_workspace_bytes(1, 512, 2, 4, 4, 128, 0, gla.GLA_BF16, ctypes.byref(n)) == 0
    assert n.value > 64 << 20
    fake = [ctypes.c_void_p((i + 1) << 32) for i in range(5)]
    st = lib.gla_forward_noalloc(*fake, 1, 512, 2, 4, 4, 128, 0, 1e4, 1e-6, gla.GLA_BF16, None)
    assert st == gla.GLA_ERR_UNSUPPORTED
    assert "scratch" in gla.gla_last_error()
