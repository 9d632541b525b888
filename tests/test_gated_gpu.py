"""Parity of the gated mixer (gla_gated_forward: write gate beta and RMSNorm
of num/den, "SANA-Video 2.0" Section 2 Eq. (1) short of W_o) with the fp64
oracle, through the C ABI.  Bar: max |gpu - oracle| / (|oracle| + floor)
<= 1e-4 (fp32), <= 1e-2 (bf16), with the operator's floor of 1e-3 without
the RMSNorm.  The RMSNorm rescales every token's output to the scale of its
weight (about 1, where the plain operator's outputs are about 0.23/sqrt(N)),
so there the floor is relative to that scale, as for the gradients: 1e-2 *
max|oracle| (fp32), 1e-3 * max|oracle| (bf16).  An absolute 1e-3 would ask
fp32 for one rounding unit of the scale near zero crossings (measured: rel-l2
1.9e-7, largest error 4.5e-7 of max|oracle| on 594 tokens)."""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for, host_inputs, round_to_bf16
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _gates(B, N, H, d, dtype, seed):
    """beta = sigmoid of N(0, 1) values in (0, 1); w = 1 + 0.5 N(0, 1)."""
    rng = np.random.default_rng(seed)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, N, H))))).astype(np.float32)
    w = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    if dtype == "bf16":
        beta, w = round_to_bf16(beta), round_to_bf16(w)
    return beta, w


NORM_FLOOR = {"f32": 1e-2, "bf16": 1e-3}


def gated_err(got, ref, dtype: str, rms: bool) -> float:
    """The bar's error: the operator's floor (1e-3) without the RMSNorm, a
    floor relative to the output scale with it."""
    if not rms:
        return max_rel_err(got, ref)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = NORM_FLOOR[dtype] * float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


def _dev(a, dtype):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda().to(
        torch.bfloat16 if dtype == "bf16" else torch.float32)


# name, B, T, Hs, Ws, H, d, dtype, F
CASES = [
    ("bf16_d128", 1, 3, 5, 7, 2, 128, "bf16", 0),
    ("bf16_d128_blocks_batch2", 2, 4, 4, 5, 2, 128, "bf16", 2),
    ("bf16_d64", 1, 4, 6, 5, 3, 64, "bf16", 0),
    ("f32_d32_vector", 1, 3, 4, 5, 2, 32, "f32", 0),
    ("bf16_d112_vector", 1, 2, 5, 5, 2, 112, "bf16", 1),
]


@pytest.mark.parametrize("use_beta,use_w", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gated_matches_oracle(case, use_beta, use_w):
    import torch

    name, B, T, Hs, Ws, H, d, dtype, F = case
    print(f"case {name}: beta={use_beta} rms={use_w} grid={T}x{Hs}x{Ws} H={H} d={d} F={F}",
          flush=True)
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=300 + len(name))
    beta, w = _gates(B, T * Hs * Ws, H, d, dtype, seed=301)
    beta = beta if use_beta else None
    w = w if use_w else None
    dev = to_device(x, dtype)
    out = torch.empty_like(dev["q"])
    gla.gla_gated_forward(dev["q"], dev["k"], dev["v"], dev["g"],
                          None if beta is None else _dev(beta, dtype),
                          None if w is None else _dev(w, dtype), out, (T, Hs, Ws), F)
    torch.cuda.synchronize()
    ref = oracle.gated_forward(x["q"], x["k"], x["v"], x["g"], beta, w, (T, Hs, Ws), F)
    err = gated_err(to_host_f32(out), ref, dtype, w is not None)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("d,dtype,F", [(128, "bf16", 0), (32, "f32", 2)])
def test_no_gates_is_the_plain_operator(d, dtype, F):
    import torch

    B, T, Hs, Ws, H = 1, 4, 4, 5, 2
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=31)
    dev = to_device(x, dtype)
    a = torch.empty_like(dev["q"])
    b = torch.empty_like(dev["q"])
    gla.gla_gated_forward(dev["q"], dev["k"], dev["v"], dev["g"], None, None, a, (T, Hs, Ws), F)
    nbytes = gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, F, gla.GLA_BF16 if dtype == "bf16"
                                     else gla.GLA_F32)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], b, (T, Hs, Ws), ws, F)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(a.view(bits), b.view(bits))


@pytest.mark.slow
def test_full_size_gated_720p():
    import torch

    w_ = WORKLOADS["720p_81f"]
    print(f"workload {w_.name} gated: grid {w_.T}x{w_.Hs}x{w_.Ws} H={w_.H}", flush=True)
    dev = device_inputs_for(w_)
    beta, w = _gates(w_.B, w_.N, w_.H, w_.d, "bf16", seed=302)
    out = torch.empty_like(dev["q"])
    gla.gla_gated_forward(dev["q"], dev["k"], dev["v"], dev["g"], _dev(beta, "bf16"),
                          _dev(w, "bf16"), out, w_.grid)
    torch.cuda.synchronize()
    host = {n: t.float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.gated_forward(host["q"], host["k"], host["v"], host["g"], beta, w, w_.grid)
    err = gated_err(out.float().cpu().numpy(), ref, "bf16", True)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
