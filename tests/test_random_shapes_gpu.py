"""48 seeded random shapes through every entry point against the fp64 oracle:
batch 1-2, grids up to 12 x 24 x 30 (one to several token ranges, ragged
tails), 1-3 heads, bf16 at d = 64, 128 (matrix-core kernels) and fp32 at
d = 16..128 (vector kernels), non-causal and block-causal.  Each case runs the
forward (block-causal cases also streamed through the block step), the
token-causal form, the gradients and the gated mixer (beta and RMSNorm) with
the bars of their own tests; dq and dk of blocks under four
tokens are left to test_one_token_blocks_backward (their terms cancel).
The floor of dq's bar is relative to the larger of max|dq| and its two
quotient-rule terms (S dnum and dden z), which cancel because the output is
invariant to scaling q: a d = 16 case whose terms are 37 times max|dq|
had errors of 7e-8 of the terms (one fp32 rounding), which the tensor-scale
floor alone scored 2.7e-4 against the bar of 1e-4."""
import random

import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err
from tests.test_backward_gpu import dq_term_scale, grad_err
from tests.test_gated_gpu import gated_err
from tests.test_token_causal_gpu import token_causal_err

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _cases(seed: int, n: int, first: int = 0):
    rng = random.Random(seed)
    out = []
    for i in range(first, first + n):
        big = i % 3 == 2
        B = rng.choice([1, 1, 2])
        T = rng.randint(1, 12 if big else 6)
        Hs = rng.randint(1, 24 if big else 9)
        Ws = rng.randint(1, 30 if big else 11)
        H = rng.randint(1, 3)
        dtype = rng.choice(["bf16"] * 4 + ["f32"])
        d = rng.choice([64, 128]) if dtype == "bf16" else rng.choice([16, 32, 64, 128])
        F = rng.choice([0] + [f for f in range(1, T + 1) if T % f == 0])
        out.append((i, B, T, Hs, Ws, H, d, dtype, F))
    return out


@pytest.mark.parametrize("case", _cases(2024, 24) + _cases(2025, 24, first=24),
                         ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    import torch

    i, B, T, Hs, Ws, H, d, dtype, F = case
    print(f"case {i}: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} {dtype} F={F}", flush=True)
    tol = TOL[dtype]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=7000 + i)
    dev = {n: torch.from_numpy(a).cuda().to(tdt) for n, a in x.items()}
    grid = (T, Hs, Ws)

    out = torch.empty_like(dev["q"])
    if F:
        gla.gla_block_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], out, grid, F)
    else:
        gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], out, grid)
    out_tc = torch.empty_like(dev["q"])
    gla.gla_token_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], out_tc, grid)
    torch.cuda.synchronize()
    ref_fwd = oracle.forward(x["q"], x["k"], x["v"], x["g"], grid, F)
    assert max_rel_err(out.float().cpu().numpy(), ref_fwd) <= tol
    if F:
        # the same layer streamed block by block through gla_block_step (the
        # inclusive step equals the block-causal output of its block)
        hw = Hs * Ws
        S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
        z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
        out_bs = torch.empty_like(dev["q"])
        for t0 in range(0, T, F):
            sl = slice(t0 * hw, (t0 + F) * hw)
            blk = {n: t[:, sl].contiguous() for n, t in dev.items()}
            o = torch.empty_like(blk["q"])
            gla.gla_block_step(blk["q"], blk["k"], blk["v"], blk["g"], o, S, z, (F, Hs, Ws), t0,
                               True)
            out_bs[:, sl] = o
        torch.cuda.synchronize()
        assert max_rel_err(out_bs.float().cpu().numpy(), ref_fwd) <= tol
    assert token_causal_err(out_tc.float().cpu().numpy(),
                            oracle.token_causal(x["q"], x["k"], x["v"], x["g"], grid),
                            x, grid, dtype) <= tol

    dout = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=8000 + i)["q"]
    grads = [torch.empty_like(dev["q"]) for _ in range(4)]
    gla.gla_backward(dev["q"], dev["k"], dev["v"], dev["g"],
                     torch.from_numpy(dout).cuda().to(tdt), *grads, grid, F)
    torch.cuda.synchronize()
    refs = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, grid, F)
    small_blocks = (F or T) * Hs * Ws < 4
    # dq's floor also covers its two quotient-rule terms, which cancel
    sq = dq_term_scale(x, dout, ref_fwd, grid, F)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), grads, refs):
        if small_blocks and name in ("dq", "dk"):
            continue
        assert grad_err(a.float().cpu().numpy(), r, dtype, sq if name == "dq" else 0.0) <= tol, name

    rng = np.random.default_rng(9000 + i)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T * Hs * Ws, H))))).astype(np.float32)
    w = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    beta_d, w_d = torch.from_numpy(beta).cuda().to(tdt), torch.from_numpy(w).cuda().to(tdt)
    out_g = torch.empty_like(dev["q"])
    gla.gla_gated_forward(dev["q"], dev["k"], dev["v"], dev["g"], beta_d, w_d, out_g, grid, F)
    torch.cuda.synchronize()
    ref_g = oracle.gated_forward(x["q"], x["k"], x["v"], x["g"], beta_d.float().cpu().numpy(),
                                 w_d.float().cpu().numpy(), grid, F)
    assert gated_err(out_g.float().cpu().numpy(), ref_g, dtype, True) <= tol
