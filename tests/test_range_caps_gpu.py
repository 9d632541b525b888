"""A shape where the 32-bit buffer-offset caps of the matrix-core kernels bind.

With 128 heads of d = 128 a token row of all heads is 32 KiB, so a chunk or
range of a head may span at most about 65,000 tokens before its byte offsets
leave 31 bits.  At 42 x 45 x 80 (151,200 tokens, 4.95 GB per tensor) the
state stage would take two chunks of 75,648 tokens per head; the cap cuts
them to three of 64,960, and the token-causal plan is cut the same way.  The
GPU computes every head; the oracle checks two heads over every token.
"""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import device_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

B, T, Hs, Ws, H, d = 1, 42, 45, 80, 128, 128
HEADS = [0, 127]


@pytest.fixture(scope="module")
def inputs():
    import torch

    x = device_inputs(B, T, Hs, Ws, H, d, "bf16", seed=71)
    idx = torch.tensor(HEADS, device="cuda")
    host = {n: t.index_select(2, idx).float().cpu().numpy() for n, t in x.items()}
    yield x, host
    del x
    torch.cuda.empty_cache()


def test_forward_where_the_range_caps_bind(inputs):
    import torch

    x, host = inputs
    print(f"case: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} forward, heads {HEADS}", flush=True)
    out = torch.empty_like(x["q"])
    gla.gla_forward(x["q"], x["k"], x["v"], x["g"], out, (T, Hs, Ws))
    torch.cuda.synchronize()
    got = out.index_select(2, torch.tensor(HEADS, device="cuda")).float().cpu().numpy()
    del out
    S, z = oracle.state(host["k"], host["v"], (T, Hs, Ws), 0, 1e4)
    ref = oracle.apply(host["q"], host["g"], S, z, (T, Hs, Ws), 0, 1e4, 1e-6)
    err, l2 = max_rel_err(got, ref), rel_l2(got, ref)
    print(f"  max rel err {err:.3e}  rel l2 {l2:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert l2 <= 3e-3


def test_token_causal_where_the_range_caps_bind(inputs):
    import torch

    x, host = inputs
    print(f"case: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} token-causal, heads {HEADS}", flush=True)
    out = torch.empty_like(x["q"])
    gla.gla_token_causal_forward(x["q"], x["k"], x["v"], x["g"], out, (T, Hs, Ws))
    torch.cuda.synchronize()
    got = out.index_select(2, torch.tensor(HEADS, device="cuda")).float().cpu().numpy()
    del out
    ref = oracle.token_causal(host["q"], host["k"], host["v"], host["g"], (T, Hs, Ws))
    err = max_rel_err(got, ref)
    print(f"  max rel err {err:.3e}  rel l2 {rel_l2(got, ref):.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert np.isfinite(got).all()
