"""The RoPE table that the library caches per (device, shape, theta, t0).

The first call of a shape computes the table on its stream; a call on a
second stream right after it must wait for that work, a change of theta must
not reuse the table, and a call captured into a HIP graph before the table
exists (or after it) must give the eager result on every replay.  Each case
uses a grid no other test uses, so that it meets the cache empty.
"""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def test_first_call_on_one_stream_then_another():
    import torch

    B, T, Hs, Ws, H, d, theta = 1, 5, 7, 11, 2, 128, 1234.5
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=41)
    dev = to_device(x, "bf16")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1, o2 = torch.empty_like(dev["q"]), torch.empty_like(dev["q"])
    torch.cuda.synchronize()
    print("case: new grid 5x7x11 on stream 1, then at once on stream 2", flush=True)
    gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], o1, (T, Hs, Ws), theta, stream=s1)
    gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], o2, (T, Hs, Ws), theta, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), 0, theta, 1e-6)
    assert max_rel_err(to_host_f32(o2), ref) <= TOL["bf16"]


def test_theta_is_part_of_the_key():
    import torch

    B, T, Hs, Ws, H, d = 1, 4, 9, 5, 2, 64
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=42)
    dev = to_device(x, "bf16")
    outs = {}
    for theta in (10000.0, 3.0, 10000.0):
        print(f"case: grid 4x9x5 theta {theta}", flush=True)
        out = torch.empty_like(dev["q"])
        gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], out, (T, Hs, Ws), theta)
        torch.cuda.synchronize()
        got = to_host_f32(out)
        ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), 0, theta, 1e-6)
        assert max_rel_err(got, ref) <= TOL["bf16"]
        outs.setdefault(theta, []).append(got)
    assert np.array_equal(outs[10000.0][0], outs[10000.0][1])
    assert not np.allclose(outs[10000.0][0], outs[3.0][0])


@pytest.mark.parametrize("warm", [False, True], ids=["captured_first", "cached_first"])
def test_graph_replays_match_eager(warm):
    import torch

    B, T, Hs, Ws, H, d, F, theta = 1, 6, 5, 9, 3, 128, 2, 777.0 + warm
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=43 + warm)
    dev = to_device(x, "bf16")
    ws = torch.empty(gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, F), dtype=torch.uint8,
                     device="cuda")
    eager = torch.empty_like(dev["q"])
    if warm:
        gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], eager, (T, Hs, Ws), ws, F, theta)
        torch.cuda.synchronize()
    out = torch.empty_like(dev["q"])
    print(f"case: capture grid 6x5x9 F=2 ({'after' if warm else 'before'} the table is cached)",
          flush=True)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], out, (T, Hs, Ws), ws, F,
                               theta, stream=side)
    torch.cuda.synchronize()
    if not warm:
        gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], eager, (T, Hs, Ws), ws, F, theta)
        torch.cuda.synchronize()
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), F, theta, 1e-6)
    assert max_rel_err(to_host_f32(eager), ref) <= TOL["bf16"]
    for rep in range(3):
        out.zero_()
        scratch = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        print(f"  replay {rep} (eager sum {float(scratch):.2f})", flush=True)
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
