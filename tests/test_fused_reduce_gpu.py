"""The reduce folded into the state kernel (one temporal block, matrix-core
path): the last workgroup of each (batch, head) sums its chunk partials,
picked by a counter that it puts back to zero.

Eager calls use the fold; a call captured into a HIP graph runs the separate
reduce kernel instead.  Both must give the same bits, every repeated call on
one stream must give the same bits (the counters were reset), and the result
must match the oracle.
"""
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

# B, T, Hs, Ws, H, d
SHAPES = [(1, 6, 9, 13, 3, 128), (2, 5, 8, 8, 5, 64), (1, 40, 12, 16, 2, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=["d128", "d64_batch2", "d128_long"])
def test_fused_reduce_matches_separate_reduce(shape):
    import torch

    B, T, Hs, Ws, H, d = shape
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=51 + d)
    dev = to_device(x, "bf16")
    grid = (T, Hs, Ws)
    ws = torch.empty(gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, 0), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.Stream()
    eager = [torch.empty_like(dev["q"]) for _ in range(3)]
    print(f"case: B={B} grid={T}x{Hs}x{Ws} H={H} d={d}, three eager calls on one stream",
          flush=True)
    for o in eager:
        gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], o, grid, ws, stream=s)
    torch.cuda.synchronize()
    for o in eager[1:]:
        assert torch.equal(o.view(torch.int16), eager[0].view(torch.int16))
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], grid, 0, 1e4, 1e-6)
    assert max_rel_err(to_host_f32(eager[0]), ref) <= TOL["bf16"]

    print("  captured call (separate reduce kernel)", flush=True)
    out = torch.empty_like(dev["q"])
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], out, grid, ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16)), f"replay {rep}"
