"""The training pair through the C ABI: gla_forward_train (the forward, which
also keeps the reduced state of every (batch, head, temporal block)) and
gla_backward_saved (the gradients from that state, without re-running the
state stage).

- The forward's output is gla_forward_ws's, bit for bit.
- The saved records hold the oracle's block sums (S, z over blocks 0..b),
  to the bar of the state export (S: 4e-3 of max|S| for bf16, 1e-5 for
  fp32; z: 1e-5 relative).
- The gradients are gla_backward's bit for bit (the same kernels on the same
  state) and the oracle's to the gradient bar."""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32
from tests.test_backward_gpu import _dout, _run, grad_err

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

# name, B, T, Hs, Ws, H, d, dtype, F
CASES = [
    ("bf16_d128", 1, 3, 5, 7, 2, 128, "bf16", 0),
    ("bf16_d128_blocks_batch2", 2, 4, 4, 5, 2, 128, "bf16", 2),
    ("bf16_d64_many_ranges_blocks", 1, 6, 13, 11, 2, 64, "bf16", 2),
    ("bf16_d128_many_ranges", 1, 7, 13, 11, 2, 128, "bf16", 0),
    ("f32_d32", 1, 2, 4, 5, 2, 32, "f32", 0),
    ("f32_d64_blocks", 1, 4, 3, 5, 2, 64, "f32", 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_training_pair(case):
    import torch

    name, B, T, Hs, Ws, H, d, dtype, F = case
    grid = (T, Hs, Ws)
    print(f"case {name}: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} {dtype} F={F}", flush=True)
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=900 + len(name))
    dout = _dout(x["q"].shape, dtype, seed=901)
    dev = to_device(x, dtype)
    ddev = to_device({"o": dout}, dtype)["o"]
    nb = oracle.num_blocks(T, F)
    nbytes = gla.gla_saved_state_bytes(B, H, T, Hs, Ws, d, F)
    assert nbytes == B * H * nb * (d * d + d) * 4
    # NaN-filled, so that a record the forward does not write fails below
    saved = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")

    out = torch.empty_like(dev["q"])
    gla.gla_forward_train(dev["q"], dev["k"], dev["v"], dev["g"], out, saved, grid, F)
    ref_out = torch.empty_like(dev["q"])
    ws = torch.empty(gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, F,
                                             gla.GLA_BF16 if dtype == "bf16" else gla.GLA_F32),
                     dtype=torch.uint8, device="cuda")
    gla.gla_forward_ws(dev["q"], dev["k"], dev["v"], dev["g"], ref_out, grid, ws, F)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(out.view(bits), ref_out.view(bits))

    rec = saved.view(B, H, nb, d * d + d).cpu().numpy().astype(np.float64)
    S, z = rec[..., :d * d].reshape(B, H, nb, d, d), rec[..., d * d:]
    Sr, zr = oracle.state(x["k"], x["v"], grid, F, 1e4)  # block b: sums over blocks 0..b
    s_tol = 4e-3 if dtype == "bf16" else 1e-5
    serr = np.max(np.abs(S - Sr)) / np.max(np.abs(Sr))
    zerr = np.max(np.abs(z - zr) / (np.abs(zr) + 1e-6))
    print(f"  saved S err {serr:.3e}  z err {zerr:.3e}", flush=True)
    assert serr <= s_tol and zerr <= 1e-5

    got = [torch.empty_like(dev["q"]) for _ in range(4)]
    gla.gla_backward_saved(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *got, saved, grid, F)
    torch.cuda.synchronize()
    full = _run(dev, ddev, grid, F)
    for gname, a, b in zip(("dq", "dk", "dv", "dg"), got, full):
        assert torch.equal(a.view(bits), b.view(bits)), gname
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, grid, F)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        err = grad_err(to_host_f32(a), r, dtype)
        print(f"  {gname}: err {err:.3e}", flush=True)
        assert err <= TOL[dtype], gname


def test_training_pair_with_workspaces_and_bad_saved_state():
    # caller workspaces give the same bits; a saved buffer inside a tensor
    # or misaligned is refused before any launch
    import torch

    B, T, Hs, Ws, H, d, F = 1, 4, 5, 6, 2, 128, 2
    grid = (T, Hs, Ws)
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=77)
    dev = to_device(x, "bf16")
    ddev = to_device({"o": _dout(x["q"].shape, "bf16", 78)}, "bf16")["o"]
    nbytes = gla.gla_saved_state_bytes(B, H, T, Hs, Ws, d, F)
    saved = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty_like(dev["q"])
    gla.gla_forward_train(dev["q"], dev["k"], dev["v"], dev["g"], out, saved, grid, F)
    a = [torch.empty_like(dev["q"]) for _ in range(4)]
    gla.gla_backward_saved(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *a, saved, grid, F)

    saved2 = torch.empty_like(saved)
    fws = torch.empty(gla.gla_workspace_bytes(B, H, T, Hs, Ws, d, F), dtype=torch.uint8,
                      device="cuda")
    bws = torch.empty(gla.gla_backward_workspace_bytes(B, H, T, Hs, Ws, d, F), dtype=torch.uint8,
                      device="cuda")
    out2 = torch.empty_like(dev["q"])
    gla.gla_forward_train(dev["q"], dev["k"], dev["v"], dev["g"], out2, saved2, grid, F,
                          workspace=fws)
    b = [torch.empty_like(dev["q"]) for _ in range(4)]
    gla.gla_backward_saved(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *b, saved2, grid, F,
                           workspace=bws)
    torch.cuda.synchronize()
    assert torch.equal(saved.view(torch.int32), saved2.view(torch.int32))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    for u, v_ in zip(a, b):
        assert torch.equal(u.view(torch.int16), v_.view(torch.int16))

    inside_q = dev["q"].view(-1)[: nbytes // 2].view(torch.float32)
    with pytest.raises(gla.GlaError):
        gla.gla_forward_train(dev["q"], dev["k"], dev["v"], dev["g"], out, inside_q, grid, F)
    with pytest.raises(gla.GlaError):
        gla.gla_backward_saved(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *b, inside_q, grid,
                               F)
    big = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    with pytest.raises(gla.GlaError):
        gla.gla_backward_saved(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *b, big[4:], grid,
                               F)


def test_training_pair_unaligned_tensors():
    # misaligned tensors take the vector kernels on both sides; the saved
    # records are the same state, so the gradients still match gla_backward
    # bit for bit and the oracle to the bar
    import torch

    from tests.gpu_util import unaligned_copies

    B, T, Hs, Ws, H, d, F = 1, 4, 5, 6, 2, 128, 2
    grid = (T, Hs, Ws)
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=79)
    dout = _dout(x["q"].shape, "bf16", 80)
    ts, place = unaligned_copies(dict(x, o=dout))
    saved = torch.empty(gla.gla_saved_state_bytes(B, H, T, Hs, Ws, d, F) // 4,
                        dtype=torch.float32, device="cuda")
    out = place(ts["q"].shape)
    gla.gla_forward_train(ts["q"], ts["k"], ts["v"], ts["g"], out, saved, grid, F)
    got = [place(ts["q"].shape) for _ in range(4)]
    gla.gla_backward_saved(ts["q"], ts["k"], ts["v"], ts["g"], ts["o"], *got, saved, grid, F)
    full = [place(ts["q"].shape) for _ in range(4)]
    gla.gla_backward(ts["q"], ts["k"], ts["v"], ts["g"], ts["o"], *full, grid, F)
    torch.cuda.synchronize()
    for a, b in zip(got, full):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert max_rel_err(to_host_f32(out), oracle.forward(x["q"], x["k"], x["v"], x["g"], grid, F)) \
        <= TOL["bf16"]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, grid, F)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert grad_err(to_host_f32(a), r) <= TOL["bf16"], gname
