"""Parity of the streaming block-causal step (gla_block_step) with the fp64
oracle, through the C ABI.

"SANA-Video" notes page, Section 3.4 and its Algorithm 1: a block of latent
frames is produced against a cache of the sums of the earlier blocks; the
cache then takes the block's own sums.  The bar is the operator's:
max |gpu - oracle| / (|oracle| + 1e-3) <= 1e-4 (fp32), <= 1e-2 (bf16).
"""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for, host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _zero_cache(B, H, d):
    import torch

    return (torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda"),
            torch.zeros((B, H, d), dtype=torch.float32, device="cuda"))


def _block(dev, b0, Tb, Hs, Ws):
    per = Tb * Hs * Ws
    return {n: t[:, b0 * Hs * Ws: b0 * Hs * Ws + per].contiguous() for n, t in dev.items()}


def _stream_gpu(dev, grid, Tb, theta=1e4, workspace=None):
    import torch

    B, N, H, d = dev["k"].shape
    T, Hs, Ws = grid
    S, z = _zero_cache(B, H, d)
    outs = []
    for b0 in range(0, T, Tb):
        blk = _block(dev, b0, Tb, Hs, Ws)
        out = torch.empty_like(blk["q"])
        gla.gla_block_step(blk["q"], blk["k"], blk["v"], blk["g"], out, S, z, (Tb, Hs, Ws), b0,
                           True, theta, 1e-6, workspace=workspace)
        outs.append(out)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), S, z


# name, B, T, Hs, Ws, H, d, dtype, Tb
CASES = [
    ("bf16_d128_Tb1", 1, 4, 5, 7, 2, 128, "bf16", 1),
    ("bf16_d128_Tb2_batch2", 2, 6, 4, 9, 2, 128, "bf16", 2),
    ("bf16_d64_Tb3", 1, 6, 6, 5, 3, 64, "bf16", 3),
    ("f32_d32_Tb2", 1, 4, 3, 5, 2, 32, "f32", 2),
    ("bf16_d112_vector_Tb1", 1, 3, 4, 4, 2, 112, "bf16", 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_streaming_matches_oracle(case):
    name, B, T, Hs, Ws, H, d, dtype, Tb = case
    print(f"case {name}: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} {dtype} Tb={Tb}", flush=True)
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=200 + len(name))
    got, S, z = _stream_gpu(to_device(x, dtype), (T, Hs, Ws), Tb)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), Tb)
    err = max_rel_err(to_host_f32(got), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    # the final cache holds the state of the whole grid
    Sr, zr = oracle.state(x["k"], x["v"], (T, Hs, Ws))
    s_tol = 4e-3 if dtype == "bf16" else 1e-5
    serr = np.max(np.abs(S.cpu().numpy() - Sr[:, :, 0])) / np.max(np.abs(Sr))
    zerr = np.max(np.abs(z.cpu().numpy() - zr[:, :, 0]) / (np.abs(zr[:, :, 0]) + 1e-6))
    print(f"  cache: S err {serr:.3e}  z err {zerr:.3e}", flush=True)
    assert serr <= s_tol and zerr <= 1e-5


def test_streaming_matches_one_call_block_causal():
    import torch

    B, T, Hs, Ws, H, d, F = 1, 6, 5, 7, 2, 128, 2
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=21)
    dev = to_device(x, "bf16")
    got, _, _ = _stream_gpu(dev, (T, Hs, Ws), F)
    one = torch.empty_like(dev["q"])
    gla.gla_block_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], one, (T, Hs, Ws), F)
    torch.cuda.synchronize()
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), F)
    assert max_rel_err(to_host_f32(got), ref) <= TOL["bf16"]
    assert max_rel_err(to_host_f32(one), ref) <= TOL["bf16"]
    assert max_rel_err(to_host_f32(got), to_host_f32(one).astype(np.float64)) <= TOL["bf16"]


def _random_cache(B, H, d, n_tokens, seed):
    # a cache shaped like the sums of n_tokens earlier tokens: S entries grow
    # like sqrt(n), z entries like n (phi(k) >= 0)
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((B, H, d, d)) * np.sqrt(n_tokens) * 0.3
    z = np.abs(rng.standard_normal((B, H, d))) * 0.4 * n_tokens
    return S.astype(np.float32), z.astype(np.float32)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (32, "f32")])
def test_large_offset_with_carried_cache(d, dtype):
    import torch

    B, Tb, Hs, Ws, H, t0 = 1, 2, 5, 6, 2, 240
    x = host_inputs(B, Tb, Hs, Ws, H, d, dtype, seed=22)
    S0, z0 = _random_cache(B, H, d, 5000, seed=23)
    dev = to_device(x, dtype)
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    out = torch.empty_like(dev["q"])
    gla.gla_block_step(dev["q"], dev["k"], dev["v"], dev["g"], out, S, z, (Tb, Hs, Ws), t0, True)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.block_step(x["q"], x["k"], x["v"], x["g"], S0, z0, (Tb, Hs, Ws), t0)
    err = max_rel_err(to_host_f32(out), ref)
    print(f"d={d} {dtype}: max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    serr = np.max(np.abs(S.cpu().numpy() - S_ref)) / np.max(np.abs(S_ref))
    assert serr <= (4e-3 if dtype == "bf16" else 1e-5)
    assert np.max(np.abs(z.cpu().numpy() - z_ref) / (np.abs(z_ref) + 1e-6)) <= 1e-5


def test_update_flag_and_cache_only_update():
    import torch

    B, Tb, Hs, Ws, H, d, t0 = 1, 2, 4, 5, 2, 128, 6
    x = host_inputs(B, Tb, Hs, Ws, H, d, "bf16", seed=24)
    S0, z0 = _random_cache(B, H, d, 800, seed=25)
    dev = to_device(x, "bf16")
    grid = (Tb, Hs, Ws)

    def fresh():
        return torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda()

    S1, z1 = fresh()
    out1 = torch.empty_like(dev["q"])
    gla.gla_block_step(dev["q"], dev["k"], dev["v"], dev["g"], out1, S1, z1, grid, t0, True)
    # update = 0: the same output, the cache untouched
    S2, z2 = fresh()
    out2 = torch.empty_like(dev["q"])
    gla.gla_block_step(dev["q"], dev["k"], dev["v"], dev["g"], out2, S2, z2, grid, t0, False)
    # out = None: the same cache update, no output
    S3, z3 = fresh()
    gla.gla_block_step(None, dev["k"], dev["v"], None, None, S3, z3, grid, t0, True)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert np.array_equal(S2.cpu().numpy(), S0) and np.array_equal(z2.cpu().numpy(), z0)
    assert torch.equal(S3, S1) and torch.equal(z3, z1)
    assert not torch.equal(S1, S2)
    with pytest.raises(gla.GlaError):
        gla.gla_block_step(None, dev["k"], dev["v"], None, None, S3, z3, grid, t0, False)


def test_caller_workspace_matches_allocating_call():
    import torch

    B, T, Hs, Ws, H, d, Tb = 1, 4, 5, 6, 2, 128, 2
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=26)
    dev = to_device(x, "bf16")
    a, Sa, za = _stream_gpu(dev, (T, Hs, Ws), Tb)
    nbytes = gla.gla_workspace_bytes(B, H, Tb, Hs, Ws, d, 0, gla.GLA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b, Sb, zb = _stream_gpu(dev, (T, Hs, Ws), Tb, workspace=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(Sa, Sb) and torch.equal(za, zb)


@pytest.mark.slow
def test_full_size_streaming_block_causal():
    # the 720p block-causal layer (7 blocks of 3 latent frames, 24 heads)
    # produced block by block through the cache
    import torch

    w = WORKLOADS["720p_block_causal"]
    print(f"workload {w.name} streamed: grid {w.T}x{w.Hs}x{w.Ws} H={w.H} Tb={w.frames_per_block}",
          flush=True)
    dev = device_inputs_for(w)
    got, _, _ = _stream_gpu(dev, w.grid, w.frames_per_block)
    one = torch.empty_like(dev["q"])
    gla.gla_block_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], one, w.grid,
                                 w.frames_per_block)
    torch.cuda.synchronize()
    host = {n: t.float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.forward(host["q"], host["k"], host["v"], host["g"], w.grid, w.frames_per_block)
    err = max_rel_err(got.float().cpu().numpy(), ref)
    print(f"  streamed max rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert max_rel_err(got.float().cpu().numpy(), one.float().cpu().numpy().astype(np.float64)) \
        <= TOL["bf16"]
