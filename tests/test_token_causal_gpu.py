"""Parity of the token-causal form (gla_token_causal_forward) with the fp64
oracle, through the C ABI.

"SANA-Video" notes page, Section 3.4 (the causal output of token i): token i
attends to tokens 0..i.  The bar is the operator's:
max |gpu - oracle| / (|oracle| + 1e-3) <= 1e-4 (fp32), <= 1e-2 (bf16).
The cases span several tiles and ranges (the chunk prefixes) and ragged
tails; the sizes that give more than one range depend on the device's
compute-unit count, so some cases are long enough to be cut on any device.
"""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for, host_inputs
from tests.gpu_util import TOL, have_gpu, max_rel_err, to_device, to_host_f32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _run(dev, grid, theta=1e4, workspace=None):
    import torch

    out = torch.empty_like(dev["q"])
    gla.gla_token_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], out, grid, theta,
                                 workspace=workspace)
    torch.cuda.synchronize()
    return out


def _term_scales(x, grid, theta=1e4, eps=1e-6):
    """Per output element, the size of the terms the token-causal output sums:
    s_i * sum_{j<=i} (|RoPE(phi(q_i))| . |RoPE(phi(k_j))|) |v_j| / den_i, with
    s = sigma(g) (fp64; rotations from the oracle).  Python loops over tokens:
    tiny grids only."""
    q, k, v, g = (np.asarray(x[n], dtype=np.float64) for n in ("q", "k", "v", "g"))
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    pos = [(n // (Hs * Ws), (n // Ws) % Hs, n % Ws) for n in range(N)]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            pq, pk = np.maximum(q[b, :, h], 0.0), np.maximum(k[b, :, h], 0.0)
            rq = np.abs(np.stack([oracle.rope(pq[i], pos[i], theta) for i in range(N)]))
            rk = np.abs(np.stack([oracle.rope(pk[j], pos[j], theta) for j in range(N)]))
            den = np.cumsum(pk, axis=0)
            den = np.einsum("ip,ip->i", pq, den) + eps
            terms = np.tril(rq @ rk.T) @ np.abs(v[b, :, h])
            out[b, :, h] = terms / den[:, None] / (1.0 + np.exp(-g[b, :, h]))
    return out


def token_causal_err(got, ref, x, grid, dtype, theta=1e4):
    """The token-causal bar.  bf16: max |got - ref| / (|ref| + 1e-3).  fp32:
    the floor is also at least 1e-2 of each element's term scale: an early
    token's output can cancel to 1e-4 of the terms it sums (outputs of 5e-5
    from terms of about 1), and fp32 leaves errors of a few rounding units of
    the terms, which against the plain 1e-3 floor reach 1e-4.  Elements that
    do not cancel are still held to 1e-4 relative."""
    got = np.asarray(got, dtype=np.float64)
    if dtype == "bf16":
        return max_rel_err(got, ref)
    floor = np.maximum(1e-3, 1e-2 * _term_scales(x, grid, theta))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


# name, B, T, Hs, Ws, H, d, dtype, theta
CASES = [
    ("f32_d32", 1, 2, 4, 5, 2, 32, "f32", 1e4),
    ("f32_d16_ragged", 1, 3, 7, 5, 1, 16, "f32", 1e4),
    ("bf16_d128", 1, 3, 5, 7, 2, 128, "bf16", 1e4),
    ("bf16_d128_batch2", 2, 4, 4, 5, 2, 128, "bf16", 1e4),
    ("bf16_d64", 1, 4, 6, 5, 3, 64, "bf16", 1e4),
    ("bf16_d112", 1, 2, 5, 5, 2, 112, "bf16", 1e4),
    ("bf16_d128_no_rotation", 1, 2, 6, 6, 2, 128, "bf16", 0.0),
    ("bf16_d128_many_ranges", 1, 8, 12, 16, 2, 128, "bf16", 1e4),
    ("bf16_d64_many_ranges_ragged", 1, 7, 13, 11, 2, 64, "bf16", 1e4),
    ("f32_d128_many_ranges", 1, 6, 10, 16, 1, 128, "f32", 1e4),
    ("bf16_d128_single_token", 1, 1, 1, 1, 2, 128, "bf16", 1e4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_token_causal_matches_oracle(case):
    name, B, T, Hs, Ws, H, d, dtype, theta = case
    print(f"case {name}: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} {dtype}", flush=True)
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=500 + len(name))
    got = _run(to_device(x, dtype), (T, Hs, Ws), theta)
    ref = oracle.token_causal(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws), theta)
    err = token_causal_err(to_host_f32(got), ref, x, (T, Hs, Ws), dtype, theta)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


def test_one_token_frames_match_block_causal_and_last_token_noncausal():
    import torch

    # one token per frame and blocks of one frame: block-causal is token-causal
    B, T, H, d = 1, 40, 2, 128
    x = host_inputs(B, T, 1, 1, H, d, "bf16", seed=51)
    dev = to_device(x, "bf16")
    got = _run(dev, (T, 1, 1))
    blk = torch.empty_like(dev["q"])
    gla.gla_block_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], blk, (T, 1, 1), 1)
    full = torch.empty_like(dev["q"])
    gla.gla_forward(dev["q"], dev["k"], dev["v"], dev["g"], full, (T, 1, 1))
    torch.cuda.synchronize()
    ref = oracle.token_causal(x["q"], x["k"], x["v"], x["g"], (T, 1, 1))
    assert max_rel_err(to_host_f32(got), ref) <= TOL["bf16"]
    assert max_rel_err(to_host_f32(blk), ref) <= TOL["bf16"]
    # the last token sees the whole sequence
    assert max_rel_err(to_host_f32(got)[:, -1:], to_host_f32(full)[:, -1:].astype(np.float64)) \
        <= TOL["bf16"]


@pytest.mark.parametrize("key", [0, 5, 17, 38, 63, 64, 101, 127])
def test_single_key_probe(key):
    # Every key zero but one (token `key` of two 64-token steps): each later
    # query reads it through exactly one score, on the diagonal tile when
    # they share a 16-token tile.  A lost accumulation step of a score tile
    # (a vector read of a matrix-core result issued before the result was
    # complete) once showed on such probes as 4/3 of the right value.
    B, T, Hs, Ws, H, d = 1, 2, 8, 8, 2, 128
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=53 + key)
    k = np.zeros_like(x["k"])
    k[:, key] = np.abs(x["k"][:, key])
    x["k"] = k
    got = _run(to_device(x, "bf16"), (T, Hs, Ws))
    ref = oracle.token_causal(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws))
    assert np.max(np.abs(ref[:, key:])) > 1e-2  # the probe reaches the later queries
    err = max_rel_err(to_host_f32(got), ref)
    print(f"key {key}: max rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_deterministic_and_caller_workspace():
    import torch

    B, T, Hs, Ws, H, d = 1, 6, 10, 12, 2, 128
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=52)
    dev = to_device(x, "bf16")
    a = _run(dev, (T, Hs, Ws))
    b = _run(dev, (T, Hs, Ws))
    nbytes = gla.gla_token_causal_workspace_bytes(B, H, T, Hs, Ws, d, gla.GLA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    c = _run(dev, (T, Hs, Ws), workspace=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    with pytest.raises(gla.GlaError):
        _run(dev, (T, Hs, Ws), workspace=ws[: nbytes // 2])


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["480p_81f", "720p_81f"])
def test_full_size_token_causal(wname):
    w = WORKLOADS[wname]
    print(f"workload {w.name} token-causal: grid {w.T}x{w.Hs}x{w.Ws} H={w.H}", flush=True)
    dev = device_inputs_for(w)
    got = _run(dev, w.grid)
    host = {n: t.float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.token_causal(host["q"], host["k"], host["v"], host["g"], w.grid)
    err = max_rel_err(got.float().cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.slow
def test_long_video_token_causal_sampled_heads():
    # the 60 s video (867,600 tokens x 24 heads, tensors of 2.67e9 elements):
    # the GPU computes every head, the oracle five of them over every token
    import torch

    w = WORKLOADS["720p_60s"]
    print(f"workload {w.name} token-causal: N={w.N} H={w.H}", flush=True)
    dev = device_inputs_for(w)
    got = _run(dev, w.grid)
    heads = [0, 5, 11, 17, 23]
    idx = torch.tensor(heads, device="cuda")
    hs = {n: t.index_select(2, idx).float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.token_causal(hs["q"], hs["k"], hs["v"], hs["g"], w.grid)
    err = max_rel_err(got.index_select(2, idx).float().cpu().numpy(), ref)
    print(f"  {len(heads)} heads x {w.N} tokens: max rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_unaligned_tensors_and_other_stream():
    # tensors one element into their allocations take the vector tile kernel;
    # a call on a non-default stream gives the default stream's bits
    import torch

    from tests.gpu_util import unaligned_copies

    B, T, Hs, Ws, H, d = 1, 3, 7, 9, 2, 128
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=53)
    ts, place = unaligned_copies(x)
    out = place(ts["q"].shape)
    gla.gla_token_causal_forward(ts["q"], ts["k"], ts["v"], ts["g"], out, (T, Hs, Ws))
    torch.cuda.synchronize()
    ref = oracle.token_causal(x["q"], x["k"], x["v"], x["g"], (T, Hs, Ws))
    assert max_rel_err(to_host_f32(out), ref) <= TOL["bf16"]

    dev = to_device(x, "bf16")
    a = _run(dev, (T, Hs, Ws))
    s = torch.cuda.Stream()
    b = torch.empty_like(dev["q"])
    with torch.cuda.stream(s):
        gla.gla_token_causal_forward(dev["q"], dev["k"], dev["v"], dev["g"], b, (T, Hs, Ws),
                                     stream=s)
    s.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
