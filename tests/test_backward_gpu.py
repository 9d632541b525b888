"""Parity of the gradients (gla_backward) with the fp64 oracle's, through the
C ABI.  Gradients of the loss sum(dout * out); dout ~ N(0, 1), seeded.

Bar: max |gpu - oracle| / (|oracle| + 1e-3 * max |oracle|) <= 1e-4 for fp32
tensors and <= 1e-2 for bf16 tensors, per gradient tensor.  The floor is
relative to the tensor's own scale because the four gradients differ in
magnitude by orders (the forward's absolute floor of 1e-3 would hide all
of dg at large N); bf16 gradients are rounded once to bf16 (2^-9)."""
import numpy as np
import pytest

import oracle
from relu_linear_attention_amd import gla
from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for, host_inputs
from tests.gpu_util import TOL, have_gpu, to_device, to_host_f32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


# Floor of the gradient bar, relative to each tensor's own scale.  The
# gradients sum products over every token of a (batch, head) and over d
# features, and dq, dk combine two terms of the quotient rule that cancel in
# part, so fp32 arithmetic leaves absolute errors of about sqrt(N) rounding
# units of the tensor's largest terms (measured: up to 5.5e-7 of max|dq| on
# 594 tokens).  With the fp32 bar of 1e-4 the floor 1e-2 * max admits those
# (1e-6 * max); large elements are still held to 1e-4 relative.  The bf16
# paths carry about 16 bits through the matrix cores: floor 1e-3 * max.
GRAD_FLOOR = {"f32": 1e-2, "bf16": 1e-3}


def grad_err(got, ref, dtype: str = "bf16", scale: float = 0.0) -> float:
    """The gradient bar's error; the floor is relative to the larger of the
    tensor's own scale and `scale` (the magnitude of terms that cancel in it,
    when known)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = GRAD_FLOOR[dtype] * max(float(np.max(np.abs(ref))), scale)
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


def dq_term_scale(x, dout, out, grid, F, theta=1e4, eps=1e-6) -> float:
    """Largest magnitude of the two quotient-rule terms of dq, S dnum_i and
    dden_i z (before RoPE^T, which keeps pair norms), from the oracle's block
    states and its forward output `out` (y = out / sigmoid(g)); vectorised.
    The output is invariant to scaling q up to eps, so dq is the difference
    of these terms and can be far smaller than either, while the
    arithmetic's errors scale with the terms."""
    q, g, do, o = (np.asarray(a, dtype=np.float64) for a in (x["q"], x["g"], dout, out))
    B, N, H, d = q.shape
    S, z = oracle.state(x["k"], x["v"], grid, F, theta)  # block b: sums over blocks 0..b
    nb = S.shape[2]
    L = N // nb
    s = 1.0 / (1.0 + np.exp(-g))
    y = o / s
    pq = np.maximum(q, 0.0)
    scale = 0.0
    for b in range(B):
        for h in range(H):
            for blk in range(nb):
                sl = slice(blk * L, (blk + 1) * L)
                den = pq[b, sl, h] @ z[b, h, blk] + eps
                sd = s[b, sl, h] * do[b, sl, h]
                dnum = sd / den[:, None]
                dden = -np.sum(sd * y[b, sl, h], axis=1) / den
                scale = max(scale, float(np.max(np.abs(dnum @ S[b, h, blk].T))),
                            float(np.max(np.abs(dden))) * float(np.max(np.abs(z[b, h, blk]))))
    return scale


def _run(dev, dout, grid, F, workspace=None):
    import torch

    outs = [torch.empty_like(dev["q"]) for _ in range(4)]
    gla.gla_backward(dev["q"], dev["k"], dev["v"], dev["g"], dout, *outs, grid, F,
                     workspace=workspace)
    torch.cuda.synchronize()
    return outs


def _dout(shape, dtype, seed):
    from relu_linear_attention_amd.inputs import round_to_bf16

    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


# name, B, T, Hs, Ws, H, d, dtype, F
CASES = [
    ("f32_d32", 1, 2, 4, 5, 2, 32, "f32", 0),
    ("f32_d64_blocks", 1, 4, 3, 5, 2, 64, "f32", 1),
    ("bf16_d128", 1, 3, 5, 7, 2, 128, "bf16", 0),
    ("bf16_d128_blocks_batch2", 2, 4, 4, 5, 2, 128, "bf16", 2),
    ("bf16_d64", 1, 4, 6, 5, 3, 64, "bf16", 0),
    ("bf16_d112", 1, 2, 5, 5, 2, 112, "bf16", 1),
    ("f32_d16_ragged", 1, 3, 7, 5, 1, 16, "f32", 0),
    # long enough for several token ranges per (batch, head, block), ragged tails
    ("bf16_d128_many_ranges", 1, 7, 13, 11, 2, 128, "bf16", 0),
    ("bf16_d64_many_ranges_blocks", 1, 6, 13, 11, 2, 64, "bf16", 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, T, Hs, Ws, H, d, dtype, F = case
    print(f"case {name}: B={B} grid={T}x{Hs}x{Ws} H={H} d={d} {dtype} F={F}", flush=True)
    x = host_inputs(B, T, Hs, Ws, H, d, dtype, seed=400 + len(name))
    dout = _dout(x["q"].shape, dtype, seed=401)
    dev = to_device(x, dtype)
    ddev = to_device({"o": dout}, dtype)["o"]
    got = _run(dev, ddev, (T, Hs, Ws), F)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, (T, Hs, Ws), F)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        err = grad_err(to_host_f32(a), r, dtype)
        print(f"  {gname}: err {err:.3e}", flush=True)
        assert err <= TOL[dtype], gname


def test_backward_is_deterministic_and_workspace_matches():
    import torch

    B, T, Hs, Ws, H, d, F = 1, 4, 5, 6, 2, 128, 2
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=41)
    dev = to_device(x, "bf16")
    ddev = to_device({"o": _dout(x["q"].shape, "bf16", 42)}, "bf16")["o"]
    a = _run(dev, ddev, (T, Hs, Ws), F)
    b = _run(dev, ddev, (T, Hs, Ws), F)
    nbytes = gla.gla_backward_workspace_bytes(B, H, T, Hs, Ws, d, F, gla.GLA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    c = _run(dev, ddev, (T, Hs, Ws), F, workspace=ws)
    for u, v_, w in zip(a, b, c):
        assert torch.equal(u.view(torch.int16), v_.view(torch.int16))
        assert torch.equal(u.view(torch.int16), w.view(torch.int16))


@pytest.mark.slow
def test_full_size_backward_480p():
    import torch

    w = WORKLOADS["480p_81f"]
    print(f"workload {w.name} backward: grid {w.T}x{w.Hs}x{w.Ws} H={w.H}", flush=True)
    dev = device_inputs_for(w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 7)
    dout = torch.randn(dev["q"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    got = _run(dev, dout, w.grid, 0)
    host = {n: t.float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.backward(host["q"], host["k"], host["v"], host["g"], dout.float().cpu().numpy(),
                          w.grid, 0)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        err = grad_err(a.float().cpu().numpy(), r)
        print(f"  {gname}: err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], gname


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["720p_81f", "720p_block_causal"])
def test_full_size_backward_sampled_heads(wname):
    # the full 720p layers (non-causal and 7 blocks of 3 frames): the GPU
    # computes every head, the oracle three of them over every token (heads
    # are independent)
    import torch

    w = WORKLOADS[wname]
    print(f"workload {w.name} backward: grid {w.T}x{w.Hs}x{w.Ws} H={w.H} F={w.frames_per_block}",
          flush=True)
    dev = device_inputs_for(w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 9)
    dout = torch.randn(dev["q"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    got = _run(dev, dout, w.grid, w.frames_per_block)
    heads = [0, 13, w.H - 1]
    idx = torch.tensor(heads, device="cuda")
    hs = {n: t.index_select(2, idx).float().cpu().numpy() for n, t in dev.items()}
    ref = oracle.backward(hs["q"], hs["k"], hs["v"], hs["g"],
                          dout.index_select(2, idx).float().cpu().numpy(), w.grid,
                          w.frames_per_block)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        err = grad_err(a.index_select(2, idx).float().cpu().numpy(), r)
        print(f"  {gname}: err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], gname


def test_unaligned_tensors_other_stream_and_small_workspace():
    # misaligned tensors take the vector gradient kernels; a non-default
    # stream gives the default stream's bits; a short workspace is refused
    import torch

    from tests.gpu_util import unaligned_copies

    B, T, Hs, Ws, H, d, F = 1, 4, 5, 6, 2, 128, 2
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=55)
    dout = _dout(x["q"].shape, "bf16", 56)
    ts, place = unaligned_copies(dict(x, o=dout))
    outs = [place(ts["q"].shape) for _ in range(4)]
    gla.gla_backward(ts["q"], ts["k"], ts["v"], ts["g"], ts["o"], *outs, (T, Hs, Ws), F)
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, (T, Hs, Ws), F)
    for gname, a, r in zip(("dq", "dk", "dv", "dg"), outs, ref):
        assert grad_err(to_host_f32(a), r) <= TOL["bf16"], gname

    dev = to_device(x, "bf16")
    ddev = to_device({"o": dout}, "bf16")["o"]
    a = _run(dev, ddev, (T, Hs, Ws), F)
    s = torch.cuda.Stream()
    b = [torch.empty_like(dev["q"]) for _ in range(4)]
    with torch.cuda.stream(s):
        gla.gla_backward(dev["q"], dev["k"], dev["v"], dev["g"], ddev, *b, (T, Hs, Ws), F,
                         stream=s)
    s.synchronize()
    for u, v_ in zip(a, b):
        assert torch.equal(u.view(torch.int16), v_.view(torch.int16))
    nbytes = gla.gla_backward_workspace_bytes(B, H, T, Hs, Ws, d, F, gla.GLA_BF16)
    ws = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(gla.GlaError):
        _run(dev, ddev, (T, Hs, Ws), F, workspace=ws)


def _quotient_term_scales(q, k, v, g, dout, grid, F, theta=1e4, eps=1e-6):
    """Largest magnitudes of the two quotient-rule terms of dq (RoPE^-1(S dnum)
    and dden z) and of dk (RoPE^-1(G v) and Gz), from the oracle's block
    states (fp64; the rotations keep pair norms, so the unrotated products
    give the scale).  Python loops: tiny grids only."""
    B, N, H, d = q.shape
    T, Hs, Ws = grid
    nb = oracle.num_blocks(T, F)
    L = N // nb
    S, z = oracle.state(k, v, grid, F, theta)  # block b: the sums over blocks 0..b
    pos = [(n // (Hs * Ws), (n // Ws) % Hs, n % Ws) for n in range(N)]
    sq = sk = 0.0
    for b in range(B):
        for h in range(H):
            dS, dz = np.zeros((nb, d, d)), np.zeros((nb, d))
            for i in range(N):
                blk = i // L
                pq = np.maximum(q[b, i, h], 0.0)
                rq = oracle.rope(pq, pos[i], theta)
                den = pq @ z[b, h, blk] + eps
                y = (rq @ S[b, h, blk]) / den
                s = 1.0 / (1.0 + np.exp(-g[b, i, h]))
                dnum = dout[b, i, h] * s / den
                dden = -np.sum(dout[b, i, h] * s * y) / den
                sq = max(sq, np.max(np.abs(S[b, h, blk] @ dnum)), np.max(np.abs(dden * z[b, h, blk])))
                dS[blk] += np.outer(rq, dnum)
                dz[blk] += dden * pq
            G, Gz = np.cumsum(dS[::-1], axis=0)[::-1], np.cumsum(dz[::-1], axis=0)[::-1]
            for j in range(N):
                c = j // L
                sk = max(sk, np.max(np.abs(G[c] @ v[b, j, h])), np.max(np.abs(Gz[c])))
    return sq, sk


@pytest.mark.parametrize("B,T,Hs,Ws,H,d,F", [(1, 1, 1, 1, 1, 128, 1), (2, 3, 1, 1, 2, 128, 1),
                                              (1, 2, 1, 1, 2, 64, 1)])
def test_one_token_blocks_backward(B, T, Hs, Ws, H, d, F):
    # Blocks of one token: the output is scale-invariant in q and k up to eps,
    # so dq and dk are the small difference of two quotient-rule terms that
    # nearly cancel (one token: dq, dk = O(eps)).  Their error is set by the
    # terms: the matrix-core products carry about 16 bits of them (2^-16 =
    # 1.5e-5), summed over d features, so the floor of the bar is 1e-2 of the
    # terms' scale (absolute errors up to 1e-4 of it) instead of 1e-3 of
    # max|dq|.
    x = host_inputs(B, T, Hs, Ws, H, d, "bf16", seed=1039 + T)
    dout = _dout(x["q"].shape, "bf16", 1040 + T)
    dev = to_device(x, "bf16")
    ddev = to_device({"o": dout}, "bf16")["o"]
    got = _run(dev, ddev, (T, Hs, Ws), F)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], dout, (T, Hs, Ws), F)
    f64 = [a.astype(np.float64) for a in (x["q"], x["k"], x["v"], x["g"], dout)]
    scales = _quotient_term_scales(*f64, (T, Hs, Ws), F)
    for gname, a, r, sc in zip(("dq", "dk"), got[:2], ref[:2], scales):
        e = np.abs(to_host_f32(a).astype(np.float64) - r) / (np.abs(r) + 1e-2 * sc)
        print(f"  {gname}: max|ref| {np.max(np.abs(r)):.2e} term scale {sc:.2e} err {e.max():.3e}",
              flush=True)
        assert e.max() <= TOL["bf16"], gname
    for gname, a, r in zip(("dv", "dg"), got[2:], ref[2:]):
        assert grad_err(to_host_f32(a), r) <= TOL["bf16"], gname
