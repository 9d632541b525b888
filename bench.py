"""Throughput of the gated ReLU linear-attention token mixer on one MI355X.

One step = one call of the whole operator over one batch of synthetic inputs
already resident in HBM, through the C ABI (gla_forward_ws with a
pre-allocated workspace): the state kernel (chunk partials, with the reduce
folded into each unit's last workgroup) and the apply kernel; the RoPE table
comes from the library's per-shape cache after the first call.

    python bench.py [--steps K] [--warmup W] [--workload 720p_81f]

Prints one JSON line: tokens/s of the whole job (K timed steps), the
per-stage launch times (HIP events on the launch stream, recorded by the
library around each kernel in a second pass of K steps), the HBM roofline of
the dominant kernel, and the fp64 oracle timed on the host cores as a CPU
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector, published
PEAK_BF16_MFMA_FLOPS = 2.5e15  # MI355X dense bf16 matrix cores, published
DEFAULT_WORKLOAD = "720p_81f"
CSRC = os.path.join(ROOT, "relu_linear_attention_amd", "csrc")


def source_digest() -> str:
    """sha256[:16] over every kernel and launcher source (a change to any of
    them invalidates the recorded counters)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of each kernel from the committed rocprofv3
    counter summary, or {} when there is none or the kernels have changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    digest, scale_f, scale_w, kernels = None, None, None, {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#"):
                continue
            if parts[0] == "source_digest":
                digest = parts[1]
            elif parts[0] == "copy_scale_fetch":
                scale_f = float(parts[1])
            elif parts[0] == "copy_scale_write":
                scale_w = float(parts[1])
            elif parts[0] == "kernel":
                kernels[parts[1]] = (float(parts[2]), float(parts[3]))
    if digest != source_digest() or scale_f is None or scale_w is None:
        return {}
    return {k: (fk * scale_f + wk * scale_w) * 1024.0 for k, (fk, wk) in kernels.items()}


def measured_counters(workload: str):
    """Normalised matrix-core busy fraction per kernel from the committed
    rocprofv3 counter summary (lines "mfma_busy <kernel> <fraction>"), or {}
    when there is none or the kernels have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return {}
    digest, busy = None, {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#"):
                continue
            if parts[0] == "source_digest":
                digest = parts[1]
            elif parts[0] == "mfma_busy":
                busy[parts[1]] = float(parts[2])
    return busy if digest == source_digest() else {}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_call_ms(call, n: int, stream) -> list:
    """n calls, each between its own pair of events on `stream` (the events
    sit between calls, outside any kernel): per-call durations in ms."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def cpu_baseline(w, dev_inputs):
    """The fp64 oracle, as it stands, on one full forward of the workload."""
    import oracle

    host = {n: t.float().cpu().numpy() for n, t in dev_inputs.items()}
    t0 = time.perf_counter()
    out = oracle.forward(host["q"], host["k"], host["v"], host["g"], w.grid,
                         w.frames_per_block, w.theta, w.eps)
    dt = time.perf_counter() - t0
    del out, host
    return {
        "value": w.B * w.N / dt,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"one full fp64 forward of the {w.name} layer ({w.B}x{w.N} tokens, "
                   f"{w.H} heads, d={w.d}) on the host, inputs copied from HBM; "
                   f"{dt:.2f} s"),
    }


def timed_calls(call, steps: int, stream, profile: bool):
    """`steps` calls bracketed by events on `stream`, with a device
    synchronization on both sides.  Returns (ms per call, wall seconds, the
    library's per-stage records or None).  With `profile` the library also
    brackets every kernel launch with HIP events on the stream; those events
    cost a few microseconds per launch, so the headline timing runs without
    them and the stage durations come from a second pass with them."""
    import torch

    from relu_linear_attention_amd import gla

    if profile:
        gla.gla_profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        call()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = None
    if profile:
        stages = gla.gla_profile_read()
        gla.gla_profile_enable(False)
    return start.elapsed_time(stop) / steps, wall, stages


def same_bytes_reference(x, steps: int, warmup: int) -> dict:
    """A library elementwise kernel over the apply kernel's algorithmic bytes:
    torch.add(q, g) into a third tensor (two tensors read, one written, the
    same shapes and dtype), timed like the headline pass.  Context for the
    apply kernel's roofline fraction: what a plain two-in/one-out stream of
    these tensors reaches on the same GPU in the same run."""
    import torch

    q, g = x["q"], x["g"]
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def call():
        torch.add(q, g, out=o)

    for _ in range(warmup):
        call()
    ms, _, _ = timed_calls(call, steps, stream, profile=False)
    nbytes = 3 * q.numel() * q.element_size()
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"op": f"torch.add(q, g, out=o), {str(q.dtype).replace('torch.', '')}",
            "bytes_per_call": nbytes, "ms_per_call": ms, "GBps": gbps,
            "frac": gbps / PEAK_HBM_GBPS}


def block_step_leg(steps: int, warmup: int, workload: str = "720p_block_causal"):
    """The streaming block-causal step (gla_block_step): the layer's blocks of
    frames_per_block latent frames fed one at a time through the fp32 cache,
    each step updating it.  One pass = every block of the layer once."""
    import torch

    from relu_linear_attention_amd import gla
    from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for

    w = WORKLOADS[workload]
    Tb, hw = w.frames_per_block, w.Hs * w.Ws
    x = device_inputs_for(w)
    out = torch.empty_like(x["q"])
    blocks = [{n: t[:, b0 * hw:(b0 + Tb) * hw] for n, t in list(x.items()) + [("out", out)]}
              for b0 in range(0, w.T, Tb)]
    S = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device="cuda")
    z = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(gla.gla_workspace_bytes(w.B, w.H, Tb, w.Hs, w.Ws, w.d, 0, gla.GLA_BF16),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def one_pass():
        S.zero_()
        z.zero_()
        for i, blk in enumerate(blocks):
            gla.gla_block_step(blk["q"], blk["k"], blk["v"], blk["g"], blk["out"], S, z,
                               (Tb, w.Hs, w.Ws), i * Tb, True, w.theta, w.eps, workspace=ws,
                               stream=stream)

    for _ in range(warmup):
        one_pass()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        one_pass()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_pass = start.elapsed_time(stop) / steps
    nblk = len(blocks)
    tensor_bytes = 5 * w.B * w.N * w.H * w.d * w.elem_bytes
    cache_bytes = nblk * 2 * 4 * w.B * w.H * (w.d * w.d + w.d)  # read + write per step
    gbps = (tensor_bytes + cache_bytes) / (ms_pass * 1e-3) / 1e9
    del x, out, blocks
    return {
        "workload": w.name, "blocks": nblk, "frames_per_block": Tb, "B": w.B, "H": w.H,
        "tokens_per_block": Tb * hw, "ms_per_pass": ms_pass, "ms_per_step": ms_pass / nblk,
        "tokens_per_s": w.B * w.N / (ms_pass * 1e-3),
        "algorithmic_bytes_per_pass": tensor_bytes + cache_bytes, "GBps": gbps,
        "frac_of_peak": gbps / PEAK_HBM_GBPS,
    }


def gated_leg(w, x, ws, steps: int, warmup: int):
    """The gated mixer (gla_gated_forward) on the same workload: the write gate
    beta [B, N, H] and the RMSNorm weight [d], both bf16, on top of the
    operator.  Algorithmic bytes add beta (2 bytes per token-head)."""
    import torch

    from relu_linear_attention_amd import gla

    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 100)
    beta = torch.sigmoid(torch.randn((w.B, w.N, w.H), device="cuda", generator=gen)).to(
        torch.bfloat16)
    rms_w = (1.0 + 0.5 * torch.randn((w.d,), device="cuda", generator=gen)).to(torch.bfloat16)
    out = torch.empty_like(x["q"])
    stream = torch.cuda.current_stream()

    def call():
        gla.gla_gated_forward(x["q"], x["k"], x["v"], x["g"], beta, rms_w, out, w.grid,
                              w.frames_per_block, w.theta, w.eps, 1e-6, workspace=ws,
                              stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = 5 * w.B * w.N * w.H * w.d * w.elem_bytes + w.B * w.N * w.H * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "beta": "[B, N, H] bf16", "rms_weight": "[d] bf16",
            "ms_per_call": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
            "algorithmic_bytes_per_call": nbytes, "GBps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS}


def backward_leg(w, x, steps: int, warmup: int):
    """Gradients (gla_backward) of sum(dout * out) on the same workload: the
    state stage re-run, then the gradient kernels.  Algorithmic bytes: q, k,
    v, g, dout read once and dq, dk, dv, dg written once."""
    import torch

    from relu_linear_attention_amd import gla

    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 200)
    dout = torch.randn(x["q"].shape, device="cuda", generator=gen).to(x["q"].dtype)
    grads = [torch.empty_like(x["q"]) for _ in range(4)]
    ws = torch.empty(gla.gla_backward_workspace_bytes(w.B, w.H, w.T, w.Hs, w.Ws, w.d,
                                                      w.frames_per_block,
                                                      gla.GLA_BF16 if w.dtype == "bf16"
                                                      else gla.GLA_F32),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        gla.gla_backward(x["q"], x["k"], x["v"], x["g"], dout, *grads, w.grid, w.frames_per_block,
                         w.theta, w.eps, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    ms, _, _ = timed_calls(call, steps, stream, profile=False)
    _, _, stages = timed_calls(call, steps, stream, profile=True)
    nbytes = 9 * w.B * w.N * w.H * w.d * w.elem_bytes
    gbps = nbytes / (ms * 1e-3) / 1e9
    stage_ms = {k: (v / n if n else None) for k, (n, v) in stages.items()}
    mfma = gla.gla_uses_matrix_cores(w.T, w.Hs, w.Ws, w.d, gla.GLA_BF16 if w.dtype == "bf16"
                                     else gla.GLA_F32) == 1
    grad_ms = stage_ms["backward"]
    if mfma:
        # the gradient kernels' algorithmic bytes are nine tensor passes (q, g,
        # dout, k, v read; dq, dg, dk, dv written); the state pass reads q, g
        # and dout a second time, which the measured traffic shows
        names = ("bwd_token_mfma_kernel", "bwd_dstate_mfma_kernel", "bwd_reduce_kernel",
                 "bwd_kv_mfma_kernel")
        measured = measured_traffic(w.name)
        roof = {"bound": "hbm", "kernel": " + ".join(names),
                "achieved": nbytes / (grad_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "traffic": (sum(measured[n] for n in names)
                            if w.frames_per_block == 0 and all(n in measured for n in names)
                            else None),
                "algorithmic_bytes_per_launch": nbytes}
        roof["frac"] = roof["achieved"] / PEAK_HBM_GBPS
        kernels = ("matrix-core gradient kernels (query side: token pass and state pass; block "
                   "sums; key/value side)")
    else:
        # fp32 FMA work on the vector units: per token-head, five d x d products
        # (num, S dnum and the dS outer product on the query side; G v and
        # RoPE(phi(k)) G on the key/value side)
        flops = 2 * 5 * w.d * w.d * w.B * w.N * w.H
        tflops = flops / (grad_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "kernel": "bwd_q_kernel + bwd_reduce_kernel + bwd_kv_kernel",
                "achieved": tflops, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_FP32_VALU_TFLOPS, "traffic": None,
                "algorithmic_flops_per_launch": flops}
        kernels = "vector (fp32 VALU) gradient kernels"
    # The training pair: the forward keeps its reduced state (gla_forward_train)
    # and the gradients take it (gla_backward_saved), as an autograd step
    # would, so the state stage is not run twice.  Timed alone and as whole
    # steps (forward + gradients).
    dt = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_F32
    saved = torch.empty(gla.gla_saved_state_bytes(w.B, w.H, w.T, w.Hs, w.Ws, w.d,
                                                  w.frames_per_block) // 4,
                        dtype=torch.float32, device="cuda")
    out = torch.empty_like(x["q"])
    fws = torch.empty(gla.gla_workspace_bytes(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.frames_per_block,
                                              dt), dtype=torch.uint8, device="cuda")

    def fwd_train():
        gla.gla_forward_train(x["q"], x["k"], x["v"], x["g"], out, saved, w.grid,
                              w.frames_per_block, w.theta, w.eps, workspace=fws, stream=stream)

    def bwd_saved():
        gla.gla_backward_saved(x["q"], x["k"], x["v"], x["g"], dout, *grads, saved, w.grid,
                               w.frames_per_block, w.theta, w.eps, workspace=ws, stream=stream)

    def train_step():
        fwd_train()
        bwd_saved()

    fwd_train()
    for _ in range(warmup):
        bwd_saved()
    ms_saved, _, _ = timed_calls(bwd_saved, steps, stream, profile=False)
    for _ in range(warmup):
        train_step()
    ms_step, _, _ = timed_calls(train_step, steps, stream, profile=False)
    return {"workload": w.name, "ms_per_call": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
            "stages_ms": stage_ms, "algorithmic_bytes_per_call": nbytes, "GBps": gbps,
            "frac_of_peak": gbps / PEAK_HBM_GBPS, "roofline": roof,
            "kernels": kernels + "; the forward state re-run on the matrix cores",
            "saved_state": {"ms_per_call": ms_saved,
                            "training_step_ms": ms_step,
                            "what": "gla_backward_saved after gla_forward_train (the forward's "
                                    "S, z kept, no state re-run); training_step_ms: one "
                                    "gla_forward_train + gla_backward_saved"}}


def token_causal_leg(w, x, steps: int, warmup: int, oracle_frames: int = 2):
    """The token-causal form (gla_token_causal_forward) on the same workload:
    state partials, the range prefixes and the tile kernel.  Algorithmic
    bytes: q, k, v, g read once and out written once.  The fp64 oracle is
    timed beside it on the first `oracle_frames` latent frames (every head)."""
    import torch

    from relu_linear_attention_amd import gla

    out = torch.empty_like(x["q"])
    ws = torch.empty(gla.gla_token_causal_workspace_bytes(w.B, w.H, w.T, w.Hs, w.Ws, w.d,
                                                          gla.GLA_BF16 if w.dtype == "bf16"
                                                          else gla.GLA_F32),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        gla.gla_token_causal_forward(x["q"], x["k"], x["v"], x["g"], out, w.grid, w.theta, w.eps,
                                     workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    ms, _, _ = timed_calls(call, steps, stream, profile=False)
    _, _, stages = timed_calls(call, steps, stream, profile=True)
    nbytes = 5 * w.B * w.N * w.H * w.d * w.elem_bytes
    gbps = nbytes / (ms * 1e-3) / 1e9
    stage_ms = {k: (v / n if n else None) for k, (n, v) in stages.items()}
    tile_ms = stage_ms["causal_apply"]
    mfma = gla.gla_uses_matrix_cores(w.T, w.Hs, w.Ws, w.d, gla.GLA_BF16 if w.dtype == "bf16"
                                     else gla.GLA_F32) == 1
    kname = "causal_mfma_kernel" if mfma else "causal_vector_kernel"
    tile_gbps = nbytes / (tile_ms * 1e-3) / 1e9
    res = {"workload": w.name, "ms_per_call": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
           "stages_ms": stage_ms, "algorithmic_bytes_per_call": nbytes, "GBps": gbps,
           "frac_of_peak": gbps / PEAK_HBM_GBPS,
           # the tile kernel reads q, k, v, g and writes out: the same five
           # tensor passes as the whole call (the state stage re-reads k, v)
           "roofline": {"bound": "hbm", "kernel": kname, "achieved": tile_gbps,
                        "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": tile_gbps / PEAK_HBM_GBPS,
                        "traffic": measured_traffic(w.name).get(kname),
                        "algorithmic_bytes_per_launch": nbytes}}
    if oracle_frames <= 0:
        return res
    try:
        import oracle

        n = oracle_frames * w.Hs * w.Ws
        host = {k_: t[:, :n].float().cpu().numpy() for k_, t in x.items()}
        t0 = time.perf_counter()
        oracle.token_causal(host["q"], host["k"], host["v"], host["g"],
                            (oracle_frames, w.Hs, w.Ws), w.theta, w.eps)
        sec = time.perf_counter() - t0
        res["oracle"] = {"tokens_per_s": w.B * n / sec, "seconds": sec,
                         "sample": f"first {oracle_frames} latent frames ({n} tokens), all heads",
                         "cores": oracle.num_threads()}
    except Exception as e:  # the oracle is a reported baseline; the GPU figures stand alone
        res["oracle"] = {"error": str(e)}
    return res


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (FETCH_SIZE, WRITE_SIZE) of the kernels."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "ms": ms, "GBps_read_plus_write": 2 * nbytes / ms / 1e6}))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU reaches its steady clocks only after a few dozen calls: with 8
    # untimed calls the 720p/81f layer measures ~9% slower than after 50.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block-step", action="store_true",
                    help="skip the streaming block-step measurement")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the gated-mixer (write gate + RMSNorm) measurement")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gradient measurement")
    ap.add_argument("--no-token-causal", action="store_true",
                    help="skip the token-causal measurement")
    ap.add_argument("--only-leg", choices=["gated", "backward", "token_causal", "block_step"],
                    help="run only this measurement and print its JSON (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the operator is "
              "benchmarked at one GPU's share; more GPUs would shard the (batch, head) units or the "
              "token axis, which is not built",
              file=sys.stderr)
        return 2

    import torch

    from relu_linear_attention_amd import gla
    from relu_linear_attention_amd.inputs import WORKLOADS, device_inputs_for

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return 0

    w = WORKLOADS[args.workload]
    if args.only_leg == "block_step":
        print(json.dumps({"block_step": block_step_leg(args.steps, args.warmup)}))
        return 0
    x = device_inputs_for(w)
    if args.only_leg == "backward":
        print(json.dumps({"backward": backward_leg(w, x, args.steps, args.warmup)}))
        return 0
    if args.only_leg == "token_causal":
        print(json.dumps({"token_causal": token_causal_leg(w, x, args.steps, args.warmup,
                                                           oracle_frames=0)}))
        return 0
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    out = torch.empty_like(q)
    dtype_code = gla.GLA_BF16 if w.dtype == "bf16" else gla.GLA_F32
    ws = torch.empty(gla.gla_workspace_bytes(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.frames_per_block,
                                             dtype_code), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    if args.only_leg == "gated":
        print(json.dumps({"gated": gated_leg(w, x, ws, args.steps, args.warmup)}))
        return 0

    def step():
        gla.gla_forward_ws(q, k, v, g, out, w.grid, ws, w.frames_per_block, w.theta, w.eps,
                           stream=stream)

    # the W untimed warm-up calls, each between its own events (its duration
    # is reported, not counted: the first calls of a process run slower)
    warm_ms = per_call_ms(step, args.warmup, stream) if args.warmup else []

    # timed region: K steps between events on `stream`; then K more steps with
    # every kernel bracketed by HIP events on `stream` for the per-kernel
    # durations (the roofline of the dominant kernel); then K more, each
    # between its own events, for the per-call median, min and max
    ms_per_step, wall, _ = timed_calls(step, args.steps, stream, profile=False)
    _, _, stages = timed_calls(step, args.steps, stream, profile=True)
    calls_ms = sorted(per_call_ms(step, args.steps, stream))
    tokens = w.B * w.N
    elem = w.B * w.N * w.H * w.d * w.elem_bytes
    algo_bytes = {"state_partials": 2 * elem, "apply": 3 * elem}

    stage_ms = {name: (ms / n if n else None) for name, (n, ms) in stages.items()}
    dominant = max(("state_partials", "apply"), key=lambda s: stages[s][1])
    dom_ms = stage_ms[dominant]
    achieved = algo_bytes[dominant] / (dom_ms * 1e-3) / 1e9
    mfma = gla.gla_uses_matrix_cores(w.T, w.Hs, w.Ws, w.d, dtype_code) == 1
    kernel_names = {"state_partials": "state_mfma_kernel" if mfma else "state_vector_kernel",
                    "apply": "apply_mfma_kernel" if mfma else "apply_vector_kernel"}
    traffic = measured_traffic(w.name).get(kernel_names[dominant])
    # matrix-core work issued per launch (flops of the bf16 products as
    # issued, hi/lo splits included): state 2 products of d x d per token and
    # head, apply 3 plus the 16-row normaliser product per 32 features
    hd = w.B * w.N * w.H
    mfma_flops = {"state_partials": 2 * 2 * hd * w.d * w.d,
                  "apply": 3 * 2 * hd * w.d * w.d + 2 * 16 * hd * w.d}
    busy = measured_counters(w.name)
    mfma_util = {}
    for st, kname in kernel_names.items():
        if mfma and stage_ms.get(st):
            mfma_util[kname] = {
                "issued_flops_frac": mfma_flops[st] / (stage_ms[st] * 1e-3) / PEAK_BF16_MFMA_FLOPS,
                "busy_counter": busy.get(kname)}

    result = {
        "metric": "GLA fwd tokens/s at 720p/81f (32 heads, d=128, bf16) + % of HBM roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hs": w.Hs, "Ws": w.Ws, "N": w.N,
                   "H": w.H, "d": w.d, "frames_per_block": w.frames_per_block,
                   "rope_theta": w.theta, "eps": w.eps, "seed": w.seed,
                   "kernels": "matrix-core" if mfma else "vector"},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_names[dominant],
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes[dominant],
            "mfma_busy": busy.get(kernel_names[dominant]),
            "mfma_busy_note": ("SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x CUs x GRBM_GUI_ACTIVE / 8 "
                               "XCDs): the fraction of the kernel's cycles its SIMDs spent in "
                               "matrix-core instructions, from the committed counter summary"),
        },
        "mfma_utilisation": mfma_util,
        "per_call_ms": {"median": calls_ms[len(calls_ms) // 2], "min": calls_ms[0],
                        "max": calls_ms[-1], "n": len(calls_ms),
                        "note": "one event pair per call, after the timed pass"},
        "warmup_calls_ms": warm_ms,
        "stages_ms": stage_ms,
        "same_bytes_reference": same_bytes_reference(x, args.steps, min(args.warmup, 20)),
        "path": {
            "algorithmic_bytes_per_step": 5 * elem,
            "GBps": 5 * elem / (ms_per_step * 1e-3) / 1e9,
            "frac_of_peak": 5 * elem / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "wall_s": wall,
        },
        "cpu_baseline": None,
    }
    if not args.no_gated and mfma:
        result["gated"] = gated_leg(w, x, ws, max(3, args.steps // 2), 10)
    if not args.no_backward:
        result["backward"] = backward_leg(w, x, max(3, args.steps // 10), 3)
    if not args.no_token_causal:
        result["token_causal"] = token_causal_leg(w, x, max(3, args.steps // 4), 5)
    if not args.no_block_step:
        result["block_step"] = block_step_leg(max(3, args.steps // 4), 5)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
