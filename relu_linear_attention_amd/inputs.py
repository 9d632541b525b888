"""Seeded synthetic inputs for the gated linear-attention token mixer.

This module only draws random numbers and rounds them; it holds none of the
operator's arithmetic.  Both the fp64 oracle and the HIP path are fed from it.

Recipe (the same for every workload):

* one generator per workload, seeded with that workload's seed;
* q, k, v, g are drawn in that order, each as B*N*H*d iid N(0, 1) float32
  values in [B, N, H, d] C-order, N = T*Hs*Ws in t-major token order;
* bf16 workloads round each value to bfloat16 with round-to-nearest-even.

Two generators implement the recipe:

* :func:`host_inputs` - numpy PCG64 on the host (sizes the oracle runs whole);
* :func:`device_inputs` - torch's device Philox generator, for the
  full-size video workloads whose tensors (up to 5.3 GB each) are drawn
  directly in HBM; the oracle then reads back the slices it needs.

Workload shapes follow the 480p/720p video latents of the pages: a
4 x 16 x 16 (time x height x width) latent compression of 81-frame clips.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hs: int
    Ws: int
    H: int
    d: int
    dtype: str  # "bf16" or "f32"
    seed: int
    frames_per_block: int = 0  # 0: non-causal
    theta: float = 10000.0
    eps: float = 1e-6
    notes: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def grid(self):
        return (self.T, self.Hs, self.Ws)

    @property
    def shape(self):
        return (self.B, self.N, self.H, self.d)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 4, 4, 2, 32, "f32", 0,
                         notes="N=32 tokens, fp32, oracle in well under a second"),
    "480p_81f": Workload("480p_81f", 1, 21, 30, 52, 24, 128, "bf16", 1,
                         notes="480p/81f layer, N=32,760"),
    "720p_81f": Workload("720p_81f", 1, 21, 45, 80, 32, 128, "bf16", 2,
                         notes="720p/81f layer at 14B width, N=75,600"),
    "720p_60s": Workload("720p_60s", 1, 241, 45, 80, 24, 128, "bf16", 3,
                         notes="720p/60s long video, N=867,600, 2.67e9 elements per tensor"),
    "720p_block_causal": Workload("720p_block_causal", 1, 21, 45, 80, 24, 128, "bf16", 4,
                                  frames_per_block=3,
                                  notes="7 temporal blocks of 3 latent frames (10,800 tokens)"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns the rounded values as float32 (exactly representable in bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32)


def host_inputs(B, T, Hs, Ws, H, d, dtype="bf16", seed=0):
    """Draw q, k, v, g on the host.

    Returns a dict of float32 numpy arrays of shape [B, N, H, d] holding the
    values the operator sees (already rounded to bf16 for bf16 workloads)."""
    N = T * Hs * Ws
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v", "g"):
        x = rng.standard_normal(B * N * H * d, dtype=np.float32).reshape(B, N, H, d)
        out[name] = round_to_bf16(x) if dtype == "bf16" else x
    return out


def host_inputs_for(w: Workload):
    return host_inputs(w.B, w.T, w.Hs, w.Ws, w.H, w.d, w.dtype, w.seed)


def device_inputs(B, T, Hs, Ws, H, d, dtype="bf16", seed=0, device="cuda"):
    """Draw q, k, v, g directly in device memory with torch's seeded generator.

    Each tensor is drawn as float32 N(0, 1) in [B, N, H, d] order and cast to
    bfloat16 (round-to-nearest-even) in slabs, so no float32 copy of a whole
    tensor is ever held."""
    import torch

    N = T * Hs * Ws
    tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    slab = max(1, (1 << 27) // max(1, H * d))  # tokens per slab (~128M values)
    for name in ("q", "k", "v", "g"):
        t = torch.empty((B, N, H, d), dtype=tdtype, device=device)
        for b in range(B):
            for n0 in range(0, N, slab):
                n1 = min(N, n0 + slab)
                x = torch.randn((n1 - n0, H, d), dtype=torch.float32, device=device,
                                generator=gen)
                t[b, n0:n1].copy_(x)
                del x
        out[name] = t
    return out


def device_inputs_for(w: Workload, device="cuda"):
    return device_inputs(w.B, w.T, w.Hs, w.Ws, w.H, w.d, w.dtype, w.seed, device)
