"""Helpers for the GPU tests: moving seeded inputs to the device and the
comparison metric.  No operator arithmetic lives here."""
from __future__ import annotations

import numpy as np


def have_gpu() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(x: dict, dtype: str):
    """float32 numpy arrays (already bf16-exact for bf16) -> device tensors."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {n: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(tdt) for n, a in x.items()}


def to_host_f32(t) -> np.ndarray:
    return t.float().cpu().numpy()


def max_rel_err(got, ref, floor=1e-3) -> float:
    """max_i |got_i - ref_i| / (|ref_i| + floor)"""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


# tolerances of the operator's outputs (max |err| / (|ref| + 1e-3))
TOL = {"f32": 1e-4, "bf16": 1e-2}


def unaligned_copies(x: dict, dtype: str = "bf16"):
    """Device copies of the arrays that start one element into their
    allocations (too misaligned for 16-byte loads), plus a maker of output
    tensors placed the same way."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def place(shape):
        n = int(np.prod(shape))
        return torch.empty(n + 1, dtype=tdt, device="cuda")[1:].view(*shape)

    ts = {}
    for name, a in x.items():
        t = place(a.shape)
        t.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(tdt))
        ts[name] = t
    return ts, place
