"""Shared helpers of the test suite (no test functions here)."""
import numpy as np
import torch

from gated_deltanet_sequence_amd import inputs

# Tolerances on max-abs-normwise error: max|x - x*| / max|x*|, per tensor.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def maxrel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(den, 1e-300))


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu").float().numpy()


def to_dev(x: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def oracle_inputs(x: dict, chains=None):
    """fp32 numpy views of a forward workload (optionally a subset of the
    flattened (b,h) chains, returned as B=1, H=len(chains))."""
    arrs = [inputs.to_f32_numpy(x[n]) for n in ("q", "k", "v")]
    arrs += [x["alpha"].numpy(), x["beta"].numpy()]
    s0 = x["s0"].numpy() if x.get("s0") is not None else None
    if chains is None:
        return arrs, s0
    out = []
    for a in arrs:
        flat = a.reshape((-1,) + a.shape[2:])
        out.append(np.ascontiguousarray(flat[chains])[None])
    if s0 is not None:
        s0 = np.ascontiguousarray(s0.reshape((-1,) + s0.shape[2:])[chains])[None]
    return out, s0
