"""Seeded synthetic inputs for the chunked gated-delta-rule forward and its
decode step.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no arithmetic of the recurrence itself: it only draws random numbers
and shapes them into the workloads' value distributions.

Recipe (fixed order of draws from one ``numpy.random.default_rng(seed)``,
all as float32 standard normals):
  q, k, v, z_alpha, z_beta, [S0]
  * q and k are L2-normalised per token over d, in fp32;
  * bf16 workloads round q, k, v to bf16 with round-to-nearest-even
    (``torch`` CPU cast);
  * alpha = exp(-softplus(z_alpha)) in (0,1),  beta = sigmoid(z_beta) in (0,1),
    both evaluated in fp64 and rounded once to fp32;
  * "slow" gates use alpha = exp(-0.01 * softplus(z_alpha)) (alpha close to 1,
    i.e. a state that forgets slowly);
  * "fast" gates use alpha = exp(-4 * softplus(z_alpha)) (a chunk of 64 tokens
    decays by far more than 2^-120);
  * "resets" gates are the default ones with alpha = 0 exactly where
    z_alpha > 2.3 (about 1% of tokens: the state is wiped there);
  * "beta2" gates are the default alpha with beta = 2 sigmoid(z_beta) in (0,2);
  * S0, when requested, is N(0, 0.1) (standard deviation 0.1), fp32.

Every returned tensor is a contiguous CPU tensor; the caller moves it to the
device.  The same tensors (widened exactly to fp32) are what the oracle sees.

``make_fwd_inputs_on_device`` draws the same distributions (default gates)
with torch's generator on the device, for inputs too large to draw on the
host; its values differ from ``make_fwd_inputs`` for the same seed.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = ["make_fwd_inputs", "make_fwd_inputs_on_device", "make_decode_inputs", "CONFIGS", "to_f32_numpy"]


def _softplus64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _sigmoid64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def _l2norm_f32(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    n = np.maximum(n, np.float32(1e-12))
    return (x / n).astype(np.float32)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    if dtype == "f32":
        return t.float().contiguous()
    raise ValueError("dtype must be 'bf16' or 'f32'")


def _gates(rng, shape, gate: str):
    z_a = rng.standard_normal(shape, dtype=np.float32)
    z_b = rng.standard_normal(shape, dtype=np.float32)
    if gate in ("default", "beta2"):
        alpha = np.exp(-_softplus64(z_a))
    elif gate == "slow":
        alpha = np.exp(-0.01 * _softplus64(z_a))
    elif gate == "fast":
        alpha = np.exp(-4.0 * _softplus64(z_a))
    elif gate == "resets":
        alpha = np.where(z_a > 2.3, 0.0, np.exp(-_softplus64(z_a)))
    else:
        raise ValueError("gate must be one of 'default', 'slow', 'fast', 'resets', 'beta2'")
    beta = _sigmoid64(z_b) * (2.0 if gate == "beta2" else 1.0)
    return (torch.from_numpy(alpha.astype(np.float32)).contiguous(),
            torch.from_numpy(beta.astype(np.float32)).contiguous())


def make_vec_alpha(B: int, H: int, T: int, d: int, seed: int, gate: str = "default") -> torch.Tensor:
    """Per-dimension gate alpha [B,H,T,d] fp32: the scalar gate laws of
    ``_gates`` drawn independently per token and key dimension from
    ``numpy.random.default_rng(seed)`` ('default': exp(-softplus(z)); 'slow':
    exp(-0.01 softplus(z)); 'fast': exp(-4 softplus(z)); 'resets': 0 where
    z > 2.3, else exp(-softplus(z)))."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, H, T, d), dtype=np.float32)
    sp = _softplus64(z)
    if gate == "default":
        alpha = np.exp(-sp)
    elif gate == "slow":
        alpha = np.exp(-0.01 * sp)
    elif gate == "fast":
        alpha = np.exp(-4.0 * sp)
    elif gate == "resets":
        alpha = np.where(z > 2.3, 0.0, np.exp(-sp))
    else:
        raise ValueError("gate must be one of 'default', 'slow', 'fast', 'resets'")
    return torch.from_numpy(alpha.astype(np.float32)).contiguous()


def make_fwd_inputs(B: int, H: int, T: int, d: int, dtype: str = "bf16",
                    seed: int = 0, init_state: bool = False,
                    gate: str = "default", dv: int | None = None) -> dict:
    """Inputs of one chunked-forward call.

    Returns dict with q, k [B,H,T,d], v [B,H,T,dv] in ``dtype``; alpha, beta
    [B,H,T] fp32; s0 [B,H,dv,d] fp32 or None.
    """
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    q = _l2norm_f32(rng.standard_normal((B, H, T, d), dtype=np.float32))
    k = _l2norm_f32(rng.standard_normal((B, H, T, d), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    alpha, beta = _gates(rng, (B, H, T), gate)
    s0 = None
    if init_state:
        s0 = torch.from_numpy(
            (0.1 * rng.standard_normal((B, H, dv, d), dtype=np.float32)).astype(np.float32)
        ).contiguous()
    return {"q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
            "alpha": alpha, "beta": beta, "s0": s0}


def make_fwd_inputs_on_device(B: int, H: int, T: int, d: int, seed: int, device) -> dict:
    """bf16 inputs of one chunked-forward call drawn on ``device`` with
    ``torch.Generator(device).manual_seed(seed)``, in the order q, k, v,
    z_alpha, z_beta (fp32 standard normals; default gates, evaluated in fp32;
    no initial state).  Each tensor is made in place of its draw, so the peak
    footprint is about one fp32 copy of q."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        x = torch.randn((B, H, T, d), generator=g, device=device, dtype=torch.float32)
        if name != "v":
            x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min_(1e-12)
        out[name] = x.to(torch.bfloat16)
        del x
    z_a = torch.randn((B, H, T), generator=g, device=device, dtype=torch.float32)
    z_b = torch.randn((B, H, T), generator=g, device=device, dtype=torch.float32)
    out["alpha"] = torch.exp(-torch.nn.functional.softplus(z_a)).contiguous()
    out["beta"] = torch.sigmoid(z_b).contiguous()
    out["s0"] = None
    return out


def make_decode_inputs(N: int, H: int, d: int, steps: int, dtype: str = "bf16",
                       seed: int = 0, gate: str = "default") -> dict:
    """Inputs of ``steps`` consecutive decode steps.

    The state [N,H,d,d] ~ N(0, 0.1) fp32 is drawn first, then per step, in
    order: q, k, v, z_alpha, z_beta (each step gets fresh tokens).  Returns dict
    with s0 and lists q, k, v, alpha, beta of length ``steps``.
    """
    rng = np.random.default_rng(seed)
    s0 = torch.from_numpy(
        (0.1 * rng.standard_normal((N, H, d, d), dtype=np.float32)).astype(np.float32)
    ).contiguous()
    out = {"s0": s0, "q": [], "k": [], "v": [], "alpha": [], "beta": []}
    for _ in range(steps):
        q = _l2norm_f32(rng.standard_normal((N, H, d), dtype=np.float32))
        k = _l2norm_f32(rng.standard_normal((N, H, d), dtype=np.float32))
        v = rng.standard_normal((N, H, d), dtype=np.float32)
        alpha, beta = _gates(rng, (N, H), gate)
        out["q"].append(_cast(q, dtype))
        out["k"].append(_cast(k, dtype))
        out["v"].append(_cast(v, dtype))
        out["alpha"].append(alpha)
        out["beta"].append(beta)
    return out


def to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 widening of a CPU tensor (bf16 or fp32) as a numpy array."""
    return t.detach().to("cpu").float().contiguous().numpy()


# The five workloads: name -> keyword arguments.  Seeds 1..5 in this order.
CONFIGS = {
    "tiny": dict(B=1, H=1, T=256, d=64, C=64, dtype="f32", seed=1, init_state=False),
    "loop": dict(B=1, H=4, T=8192, d=64, C=64, dtype="bf16", seed=2, init_state=False),
    "main": dict(B=4, H=16, T=8192, d=128, C=64, dtype="bf16", seed=3, init_state=False),
    "long": dict(B=1, H=16, T=131072, d=128, C=64, dtype="bf16", seed=4, init_state=True),
    "decode": dict(N=256, H=16, d=128, steps=64, dtype="bf16", seed=5),
}
