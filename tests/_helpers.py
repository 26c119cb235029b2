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


def grouped_oracle_errors(x: dict, go: np.ndarray, gs: np.ndarray, group: int = 4):
    """Max-abs-normwise errors of GPU outputs (go [B,H,T,dv], gs [B,H,dv,dk])
    against the fp64 oracle over EVERY (b,h) chain, with the oracle run on
    `group` chains at a time so that its fp64 outputs for a long workload never
    all sit in host memory at once.  The normalisation is over the whole tensor,
    as in maxrel."""
    import oracle
    B, H = x["q"].shape[:2]
    n = B * H
    go = go.reshape((n,) + go.shape[2:])
    gs = gs.reshape((n,) + gs.shape[2:])
    dmax_o = rmax_o = dmax_s = rmax_s = 0.0
    for c0 in range(0, n, group):
        chains = list(range(c0, min(n, c0 + group)))
        (q, k, v, a, b), s0 = oracle_inputs(x, chains)
        ro, rs = oracle.oracle_fwd(q, k, v, a, b, s0)
        dmax_o = max(dmax_o, float(np.max(np.abs(go[chains][None].astype(np.float64) - ro))))
        dmax_s = max(dmax_s, float(np.max(np.abs(gs[chains][None].astype(np.float64) - rs))))
        rmax_o = max(rmax_o, float(np.max(np.abs(ro))))
        rmax_s = max(rmax_s, float(np.max(np.abs(rs))))
        assert np.all(np.isfinite(go[chains])) and np.all(np.isfinite(gs[chains]))
        del ro, rs, q, k, v
    return dmax_o / max(rmax_o, 1e-300), dmax_s / max(rmax_s, 1e-300)
