"""GPU parity of the decode steps with a per-dimension gate
(gdn_recurrent_step_vecgate) and without the delta rule (gla_recurrent_step).

Chaining the steps over T tokens is the token loop of the matching forward
oracle (oracle_fwd_vecgate, oracle_gla_fwd, both pinned on the CPU), so every
step's output and the final state are compared with that oracle run over the
same T tokens from the same initial state, with the workloads' bars (2e-2
bf16, 1e-4 fp32, max-abs-normwise).  The chained steps are also checked
against the chunked forward entry point of the same recurrence on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (GDNError, gdn_chunk_fwd_vecgate, gdn_recurrent_step,
                                                 gdn_recurrent_step_vecgate, gla_chunk_fwd, gla_recurrent_step)

from _helpers import TOL, maxrel, to_np

pytestmark = pytest.mark.gpu


def _draw(N, H, d, steps, dtype, seed, kind, gate="default"):
    """Decode inputs stacked over the steps as a forward workload: q, k, v
    [N,H,steps,d], alpha [N,H,steps] (scalar) or [N,H,steps,d] (per
    dimension), beta [N,H,steps], s0 [N,H,d,d]."""
    x = inputs.make_decode_inputs(N, H, d, steps, dtype, seed=seed, gate=gate if kind == "gla" else "default")
    f = {n: torch.stack(x[n], dim=2).contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    if kind == "vec":
        f["alpha"] = inputs.make_vec_alpha(N, H, steps, d, seed=seed + 100, gate=gate)
    f["s0"] = x["s0"]
    return f


def _oracle(f, kind):
    q, k, v = (inputs.to_f32_numpy(f[n]) for n in ("q", "k", "v"))
    a, b, s0 = f["alpha"].numpy(), f["beta"].numpy(), f["s0"].numpy()
    if kind == "vec":
        return oracle.oracle_fwd_vecgate(q, k, v, a, b, s0)
    return oracle.oracle_gla_fwd(q, k, v, a, b, s0)


def _run_steps(f, kind):
    """The chained GPU steps: outputs [N,H,steps,d] and the final state."""
    step = gdn_recurrent_step_vecgate if kind == "vec" else gla_recurrent_step
    state = f["s0"].cuda()
    outs = []
    for t in range(f["q"].shape[2]):
        sl = lambda n: f[n][:, :, t].contiguous().cuda()
        outs.append(step(sl("q"), sl("k"), sl("v"), sl("alpha"), sl("beta"), state))
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2), state


CASES = [
    # kind, d, dtype, gate
    ("vec", 64, "f32", "default"), ("vec", 128, "f32", "slow"), ("vec", 64, "bf16", "resets"),
    ("vec", 128, "bf16", "default"), ("vec", 128, "bf16", "fast"),
    ("gla", 64, "f32", "default"), ("gla", 128, "f32", "slow"), ("gla", 64, "bf16", "resets"),
    ("gla", 128, "bf16", "default"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_d%d_%s_%s" % c)
def test_step_variant_against_oracle(case):
    kind, d, dtype, gate = case
    N, H, steps = 3, 5, 9
    print("case step", case, flush=True)
    f = _draw(N, H, d, steps, dtype, seed=2300 + d, kind=kind, gate=gate)
    ro, rs = _oracle(f, kind)
    o, sT = _run_steps(f, kind)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("kind", ["vec", "gla"])
def test_step_variant_decode_shape(kind):
    """The decode workload's shape (256 sequences x 16 heads, d = 128, bf16,
    state ~ N(0, 0.1)) over 16 steps, every output and the final state."""
    N, H, d, steps = 256, 16, 128, 16
    print("case step decode shape", kind, flush=True)
    f = _draw(N, H, d, steps, "bf16", seed=2400, kind=kind)
    ro, rs = _oracle(f, kind)
    o, sT = _run_steps(f, kind)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S %.3e" % (eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("kind", ["vec", "gla"])
def test_chained_steps_equal_the_chunked_pass(kind):
    """T single-token steps and the chunked forward pass of the same recurrence
    (32-token chunks with a per-dimension gate, 64-token chunks for gated
    linear attention) agree within the bf16 bar."""
    N, H, d, steps = 2, 3, 128, 70
    print("case steps vs chunked", kind, flush=True)
    f = _draw(N, H, d, steps, "bf16", seed=2500, kind=kind)
    o_steps, s_steps = _run_steps(f, kind)
    dev = {n: f[n].cuda() for n in ("q", "k", "v", "alpha", "beta", "s0")}
    fwd = gdn_chunk_fwd_vecgate if kind == "vec" else gla_chunk_fwd
    o, sT = fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["s0"])
    torch.cuda.synchronize()
    assert maxrel(to_np(o_steps), to_np(o)) <= TOL["bf16"]
    assert maxrel(to_np(s_steps), to_np(sT)) <= TOL["bf16"]


def test_vecgate_step_with_a_uniform_gate_is_the_scalar_step():
    """A per-dimension gate with one value per head is the scalar gate: the two
    steps agree to fp32 rounding (the decay is applied to the row-dot vectors
    instead of the dot products)."""
    N, H, d = 4, 4, 128
    x = inputs.make_decode_inputs(N, H, d, 1, "f32", seed=2600)
    dev = {n: x[n][0].cuda() for n in ("q", "k", "v", "alpha", "beta")}
    avec = dev["alpha"][..., None].expand(N, H, d).contiguous()
    s1, s2 = x["s0"].cuda(), x["s0"].cuda()
    o1 = gdn_recurrent_step(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], s1)
    o2 = gdn_recurrent_step_vecgate(dev["q"], dev["k"], dev["v"], avec, dev["beta"], s2)
    torch.cuda.synchronize()
    assert maxrel(to_np(o2), to_np(o1)) <= 1e-6 and maxrel(to_np(s2), to_np(s1)) <= 1e-6


def test_step_variant_errors():
    N, H, d = 2, 2, 64
    x = inputs.make_decode_inputs(N, H, d, 1, "bf16", seed=2700)
    dev = {n: x[n][0].cuda() for n in ("q", "k", "v", "alpha", "beta")}
    state = x["s0"].cuda()
    with pytest.raises(ValueError):   # a scalar gate where the per-dimension step wants [N,H,dk]
        gdn_recurrent_step_vecgate(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], state)
    # the output may not overlap the state: the library rejects it before launching
    o_alias = state.view(-1)[: N * H * d].view(torch.bfloat16)[: N * H * d].view(N, H, d)
    avec = torch.rand(N, H, d, device="cuda")
    with pytest.raises(GDNError) as ei:
        gdn_recurrent_step_vecgate(dev["q"], dev["k"], dev["v"], avec, dev["beta"], state, o=o_alias)
    assert ei.value.code == 1
    with pytest.raises(GDNError) as ei:
        gla_recurrent_step(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], state, o=o_alias)
    assert ei.value.code == 1
    # the state is untouched by the rejected calls
    assert torch.equal(state.cpu(), x["s0"])
