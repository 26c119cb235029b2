"""GPU parity of the token-by-token forward pass (gdn_recurrent_fwd, and
gdn_recurrent_fwd_vecgate with a per-dimension gate) against the fp64
oracles (oracle_fwd, oracle_fwd_vecgate), max-abs-normwise on o and the final
state with the workloads' bars (2e-2 bf16, 1e-4 fp32): short and ragged
lengths around the 32-token staging tile, few and many (512) sequences,
d = 64 and 128, zero and random initial states, every gate law, the decode
workload's shape with eight new tokens per sequence, a final state aliasing
the initial one, and zero tokens."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import GDNError, gdn_recurrent_fwd, gdn_recurrent_fwd_vecgate

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, T, d, initial state, gate, dtype, per-dimension gate
    (1, 1, 1, 64, False, "default", "f32", False),
    (2, 3, 5, 128, True, "default", "bf16", False),
    (1, 2, 31, 64, True, "slow", "f32", False),
    (2, 2, 33, 128, True, "resets", "bf16", False),
    (1, 3, 100, 64, True, "fast", "bf16", False),
    (1, 2, 1000, 128, True, "default", "f32", False),
    (2, 1, 7, 64, True, "default", "f32", True),
    (1, 2, 65, 128, True, "slow", "bf16", True),
    (2, 2, 300, 64, False, "resets", "bf16", True),
    (1, 1, 500, 128, True, "default", "f32", True),
    # many sequences (512)
    (32, 16, 1, 128, True, "default", "bf16", False),
    (16, 32, 17, 64, True, "slow", "f32", False),
    (64, 8, 40, 128, False, "resets", "f32", False),
    (32, 16, 16, 128, True, "fast", "bf16", True),
    (8, 64, 33, 64, True, "default", "f32", True),
]


def _inputs(B, H, T, d, init, gate, dtype, vec, seed):
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=seed, init_state=init, gate="default" if vec else gate)
    if vec:
        x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=seed + 100, gate=gate)
    return x


def _run(xd, vec, **kw):
    f = gdn_recurrent_fwd_vecgate if vec else gdn_recurrent_fwd
    o, sT = f(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], **kw)
    torch.cuda.synchronize()
    return o, sT


def _oracle(x, vec):
    (q, k, v, a, b), s0 = oracle_inputs(x)
    if vec:
        return oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    return oracle.oracle_fwd(q, k, v, a, b, s0)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s%s" % (
    c[0], c[1], c[2], c[3], "s0" if c[4] else "z", c[5], c[6], "_vec" if c[7] else ""))
def test_recurrent_fwd_against_oracle(case):
    B, H, T, d, init, gate, dtype, vec = case
    print("case recurrent fwd", case, flush=True)
    x = _inputs(B, H, T, d, init, gate, dtype, vec, seed=900 + T + d)
    o, sT = _run(to_dev(x), vec)
    ro, rs = _oracle(x, vec)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_recurrent_fwd_decode_shape_eight_tokens():
    """256 sequences x 16 heads, d = 128, bf16, a state ~ N(0, 0.1) and eight
    new tokens per sequence (e.g. drafted tokens to verify): every output
    and the final state against the oracle."""
    N, H, T, d = 256, 16, 8, 128
    print("case recurrent fwd decode shape", flush=True)
    x = inputs.make_fwd_inputs(N, H, T, d, "bf16", seed=950, init_state=True)
    x["s0"] = x["s0"] * (0.1 / float(x["s0"].std()))
    o, sT = _run(to_dev(x), False)
    ro, rs = _oracle(x, False)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e" % (eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("vec", [False, True])
@pytest.mark.parametrize("heads", [4, 512])
def test_recurrent_fwd_aliasing_and_edges(vec, heads):
    x = _inputs(heads // 2, 2, 77, 128, True, "default", "bf16", vec, seed=960)
    xd = to_dev(x)
    ref_o, ref_s = _run(xd, vec)
    s = xd["s0"].clone()
    f = gdn_recurrent_fwd_vecgate if vec else gdn_recurrent_fwd
    o, s2 = f(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, final_state=s)
    torch.cuda.synchronize()
    assert s2.data_ptr() == s.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
    # no initial state: a zero start
    xz = dict(x, s0=None)
    o, sT = _run(to_dev(xz), vec)
    ro, rs = _oracle(xz, vec)
    assert maxrel(to_np(o), ro) <= TOL["bf16"] and maxrel(to_np(sT), rs) <= TOL["bf16"]
    # zero tokens: the final state is the initial one
    x0 = _inputs(heads // 2, 2, 0, 64, True, "default", "bf16", vec, seed=961)
    o, sT = _run(to_dev(x0), vec)
    assert o.shape == (heads // 2, 2, 0, 64) and torch.equal(sT.cpu(), x0["s0"])
    # no sequences
    xn = _inputs(0, 3, 10, 64, True, "default", "bf16", vec, seed=962)
    o, sT = _run(to_dev(xn), vec)
    assert o.numel() == 0 and sT.numel() == 0


def test_recurrent_fwd_rejects_unsupported_widths():
    x = inputs.make_fwd_inputs(1, 1, 10, 96, "bf16", seed=970)
    xd = to_dev(x)
    with pytest.raises(GDNError) as ei:
        gdn_recurrent_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None)
    assert ei.value.code == 2
