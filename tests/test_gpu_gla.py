"""GPU parity of gated linear attention without the delta rule
(gla_chunk_fwd, [P3] §2.3) against its fp64 oracle (oracle_gla_fwd), with
the bf16 bar of the main path: max-abs-normwise error <= 2e-2 on o and on
the final state.  Sizes span several chunks with ragged tails, d = 64 and
128, zero and random initial states, and the gate laws of the delta-rule
cases."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import GDNError, gla_chunk_fwd

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, T, d, initial state, gate
    (1, 1, 64, 128, False, "default"),
    # 1 to 3 chunks: the loader's two-chunk lookahead at its boundaries
    (1, 2, 1, 128, True, "default"),
    (1, 2, 128, 64, True, "default"),
    (2, 1, 150, 128, True, "default"),
    (1, 1, 192, 128, False, "default"),
    (2, 2, 65, 128, True, "default"),
    (2, 4, 1000, 128, True, "default"),
    (1, 3, 300, 64, True, "default"),
    (1, 2, 2048, 128, True, "slow"),
    (2, 2, 700, 128, True, "resets"),
    (4, 16, 1024, 128, False, "default"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "s0" if c[4] else "z", c[5]))
def test_gla_against_oracle(case):
    B, H, T, d, init, gate = case
    print("case gla", case, flush=True)
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=300 + T + d, init_state=init, gate=gate)
    xd = to_dev(x)
    o, sT = gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64)
    torch.cuda.synchronize()
    (q, k, v, a, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_gla_fwd(q, k, v, a, b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e" % (eo, es), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_gla_rejects_fp32():
    x = inputs.make_fwd_inputs(1, 1, 64, 64, "f32", seed=1)
    xd = to_dev(x)
    with pytest.raises(GDNError):
        gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, 64)
