"""The grouped oracle comparison used by the long-context GPU tests, on the
CPU: run group by group, it must give exactly the whole-tensor max-abs-
normwise errors (numerator and denominator maxed over all chains)."""
import numpy as np

import oracle
from gated_deltanet_sequence_amd import inputs

from _helpers import grouped_oracle_errors, maxrel, oracle_inputs


def test_grouped_errors_equal_the_whole_tensor_errors():
    x = inputs.make_fwd_inputs(2, 3, 70, 8, "f32", seed=11, init_state=True)
    (q, k, v, a, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, s0)
    rng = np.random.default_rng(0)
    go = ro + 1e-3 * rng.standard_normal(ro.shape)
    gs = rs.copy()
    gs[1, 2, 3, 4] += 0.05          # one planted error in the last chain
    eo, es = grouped_oracle_errors(x, go, gs, group=4)
    assert abs(eo - maxrel(go, ro)) <= 1e-15 * max(1.0, eo)
    assert abs(es - maxrel(gs, rs)) <= 1e-15 * max(1.0, es)
    assert es > 0.0
