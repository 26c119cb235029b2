"""GPU parity of the parallel-scan route (gdn_scan_fwd) against the fp64
oracle of the same recurrence, with the workloads' bars: max-abs-normwise
error <= 2e-2 for bf16 inputs and <= 1e-4 for fp32 inputs, on o and on the
final state.  Cases cover one block (no scan) and many, ragged tails,
d = 64 and 128 in both dtypes, initial states, slow and reset gates, the
tiny and loop workloads in full, and agreement with the chunked route."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (GDNError, gdn_chunk_fwd, gdn_scan_fwd,
                                                 gdn_scan_fwd_workspace)

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_scan(x, **kw):
    xd = to_dev(x)
    o, sT = gdn_scan_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], **kw)
    torch.cuda.synchronize()
    return o, sT


def check(x, dtype, label):
    print("case scan", label, tuple(x["q"].shape), dtype, flush=True)
    o, sT = run_scan(x)
    (q, k, v, a, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


CASES = [
    # B, H, T, d, dtype, initial state, gate
    (1, 1, 40, 64, "f32", True, "default"),       # shorter than one block
    (1, 2, 1000, 64, "f32", True, "default"),
    (2, 1, 777, 128, "f32", True, "slow"),
    (1, 3, 1500, 64, "bf16", False, "default"),
    (2, 2, 2100, 128, "bf16", True, "resets"),
    (1, 2, 3000, 128, "bf16", True, "beta2"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "s0" if c[5] else "z", c[6]))
def test_scan_against_oracle(case):
    B, H, T, d, dtype, init, gate = case
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=400 + T + d, init_state=init, gate=gate)
    check(x, dtype, "small")


def test_scan_config_tiny():
    c = dict(inputs.CONFIGS["tiny"])
    x = inputs.make_fwd_inputs(c["B"], c["H"], c["T"], c["d"], c["dtype"], seed=c["seed"],
                               init_state=c["init_state"])
    check(x, c["dtype"], "tiny")


def test_scan_config_loop():
    c = dict(inputs.CONFIGS["loop"])
    x = inputs.make_fwd_inputs(c["B"], c["H"], c["T"], c["d"], c["dtype"], seed=c["seed"],
                               init_state=c["init_state"])
    check(x, c["dtype"], "loop")


def test_scan_matches_chunked_route():
    x = inputs.make_fwd_inputs(2, 2, 2000, 128, "bf16", seed=41, init_state=True, gate="slow")
    o1, s1 = run_scan(x)
    xd = to_dev(x)
    o2, s2 = gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64)
    torch.cuda.synchronize()
    assert maxrel(to_np(o1), to_np(o2).astype(np.float64)) <= TOL["bf16"]
    assert maxrel(to_np(s1), to_np(s2).astype(np.float64)) <= TOL["bf16"]


def test_scan_rejects_small_workspace():
    x = inputs.make_fwd_inputs(1, 1, 500, 64, "f32", seed=42)
    need = gdn_scan_fwd_workspace(1, 1, 500, 64, 64, torch.float32)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(GDNError):
        run_scan(x, workspace=ws)
