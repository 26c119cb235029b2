"""GPU parity of the sequence-split forward pass (gdn_chunk_fwd_split)
against the fp64 oracle, with the same bar as the plain pass: max-abs-
normwise error <= 2e-2 for bf16 inputs, on o and on the final state.

The split runs each sequence as G segments: first the state from zero and
the transition matrix of each of the first G-1 segments, then the start
state of every segment, then every segment from its start state.  These
cases check that G > 1 really happens (non-zero workspace), cover d = 64 and
128, ragged tails, an initial state, aliasing of the final and initial
state, the fallback to the plain pass, and the long-context workload.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (GDNError, gdn_chunk_fwd, gdn_chunk_fwd_split,
                                                 gdn_chunk_fwd_split_workspace)

from _helpers import grouped_oracle_errors, TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def run_split(x, **kw):
    xd = to_dev(x)
    o, sT = gdn_chunk_fwd_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64, **kw)
    torch.cuda.synchronize()
    return o, sT


def run_plain(x):
    xd = to_dev(x)
    o, sT = gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64)
    torch.cuda.synchronize()
    return o, sT


def workspace(x):
    B, H, T, d = x["q"].shape
    return gdn_chunk_fwd_split_workspace(B, H, T, d, x["v"].shape[3], 64, x["q"].dtype)


def check_split_against_oracle(x, chains=None, label=""):
    _say("case split", label, "shape", tuple(x["q"].shape), "workspace", workspace(x))
    o, sT = run_split(x)
    (q, k, v, a, b), s0 = oracle_inputs(x, chains)
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, s0)
    go, gs = to_np(o), to_np(sT)
    if chains is not None:
        go = go.reshape((-1,) + go.shape[2:])[chains][None]
        gs = gs.reshape((-1,) + gs.shape[2:])[chains][None]
    eo, es = maxrel(go, ro), maxrel(gs, rs)
    _say("  err o %.3e  err S_T %.3e" % (eo, es))
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gs))
    assert eo <= TOL["bf16"], "output error %.3e" % eo
    assert es <= TOL["bf16"], "final-state error %.3e" % es


SPLIT_CASES = [
    # B, H, T, d, initial state, gate
    (1, 2, 3000, 128, True, "default"),
    (1, 1, 1600, 128, False, "default"),   # T/512 = 3 segments: the smallest split
    (1, 3, 2000, 64, False, "default"),
    (2, 1, 2500, 64, True, "slow"),        # long memory: the start states matter
    (1, 2, 4096, 128, True, "resets"),
    # the start-state walk runs whole groups of 4 (d = 64) or 3 (d = 128)
    # segments, then the rest: one group and a rest of 3, groups and no rest
    (1, 1, 4096, 64, True, "slow"),        # G = 8
    (1, 1, 4608, 64, False, "default"),    # G = 9
    (1, 1, 3584, 128, True, "slow"),       # G = 7
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "s0" if c[4] else "z", c[5]))
def test_split_small(case):
    B, H, T, d, init, gate = case
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=200 + T + d, init_state=init, gate=gate)
    assert workspace(x) > 0, "the split did not engage"
    check_split_against_oracle(x, label="small")


def test_split_matches_plain_pass():
    x = inputs.make_fwd_inputs(1, 2, 3000, 128, "bf16", seed=31, init_state=True, gate="slow")
    o1, s1 = run_split(x)
    o2, s2 = run_plain(x)
    eo = maxrel(to_np(o1), to_np(o2).astype(np.float64))
    es = maxrel(to_np(s1), to_np(s2).astype(np.float64))
    _say("  split vs plain: o %.3e  S_T %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_split_final_state_aliases_initial_state():
    x = inputs.make_fwd_inputs(1, 2, 2000, 128, "bf16", seed=32, init_state=True)
    ref_o, ref_s = run_split(x)
    xd = to_dev(x)
    s = xd["s0"].clone()
    o, s2 = gdn_chunk_fwd_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, 64,
                                final_state=s)
    torch.cuda.synchronize()
    assert s2.data_ptr() == s.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


def test_split_falls_back_to_plain_pass():
    x = inputs.make_fwd_inputs(8, 8, 512, 128, "bf16", seed=33, init_state=True)
    assert workspace(x) == 0
    o1, s1 = run_split(x)
    o2, s2 = run_plain(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("d", [64, 128])
def test_split_fp32_takes_plain_pass(d):
    """fp32 inputs are never split: the split entry point is gdn_chunk_fwd."""
    x = inputs.make_fwd_inputs(1, 2, 3000, d, "f32", seed=35 + d, init_state=True)
    assert workspace(x) == 0
    o1, s1 = run_split(x)
    o2, s2 = run_plain(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_split_rejects_small_workspace():
    x = inputs.make_fwd_inputs(1, 2, 3000, 128, "bf16", seed=34)
    need = workspace(x)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(GDNError):
        run_split(x, workspace=ws)


def test_config_long_split_full():
    """The long-context workload through the split entry point: every
    sequence against the oracle (four sequences at a time)."""
    c = dict(inputs.CONFIGS["long"])
    x = inputs.make_fwd_inputs(c["B"], c["H"], c["T"], c["d"], c["dtype"], seed=c["seed"],
                               init_state=c["init_state"])
    assert workspace(x) > 0
    _say("case split long, all 16 sequences, workspace", workspace(x))
    o, sT = run_split(x)
    eo, es = grouped_oracle_errors(x, to_np(o), to_np(sT))
    _say("  err o %.3e  err S_T %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_config_loop_split():
    """The pages' loop case (B=1, H=4, T=8192, d=64) in full through the split
    entry point, as timed by the benchmark (16 segments of 512 tokens)."""
    c = dict(inputs.CONFIGS["loop"])
    x = inputs.make_fwd_inputs(c["B"], c["H"], c["T"], c["d"], c["dtype"], seed=c["seed"],
                               init_state=c["init_state"])
    assert workspace(x) > 0
    check_split_against_oracle(x, label="loop")


def _plan(nseq, T, dv, ncu):
    """The segment plan as documented for gdn_chunk_fwd_split: the most
    segments whose first launch (2 (G-1) chains of dv/32 workgroups per
    sequence) fits the CUs in one wave, each at least 512 tokens, in
    multiples of 64 tokens; fewer than 3 segments means no split."""
    g = min(1 + ncu // (2 * nseq * (dv // 32)), T // 512)
    if g < 3:
        return 1
    L = ((T + g - 1) // g + 63) // 64 * 64
    G = (T + L - 1) // L
    return G if G >= 3 else 1


@pytest.mark.parametrize("shape", [(1, 1, 1100, 128), (1, 1, 1535, 128), (1, 1, 1536, 128), (1, 1, 1600, 128),
                                   (1, 16, 131072, 128), (1, 4, 8192, 64), (2, 16, 8192, 128), (4, 16, 8192, 128),
                                   (1, 8, 16384, 64), (1, 2, 32768, 128)])
def test_split_plan_and_workspace(shape):
    B, H, T, d = shape
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    G = _plan(B * H, T, d, ncu)
    want = 0 if G == 1 else (2 * (G - 1) + G) * B * H * d * d * 4
    got = gdn_chunk_fwd_split_workspace(B, H, T, d, d, 64, torch.bfloat16)
    _say("  plan", shape, "CUs", ncu, "G", G, "workspace", got)
    assert got == want
