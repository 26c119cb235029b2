"""GPU parity of the delta rule with a per-dimension gate on the key columns
(gdn_scan_fwd_vecgate, scan route; gdn_chunk_fwd_vecgate, chunked route)
against its fp64 oracle (oracle_fwd_vecgate), with the workloads' bars
(2e-2 bf16, 1e-4 fp32, max-abs-normwise on o and the final state).

Gates: alpha_t[j] = exp(-softplus(z)) drawn per token and key dimension from
the seeded generator (the scalar-gate law of the workloads, per dimension);
one case with a uniform gate must also match the scalar-gate route."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (GDNError, gdn_chunk_fwd, gdn_chunk_fwd_vecgate,
                                                 gdn_chunk_fwd_vecgate_split,
                                                 gdn_chunk_fwd_vecgate_split_workspace, gdn_scan_fwd,
                                                 gdn_scan_fwd_vecgate)

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu


def vec_alpha(B, H, T, d, seed, slow=False):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, H, T, d)).astype(np.float64)
    sp = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    return torch.from_numpy(np.exp(-(0.01 if slow else 1.0) * sp).astype(np.float32)).contiguous()


CASES = [
    # B, H, T, d, dtype, initial state, slow gates
    (1, 1, 50, 64, "f32", True, False),
    (1, 2, 1200, 64, "f32", True, True),
    (2, 1, 900, 128, "f32", False, False),
    (1, 3, 2000, 128, "bf16", True, True),
    (2, 2, 1500, 64, "bf16", True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "s0" if c[5] else "z", "slow" if c[6] else "default"))
def test_vecgate_against_oracle(case):
    B, H, T, d, dtype, init, slow = case
    print("case vecgate", case, flush=True)
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=500 + T + d, init_state=init)
    x["alpha"] = vec_alpha(B, H, T, d, seed=600 + T, slow=slow)
    xd = to_dev(x)
    o, sT = gdn_scan_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    (q, k, v, _, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(to_np(o)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_uniform_vecgate_matches_scalar_gate():
    x = inputs.make_fwd_inputs(1, 2, 1000, 128, "f32", seed=51, init_state=True)
    xd = to_dev(x)
    av = xd["alpha"][..., None].expand(-1, -1, -1, 128).contiguous()
    o1, s1 = gdn_scan_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"], xd["s0"])
    o2, s2 = gdn_scan_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# Chunked route (32-token chunks).  Gates per dimension with the gate laws
# of the workloads: default, slow (long memory), fast (every chunk decays
# below 2^-100 in some column: the exact element-wise products) and resets
# (a gate of 0 in ~1 % of the entries: the exact path for the chunks that
# hold one).
CHUNK_CASES = [
    # B, H, T, d, initial state, gate, dtype
    (1, 1, 1, 128, True, "default", "bf16"),
    (1, 2, 31, 64, False, "default", "bf16"),
    (2, 1, 33, 128, True, "default", "bf16"),
    (1, 3, 1000, 64, True, "default", "bf16"),
    (2, 2, 777, 128, True, "slow", "bf16"),
    (1, 2, 2048, 128, True, "slow", "bf16"),
    (1, 2, 300, 128, True, "fast", "bf16"),
    (2, 1, 500, 64, True, "resets", "bf16"),
    (1, 2, 640, 128, False, "resets", "bf16"),
    (8, 1, 256, 128, True, "default", "bf16"),   # 8 sequences: XCD-grouped mapping
    (1, 1, 50, 64, True, "default", "f32"),
    (2, 1, 900, 128, False, "default", "f32"),
    (1, 2, 1200, 64, True, "slow", "f32"),
    (1, 2, 300, 128, True, "fast", "f32"),
    (1, 2, 640, 128, True, "resets", "f32"),
]


def run_chunk_vec(x):
    xd = to_dev(x)
    o, sT = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    return o, sT


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], "s0" if c[4] else "z", c[5], c[6]))
def test_chunked_vecgate_against_oracle(case):
    B, H, T, d, init, gate, dtype = case
    print("case chunked vecgate", case, flush=True)
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=700 + T + d, init_state=init)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=800 + T, gate=gate)
    o, sT = run_chunk_vec(x)
    (q, k, v, _, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_chunked_vecgate_main_shape():
    """The main workload's shape (B=4, H=16, T=8192, d=128) with a per-
    dimension default gate, every output and the final state."""
    B, H, T, d = 4, 16, 8192, 128
    print("case chunked vecgate main shape", flush=True)
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=3)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=33)
    o, sT = run_chunk_vec(x)
    (q, k, v, _, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e" % (eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_chunked_uniform_vecgate_matches_scalar_gate():
    """A gate that is the same in every key column is the scalar gate: the
    chunked vector-gate route against the scalar chunked route (both bf16,
    different chunk sizes and decay bookkeeping: equal within the bar)."""
    x = inputs.make_fwd_inputs(2, 2, 700, 128, "bf16", seed=52, init_state=True)
    xd = to_dev(x)
    av = xd["alpha"][..., None].expand(-1, -1, -1, 128).contiguous()
    o1, s1 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"], xd["s0"])
    o2, s2 = gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64)
    torch.cuda.synchronize()
    assert maxrel(to_np(o1), to_np(o2)) <= TOL["bf16"] and maxrel(to_np(s1), to_np(s2)) <= TOL["bf16"]


def test_chunked_vecgate_rejects_other_chunk_sizes():
    for dtype in ("f32", "bf16"):
        x = inputs.make_fwd_inputs(1, 1, 64, 64, dtype, seed=1)
        x["alpha"] = inputs.make_vec_alpha(1, 1, 64, 64, seed=2)
        xd = to_dev(x)
        for C in (16, 64):
            with pytest.raises(GDNError):
                gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, C)


def test_chunked_uniform_vecgate_matches_scalar_gate_fp32():
    """fp32 at d = 128: the scalar-gate path runs the same 32-token kernel
    with one gate per token, the vector-gate path with that gate repeated over
    the key columns; the decay tables hold the same values, so the two agree
    bit for bit."""
    x = inputs.make_fwd_inputs(2, 2, 500, 128, "f32", seed=53, init_state=True)
    xd = to_dev(x)
    av = xd["alpha"][..., None].expand(-1, -1, -1, 128).contiguous()
    o1, s1 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"], xd["s0"])
    o2, s2 = gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# Sequence split of the chunked vector-gate route: few sequences, long
# enough for at least three segments (the workspace query says whether the
# split engages).  Against the oracle, at the bars above.
SPLIT_CASES = [
    # B, H, T, d, dtype, initial state, gate
    (1, 8, 16384, 64, "bf16", False, "default"),   # the pages' route-comparison shape
    (1, 2, 8192, 128, "bf16", True, "slow"),
    (2, 1, 3000, 128, "bf16", True, "fast"),
    (1, 2, 4096, 64, "f32", True, "resets"),
    (1, 1, 2000, 128, "f32", True, "default"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "s0" if c[5] else "z", c[6]))
def test_chunked_vecgate_split_against_oracle(case):
    B, H, T, d, dtype, init, gate = case
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=900 + T + d, init_state=init)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=950 + T, gate=gate)
    ws = gdn_chunk_fwd_vecgate_split_workspace(B, H, T, d, d, 32, x["q"].dtype)
    print("case chunked vecgate split", case, "workspace", ws, flush=True)
    assert ws > 0, "the split is expected to engage for this shape"
    xd = to_dev(x)
    o, sT = gdn_chunk_fwd_vecgate_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    (q, k, v, _, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
    print("  err o %.3e  err S_T %.3e (tol %.0e)" % (eo, es, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_chunked_vecgate_split_falls_back_and_aliases():
    """With many sequences no split is planned (workspace 0) and the entry
    point is the plain chunked route, bit for bit; a final state aliasing the
    initial state gives the same result as separate buffers."""
    x = inputs.make_fwd_inputs(8, 8, 512, 64, "bf16", seed=71, init_state=True)
    x["alpha"] = inputs.make_vec_alpha(8, 8, 512, 64, seed=72)
    assert gdn_chunk_fwd_vecgate_split_workspace(8, 8, 512, 64, 64, 32, torch.bfloat16) == 0
    xd = to_dev(x)
    o1, s1 = gdn_chunk_fwd_vecgate_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    o2, s2 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)

    y = inputs.make_fwd_inputs(1, 2, 6000, 64, "bf16", seed=73, init_state=True)
    y["alpha"] = inputs.make_vec_alpha(1, 2, 6000, 64, seed=74)
    assert gdn_chunk_fwd_vecgate_split_workspace(1, 2, 6000, 64, 64, 32, torch.bfloat16) > 0
    yd = to_dev(y)
    ref_o, ref_s = gdn_chunk_fwd_vecgate_split(yd["q"], yd["k"], yd["v"], yd["alpha"], yd["beta"], yd["s0"])
    s = yd["s0"].clone()
    o, s3 = gdn_chunk_fwd_vecgate_split(yd["q"], yd["k"], yd["v"], yd["alpha"], yd["beta"], s, final_state=s)
    torch.cuda.synchronize()
    assert s3.data_ptr() == s.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


def test_chunked_vecgate_split_rejects_small_workspace():
    x = inputs.make_fwd_inputs(1, 2, 6000, 64, "bf16", seed=75)
    x["alpha"] = inputs.make_vec_alpha(1, 2, 6000, 64, seed=76)
    need = gdn_chunk_fwd_vecgate_split_workspace(1, 2, 6000, 64, 64, 32, torch.bfloat16)
    assert need > 0
    xd = to_dev(x)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(GDNError):
        gdn_chunk_fwd_vecgate_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, workspace=ws)
