"""GPU parity of the two-pass chunked route with a per-dimension gate
(gdn_chunk_fwd_vecgate_2pass) against the fp64 oracle (oracle_fwd_vecgate),
with the workloads' bars (2e-2 bf16, 1e-4 fp32, max-abs-normwise on o and
the final state).  fp32 records are walked by the 32-token kernel's own
products in the same order as the single-pass route, so fp32 results match it
bit for bit; bf16 records are walked by the pipelined second pass, whose
MFMA sums run in another order, so bf16 results match it within the bar.  The
tile length (set by the workspace size) does not change the result.  With few
sequences the route splits them into segments (when the workspace holds the
split), which changes the rounding only."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (GDNError, gdn_chunk_fwd_vecgate, gdn_chunk_fwd_vecgate_2pass,
                                                 gdn_chunk_fwd_vecgate_2pass_workspace)

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, T, d, initial state, gate, dtype
    (1, 1, 1, 128, True, "default", "bf16"),
    (1, 2, 31, 64, False, "default", "bf16"),
    (2, 1, 33, 128, True, "default", "bf16"),
    (1, 3, 1000, 64, True, "default", "bf16"),
    (2, 2, 777, 128, True, "slow", "bf16"),
    (1, 2, 12000, 128, True, "slow", "bf16"),   # 375 chunks: split, and unsplit two tiles of at most 256
    (1, 2, 300, 128, True, "fast", "bf16"),
    (2, 1, 2500, 64, True, "resets", "bf16"),
    (8, 1, 256, 128, True, "default", "bf16"),  # 8 sequences: XCD-grouped mapping
    # enough value slices to fill the device twice: two slices per workgroup
    # of the second pass
    (8, 8, 100, 128, True, "default", "bf16"),
    (8, 16, 70, 64, True, "resets", "bf16"),
    # more slices than the device holds at two per workgroup: four value
    # slices per workgroup of the bf16 second pass (128 sequences at d = 128,
    # 512 at d = 64 on a 256-CU device)
    (8, 16, 100, 128, True, "slow", "bf16"),
    (16, 32, 40, 64, False, "fast", "bf16"),
    (8, 8, 40, 128, True, "default", "f32"),
    (1, 1, 50, 64, True, "default", "f32"),
    (2, 1, 2100, 128, False, "default", "f32"),
    (1, 2, 1200, 64, True, "slow", "f32"),
    (1, 2, 640, 128, True, "resets", "f32"),
    # few long sequences: sequence split where the device plans one
    (1, 2, 6000, 64, True, "default", "bf16"),
    (1, 1, 9000, 128, True, "slow", "bf16"),
    (2, 1, 4000, 64, False, "fast", "f32"),
    (1, 2, 3333, 128, True, "resets", "f32"),
]


def _inputs(B, H, T, d, dtype, init, gate, seed):
    x = inputs.make_fwd_inputs(B, H, T, d, dtype, seed=seed, init_state=init)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=seed + 100, gate=gate)
    return x


def _record_bytes(d, dtype=torch.bfloat16):
    # the workspace of one sequence and one chunk: the carried state and one record
    return gdn_chunk_fwd_vecgate_2pass_workspace(1, 1, 32, d, d, 32, dtype) - d * d * 4


def _tiled_bytes(B, H, T, d, dtype):
    """Workspace of the tiled (unsplit) plan; the query returns more exactly
    when a sequence split is planned."""
    nch = (T + 31) // 32
    return B * H * (d * d * 4 + max(1, min(nch, 256)) * _record_bytes(d, dtype))


def _run2(xd, **kw):
    o, sT = gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], **kw)
    torch.cuda.synchronize()
    return o, sT


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%dd%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], "s0" if c[4] else "z", c[5], c[6]))
def test_2pass_against_oracle_and_single_pass(case):
    B, H, T, d, init, gate, dtype = case
    print("case vecgate 2pass", case, flush=True)
    x = _inputs(B, H, T, d, dtype, init, gate, seed=1700 + T + d)
    xd = to_dev(x)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tiled = _tiled_bytes(B, H, T, d, tdt)
    split = gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, d, d, 32, tdt) > tiled
    (q, k, v, _, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd_vecgate(q, k, v, x["alpha"].numpy(), b, s0)
    o1, s1 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    # the planned route (a split where planned), then the tiled plan
    for ws_bytes in ([None, tiled] if split else [None]):
        ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        o, sT = _run2(xd, workspace=ws)
        eo, es = maxrel(to_np(o), ro), maxrel(to_np(sT), rs)
        print("  %s: err o %.3e  err S_T %.3e (tol %.0e)" % ("split" if split and ws is None else "tiles", eo, es,
                                                             TOL[dtype]), flush=True)
        assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(sT)))
        assert eo <= TOL[dtype] and es <= TOL[dtype]
        if not (split and ws is None):
            if dtype == "f32":
                assert torch.equal(o, o1) and torch.equal(sT, s1)
            else:
                assert maxrel(to_np(o), to_np(o1)) <= TOL[dtype] and maxrel(to_np(sT), to_np(s1)) <= TOL[dtype]


def test_2pass_tile_length_does_not_change_the_result():
    """Workspaces for tiles of 1, 3, 64 and 94 chunks (B=2, H=2, T=3000: 94 chunks)
    give the same outputs and final state bit for bit; the state passes from
    tile to tile through the workspace in fp32."""
    B, H, T, d = 2, 2, 3000, 128
    x = _inputs(B, H, T, d, "bf16", True, "default", seed=1901)
    xd = to_dev(x)
    rec = _record_bytes(d)
    ref = None
    for tile in (1, 3, 64, 94):
        ws = torch.empty(B * H * (d * d * 4 + tile * rec), dtype=torch.uint8, device="cuda")
        print("  tile", tile, "workspace", ws.numel(), flush=True)
        o, sT = _run2(xd, workspace=ws)
        if ref is None:
            ref = (o.clone(), sT.clone())
        else:
            assert torch.equal(o, ref[0]) and torch.equal(sT, ref[1])


def test_2pass_main_shape_matches_single_pass():
    """The main workload's shape (B=4, H=16, T=8192, d=128, bf16, per-dimension
    default gate): the single-pass route, which is checked against the oracle
    on every output by the single-pass suite, within the bf16 bar (the
    pipelined second pass sums in another order)."""
    B, H, T, d = 4, 16, 8192, 128
    print("case vecgate 2pass main shape", flush=True)
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=3)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=33)
    xd = to_dev(x)
    o, sT = _run2(xd)
    o1, s1 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    torch.cuda.synchronize()
    # max-abs-normwise, on the GPU (2^28 outputs)
    def rel(a, b):
        return float((a.float() - b.float()).abs().max() / b.float().abs().max())

    eo, es = rel(o, o1), rel(sT, s1)
    print("  two-pass vs single-pass: o %.3e  S_T %.3e" % (eo, es), flush=True)
    assert bool(torch.isfinite(o).all()) and eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_2pass_aliasing_and_errors():
    x = _inputs(1, 2, 2500, 64, "bf16", True, "default", seed=1911)
    xd = to_dev(x)
    # the planned route (a split on a GPU with enough CUs) and the tiled one
    for ws_bytes in (None, _tiled_bytes(1, 2, 2500, 64, torch.bfloat16)):
        ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        ref_o, ref_s = _run2(xd, workspace=ws)
        s = xd["s0"].clone()
        o, s2 = gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, final_state=s,
                                            workspace=ws)
        torch.cuda.synchronize()
        assert s2.data_ptr() == s.data_ptr()
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
    rec = _record_bytes(64)
    small = torch.empty(2 * (64 * 64 * 4 + rec) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(GDNError) as ei:
        gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, workspace=small)
    assert ei.value.code == 1
    with pytest.raises(GDNError) as ei:
        gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, 64)
    assert ei.value.code == 2
