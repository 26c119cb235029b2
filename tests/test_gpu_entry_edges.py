"""Edge cases of the sequence-split, scan, vector-gate (scan and chunked),
GLA (64- and 32-token chunks, bf16 and fp32), fp32 chunked, 32-token chunked
and two-pass per-dimension-gate entry points on the GPU: zero tokens (the final state is the initial one, or zero), no
sequences, fewer tokens than one chunk or block, and a final state that
aliases the initial state.  Results are compared with the fp64 oracles or
with exact expectations."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (gdn_chunk_fwd, gdn_chunk_fwd_split, gdn_chunk_fwd_vecgate,
                                                 gdn_chunk_fwd_vecgate_2pass,
                                                 gdn_scan_fwd, gdn_scan_fwd_vecgate, gla_chunk_fwd)

from _helpers import TOL, maxrel, oracle_inputs, to_dev, to_np

pytestmark = pytest.mark.gpu


def _vec(alpha, d):
    return alpha[..., None].expand(*alpha.shape, d).contiguous()


ENTRIES = {
    "split": lambda xd: gdn_chunk_fwd_split(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64),
    "scan": lambda xd: gdn_scan_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"]),
    "scan_vecgate": lambda xd: gdn_scan_fwd_vecgate(xd["q"], xd["k"], xd["v"], _vec(xd["alpha"], xd["q"].shape[3]),
                                                    xd["beta"], xd["s0"]),
    "gla": lambda xd: gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 64),
    "chunk_vecgate": lambda xd: gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], _vec(xd["alpha"], xd["q"].shape[3]),
                                                      xd["beta"], xd["s0"]),
    "chunk_vecgate_2pass": lambda xd: gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"],
                                                                  _vec(xd["alpha"], xd["q"].shape[3]), xd["beta"],
                                                                  xd["s0"]),
    # chunk_size 32: the 32-token kernel on the bf16 inputs
    "c32": lambda xd: gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 32),
    # the same bf16-rounded inputs as fp32: the fp32 chunked path
    "fp32": lambda xd: gdn_chunk_fwd(xd["q"].float(), xd["k"].float(), xd["v"].float(), xd["alpha"], xd["beta"],
                                     xd["s0"], 64),
    # gated linear attention on the 32-token kernel: chunk_size 32, and fp32
    "gla_c32": lambda xd: gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], 32),
    "gla_fp32": lambda xd: gla_chunk_fwd(xd["q"].float(), xd["k"].float(), xd["v"].float(), xd["alpha"],
                                         xd["beta"], xd["s0"], 64),
}


@pytest.mark.parametrize("name", sorted(ENTRIES))
def test_zero_tokens_keeps_state(name):
    x = inputs.make_fwd_inputs(2, 3, 0, 128, "bf16", seed=61, init_state=True)
    o, sT = ENTRIES[name](to_dev(x))
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 128)
    assert torch.equal(sT.cpu(), x["s0"])
    x["s0"] = None
    o, sT = ENTRIES[name](to_dev(x))
    torch.cuda.synchronize()
    assert torch.count_nonzero(sT).item() == 0


@pytest.mark.parametrize("name", sorted(ENTRIES))
def test_no_sequences(name):
    x = inputs.make_fwd_inputs(0, 4, 100, 64, "bf16", seed=62, init_state=True)
    o, sT = ENTRIES[name](to_dev(x))
    torch.cuda.synchronize()
    assert o.numel() == 0 and sT.numel() == 0


@pytest.mark.parametrize("name", ["split", "scan", "scan_vecgate", "chunk_vecgate", "chunk_vecgate_2pass", "c32",
                                  "fp32"])
@pytest.mark.parametrize("T", [1, 17, 31, 33, 63])
def test_short_sequences_match_oracle(name, T):
    x = inputs.make_fwd_inputs(1, 2, T, 64, "bf16", seed=63 + T, init_state=True)
    o, sT = ENTRIES[name](to_dev(x))
    torch.cuda.synchronize()
    (q, k, v, a, b), s0 = oracle_inputs(x)
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, s0)
    tol = TOL["f32"] if name == "fp32" else TOL["bf16"]
    assert maxrel(to_np(o), ro) <= tol and maxrel(to_np(sT), rs) <= tol


@pytest.mark.parametrize("name", ["scan", "gla", "chunk_vecgate", "chunk_vecgate_2pass", "c32", "fp32", "gla_c32",
                                  "gla_fp32"])
def test_final_state_aliases_initial_state(name):
    x = inputs.make_fwd_inputs(1, 2, 700, 128, "bf16", seed=64, init_state=True)
    xd = to_dev(x)
    ref_o, ref_s = ENTRIES[name](xd)
    torch.cuda.synchronize()
    s = xd["s0"].clone()
    if name == "scan":
        o, s2 = gdn_scan_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, final_state=s)
    elif name == "gla":
        o, s2 = gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, 64, final_state=s)
    elif name == "chunk_vecgate":
        o, s2 = gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], _vec(xd["alpha"], 128), xd["beta"], s,
                                      final_state=s)
    elif name == "chunk_vecgate_2pass":
        o, s2 = gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], _vec(xd["alpha"], 128), xd["beta"], s,
                                            final_state=s)
    elif name == "c32":
        o, s2 = gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, 32, final_state=s)
    elif name == "gla_c32":
        o, s2 = gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], s, 32, final_state=s)
    elif name == "gla_fp32":
        o, s2 = gla_chunk_fwd(xd["q"].float(), xd["k"].float(), xd["v"].float(), xd["alpha"], xd["beta"], s, 64,
                              final_state=s)
    else:
        o, s2 = gdn_chunk_fwd(xd["q"].float(), xd["k"].float(), xd["v"].float(), xd["alpha"], xd["beta"], s, 64,
                              final_state=s)
    torch.cuda.synchronize()
    assert s2.data_ptr() == s.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


T_MAX = (2 ** 31 - 1) // (128 * 2)  # longest bf16 sequence at d = 128: q, k, v under 2^31 bytes


def test_maximum_sequence_length_tail_matches_oracle():
    """The longest sequence the bf16 path takes at d = 128 (8,388,607 tokens;
    buffer offsets up to 2^31 - 1 bytes), on the plain and the sequence-split
    entry points and at chunk_size 32 (the 32-token kernel).  alpha = 0 at
    token t0 wipes the state (up to the 2^-200 clamp of log2 alpha), so the
    outputs from t0 on and the final state equal the oracle's run over the
    tokens from t0 on, from a zero state."""
    from gated_deltanet_sequence_amd.binding import gdn_chunk_fwd, gdn_chunk_fwd_split
    T, d = T_MAX, 128
    print("case max length T", T, "d", d, flush=True)
    x = inputs.make_fwd_inputs_on_device(1, 1, T, d, seed=71, device="cuda")
    t0 = T - 777
    x["alpha"][0, 0, t0] = 0.0
    tail = {n: x[n][:, :, t0:].contiguous().cpu() for n in ("q", "k", "v", "alpha", "beta")}
    (q, k, v, a, b), _ = oracle_inputs(dict(tail, s0=None))
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, None)
    for name, run in (("plain", lambda: gdn_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], None, 64)),
                      ("split", lambda: gdn_chunk_fwd_split(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                                            None, 64)),
                      ("chunk_size 32", lambda: gdn_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                                              None, 32))):
        print("  entry", name, flush=True)
        o, sT = run()
        torch.cuda.synchronize()
        eo, es = maxrel(to_np(o[:, :, t0:]), ro), maxrel(to_np(sT), rs)
        print("  err o %.3e  err S_T %.3e" % (eo, es), flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
        del o, sT
