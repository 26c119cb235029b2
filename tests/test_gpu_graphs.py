"""The entry points under HIP graph capture.  The library allocates nothing
and never synchronises, so a caller can capture its launches into a graph and
replay them (a serving loop of decode steps, a fixed-shape forward pass).
Each captured sequence is replayed three times; before every replay the
outputs are poisoned and another eager call runs on other buffers, and every
replay must equal the eager result bit for bit."""
import pytest
import torch

from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (gdn_chunk_fwd, gdn_chunk_fwd_vecgate_2pass,
                                                 gdn_chunk_fwd_vecgate_2pass_workspace, gdn_recurrent_step,
                                                 gla_chunk_fwd)

from _helpers import to_dev

pytestmark = pytest.mark.gpu


def _replay_and_check(g, outs, refs, eager_other):
    for rep in range(3):
        print("  replay", rep, flush=True)
        for t in outs:
            t.fill_(float("nan"))
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), "replay %d differs" % rep


@pytest.mark.parametrize("entry,dtype,C", [("gdn", "bf16", 64), ("gdn", "f32", 64), ("gdn", "bf16", 32),
                                           ("gla", "bf16", 64)])
def test_forward_pass_replays_from_a_graph(entry, dtype, C):
    print("case graph", entry, dtype, C, flush=True)
    fwd = gdn_chunk_fwd if entry == "gdn" else gla_chunk_fwd
    B, H, T, d = 2, 4, 1000, 128
    xd = to_dev(inputs.make_fwd_inputs(B, H, T, d, dtype, seed=810, init_state=True))
    yd = to_dev(inputs.make_fwd_inputs(1, 2, 300, 64, dtype, seed=811, init_state=True))
    a = (xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"], C)
    o_ref, s_ref = fwd(*a)
    torch.cuda.synchronize()
    o, s = torch.empty_like(o_ref), torch.empty_like(s_ref)
    o_y, s_y = torch.empty_like(yd["v"]), torch.empty_like(yd["s0"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(*a, o=o, final_state=s)
    torch.cuda.synchronize()
    _replay_and_check(g, [o, s], [o_ref, s_ref],
                      lambda: fwd(yd["q"], yd["k"], yd["v"], yd["alpha"], yd["beta"], yd["s0"], C, o=o_y,
                                  final_state=s_y))


def test_two_pass_route_replays_from_a_graph():
    """The two-pass per-dimension-gate route with a caller's workspace (its
    records and carried state are rewritten by every call)."""
    B, H, T, d = 1, 2, 3000, 128
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=812, init_state=True)
    x["alpha"] = inputs.make_vec_alpha(B, H, T, d, seed=813)
    xd = to_dev(x)
    ws = torch.empty(gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, d, d, 32, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    a = (xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd["s0"])
    o_ref, s_ref = gdn_chunk_fwd_vecgate_2pass(*a, workspace=ws)
    torch.cuda.synchronize()
    o, s = torch.empty_like(o_ref), torch.empty_like(s_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn_chunk_fwd_vecgate_2pass(*a, o=o, final_state=s, workspace=ws)
    torch.cuda.synchronize()
    # the other call writes the same workspace
    y = inputs.make_fwd_inputs(1, 1, 500, 128, "bf16", seed=814, init_state=True)
    y["alpha"] = inputs.make_vec_alpha(1, 1, 500, 128, seed=815)
    yd = to_dev(y)
    _replay_and_check(g, [o, s], [o_ref, s_ref],
                      lambda: gdn_chunk_fwd_vecgate_2pass(yd["q"], yd["k"], yd["v"], yd["alpha"], yd["beta"],
                                                          yd["s0"], workspace=ws))


def test_decode_loop_replays_from_a_graph():
    """Eight decode steps on one state, captured as one graph: the serving
    loop's launches without per-step host work.  The state is reset (eagerly)
    before each replay; outputs of every step and the final state match the
    eager loop bit for bit."""
    N, H, d, steps = 64, 16, 128, 8
    x = inputs.make_decode_inputs(N, H, d, steps, "bf16", seed=816)
    dev = {n: [t.cuda() for t in x[n]] for n in ("q", "k", "v", "alpha", "beta")}
    s0 = x["s0"].cuda()
    state = s0.clone()
    o_ref = [gdn_recurrent_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["alpha"][t], dev["beta"][t], state)
             for t in range(steps)]
    torch.cuda.synchronize()
    s_ref = state.clone()
    outs = [torch.empty_like(o) for o in o_ref]
    state.copy_(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            gdn_recurrent_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["alpha"][t], dev["beta"][t], state,
                               o=outs[t])
    torch.cuda.synchronize()
    other = s0.clone()

    def reset_and_other():
        state.copy_(s0)
        gdn_recurrent_step(dev["q"][0], dev["k"][0], dev["v"][0], dev["alpha"][0], dev["beta"][0], other)

    _replay_and_check(g, outs, o_ref, reset_and_other)
    assert torch.equal(state, s_ref)
