"""GPU test of gdn_chunk_fwd_split_noalloc, the allocation-free variant of
the sequence-split entry point (its segment states live in the library's
static per-GPU scratch instead of a caller's workspace).

It is compared, through the C ABI, with gdn_chunk_fwd_split on the same
inputs: both run the same kernels with the same segment plan, so the outputs
must be bit-identical.  Two split calls run in a row, the second with a
smaller plan, so stale scratch contents of the first call must not leak into
the second; a third call plans no split and must equal gdn_chunk_fwd.
"""
import pytest
import torch

from gated_deltanet_sequence_amd import inputs
from gated_deltanet_sequence_amd.binding import (SPLIT_NOALLOC_SCRATCH_BYTES, gdn_chunk_fwd,
                                                 gdn_chunk_fwd_split, gdn_chunk_fwd_split_noalloc,
                                                 gdn_chunk_fwd_split_workspace)

pytestmark = pytest.mark.gpu

# (B, H, T, d, S0): the long-context shape (the largest plan: 7 MiB of scratch on
# 256 CUs), then the pages' loop case (3 MiB), then enough sequences that no split
# is planned.
CASES = [(1, 16, 131072, 128, True), (1, 4, 8192, 64, False), (8, 16, 1024, 128, True)]


def _inputs(B, H, T, d, s0, seed, dev):
    x = inputs.make_fwd_inputs_on_device(B, H, T, d, seed, dev)
    if s0:
        g = torch.Generator(device=dev)
        g.manual_seed(seed + 1)
        x["s0"] = 0.1 * torch.randn((B, H, d, d), generator=g, device=dev, dtype=torch.float32)
    return x


def test_noalloc_split_matches_the_workspace_split_on_consecutive_calls():
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    for i, (B, H, T, d, s0) in enumerate(CASES):
        print("noalloc case", i, (B, H, T, d, s0), flush=True)
        need = gdn_chunk_fwd_split_workspace(B, H, T, d, d, 64, torch.bfloat16)
        assert need <= SPLIT_NOALLOC_SCRATCH_BYTES
        if i < 2:
            assert need > 0, "the case must plan a split"
        else:
            assert need == 0, "the case must plan no split"
        x = _inputs(B, H, T, d, s0, 100 + i, dev)
        a = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"], 64)
        o1 = torch.full((B, H, T, d), float("nan"), dtype=torch.bfloat16, device=dev)
        s1 = torch.full((B, H, d, d), float("nan"), dtype=torch.float32, device=dev)
        gdn_chunk_fwd_split_noalloc(*a, o=o1, final_state=s1, stream=stream)
        torch.cuda.synchronize()
        if need > 0:
            o2, s2 = gdn_chunk_fwd_split(*a, stream=stream)
        else:
            o2, s2 = gdn_chunk_fwd(*a, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), "case %d: o differs" % i
        assert torch.equal(s1, s2), "case %d: final state differs" % i
        del x, o1, s1, o2, s2
        torch.cuda.empty_cache()


def test_noalloc_split_replays_from_a_captured_graph():
    """Callers that cannot allocate include code under graph capture.  The
    allocation-free split is captured into a HIP graph once and replayed three
    times; between the replays an eager call with another plan overwrites the
    shared scratch and the outputs are poisoned.  Every replay must equal the
    eager call bit for bit (nothing in the scratch has to start at zero)."""
    dev = torch.device("cuda:0")
    B, H, T, d = 1, 4, 8192, 64           # the pages' loop case: a 16-segment plan
    assert gdn_chunk_fwd_split_workspace(B, H, T, d, d, 64, torch.bfloat16) > 0
    x = _inputs(B, H, T, d, True, 200, dev)
    a = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"], 64)
    o_ref = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    s_ref = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    gdn_chunk_fwd_split_noalloc(*a, o=o_ref, final_state=s_ref)   # eager; also looks up the scratch
    torch.cuda.synchronize()
    # another plan that writes the same scratch between the replays
    y = _inputs(1, 2, 16384, 128, True, 201, dev)
    b = (y["q"], y["k"], y["v"], y["alpha"], y["beta"], y["s0"], 64)
    assert gdn_chunk_fwd_split_workspace(1, 2, 16384, 128, 128, 64, torch.bfloat16) > 0
    o_y = torch.empty((1, 2, 16384, 128), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((1, 2, 128, 128), dtype=torch.float32, device=dev)

    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn_chunk_fwd_split_noalloc(*a, o=o, final_state=s)
    torch.cuda.synchronize()
    for rep in range(3):
        print("graph replay", rep, flush=True)
        o.fill_(float("nan"))
        s.fill_(float("nan"))
        gdn_chunk_fwd_split_noalloc(*b, o=o_y, final_state=s_y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d: o differs" % rep
        assert torch.equal(s, s_ref), "replay %d: final state differs" % rep
