"""Reads of LDS that no code wrote.  libgdn_debug.so is the same sources
built with GDN_POISON_LDS=1: every kernel first fills its LDS with a NaN
pattern.  A kernel that read LDS before writing it (a missing initialisation,
or a read that races ahead of the write it should wait for) would then see
NaN where the release build sees leftover data, so every entry point is run
with both builds on the same inputs and the outputs must be finite and equal
bit for bit.  (The kernels use no atomics, so the results are deterministic.)"""
import pytest
import torch

from gated_deltanet_sequence_amd import _build, binding, inputs

from _helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    release = binding.load_library()
    debug = binding.load_library(_build.DEBUG_LIB)
    yield release, debug
    binding._lib = release


def _vec(x, d, seed):
    B, H, T = x["alpha"].shape
    return inputs.make_vec_alpha(B, H, T, d, seed=seed).cuda()


CASES = {
    # name: (B, H, T, d, dtype, call)
    "chunk_d128": (2, 2, 300, 128, "bf16", lambda a, av: binding.gdn_chunk_fwd(*a, 64)),
    "chunk_d64": (1, 2, 200, 64, "bf16", lambda a, av: binding.gdn_chunk_fwd(*a, 64)),
    "chunk_c32": (2, 1, 150, 128, "bf16", lambda a, av: binding.gdn_chunk_fwd(*a, 32)),
    "chunk_fp32": (1, 2, 130, 128, "f32", lambda a, av: binding.gdn_chunk_fwd(*a, 64)),
    "split_d64": (1, 2, 6000, 64, "bf16", lambda a, av: binding.gdn_chunk_fwd_split(*a, 64)),
    "split_d128": (1, 1, 9000, 128, "bf16", lambda a, av: binding.gdn_chunk_fwd_split(*a, 64)),
    "noalloc_split": (1, 2, 6000, 64, "bf16", lambda a, av: binding.gdn_chunk_fwd_split_noalloc(*a, 64)),
    "gla": (2, 2, 300, 128, "bf16", lambda a, av: binding.gla_chunk_fwd(*a, 64)),
    "gla_fp32": (1, 2, 100, 64, "f32", lambda a, av: binding.gla_chunk_fwd(*a, 64)),
    "vecgate": (2, 1, 200, 128, "bf16", lambda a, av: binding.gdn_chunk_fwd_vecgate(*a[:3], av, *a[4:])),
    "vecgate_split": (1, 2, 6000, 64, "bf16",
                      lambda a, av: binding.gdn_chunk_fwd_vecgate_split(*a[:3], av, *a[4:])),
    "vecgate_2pass": (2, 2, 500, 128, "bf16", lambda a, av: binding.gdn_chunk_fwd_vecgate_2pass(*a[:3], av, *a[4:])),
    "vecgate_2pass_split": (1, 2, 6000, 64, "bf16",
                            lambda a, av: binding.gdn_chunk_fwd_vecgate_2pass(*a[:3], av, *a[4:])),
    "scan": (1, 2, 2000, 64, "bf16", lambda a, av: binding.gdn_scan_fwd(*a)),
    "scan_vecgate": (1, 2, 1000, 128, "f32", lambda a, av: binding.gdn_scan_fwd_vecgate(*a[:3], av, *a[4:])),
    "recurrent_short": (4, 4, 20, 128, "bf16", lambda a, av: binding.gdn_recurrent_fwd(*a)),
    "recurrent_long": (1, 2, 200, 64, "bf16", lambda a, av: binding.gdn_recurrent_fwd(*a)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_poisoned_lds_changes_nothing(libs, name):
    B, H, T, d, dtype, call = CASES[name]
    print("case poison", name, flush=True)
    x = to_dev(inputs.make_fwd_inputs(B, H, T, d, dtype, seed=1300 + T, init_state=True))
    av = _vec(x, d, seed=1400 + T)
    a = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"])
    outs = []
    for lib in libs:
        binding._lib = lib
        o, sT = call(a, av)
        torch.cuda.synchronize()
        outs.append((o.clone(), sT.clone()))
    binding._lib = libs[0]
    for t in outs[1]:
        assert torch.isfinite(t).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
