"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects every invalid argument with its documented code
before touching the device.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from gated_deltanet_sequence_amd import _build
from gated_deltanet_sequence_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

A = 0x10000          # 16-byte aligned fake device addresses (never dereferenced)
MB = 1 << 20


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gdn|gla)_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if _build.is_stale():
        _build.build()
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"gdn_chunk_fwd", "gdn_recurrent_step", "gdn_strerror", "gdn_version",
                          "gla_chunk_fwd", "gla_recurrent_step", "gdn_recurrent_step_vecgate"}
    for n in names:
        assert hasattr(lib, n), n


def test_debug_build_exports_the_same_functions(lib):
    """libgdn_debug.so (LDS filled with NaN before use, for the GPU check that
    no kernel reads LDS it did not write) is a separate build of the same
    sources with the same exports."""
    debug = binding.load_library(_build.DEBUG_LIB)
    for n in declared_functions():
        assert hasattr(debug, n), n
    assert open(_build.DEBUG_LIB, "rb").read() != open(_build.LIB, "rb").read()


def test_strerror_and_version(lib):
    for code in range(0, 5):
        s = binding.strerror(code)
        assert s and s != "unknown gdn error code"
    assert binding.strerror(99) == "unknown gdn error code"
    assert re.match(r"^\d+\.\d+\.\d+$", binding.version())


def fwd(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, alpha=A + 192 * MB, beta=A + 200 * MB,
        s0=None, o=A + 256 * MB, sT=None, B=1, H=1, T=64, dk=64, dv=64, C=64, dtype=1):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn_chunk_fwd(P(q), P(k), P(v), P(alpha), P(beta), P(s0), P(o), P(sT),
                             B, H, T, dk, dv, C, dtype, None)


STEPS = ["gdn_recurrent_step", "gdn_recurrent_step_vecgate", "gla_recurrent_step"]


def step(lib, q=A, k=A + MB, v=A + 2 * MB, alpha=A + 3 * MB, beta=A + 4 * MB,
         state=A + 8 * MB, o=A + 64 * MB, N=1, H=1, dk=64, dv=64, dtype=1, fn="gdn_recurrent_step"):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(P(q), P(k), P(v), P(alpha), P(beta), P(state), P(o),
                            N, H, dk, dv, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(alpha=None), 1),
    (dict(beta=None), 1), (dict(o=None), 1),
    (dict(B=-1), 1), (dict(H=-2), 1), (dict(T=-1), 1), (dict(C=0), 1), (dict(dtype=7), 1),
    (dict(dk=32, dv=32), 2), (dict(dk=64, dv=128), 2), (dict(dk=256, dv=256), 2),
    (dict(C=16), 2), (dict(C=48), 2), (dict(C=128), 2),
    (dict(q=A + 8), 3), (dict(v=A + 128 * MB + 2), 3), (dict(o=A + 256 * MB + 4), 3),
    (dict(s0=A + 300 * MB + 8), 3), (dict(sT=A + 400 * MB + 12), 3),
    (dict(o=A + 112), 1),                  # output overlaps q
    (dict(o=A + 192 * MB), 1),             # output overlaps alpha
    (dict(sT=A + 256 * MB + 16), 1),       # final state overlaps the output
    (dict(sT=A + 64 * MB), 1),             # final state overlaps k
    (dict(sT=A + 192 * MB + 16), 1),       # final state overlaps alpha
    (dict(s0=A + 300 * MB, sT=A + 300 * MB + 16), 1),   # final state partly overlaps the initial state
])
def test_chunk_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def gla(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, alpha=A + 192 * MB, beta=A + 200 * MB,
        s0=None, o=A + 256 * MB, sT=None, B=1, H=1, T=64, dk=64, dv=64, C=64, dtype=1):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_chunk_fwd(P(q), P(k), P(v), P(alpha), P(beta), P(s0), P(o), P(sT),
                             B, H, T, dk, dv, C, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(beta=None), 1), (dict(T=-1), 1), (dict(dtype=7), 1),
    (dict(dk=32, dv=32), 2), (dict(C=16), 2), (dict(C=48), 2), (dict(C=128), 2), (dict(C=48, dtype=0), 2),
    (dict(q=A + 8), 3), (dict(sT=A + 400 * MB + 12, C=32), 3), (dict(dtype=0, o=A + 256 * MB + 4), 3),
    (dict(o=A + 112, C=32), 1), (dict(sT=A + 256 * MB + 16, dtype=0), 1),
])
def test_gla_chunk_fwd_rejects(lib, kw, code):
    """gla_chunk_fwd validates as gdn_chunk_fwd, for both kernels (64-token
    bf16; fp32 and chunk_size 32)."""
    assert gla(lib, **kw) == code


def rec_fwd(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, alpha=A + 192 * MB, beta=A + 200 * MB,
            s0=None, o=A + 256 * MB, sT=None, B=1, H=1, T=64, dk=64, dv=64, dtype=1, fn="gdn_recurrent_fwd"):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(P(q), P(k), P(v), P(alpha), P(beta), P(s0), P(o), P(sT),
                            B, H, T, dk, dv, dtype, None)


@pytest.mark.parametrize("fn", ["gdn_recurrent_fwd", "gdn_recurrent_fwd_vecgate"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(alpha=None), 1), (dict(T=-1), 1), (dict(dtype=7), 1),
    (dict(dk=96, dv=96), 2), (dict(dk=64, dv=128), 2),
    (dict(k=A + 64 * MB + 8), 3), (dict(sT=A + 400 * MB + 4), 3),
    (dict(o=A + 64 * MB), 1),              # output overlaps k
    (dict(sT=A + 128 * MB), 1),            # final state overlaps v
    (dict(s0=A + 300 * MB, sT=A + 300 * MB + 16), 1),
])
def test_recurrent_fwd_rejects(lib, kw, code, fn):
    assert rec_fwd(lib, fn=fn, **kw) == code


def test_recurrent_fwd_vecgate_checks_the_whole_gate(lib):
    # dk gate floats per token: an output 16 bytes into alpha's 64 * 64 floats overlaps it
    assert rec_fwd(lib, fn="gdn_recurrent_fwd_vecgate", o=A + 192 * MB + 4096) == 1


def test_chunk_fwd_empty_is_noop(lib):
    # no sequences, or no tokens and no state to write: nothing is launched
    assert fwd(lib, B=0) == 0
    assert fwd(lib, B=0, dtype=0, dk=128, dv=128) == 0   # fp32 at d = 128 passes the checks
    assert fwd(lib, H=0) == 0
    assert fwd(lib, T=0, sT=None) == 0
    assert fwd(lib, B=0, q=None, k=None, v=None, alpha=None, beta=None, o=None) == 0


@pytest.mark.parametrize("fn", STEPS)
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(alpha=None), 1), (dict(beta=None), 1), (dict(state=None), 1),
    (dict(o=None), 1), (dict(N=-1), 1), (dict(H=-1), 1),
    (dict(dtype=3), 1), (dict(dk=96, dv=96), 2), (dict(dk=64, dv=128), 2),
    (dict(state=A + 8 * MB + 4), 3), (dict(k=A + MB + 2), 3), (dict(alpha=A + 3 * MB + 8), 3),
    (dict(o=A + 8 * MB), 1),               # output overlaps the state
    (dict(o=A + 2 * MB + 64), 1),          # output overlaps v
    (dict(state=A + MB), 1),               # state overlaps k
    (dict(q=A + 8 * MB + 4096), 1),        # q inside the state
])
def test_recurrent_step_rejects(lib, kw, code, fn):
    assert step(lib, fn=fn, **kw) == code


def test_vecgate_step_checks_the_whole_gate_vector(lib):
    # a per-dimension gate has dk entries per head: an output 16 bytes past the
    # start of alpha overlaps it (a scalar gate would end there)
    assert step(lib, fn="gdn_recurrent_step_vecgate", o=A + 3 * MB + 16) == 1
    assert step(lib, fn="gdn_recurrent_step_vecgate", o=A + 3 * MB + 240) == 1   # last 16 of 256 bytes


@pytest.mark.parametrize("fn", STEPS)
def test_recurrent_step_empty_is_noop(lib, fn):
    assert step(lib, N=0, fn=fn) == 0
    assert step(lib, H=0, q=None, state=None, o=None, fn=fn) == 0


def fwd_split(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, alpha=A + 192 * MB, beta=A + 200 * MB,
              s0=None, o=A + 256 * MB, sT=None, B=1, H=1, T=64, dk=64, dv=64, C=64, dtype=1,
              ws=None, ws_bytes=0):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn_chunk_fwd_split(P(q), P(k), P(v), P(alpha), P(beta), P(s0), P(o), P(sT),
                                   B, H, T, dk, dv, C, dtype, P(ws), ws_bytes, None)


def test_split_rejects_invalid_arguments(lib):
    assert fwd_split(lib, B=-1) == binding.GDN_ERR_INVALID_ARG
    assert fwd_split(lib, dtype=7) == binding.GDN_ERR_INVALID_ARG
    assert fwd_split(lib, q=None) == binding.GDN_ERR_INVALID_ARG
    assert fwd_split(lib, dk=96, dv=96) == binding.GDN_ERR_UNSUPPORTED
    assert fwd_split(lib, C=32) == binding.GDN_ERR_UNSUPPORTED
    assert fwd_split(lib, k=A + 8) == binding.GDN_ERR_ALIGNMENT
    assert fwd_split(lib, o=A) == binding.GDN_ERR_INVALID_ARG  # output overlaps q


def test_split_workspace_query_is_host_only(lib):
    f = lib.gdn_chunk_fwd_split_workspace
    assert f(1, 16, 131072, 128, 128, 64, 0) == 0      # fp32: never split
    assert f(1, 16, 131072, 96, 96, 64, 1) == 0        # unsupported width
    assert f(1, 16, 131072, 128, 128, 32, 1) == 0      # unsupported chunk size
    assert f(0, 16, 131072, 128, 128, 64, 1) == 0      # nothing to do
    assert f(1, 16, 131072, 128, 128, 64, 1) >= 0      # no GPU here: 0; on a GPU: > 0


def test_scan_rejects_invalid_arguments_and_sizes_workspace(lib):
    P = lambda x: None if x is None else ctypes.c_void_p(x)

    def scan(B=1, H=1, T=64, dk=64, dv=64, dtype=1, q=A, o=A + 256 * MB, ws=A + 512 * MB, wsb=0):
        return lib.gdn_scan_fwd(P(q), P(A + 64 * MB), P(A + 128 * MB), P(A + 192 * MB),
                                P(A + 200 * MB), None, P(o), None, B, H, T, dk, dv, dtype,
                                P(ws), wsb, None)
    assert scan(B=-1) == binding.GDN_ERR_INVALID_ARG
    assert scan(dtype=9) == binding.GDN_ERR_INVALID_ARG
    assert scan(dk=96, dv=96) == binding.GDN_ERR_UNSUPPORTED
    assert scan(q=A + 4) == binding.GDN_ERR_ALIGNMENT
    assert scan(o=A) == binding.GDN_ERR_INVALID_ARG
    need = lib.gdn_scan_fwd_workspace(1, 1, 64, 64, 64, 1)
    assert need == 64 * 64 * 4                        # one block: the start-state slot only
    assert scan(wsb=need - 4) == binding.GDN_ERR_INVALID_ARG
    assert lib.gdn_scan_fwd_workspace(1, 1, 64, 128, 128, 0) == 128 * 128 * 4   # fp32 d = 128


@pytest.mark.parametrize("kw", [
    dict(B=2 ** 31), dict(H=2 ** 31), dict(T=2 ** 31), dict(B=2 ** 16, H=2 ** 16),
    dict(B=2 ** 20, H=2 ** 10, T=2 ** 20), dict(B=2 ** 62, H=2 ** 62),
])
def test_oversized_shapes_are_rejected_before_any_arithmetic_overflows(lib, kw):
    """Sizes whose byte counts would not fit int64 (or exceed the limits the
    header states) are refused with UNSUPPORTED, before anything is launched."""
    assert fwd(lib, **kw) == binding.GDN_ERR_UNSUPPORTED
    assert fwd_split(lib, **kw) == binding.GDN_ERR_UNSUPPORTED
    args = (kw.get("B", 1), kw.get("H", 1), kw.get("T", 64), 128, 128)
    assert lib.gdn_scan_fwd_workspace(*args, 1) == 0
    assert lib.gdn_chunk_fwd_split_workspace(*args, 64, 1) == 0
    if "T" not in kw:
        assert step(lib, N=kw.get("B", 1), H=kw.get("H", 1)) == binding.GDN_ERR_UNSUPPORTED


def test_sequence_over_the_bf16_length_limit_is_rejected(lib):
    """One sequence's q, k or v must stay under 2^31 bytes on the bf16
    pipelined path: T = 2^31 / (2 d) is refused before anything else is done
    with it (also by the split entry point, whatever its workspace)."""
    G = 1 << 32
    ptrs = dict(q=A, k=A + 4 * G, v=A + 8 * G, alpha=A + 12 * G, beta=A + 13 * G, o=A + 16 * G)
    T = 2 ** 31 // 256
    assert fwd(lib, T=T, dk=128, dv=128, **ptrs) == binding.GDN_ERR_UNSUPPORTED
    assert fwd_split(lib, T=T, dk=128, dv=128, **ptrs) == binding.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_fwd_split_workspace(1, 1, T, 128, 128, 64, 1) == 0
    P = lambda x: ctypes.c_void_p(x)
    assert lib.gla_chunk_fwd(P(ptrs["q"]), P(ptrs["k"]), P(ptrs["v"]), P(ptrs["alpha"]), P(ptrs["beta"]),
                             None, P(ptrs["o"]), None, 1, 1, T, 128, 128, 64, 1, None) == binding.GDN_ERR_UNSUPPORTED


def noalloc(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, alpha=A + 192 * MB, beta=A + 200 * MB,
            s0=None, o=A + 256 * MB, sT=None, B=1, H=1, T=64, dk=64, dv=64, C=64, dtype=1):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn_chunk_fwd_split_noalloc(P(q), P(k), P(v), P(alpha), P(beta), P(s0), P(o), P(sT),
                                           B, H, T, dk, dv, C, dtype, None)


def test_noalloc_split_validates_before_any_device_call(lib):
    # the same argument checks as gdn_chunk_fwd_split, all before the scratch
    # is looked up or anything is launched
    assert noalloc(lib, q=None) == binding.GDN_ERR_INVALID_ARG
    assert noalloc(lib, B=-1) == binding.GDN_ERR_INVALID_ARG
    assert noalloc(lib, dk=96, dv=96) == binding.GDN_ERR_UNSUPPORTED
    assert noalloc(lib, C=32) == binding.GDN_ERR_UNSUPPORTED
    assert noalloc(lib, v=A + 128 * MB + 8) == binding.GDN_ERR_ALIGNMENT
    assert noalloc(lib, o=A + 64 * MB) == binding.GDN_ERR_INVALID_ARG     # o overlaps k
    assert noalloc(lib, dtype=7) == binding.GDN_ERR_INVALID_ARG
    # nothing to do: no sequences
    assert noalloc(lib, B=0) == binding.GDN_OK


def test_vecgate_split_rejects_invalid_arguments_and_sizes_workspace(lib):
    P = lambda x: None if x is None else ctypes.c_void_p(x)

    def vs(B=1, H=1, T=64, dk=64, dv=64, C=32, dtype=1, q=A, o=A + 256 * MB, alpha=A + 192 * MB):
        return lib.gdn_chunk_fwd_vecgate_split(P(q), P(A + 64 * MB), P(A + 128 * MB), P(alpha),
                                               P(A + 240 * MB), None, P(o), None, B, H, T, dk, dv, C, dtype,
                                               None, 0, None)
    assert vs(B=-1) == binding.GDN_ERR_INVALID_ARG
    assert vs(dtype=5) == binding.GDN_ERR_INVALID_ARG
    assert vs(q=None) == binding.GDN_ERR_INVALID_ARG
    assert vs(C=64) == binding.GDN_ERR_UNSUPPORTED          # this route's chunk is 32 tokens
    assert vs(dk=96, dv=96) == binding.GDN_ERR_UNSUPPORTED
    assert vs(q=A + 4) == binding.GDN_ERR_ALIGNMENT
    assert vs(o=A) == binding.GDN_ERR_INVALID_ARG            # output overlaps q
    assert vs(B=0) == 0                                      # nothing to do
    f = lib.gdn_chunk_fwd_vecgate_split_workspace
    assert f(1, 8, 16384, 64, 64, 64, 1) == 0               # unsupported chunk size
    assert f(1, 8, 16384, 96, 96, 32, 1) == 0               # unsupported width
    assert f(0, 8, 16384, 64, 64, 32, 1) == 0               # nothing to do
    assert f(1, 8, 16384, 64, 64, 32, 1) >= 0               # no GPU here: 0; on a GPU: > 0


def test_vecgate_2pass_rejects_invalid_arguments_and_sizes_workspace(lib):
    """The two-pass route's checks, all before any device call, and its
    workspace size: the carried state (B*H*dk*dv floats) plus one record per
    chunk of the largest tile (at most 256 chunks per sequence); a record holds
    the scaled q and k, Kbar^T, (I+L)^-1, P, 2^(G_C) and beta of a 32-token
    chunk in their LDS layout, rounded up to whole KiB."""
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    WS = A + 512 * MB

    def tp(B=1, H=1, T=64, dk=64, dv=64, C=32, dtype=1, q=A, o=A + 256 * MB, ws=WS, wsb=64 * MB):
        return lib.gdn_chunk_fwd_vecgate_2pass(P(q), P(A + 64 * MB), P(A + 128 * MB), P(A + 192 * MB),
                                               P(A + 240 * MB), None, P(o), None, B, H, T, dk, dv, C, dtype,
                                               P(ws), wsb, None)
    assert tp(B=-1) == binding.GDN_ERR_INVALID_ARG
    assert tp(q=None) == binding.GDN_ERR_INVALID_ARG
    assert tp(C=64) == binding.GDN_ERR_UNSUPPORTED
    assert tp(dk=96, dv=96) == binding.GDN_ERR_UNSUPPORTED
    assert tp(ws=None) == binding.GDN_ERR_INVALID_ARG
    assert tp(wsb=64 * 64 * 4 + 20480 - 1) == binding.GDN_ERR_INVALID_ARG   # under one record per sequence
    assert tp(ws=WS + 8) == binding.GDN_ERR_ALIGNMENT
    assert tp(ws=A + 64 * MB) == binding.GDN_ERR_INVALID_ARG               # workspace overlaps k
    assert tp(B=0) == 0
    f = lib.gdn_chunk_fwd_vecgate_2pass_workspace
    rec = {(1, 64): 20480, (1, 128): 33792, (0, 64): 36864, (0, 128): 62464}
    for (dt, d), r in rec.items():
        assert f(1, 1, 1000, d, d, 32, dt) == d * d * 4 + 32 * r              # 32 chunks: one tile
        assert f(4, 16, 8192, d, d, 32, dt) == 64 * (d * d * 4 + 256 * r)     # one tile of 256 chunks
        assert f(1, 2, 20000, d, d, 32, dt) == 2 * (d * d * 4 + 256 * r)      # 625 chunks: tiles of 256
        assert f(1, 1, 0, d, d, 32, dt) == d * d * 4 + r
    assert f(1, 1, 1000, 64, 64, 64, 1) == 0
    assert f(1, 1, 1000, 96, 96, 32, 1) == 0
    assert f(0, 1, 1000, 64, 64, 32, 1) == 0
