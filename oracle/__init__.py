"""fp64 CPU oracle for the gated delta rule (TEST INFRASTRUCTURE).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP path.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, OpenMP over the
independent (b,h) chains).  This module only builds it with gcc, marshals
numpy arrays and returns fp64 results.

Sources (web pages, by title and section):
  [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案",
       §2.1 (delta-rule update), §2.2 (scalar gate), §1.3 / §5.3 (naive token
       loop as the correctness baseline).
  [P3] "线性注意力机制与Gated DeltaNet的优化实践", §2.1 (inclusive output),
       §2.3 (gated linear attention without the delta rule: ``oracle_gla_fwd``);
  [P1] §2.2 also allows a per-dimension gate: ``oracle_fwd_vecgate``.

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``:
composed affine maps vs. the loop (with a negative control), beta=0 pure decay,
exact retrieval with orthonormal keys, causal (gated) linear attention, a
hand-computed d=2 example under ``tests/golden/``, the d=1 closed form,
linearity, row independence, split invariance and the chunked identity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP,
    no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    f = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.gdn_oracle_fwd.argtypes = [f, f, f, f, f, f, f, f, i64, i64, i64, i64, i64]
    lib.gdn_oracle_fwd.restype = ctypes.c_int
    lib.gdn_oracle_step.argtypes = [f, f, f, f, f, f, f, i64, i64, i64, i64]
    lib.gdn_oracle_step.restype = ctypes.c_int
    lib.gla_oracle_fwd.argtypes = [f, f, f, f, f, f, f, f, i64, i64, i64, i64, i64]
    lib.gla_oracle_fwd.restype = ctypes.c_int
    lib.gdn_oracle_fwd_vecgate.argtypes = [f, f, f, f, f, f, f, f, i64, i64, i64, i64, i64]
    lib.gdn_oracle_fwd_vecgate.restype = ctypes.c_int
    lib.gdn_oracle_num_threads.argtypes = []
    lib.gdn_oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(_LIB)
    return _lib


def _f32(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def num_threads() -> int:
    """Threads the oracle's OpenMP loop uses."""
    return int(_load().gdn_oracle_num_threads())


def fwd_from_library(path):
    """``oracle_fwd`` bound to another build of the oracle source (used by the
    tests that plant mistakes in a copy of it)."""
    lib = _bind(path)
    return lambda *args, **kw: oracle_fwd(*args, _lib_override=lib, **kw)


def oracle_fwd(q, k, v, alpha, beta, s0=None, _lib_override=None):
    """Token-by-token fp64 forward pass.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; alpha, beta: [B,H,T]; s0: [B,H,dv,dk] or
    None (zero).  All inputs are taken as fp32 values (bf16 tensors must be
    passed as their exact fp32 widening).  Returns (o [B,H,T,dv] fp64,
    sT [B,H,dv,dk] fp64).
    """
    lib = _lib_override if _lib_override is not None else _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, T) and beta.shape == (B, H, T)
    if s0 is not None:
        s0 = _f32(s0)
        assert s0.shape == (B, H, dv, dk)
    o = np.zeros((B, H, T, dv), dtype=np.float64)
    sT = np.zeros((B, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(s0), _ptr(o), _ptr(sT), B, H, T, dk, dv)
    if rc != 0:
        raise RuntimeError("gdn_oracle_fwd failed with code %d" % rc)
    return o, sT


def oracle_gla_fwd(q, k, v, alpha, beta, s0=None, _lib_override=None):
    """Gated linear attention, token by token in fp64 ([P3] §2.3):
    S_t = alpha_t S_{t-1} + beta_t v_t k_t^T, o_t = S_t q_t.  Same shapes and
    returns as ``oracle_fwd``."""
    lib = _lib_override if _lib_override is not None else _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, T) and beta.shape == (B, H, T)
    if s0 is not None:
        s0 = _f32(s0)
        assert s0.shape == (B, H, dv, dk)
    o = np.zeros((B, H, T, dv), dtype=np.float64)
    sT = np.zeros((B, H, dv, dk), dtype=np.float64)
    rc = lib.gla_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(s0), _ptr(o), _ptr(sT), B, H, T, dk, dv)
    if rc != 0:
        raise RuntimeError("gla_oracle_fwd failed with code %d" % rc)
    return o, sT


def oracle_fwd_vecgate(q, k, v, alpha, beta, s0=None, _lib_override=None):
    """The delta rule with a per-dimension gate alpha [B,H,T,dk] that decays
    the key columns of the state ([P1] §2.2): S_t = S_{t-1} Diag(alpha_t)
    (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t, in fp64.
    Returns (o, sT) like ``oracle_fwd``."""
    lib = _lib_override if _lib_override is not None else _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, T, dk) and beta.shape == (B, H, T)
    if s0 is not None:
        s0 = _f32(s0)
        assert s0.shape == (B, H, dv, dk)
    o = np.zeros((B, H, T, dv), dtype=np.float64)
    sT = np.zeros((B, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_fwd_vecgate(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(s0), _ptr(o), _ptr(sT), B, H, T, dk, dv)
    if rc != 0:
        raise RuntimeError("gdn_oracle_fwd_vecgate failed with code %d" % rc)
    return o, sT


def oracle_step(q, k, v, alpha, beta, state):
    """One decode step, fp64.  q,k: [N,H,dk]; v: [N,H,dv]; alpha,beta: [N,H];
    state: [N,H,dv,dk] fp64, updated IN PLACE.  Returns o [N,H,dv] fp64."""
    lib = _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    assert state.shape == (N, H, dv, dk)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.gdn_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                             _ptr(state), _ptr(o), N, H, dk, dv)
    if rc != 0:
        raise RuntimeError("gdn_oracle_step failed with code %d" % rc)
    return o
