"""Pins of the per-dimension-gate oracle (``oracle.oracle_fwd_vecgate``,
[P1] §2.2 with a vector gate that decays the key columns of the state).
CPU only.

  * explicit d x d maps A_t = Diag(alpha_t) (I - beta_t k_t k_t^T) and
    B_t = beta_t v_t k_t^T folded as S -> S A_t + B_t in numpy (tiny sizes);
  * a gate equal in every dimension reproduces the scalar-gate oracle
    (pinned on its own in test_oracle_pins.py);
  * beta = 0: pure per-dimension decay, S_T = S_0 Diag(prod_t alpha_t) and
    o_t = S_0 Diag(prod_{r<=t} alpha_r) q_t;
  * negative control: decaying the value rows instead of the key columns
    gives a different result.
Planted mistakes in a copy of the oracle must each fail a pin.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def maxrel(x, ref):
    den = max(np.max(np.abs(ref)), 1e-300)
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref)) / den)


def case(rng, T, dk, dv):
    q = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, dv)).astype(np.float32)
    a = rng.uniform(0.2, 1.0, (1, 1, T, dk)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, (1, 1, T)).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((1, 1, dv, dk))).astype(np.float32)
    return q, k, v, a, b, S0


def pin_explicit_maps(fwd, seed=0):
    rng = np.random.default_rng(seed)
    for T, dk, dv in [(1, 2, 2), (6, 3, 4), (10, 5, 3)]:
        q, k, v, a, b, S0 = case(rng, T, dk, dv)
        o, sT = fwd(q, k, v, a, b, S0)
        S = S0[0, 0].astype(np.float64)
        for t in range(T):
            kt = k[0, 0, t].astype(np.float64)
            A = np.diag(a[0, 0, t].astype(np.float64)) @ (np.eye(dk) - float(b[0, 0, t]) * np.outer(kt, kt))
            S = S @ A + float(b[0, 0, t]) * np.outer(v[0, 0, t].astype(np.float64), kt)
            assert maxrel(o[0, 0, t], S @ q[0, 0, t].astype(np.float64)) < 1e-12
        assert maxrel(sT[0, 0], S) < 1e-12


def pin_uniform_gate_is_scalar_gate(fwd, seed=1):
    rng = np.random.default_rng(seed)
    q, k, v, _, b, S0 = case(rng, 30, 16, 8)
    a = rng.uniform(0.2, 1.0, (1, 1, 30)).astype(np.float32)
    o1, s1 = fwd(q, k, v, np.repeat(a[..., None], 16, axis=-1), b, S0)
    o2, s2 = oracle.oracle_fwd(q, k, v, a, b, S0)
    assert maxrel(o1, o2) < 1e-13 and maxrel(s1, s2) < 1e-13


def pin_pure_decay(fwd, seed=2):
    rng = np.random.default_rng(seed)
    q, k, v, a, _, S0 = case(rng, 12, 6, 5)
    zero = np.zeros((1, 1, 12), np.float32)
    o, sT = fwd(q, k, v, a, zero, S0)
    cum = np.cumprod(a[0, 0].astype(np.float64), axis=0)
    S0d = S0[0, 0].astype(np.float64)
    for t in range(12):
        assert maxrel(o[0, 0, t], (S0d * cum[t]) @ q[0, 0, t].astype(np.float64)) < 1e-12
    assert maxrel(sT[0, 0], S0d * cum[-1]) < 1e-12


PINS = [pin_explicit_maps, pin_uniform_gate_is_scalar_gate, pin_pure_decay]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_vecgate_oracle_pin(pin):
    pin(oracle.oracle_fwd_vecgate)


def test_value_row_decay_differs():
    """Negative control: the per-dimension gate acts on key columns; decaying
    value rows (Diag(alpha) S, with dv = dk) gives another result."""
    rng = np.random.default_rng(3)
    q, k, v, a, b, S0 = case(rng, 20, 8, 8)
    o, _ = oracle.oracle_fwd_vecgate(q, k, v, a, b, S0)
    S = S0[0, 0].astype(np.float64)
    for t in range(20):
        kt = k[0, 0, t].astype(np.float64)
        S = np.diag(a[0, 0, t].astype(np.float64)) @ S
        S = S @ (np.eye(8) - float(b[0, 0, t]) * np.outer(kt, kt)) + float(b[0, 0, t]) * np.outer(v[0, 0, t], kt)
    assert maxrel(S @ q[0, 0, -1].astype(np.float64), o[0, 0, -1]) > 1e-3


MUTATIONS = {
    "no_decay": ("row[j] *= (double)at[j];", "row[j] *= 1.0;"),
    "decay_after_retrieve": ("row[j] *= (double)at[j];\n                    r += row[j] * (double)kt[j];",
                             "r += row[j] * (double)kt[j];\n                    row[j] *= (double)at[j];"),
    "no_beta": ("const double u = bt * ((double)v[tok * dv + i] - r);",
                "const double u = ((double)v[tok * dv + i] - r);"),
    "one_gate_for_all": ("row[j] *= (double)at[j];", "row[j] *= (double)at[0];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_vecgate_pins_catch_planted_mistakes(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "gdn_oracle.c"), encoding="utf-8").read()
    assert src.count(old) == 1, name
    cfile = tmp_path / ("mut_%s.c" % name)
    cfile.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(cfile)], check=True)
    lib = oracle._bind(str(so))
    fwd = lambda *args, **kw: oracle.oracle_fwd_vecgate(*args, _lib_override=lib, **kw)
    caught = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
