"""Pins of the gated-linear-attention oracle (``oracle.oracle_gla_fwd``),
against results fixed independently of its loop ([P3] §2.3: the state
decays by a gate and gains beta v k^T, no erase term; output inclusive of
the current token, [P3] §2.1).  CPU only.

  * the unrolled sum, evaluated by explicit double loops on tiny inputs;
  * with orthonormal keys and a zero start the delta rule has nothing to
    erase, so both oracles must agree (the delta-rule oracle is pinned on its
    own in test_oracle_pins.py);
  * alpha = beta = 1: causal linear attention, tril(Q K^T) V and S_T = V^T K
    (numpy matrix products);
  * negative control: on generic keys the two recurrences differ.
Planted mistakes in a copy of the oracle source must each fail a pin.
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


def case(rng, T, dk, dv, s0=True, unit=True):
    q = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, dv)).astype(np.float32)
    a = rng.uniform(0.3, 1.0, (1, 1, T)).astype(np.float32)
    b = rng.uniform(0.0, 1.5, (1, 1, T)).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((1, 1, dv, dk))).astype(np.float32) if s0 else None
    return q, k, v, a, b, S0


def pin_unrolled_sum(fwd, seed=0):
    """o_t = (prod_{r<=t} a_r) S0 q_t + sum_{s<=t} (prod_{s<r<=t} a_r) b_s (k_s.q_t) v_s,
    S_T = (prod_r a_r) S0 + sum_s (prod_{s<r<=T} a_r) b_s v_s k_s^T."""
    rng = np.random.default_rng(seed)
    for T, dk, dv in [(1, 3, 2), (7, 4, 5), (12, 6, 3)]:
        q, k, v, a, b, S0 = case(rng, T, dk, dv)
        o, sT = fwd(q, k, v, a, b, S0)
        qd, kd, vd = (x[0, 0].astype(np.float64) for x in (q, k, v))
        ad, bd, Sd = a[0, 0].astype(np.float64), b[0, 0].astype(np.float64), S0[0, 0].astype(np.float64)
        for t in range(T):
            ref = np.prod(ad[:t + 1]) * (Sd @ qd[t])
            for s in range(t + 1):
                ref = ref + np.prod(ad[s + 1:t + 1]) * bd[s] * float(kd[s] @ qd[t]) * vd[s]
            assert maxrel(o[0, 0, t], ref) < 1e-12
        Sref = np.prod(ad) * Sd
        for s in range(T):
            Sref = Sref + np.prod(ad[s + 1:]) * bd[s] * np.outer(vd[s], kd[s])
        assert maxrel(sT[0, 0], Sref) < 1e-12


def pin_equals_delta_rule_on_orthonormal_keys(fwd, seed=1):
    rng = np.random.default_rng(seed)
    dk, dv, T = 32, 9, 20
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T].astype(np.float32)[None, None]
    q = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, dv)).astype(np.float32)
    a = rng.uniform(0.2, 1.0, (1, 1, T)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, (1, 1, T)).astype(np.float32)
    o1, s1 = fwd(q, k, v, a, b, None)
    o2, s2 = oracle.oracle_fwd(q, k, v, a, b, None)
    assert maxrel(o1, o2) < 1e-5 and maxrel(s1, s2) < 1e-5


def pin_linear_attention(fwd, seed=2):
    rng = np.random.default_rng(seed)
    q, k, v, _, _, _ = case(rng, 16, 8, 6, s0=False, unit=False)
    one = np.ones((1, 1, 16), np.float32)
    o, sT = fwd(q, k, v, one, one, None)
    qd, kd, vd = (x[0, 0].astype(np.float64) for x in (q, k, v))
    assert maxrel(o[0, 0], np.tril(qd @ kd.T) @ vd) < 1e-12
    assert maxrel(sT[0, 0], vd.T @ kd) < 1e-12


PINS = [pin_unrolled_sum, pin_equals_delta_rule_on_orthonormal_keys, pin_linear_attention]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_gla_oracle_pin(pin):
    pin(oracle.oracle_gla_fwd)


def test_gla_and_delta_rule_differ_on_generic_keys():
    rng = np.random.default_rng(3)
    q, k, v, a, b, S0 = case(rng, 24, 8, 8)
    o1, _ = oracle.oracle_gla_fwd(q, k, v, a, b, S0)
    o2, _ = oracle.oracle_fwd(q, k, v, a, b, S0)
    assert maxrel(o1, o2) > 1e-2


MUTATIONS = {
    "no_decay": ("row[j] = a * row[j] + w * (double)kt[j];", "row[j] = row[j] + w * (double)kt[j];"),
    "no_beta": ("const double w = b * (double)v[tok * dv + i];", "const double w = (double)v[tok * dv + i];"),
    "key_for_query": ("row[j] = a * row[j] + w * (double)kt[j];\n                    acc += row[j] * (double)qt[j];",
                      "row[j] = a * row[j] + w * (double)kt[j];\n                    acc += row[j] * (double)kt[j];"),
    "output_before_update": ("row[j] = a * row[j] + w * (double)kt[j];\n                    acc += row[j] * (double)qt[j];",
                             "row[j] = a * row[j] + w * (double)kt[j];\n                    acc += (row[j] - w * (double)kt[j]) * (double)qt[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_gla_pins_catch_planted_mistakes(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "gdn_oracle.c"), encoding="utf-8").read()
    assert src.count(old) == 1, name
    cfile = tmp_path / ("mut_%s.c" % name)
    cfile.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(cfile)], check=True)
    lib = oracle._bind(str(so))
    fwd = lambda *args, **kw: oracle.oracle_gla_fwd(*args, _lib_override=lib, **kw)
    caught = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
