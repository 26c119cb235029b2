"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each check below is independent of the oracle's own code: closed forms,
explicit affine-map composition, a hand-computed example, invariants.  A
plausible slip in the oracle (dropped decay, dropped beta, wrong sign of the
error, retrieving with q instead of k, reading the output before the update,
left- instead of right-multiplication) fails at least one of them; the
mutation test at the end plants such slips in a copy of the oracle source and
checks that they are caught.

Sources (web pages, by title and section):
  [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
       §2.1 delta rule as an affine map, §2.2 gate, §2.3 composition of affine
       maps and its associativity, §5.2 (first pitfall: composition order; test
       on d=2 random data against the naive loop).
  [P3] "线性注意力机制与Gated DeltaNet的优化实践"
       §2.1-2.2 causal linear attention and its state S = sum k v^T,
       §2.3 gated (non-delta) form S = gamma S + eta k v^T.
"""
import ctypes
import os
import random
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "worked_example_d2.txt")


# ----------------------------------------------------------------- helpers --
def rand_case(rng, B, H, T, dk, dv, unit_keys=True, s0=True):
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    alpha = rng.uniform(0.3, 1.0, (B, H, T)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, H, T)).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((B, H, dv, dk))).astype(np.float32) if s0 else None
    return q, k, v, alpha, beta, S0


def maxrel(x, ref):
    den = max(np.max(np.abs(ref)), 1e-300)
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref)) / den)


def token_maps(k, v, alpha, beta):
    """The page's left form acting on X = S^T (d_k x d_v):
    X_t = M_t X_{t-1} + N_t with M_t = alpha_t (I - beta_t k k^T) and
    N_t = beta_t k v^T  ([P1] §2.1-2.2)."""
    dk = k.shape[-1]
    Ms, Ns = [], []
    for t in range(k.shape[0]):
        kt = k[t].astype(np.float64)[:, None]
        vt = v[t].astype(np.float64)[:, None]
        Ms.append(float(alpha[t]) * (np.eye(dk) - float(beta[t]) * kt @ kt.T))
        Ns.append(float(beta[t]) * kt @ vt.T)
    return Ms, Ns


def compose(f, g):
    """Map g applied after map f ([P1] §2.3): (g o f)(X) = Mg (Mf X + Nf) + Ng."""
    Mf, Nf = f
    Mg, Ng = g
    return (Mg @ Mf, Mg @ Nf + Ng)


def fold_tree(maps, rng):
    """Fold a list of maps (earliest first) in a random bracketing."""
    if len(maps) == 1:
        return maps[0]
    cut = rng.randint(1, len(maps) - 1)
    return compose(fold_tree(maps[:cut], rng), fold_tree(maps[cut:], rng))


# ---------------------------------------------------------- pin functions --
# Each pin takes a forward function with the signature of oracle.oracle_fwd
# and raises AssertionError when it is violated.

def pin_affine_composition(fwd, seed=0):
    """P-A: sequential loop == composed affine maps under any bracketing;
    the reversed composition order must NOT match (negative control)."""
    rng = np.random.default_rng(seed)
    prng = random.Random(seed)
    for dk, dv, T in [(2, 2, 6), (3, 2, 9), (5, 4, 12), (2, 3, 16)]:
        q, k, v, alpha, beta, S0 = rand_case(rng, 1, 1, T, dk, dv)
        o, sT = fwd(q, k, v, alpha, beta, S0)
        Ms, Ns = token_maps(k[0, 0], v[0, 0], alpha[0, 0], beta[0, 0])
        X0 = S0[0, 0].astype(np.float64).T
        # explicit interval formula A_{t:1} = M_t..M_1, B_{t:1} = sum_s M_t..M_{s+1} N_s
        for t in range(1, T + 1):
            A = np.eye(dk)
            Bm = np.zeros((dk, dv))
            for s in range(t):
                P = np.eye(dk)
                for r in range(s + 1, t):
                    P = Ms[r] @ P
                Bm = Bm + P @ Ns[s]
                A = Ms[s] @ A
            Xt = A @ X0 + Bm
            ot = Xt.T @ q[0, 0, t - 1].astype(np.float64)
            assert maxrel(o[0, 0, t - 1], ot) < 1e-12
        for trial in range(5):
            M, N = fold_tree(list(zip(Ms, Ns)), prng)
            XT = M @ X0 + N
            assert maxrel(sT[0, 0].T, XT) < 1e-12
        # negative control: composing in the wrong order (earlier map applied
        # last) disagrees with the loop
        Mw, Nw = np.eye(dk), np.zeros((dk, dv))
        for t in range(T):
            Mw, Nw = compose((Ms[t], Ns[t]), (Mw, Nw))
        assert maxrel(sT[0, 0].T, Mw @ X0 + Nw) > 1e-3


def pin_pure_decay(fwd, seed=1):
    """P-B: beta = 0 gives S_T = (prod alpha) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = rand_case(rng, 2, 3, 17, 8, 6)
    beta[:] = 0.0
    o, sT = fwd(q, k, v, alpha, beta, S0)
    cum = np.cumprod(alpha.astype(np.float64), axis=-1)
    S0d = S0.astype(np.float64)
    o_ref = cum[..., None] * np.einsum("bhij,bhtj->bhti", S0d, q.astype(np.float64))
    assert maxrel(o, o_ref) < 1e-12
    assert maxrel(sT, cum[..., -1][..., None, None] * S0d) < 1e-12


def orthonormal_keys(rng, T, dk):
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    return Qm[:T].astype(np.float32)


def pin_exact_retrieval(fwd, seed=2):
    """P-C: alpha = beta = 1, orthonormal keys, S_0 = 0: S_T k_i = v_i and
    o_t = sum_{s<=t} (k_s . q_t) v_s (causal linear attention, [P3] §2.1-2.2)."""
    rng = np.random.default_rng(seed)
    for dk, dv, T in [(8, 8, 8), (16, 5, 11), (64, 64, 40)]:
        k = orthonormal_keys(rng, T, dk)
        # orthonormal rows are only approximately unit after the fp32 rounding;
        # the closed form below is evaluated on the same rounded keys, and the
        # deviation from exact orthonormality is ~1e-7
        q = rng.standard_normal((T, dk)).astype(np.float32)
        v = rng.standard_normal((T, dv)).astype(np.float32)
        one = np.ones(T, np.float32)
        o, sT = fwd(q[None, None], k[None, None], v[None, None], one[None, None],
                    one[None, None], None)
        kd, qd, vd = k.astype(np.float64), q.astype(np.float64), v.astype(np.float64)
        retrieved = (sT[0, 0] @ kd.T).T
        assert maxrel(retrieved, vd) < 1e-5
        o_ref = np.tril(qd @ kd.T) @ vd
        assert maxrel(o[0, 0], o_ref) < 1e-5


def pin_gated_linear_attention(fwd, seed=3):
    """P-D: beta = 1, orthonormal keys, any alpha, S_0 = 0 reduces to gated
    linear attention ([P3] §2.3 with eta = 1 and a scalar gamma):
    o_t = sum_{s<=t} (prod_{s<r<=t} alpha_r) (k_s . q_t) v_s."""
    rng = np.random.default_rng(seed)
    dk, dv, T = 32, 12, 24
    k = orthonormal_keys(rng, T, dk)
    q = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    alpha = rng.uniform(0.2, 1.0, T).astype(np.float32)
    one = np.ones(T, np.float32)
    o, sT = fwd(q[None, None], k[None, None], v[None, None], alpha[None, None],
                one[None, None], None)
    la = np.log(alpha.astype(np.float64))
    g = np.cumsum(la)
    decay = np.exp(g[:, None] - g[None, :]) * np.tri(T)
    o_ref = (decay * (q.astype(np.float64) @ k.astype(np.float64).T)) @ v.astype(np.float64)
    assert maxrel(o[0, 0], o_ref) < 1e-5


def read_golden(path=GOLDEN):
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rhs = (s.strip() for s in line.split("=", 1))
            rows = [[float(x) for x in r.split()] for r in rhs.split(";")]
            vals[name] = np.array(rows if len(rows) > 1 else rows[0], dtype=np.float64)
    return vals


def pin_worked_example(fwd):
    """P-E: the hand-computed d=2 example under tests/golden/."""
    g = read_golden()
    q = np.stack([g["q1"], g["q2"]])[None, None]
    k = np.stack([g["k1"], g["k2"]])[None, None]
    v = np.stack([g["v1"], g["v2"]])[None, None]
    alpha = np.array([g["alpha1"], g["alpha2"]]).reshape(1, 1, 2)
    beta = np.array([g["beta1"], g["beta2"]]).reshape(1, 1, 2)
    o, sT = fwd(q, k, v, alpha, beta, None)
    # inputs are exact in binary except 0.6/0.8 (fp32 rounding, ~3e-8)
    assert np.max(np.abs(o[0, 0, 0] - g["o1"])) < 1e-6
    assert np.max(np.abs(o[0, 0, 1] - g["o2"])) < 1e-6
    assert np.max(np.abs(sT[0, 0] - g["S2"])) < 1e-6
    assert np.max(np.abs(sT[0, 0] - g["S2_left_reading"])) > 0.05


def pin_scalar_closed_form(fwd, seed=4):
    """P-F: d = 1 reduces to s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t v_t k_t."""
    rng = np.random.default_rng(seed)
    T = 50
    q = rng.standard_normal(T).astype(np.float32)
    k = rng.standard_normal(T).astype(np.float32)
    v = rng.standard_normal(T).astype(np.float32)
    alpha = rng.uniform(0.5, 1.0, T).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, T).astype(np.float32)
    s0 = np.float32(0.7)
    o, sT = fwd(q.reshape(1, 1, T, 1), k.reshape(1, 1, T, 1), v.reshape(1, 1, T, 1),
                alpha.reshape(1, 1, T), beta.reshape(1, 1, T),
                np.array(s0, np.float32).reshape(1, 1, 1, 1))
    s = float(s0)
    ref = []
    for t in range(T):
        a, b, kk, vv = float(alpha[t]), float(beta[t]), float(k[t]), float(v[t])
        s = a * (1.0 - b * kk * kk) * s + b * vv * kk
        ref.append(s * float(q[t]))
    assert maxrel(o.reshape(T), np.array(ref)) < 1e-12
    assert abs(sT.reshape(()) - s) <= 1e-12 * max(1.0, abs(s))


def pin_linearity(fwd, seed=5):
    """P-G: for fixed q, k, alpha, beta the outputs are linear in (V, S_0)."""
    rng = np.random.default_rng(seed)
    q, k, v1, alpha, beta, S1 = rand_case(rng, 1, 2, 20, 6, 5)
    _, _, v2, _, _, S2 = rand_case(rng, 1, 2, 20, 6, 5)
    a, b = 0.75, -1.25
    o1, s1 = fwd(q, k, v1, alpha, beta, S1)
    o2, s2 = fwd(q, k, v2, alpha, beta, S2)
    v3 = (a * v1.astype(np.float64) + b * v2).astype(np.float32)
    S3 = (a * S1.astype(np.float64) + b * S2).astype(np.float32)
    o3, s3 = fwd(q, k, v3, alpha, beta, S3)
    # v3/S3 are rounded to fp32 (2^-24 relative); compare at that level
    assert maxrel(o3, a * o1 + b * o2) < 1e-6
    assert maxrel(s3, a * s1 + b * s2) < 1e-6


def pin_row_independence(fwd, seed=6):
    """P-H: each value row of S evolves alone: permuting the value dims
    permutes o and S, and a value slice run alone equals that slice."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = rand_case(rng, 1, 2, 24, 8, 8)
    o, sT = fwd(q, k, v, alpha, beta, S0)
    perm = rng.permutation(8)
    op, sp = fwd(q, k, np.ascontiguousarray(v[..., perm]), alpha, beta,
                 np.ascontiguousarray(S0[:, :, perm, :]))
    assert maxrel(op, o[..., perm]) < 1e-13
    assert maxrel(sp, sT[:, :, perm, :]) < 1e-13
    osl, ssl = fwd(q, k, np.ascontiguousarray(v[..., 2:5]), alpha, beta,
                   np.ascontiguousarray(S0[:, :, 2:5, :]))
    assert maxrel(osl, o[..., 2:5]) < 1e-13
    assert maxrel(ssl, sT[:, :, 2:5, :]) < 1e-13


def pin_split_invariance(fwd, seed=7):
    """P-I: run(T1+T2) == run(T2, init = run(T1).S)  ([P1] §2.3 interval folding).
    The hand-off state is fp32 (as the library's state is), so compare at the
    fp32 level."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = rand_case(rng, 1, 2, 30, 6, 5)
    o, sT = fwd(q, k, v, alpha, beta, S0)
    oa, sa = fwd(q[:, :, :13], k[:, :, :13], v[:, :, :13], alpha[:, :, :13],
                 beta[:, :, :13], S0)
    ob, sb = fwd(q[:, :, 13:], k[:, :, 13:], v[:, :, 13:], alpha[:, :, 13:],
                 beta[:, :, 13:], sa.astype(np.float32))
    assert maxrel(oa, o[:, :, :13]) < 1e-13
    assert maxrel(ob, o[:, :, 13:]) < 1e-6
    assert maxrel(sb, sT) < 1e-6


def chunk_form(q, k, v, alpha, beta, S0, C):
    """Chunked form of the recurrence (derived: within a chunk the unrolled
    state is S_r = e^{g_r} S + sum_{s<=r} e^{g_r - g_s} u_s k_s^T, which gives
    the unit-lower-triangular system (I + L) U = diag(beta) V -
    diag(beta e^g) K S^T).  Written here only to pin the algebra the GPU path
    uses; fp64 numpy, one (b,h) at a time."""
    T, dk = k.shape
    dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        K, Q, V = k[c0:c1], q[c0:c1], v[c0:c1]
        g = np.cumsum(np.log(alpha[c0:c1]))
        b = beta[c0:c1]
        D = np.exp(g[:, None] - g[None, :]) * np.tri(n)
        L = (b[:, None] * D * (K @ K.T)) * np.tri(n, k=-1)
        Tinv = np.linalg.inv(np.eye(n) + L)
        Ut = Tinv @ (b[:, None] * V)
        W = Tinv @ ((b * np.exp(g))[:, None] * K)
        U = Ut - W @ S.T
        P = D * (Q @ K.T)
        o[c0:c1] = np.exp(g)[:, None] * (Q @ S.T) + P @ U
        Khat = np.exp(g[-1] - g)[:, None] * K
        S = np.exp(g[-1]) * S + U.T @ Khat
    return o, S


def pin_chunk_identity(fwd, seed=8):
    """P-J: the chunked form equals the token loop for any chunk size,
    including a ragged tail chunk."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = rand_case(rng, 1, 1, 40, 6, 5)
    o, sT = fwd(q, k, v, alpha, beta, S0)
    for C in (1, 4, 8, 16, 40, 64):
        oc, Sc = chunk_form(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64),
                            v[0, 0].astype(np.float64), alpha[0, 0].astype(np.float64),
                            beta[0, 0].astype(np.float64), S0[0, 0].astype(np.float64), C)
        assert maxrel(oc, o[0, 0]) < 1e-12
        assert maxrel(Sc, sT[0, 0]) < 1e-12


PINS = [pin_affine_composition, pin_pure_decay, pin_exact_retrieval,
        pin_gated_linear_attention, pin_worked_example, pin_scalar_closed_form,
        pin_linearity, pin_row_independence, pin_split_invariance,
        pin_chunk_identity]


# ------------------------------------------------------------------ tests --
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.oracle_fwd)


def test_decode_step_equals_forward():
    """The decode step is the same token update: chaining T steps reproduces
    a T-token forward pass from the same initial state."""
    rng = np.random.default_rng(9)
    q, k, v, alpha, beta, S0 = rand_case(rng, 3, 2, 7, 16, 16)
    o, sT = oracle.oracle_fwd(q, k, v, alpha, beta, S0)
    state = S0.astype(np.float64).copy()
    for t in range(7):
        ot = oracle.oracle_step(np.ascontiguousarray(q[:, :, t]), np.ascontiguousarray(k[:, :, t]),
                                np.ascontiguousarray(v[:, :, t]), np.ascontiguousarray(alpha[:, :, t]),
                                np.ascontiguousarray(beta[:, :, t]), state)
        assert maxrel(ot, o[:, :, t]) < 1e-13
    assert maxrel(state, sT) < 1e-13


def test_zero_length_and_zero_state():
    """T = 0 returns the initial state untouched; S_0 = None means zeros."""
    rng = np.random.default_rng(10)
    q, k, v, alpha, beta, S0 = rand_case(rng, 1, 2, 0, 4, 4)
    o, sT = oracle.oracle_fwd(q, k, v, alpha, beta, S0)
    assert o.shape == (1, 2, 0, 4)
    assert np.array_equal(sT, S0.astype(np.float64))
    o, sT = oracle.oracle_fwd(q, k, v, alpha, beta, None)
    assert np.all(sT == 0.0)


# ------------------------------------------------ mutations of the oracle --
MUTATIONS = {
    "no_decay": ("row[j] *= alpha;", "row[j] *= 1.0;"),
    "no_beta": ("double u = beta * (", "double u = 1.0 * ("),
    "wrong_sign": ("(double)v[i] - r", "(double)v[i] + r"),
    "retrieve_with_q": ("r += row[j] * kd[j];", "r += row[j] * qd[j];"),
    "no_erase": ("double u = beta * ((double)v[i] - r);",
                 "double u = beta * ((double)v[i] - 0.0 * r);"),
    "output_before_update": ("acc += row[j] * qd[j];",
                             "acc += (row[j] - u * kd[j]) * qd[j];"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "gdn_oracle.c"), encoding="utf-8").read()
    assert old in src, name
    mutated = src.replace(old, new, 1)
    cfile = tmp_path / ("mut_%s.c" % name)
    cfile.write_text(mutated, encoding="utf-8")
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o",
                    str(so), str(cfile)], check=True)
    return oracle.fwd_from_library(str(so))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(tmp_path, name):
    old, new = MUTATIONS[name]
    fwd = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
