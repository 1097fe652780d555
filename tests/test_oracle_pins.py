"""Pins of the oracle to things other than itself (CPU only).

* closed forms evaluated with numpy matrix products (the parallel form of
  causal linear attention, its decayed variant, the delta rule's special cases);
* invariants of the delta rule (retrieval of the stored value along a unit key);
* exact rational evaluation of the buffered (chunkwise) form of the method,
  which must agree with the oracle's per-token recurrence up to fp64 rounding.

Shapes are non-square (d_k != d_v) so that a transposed operand fails, the
initial state is non-zero so that a dropped state term fails, and the output is
read after the token's own update so that an off-by-one in causality fails.
"""

import math
from fractions import Fraction as F

import numpy as np
import pytest

import oracle

RTOL = 1e-12


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, rtol=RTOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / scale
    assert err <= rtol, "relative error %.3e > %.1e" % (err, rtol)


# --------------------------------------------------------------------------
# Closed forms (numpy fp64 matrix products)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [1.0, 0.375])
def test_linear_parallel_form(scale):
    """Ungated: O = Q S0 + tril(Q K^T) V and S_T = S0 + K^T V (causal linear
    attention without normaliser, Katharopoulos et al., the parallel form the
    pages' references give for linear attention)."""
    T, ntiles, dk, dv = 7, 3, 3, 5
    S0 = _rand(1, ntiles, dk, dv)
    q, k, v = _rand(2, T, ntiles, dk), _unit_rows(_rand(3, T, ntiles, dk)), _rand(4, T, ntiles, dv)
    out, S = oracle.recurrent(0, S0, q, k, v, scale=scale)
    for j in range(ntiles):
        Q, K, V = scale * q[:, j], k[:, j], v[:, j]
        _close(out[:, j], Q @ S0[j] + np.tril(Q @ K.T) @ V)
        _close(S[j], S0[j] + K.T @ V)


def test_gated_parallel_form():
    """Scalar gate: O = diag(e^b) Q S0 + (tril(Q K^T) * D) V with
    D[t, i] = exp(b_t - b_i), b = cumsum(g); S_T = e^{b_T} S0 + K^T diag(e^{b_T - b}) V
    (the decayed parallel form of RetNet / Mamba-2 style scalar decay)."""
    T, ntiles, dk, dv = 9, 2, 4, 3
    S0 = _rand(5, ntiles, dk, dv)
    q, k, v = _rand(6, T, ntiles, dk), _unit_rows(_rand(7, T, ntiles, dk)), _rand(8, T, ntiles, dv)
    g = np.random.default_rng(9).uniform(-0.3, 0.0, size=(T, ntiles))
    out, S = oracle.recurrent(1, S0, q, k, v, g=g)
    for j in range(ntiles):
        Q, K, V = q[:, j], k[:, j], v[:, j]
        b = np.cumsum(g[:, j])
        D = np.exp(b[:, None] - b[None, :])
        _close(out[:, j], np.exp(b)[:, None] * (Q @ S0[j]) + (np.tril(Q @ K.T) * D) @ V)
        _close(S[j], np.exp(b[-1]) * S0[j] + K.T @ (np.exp(b[-1] - b)[:, None] * V))


def test_channel_gate_parallel_form():
    """One log-gate per key channel: with B = cumsum(g) over the tokens (a
    vector per token), O[t] = (e^{B_t} * q_t) S0 + sum_{i<=t} (q_t * e^{B_t - B_i}) . k_i  v_i
    and S_T = diag(e^{B_T}) S0 + sum_i (e^{B_T - B_i} * k_i) v_i^T (the decayed
    parallel form of gated linear attention, reference [20] of the page).
    d_k != d_v, so decaying columns instead of rows fails."""
    T, ntiles, dk, dv = 8, 2, 4, 3
    S0 = _rand(50, ntiles, dk, dv)
    q, k, v = _rand(51, T, ntiles, dk), _unit_rows(_rand(52, T, ntiles, dk)), _rand(53, T, ntiles, dv)
    g = np.random.default_rng(54).uniform(-0.4, 0.0, size=(T, ntiles, dk))
    out, S = oracle.recurrent(3, S0, q, k, v, g=g, scale=0.5)
    for j in range(ntiles):
        Q, K, V = 0.5 * q[:, j], k[:, j], v[:, j]
        B = np.cumsum(g[:, j], axis=0)  # [T, dk]
        W = np.exp(B[:, None, :] - B[None, :, :])  # [t, i, dk]
        A = np.einsum("tr,tir,ir->ti", Q, W, K) * np.tri(T)
        _close(out[:, j], (np.exp(B) * Q) @ S0[j] + A @ V)
        _close(S[j], np.exp(B[-1])[:, None] * S0[j] + (np.exp(B[-1] - B) * K).T @ V)


def test_channel_gate_equal_channels_is_scalar_gate():
    T, ntiles, dk, dv = 6, 3, 3, 5
    S0 = _rand(55, ntiles, dk, dv)
    q, k, v = _rand(56, T, ntiles, dk), _rand(57, T, ntiles, dk), _rand(58, T, ntiles, dv)
    g = np.random.default_rng(59).uniform(-0.3, 0.0, size=(T, ntiles))
    o1, S1 = oracle.recurrent(1, S0, q, k, v, g=g)
    o3, S3 = oracle.recurrent(3, S0, q, k, v, g=np.repeat(g[:, :, None], dk, axis=2))
    _close(o3, o1, 1e-14)
    _close(S3, S1, 1e-14)


def test_channel_gate_closes_one_channel():
    """A very negative gate on channel r wipes row r of the state each step:
    after any token, row r is exactly k_t[r] v_t, and the other rows are
    untouched by that channel's gate."""
    T, ntiles, dk, dv = 4, 1, 3, 2
    S0 = _rand(60, ntiles, dk, dv)
    q, k, v = _rand(61, T, ntiles, dk), _rand(62, T, ntiles, dk), _rand(63, T, ntiles, dv)
    g = np.zeros((T, ntiles, dk))
    g[:, :, 1] = -800.0  # exp underflows to 0
    _, S = oracle.recurrent(3, S0, q, k, v, g=g)
    _close(S[0, 1], k[-1, 0, 1] * v[-1, 0], 1e-15)
    _close(S[0, [0, 2]], S0[0, [0, 2]] + k[:, 0, [0, 2]].T @ v[:, 0])


def test_gate_zero_is_ungated():
    T, ntiles, dk, dv = 6, 2, 3, 4
    S0 = _rand(10, ntiles, dk, dv)
    q, k, v = _rand(11, T, ntiles, dk), _rand(12, T, ntiles, dk), _rand(13, T, ntiles, dv)
    o1, S1 = oracle.recurrent(1, S0, q, k, v, g=np.zeros((T, ntiles)))
    o0, S0_ = oracle.recurrent(0, S0, q, k, v)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(S1, S0_)


def test_delta_beta_zero_is_pure_decay():
    """beta = 0: nothing is written, S_t = e^{b_t} S0 and o_t = e^{b_t} S0^T q_t."""
    T, ntiles, dk, dv = 5, 2, 4, 3
    S0 = _rand(14, ntiles, dk, dv)
    q, k, v = _rand(15, T, ntiles, dk), _unit_rows(_rand(16, T, ntiles, dk)), _rand(17, T, ntiles, dv)
    g = np.random.default_rng(18).uniform(-0.2, 0.0, size=(T, ntiles))
    out, S = oracle.recurrent(2, S0, q, k, v, g=g, beta=np.zeros((T, ntiles)))
    for j in range(ntiles):
        b = np.cumsum(g[:, j])
        _close(out[:, j], np.exp(b)[:, None] * (q[:, j] @ S0[j]))
        _close(S[j], np.exp(b[-1]) * S0[j])


def test_delta_orthonormal_keys_store_latest_values():
    """gamma = beta = 1 and orthonormal keys: after writing T <= d_k tokens,
    reading along key i returns exactly v_i (the delta rule replaces the value
    stored under a key; DeltaNet's defining property)."""
    dk, dv, ntiles = 5, 3, 2
    T = dk
    S0 = _rand(19, ntiles, dk, dv)
    k = np.empty((T, ntiles, dk))
    for j in range(ntiles):
        Qm, _ = np.linalg.qr(_rand(20 + j, dk, dk))
        k[:, j] = Qm.T[:T]
    q, v = _rand(22, T, ntiles, dk), _rand(23, T, ntiles, dv)
    _, S = oracle.recurrent(2, S0, q, k, v, g=np.zeros((T, ntiles)), beta=np.ones((T, ntiles)))
    for j in range(ntiles):
        for i in range(T):
            _close(S[j].T @ k[i, j], v[i, j], rtol=1e-12)


def test_delta_one_step_retrieval():
    """Unit key k_t: S_t^T k_t = gamma_t (1 - beta_t) S_{t-1}^T k_t + beta_t v_t."""
    T, ntiles, dk, dv = 6, 3, 4, 5
    S0 = _rand(24, ntiles, dk, dv)
    q, k, v = _rand(25, T, ntiles, dk), _unit_rows(_rand(26, T, ntiles, dk)), _rand(27, T, ntiles, dv)
    g = np.random.default_rng(28).uniform(-0.3, 0.0, size=(T, ntiles))
    beta = np.random.default_rng(29).uniform(0.0, 1.0, size=(T, ntiles))
    _, Sprev = oracle.recurrent(2, S0, q[:-1], k[:-1], v[:-1], g=g[:-1], beta=beta[:-1])
    _, S = oracle.recurrent(2, S0, q, k, v, g=g, beta=beta)
    t = T - 1
    for j in range(ntiles):
        lhs = S[j].T @ k[t, j]
        rhs = math.exp(g[t, j]) * (1 - beta[t, j]) * (Sprev[j].T @ k[t, j]) + beta[t, j] * v[t, j]
        _close(lhs, rhs)


def test_delta_matches_explicit_projection():
    """Rule 2 against the explicit d_k x d_k matrix gamma (I - beta k k^T) S + beta k v^T."""
    T, ntiles, dk, dv = 5, 2, 4, 3
    S0 = _rand(30, ntiles, dk, dv)
    q, k, v = _rand(31, T, ntiles, dk), _unit_rows(_rand(32, T, ntiles, dk)), _rand(33, T, ntiles, dv)
    g = np.random.default_rng(34).uniform(-0.3, 0.0, size=(T, ntiles))
    beta = np.random.default_rng(35).uniform(0.0, 1.0, size=(T, ntiles))
    out, S = oracle.recurrent(2, S0, q, k, v, g=g, beta=beta)
    for j in range(ntiles):
        St = S0[j].copy()
        for t in range(T):
            P = np.eye(dk) - beta[t, j] * np.outer(k[t, j], k[t, j])
            St = math.exp(g[t, j]) * (P @ St) + beta[t, j] * np.outer(k[t, j], v[t, j])
            _close(out[t, j], St.T @ q[t, j])
        _close(S[j], St)


# --------------------------------------------------------------------------
# Exact rational chunkwise form vs the oracle's fp64 recurrence
# --------------------------------------------------------------------------

def _exact_inputs(seed, T, dk, dv, rule):
    rs = np.random.default_rng(seed)
    S0 = rs.integers(-4, 5, size=(dk, dv)) / 8.0
    q = rs.integers(-4, 5, size=(T, dk)) / 4.0
    k = rs.integers(-4, 5, size=(T, dk)) / 8.0
    v = rs.integers(-4, 5, size=(T, dv)) / 4.0
    if rule == 3:
        g = rs.uniform(-0.2, 0.0, size=(T, dk))
    else:
        g = rs.uniform(-0.2, 0.0, size=T) if rule >= 1 else np.zeros(T)
    beta = rs.integers(0, 5, size=T) / 4.0 if rule == 2 else np.zeros(T)
    return S0, q, k, v, g, beta


def _gam(rule, g):
    """exp(g) as exact Fractions: a scalar, or a vector for rule 3."""
    if rule == 3:
        return [F(math.exp(x)) for x in g]
    return F(math.exp(g)) if rule >= 1 else F(1)


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("m", [1, 3, 4])
def test_oracle_equals_exact_buffered_form(rule, m):
    """Exact (Fraction) buffered evaluation -- fold every m tokens, outputs from
    the folded state plus the decayed causal sum over the buffer -- agrees with
    the oracle's fp64 per-token recurrence to fp64 rounding."""
    from tests.exact import ExactKVBuffer

    T, dk, dv = 11, 3, 4
    S0, q, k, v, g, beta = _exact_inputs(40 + rule + 3 * m, T, dk, dv, rule)
    out, S = oracle.recurrent(rule, S0[None], q[:, None], k[:, None], v[:, None],
                              g=g[:, None], beta=beta[:, None], scale=0.5)
    ex = ExactKVBuffer(rule, [[F(x) for x in row] for row in S0], m, scale=F(1, 2))
    for t in range(T):
        o = ex.decode([F(x) for x in q[t]], [F(x) for x in k[t]], [F(x) for x in v[t]],
                      _gam(rule, g[t]), F(beta[t]))
        _close(out[t, 0], [float(x) for x in o])
    _close(S[0], [[float(x) for x in row] for row in ex.effective_state()])


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_oracle_serial_decode_equals_exact_parallel_verify(rule):
    """Drafts verified in parallel from the buffer (exact) equal the oracle's
    serial decode of the drafts from the current state."""
    from tests.exact import ExactKVBuffer

    T, n, dk, dv = 5, 4, 3, 3
    S0, q, k, v, g, beta = _exact_inputs(60 + rule, T + n, dk, dv, rule)
    Fr = lambda a: [F(x) for x in a]
    ex = ExactKVBuffer(rule, [Fr(row) for row in S0], m=8)
    for t in range(T):
        ex.decode(Fr(q[t]), Fr(k[t]), Fr(v[t]), _gam(rule, g[t]), F(beta[t]))
    outs = ex.verify([Fr(q[t]) for t in range(T, T + n)], [Fr(k[t]) for t in range(T, T + n)],
                     [Fr(v[t]) for t in range(T, T + n)],
                     [_gam(rule, g[t]) for t in range(T, T + n)],
                     [F(beta[t]) for t in range(T, T + n)])
    out, _ = oracle.recurrent(rule, S0[None], q[:, None], k[:, None], v[:, None],
                              g=g[:, None], beta=beta[:, None])
    for d in range(n):
        _close(out[T + d, 0], [float(x) for x in outs[d]])


# --------------------------------------------------------------------------
# The output magnitude |S_t|^T |scale q_t| (the scale output errors are
# measured against): triangle inequality, equality when every term is
# non-negative, and homogeneity in the query scale.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_magnitude_bounds_the_output(rule):
    T, ntiles, dk, dv = 6, 3, 4, 5
    rs = np.random.default_rng(70 + rule)
    S0 = rs.standard_normal((ntiles, dk, dv))
    q, k = rs.standard_normal((T, ntiles, dk)), _unit_rows(rs.standard_normal((T, ntiles, dk)))
    v = rs.standard_normal((T, ntiles, dv))
    g = rs.uniform(-0.1, 0.0, (T, ntiles, dk) if rule == 3 else (T, ntiles))
    beta = rs.uniform(0.0, 1.0, (T, ntiles))
    out, _, mag = oracle.recurrent(rule, S0, q, k, v, g=g, beta=beta, scale=-0.75, with_magnitude=True)
    assert np.all(mag >= np.abs(out) * (1 - 1e-12))
    # cancellation makes the output smaller than its magnitude somewhere
    assert np.max(mag - np.abs(out)) > 0.1
    _, _, mag1 = oracle.recurrent(rule, S0, q, k, v, g=g, beta=beta, scale=1.5, with_magnitude=True)
    _close(mag1, 2.0 * mag)


@pytest.mark.parametrize("rule", [0, 1, 3])
def test_magnitude_equals_output_without_cancellation(rule):
    """Non-negative state, queries, keys and values: every term of every
    output is non-negative, so the output equals its magnitude."""
    T, ntiles, dk, dv = 5, 2, 3, 4
    rs = np.random.default_rng(80 + rule)
    S0 = rs.uniform(0, 1, (ntiles, dk, dv))
    q, k, v = (rs.uniform(0, 1, (T, ntiles, n)) for n in (dk, dk, dv))
    g = rs.uniform(-0.1, 0.0, (T, ntiles, dk) if rule == 3 else (T, ntiles))
    out, _, mag = oracle.recurrent(rule, S0, q, k, v, g=g, with_magnitude=True)
    _close(mag, out)
