"""The method's three exactness claims, brute-forced in rational arithmetic.

KVBuffer: IO-aware Serving for Linear Attention (pith.science page):
  * "Core claim" / "What would settle it": deferring the state update and
    computing outputs from the state plus buffered keys and values gives the
    same results as the per-token recurrence;
  * Figure 2 caption: drafts are verified from the buffer without temporary
    states; keeping the accepted prefix must leave the request exactly where a
    serial decode of that prefix would;
  * abstract, short contexts: outputs computed from the buffered keys and values
    alone, never creating a state, equal the recurrence started from zero.

All comparisons are exact equality of Fractions (d <= 4, a few dozen tokens).
"""

import random
from fractions import Fraction as F

import pytest

from tests.exact import ExactKVBuffer, exact_recurrent, zeros


def _seq(seed, T, dk, dv, rule, zero_state=False):
    r = random.Random(seed)
    fr = lambda lo, hi, den: F(r.randint(lo, hi), den)
    S0 = zeros(dk, dv) if zero_state else [[fr(-3, 3, 4) for _ in range(dv)] for _ in range(dk)]
    q = [[fr(-3, 3, 2) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-3, 3, 4) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-3, 3, 2) for _ in range(dv)] for _ in range(T)]
    if rule == 3:  # one decay per key channel
        gam = [[fr(4, 8, 8) for _ in range(dk)] for _ in range(T)]
    else:
        gam = [fr(5, 8, 8) if rule >= 1 else F(1) for _ in range(T)]
    beta = [fr(0, 4, 4) if rule == 2 else F(0) for _ in range(T)]
    return S0, q, k, v, gam, beta


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_buffered_decode_equals_recurrent(rule, m):
    T, dk, dv = 12, 3, 2
    S0, q, k, v, gam, beta = _seq(100 + 10 * rule + m, T, dk, dv, rule)
    ref_o, ref_S = exact_recurrent(rule, S0, q, k, v, gam, beta)
    ex = ExactKVBuffer(rule, S0, m)
    for t in range(T):
        o = ex.decode(q[t], k[t], v[t], gam[t], beta[t])
        assert o == ref_o[t]
        assert ex.effective_state() == ref_S[t]
        if (t + 1) % m == 0:
            assert ex.buf == [] and ex.S == ref_S[t]  # folded state written back exactly


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("n", [1, 2, 4])
def test_verify_then_commit_equals_serial_prefix(rule, n):
    m, pre, dk, dv = 4, 3, 2, 3
    for a in range(n + 1):
        S0, q, k, v, gam, beta = _seq(200 + 10 * rule + n, pre + n + 3, dk, dv, rule)
        ex = ExactKVBuffer(rule, S0, m)
        for t in range(pre):
            ex.decode(q[t], k[t], v[t], gam[t], beta[t])
        sl = slice(pre, pre + n)
        outs = ex.verify(q[sl], k[sl], v[sl], gam[sl], beta[sl])
        # every draft's output equals the serial decode of the drafts before it
        ref_o, _ = exact_recurrent(rule, S0, q[: pre + n], k[: pre + n], v[: pre + n],
                                   gam[: pre + n], beta[: pre + n])
        assert outs == ref_o[pre:pre + n]
        ex.commit(a)
        # the request now continues exactly as if only the accepted prefix had been decoded
        keep = list(range(pre + a)) + list(range(pre + n, pre + n + 3))
        pick = lambda xs: [xs[i] for i in keep]
        ref_o2, ref_S2 = exact_recurrent(rule, S0, pick(q), pick(k), pick(v), pick(gam), pick(beta))
        assert ex.effective_state() == ref_S2[pre + a - 1] if pre + a > 0 else True
        for j, t in enumerate(range(pre + n, pre + n + 3)):
            assert ex.decode(q[t], k[t], v[t], gam[t], beta[t]) == ref_o2[pre + a + j]


def test_commit_nothing_is_a_no_op():
    S0, q, k, v, gam, beta = _seq(300, 6, 2, 2, 1)
    ex = ExactKVBuffer(1, S0, 4)
    for t in range(3):
        ex.decode(q[t], k[t], v[t], gam[t], beta[t])
    before = (ex.S, list(ex.buf))
    ex.verify(q[3:5], k[3:5], v[3:5], gam[3:5], beta[3:5])
    ex.commit(0)
    assert (ex.S, ex.buf) == before


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_direct_equals_recurrence_from_zero(rule):
    """Buffer-only attention with no state at all (S = 0, never folded) equals
    the recurrence started from a zero state."""
    T, dk, dv = 10, 3, 3
    S0, q, k, v, gam, beta = _seq(400 + rule, T, dk, dv, rule, zero_state=True)
    ref_o, ref_S = exact_recurrent(rule, S0, q, k, v, gam, beta)
    ex = ExactKVBuffer(rule, S0, m=0)  # m = 0 here: never fold
    for t in range(T):
        assert ex.decode(q[t], k[t], v[t], gam[t], beta[t]) == ref_o[t]
    # promoting it to a stateful request: folding everything gives the recurrent state
    ex.m = T
    ex.fold()
    assert ex.S == ref_S[-1]


def test_m1_is_recurrent():
    S0, q, k, v, gam, beta = _seq(500, 5, 2, 2, 2)
    ref_o, ref_S = exact_recurrent(2, S0, q, k, v, gam, beta)
    ex = ExactKVBuffer(2, S0, 1)
    for t in range(5):
        assert ex.decode(q[t], k[t], v[t], gam[t], beta[t]) == ref_o[t]
        assert ex.S == ref_S[t] and ex.buf == []


def _tree(seed, n):
    """A random draft tree: parent[d] in {-1 (the buffer), 0 .. d-1}."""
    r = random.Random(seed)
    return [r.randint(-1, d - 1) for d in range(n)]


def _path_to(parent, d):
    path = []
    while d >= 0:
        path.append(d)
        d = parent[d]
    return path[::-1]


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_verify_equals_serial_path_and_commit_keeps_it(rule, seed):
    """Every node of a draft tree, verified from the buffer, equals the serial
    decode of its root-to-node path; committing one path leaves the request
    exactly where a serial decode of that path would (the page's reference
    list includes tree speculative decoding for state-space models)."""
    m, pre, n, dk, dv = 5, 3, 6, 2, 3
    parent = _tree(600 + seed, n)
    S0, q, k, v, gam, beta = _seq(700 + 10 * rule + seed, pre + n + 3, dk, dv, rule)
    ex = ExactKVBuffer(rule, S0, m)
    for t in range(pre):
        ex.decode(q[t], k[t], v[t], gam[t], beta[t])
    sl = slice(pre, pre + n)
    outs = ex.verify_tree(q[sl], k[sl], v[sl], gam[sl], beta[sl], parent)
    for d in range(n):
        idx = list(range(pre)) + [pre + a for a in _path_to(parent, d)]
        pick = lambda xs: [xs[i] for i in idx]
        ref_o, _ = exact_recurrent(rule, S0, pick(q), pick(k), pick(v), pick(gam), pick(beta))
        assert outs[d] == ref_o[-1], d
    leaf = max(range(n), key=lambda d: len(_path_to(parent, d)))
    path = _path_to(parent, leaf)
    ex.commit_path(path)
    idx = list(range(pre)) + [pre + a for a in path] + list(range(pre + n, pre + n + 3))
    pick = lambda xs: [xs[i] for i in idx]
    ref_o, ref_S = exact_recurrent(rule, S0, pick(q), pick(k), pick(v), pick(gam), pick(beta))
    assert ex.effective_state() == ref_S[pre + len(path) - 1]
    for j, t in enumerate(range(pre + n, pre + n + 3)):
        assert ex.decode(q[t], k[t], v[t], gam[t], beta[t]) == ref_o[pre + len(path) + j]


def test_chain_tree_is_parallel_verify():
    n = 4
    S0, q, k, v, gam, beta = _seq(800, 2 + n, 2, 2, 1)
    a, b = ExactKVBuffer(1, S0, 8), ExactKVBuffer(1, S0, 8)
    for t in range(2):
        a.decode(q[t], k[t], v[t], gam[t], beta[t])
        b.decode(q[t], k[t], v[t], gam[t], beta[t])
    sl = slice(2, 2 + n)
    assert a.verify(q[sl], k[sl], v[sl], gam[sl], beta[sl]) == \
        b.verify_tree(q[sl], k[sl], v[sl], gam[sl], beta[sl], [d - 1 for d in range(n)])
