"""Host model of the operand splits the matrix-core paths use, on the seeded
inputs of the GPU precision guards (tests/test_gpu_precision.py): each guard's
bound separates the split as built from the same split with a term dropped.

* Verification: S0^T q with the fp32 state as bf16 hi + lo terms.  The
  oracle's outputs are linear in S0 for fixed drafts, so running the oracle
  from hi (or hi + lo) in place of S0 gives exactly what a product with that
  representation of the state computes, up to fp64 rounding.
* Folds of more than 32 positions: the rank-T update sum_i (w_i k_i) x_i^T
  with the fp32 weighted keys as bf16 hi + mid + lo terms (the delta rule
  splits its weighted pseudo-values the same way against exact keys).

bf16 rounding is round-to-nearest-even, as the device conversion does.
"""

import numpy as np
import pytest

import oracle
import synth
from tests.test_gpu_precision import FOLD_BOUND, VERIFY_BOUND, fold_guard_workload, verify_guard_workload


def _bf(x):
    return synth.bf16_round(np.asarray(x, np.float32)).astype(np.float64)


def _tile_rel(a, b):
    """max over tiles of max|a - b| / max|b|, a and b [tiles, ...]."""
    a = a.reshape(a.shape[0], -1)
    b = b.reshape(b.shape[0], -1)
    return float(np.max(np.max(np.abs(a - b), axis=1) / np.max(np.abs(b), axis=1)))


def _guard_state(w):
    """Initial states of the GPU guard's tiles, request-major, as the harness
    places them (a seeded permutation of the slots)."""
    nslots = w.B + 1
    pool = synth.initial_state(w, nslots)
    slots = synth.slot_permutation(w, nslots)[: w.B]
    return pool[slots].reshape(w.B * w.H, w.dk, w.dv).astype(np.float64)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_verify_bound_separates_the_state_split(n):
    w = verify_guard_workload()
    S0 = _guard_state(w)
    inp = synth.token_inputs(w, 0, n=n, stream_base=100)  # the first call: occupancy 0
    drafts = lambda x: np.swapaxes(x, 1, 2).reshape(w.B * w.H, n, *x.shape[3:]).swapaxes(0, 1)
    args = [drafts(inp[k]) for k in ("q", "k", "v", "g")]
    exact, _ = oracle.recurrent(1, S0, *args)
    hi = _bf(S0)
    lo = _bf(S0 - hi)
    two_terms, _ = oracle.recurrent(1, hi + lo, *args)
    hi_only, _ = oracle.recurrent(1, hi, *args)
    err2 = _tile_rel(np.swapaxes(two_terms, 0, 1), np.swapaxes(exact, 0, 1))
    err1 = _tile_rel(np.swapaxes(hi_only, 0, 1), np.swapaxes(exact, 0, 1))
    print("n %d: hi + lo %.2e, hi alone %.2e, bound %.0e" % (n, err2, err1, VERIFY_BOUND))
    assert err2 < VERIFY_BOUND / 2
    assert err1 > 20 * VERIFY_BOUND


def _split3(x):
    h = _bf(x)
    m = _bf(x - h)
    lo = _bf(x - h - m)
    return h, m, lo


def test_fold_bound_separates_the_operand_split():
    """Gated rule, m = 64 and 128, the GPU guard's inputs: weights
    exp(b_{T-1} - b_i) in fp32, weighted keys in fp32, values exact bf16."""
    for m in (64, 128):
        w = fold_guard_workload(1, m)
        steps = [synth.token_inputs(w, t) for t in range(m)]
        tiles = w.B * w.H
        k = np.stack([s["k"].reshape(tiles, w.dk) for s in steps], axis=1).astype(np.float64)  # [tiles, m, d]
        v = np.stack([s["v"].reshape(tiles, w.dv) for s in steps], axis=1).astype(np.float64)
        g = np.stack([s["g"].reshape(tiles) for s in steps], axis=1).astype(np.float64)
        b = np.cumsum(g, axis=1)
        wt = np.exp(b[:, -1:] - b).astype(np.float32)
        wk = (wt[:, :, None] * k.astype(np.float32)).astype(np.float64)  # fp32 products
        exact = np.einsum("tir,tic->trc", wk, v)
        h, mid, lo = _split3(wk)
        full = np.einsum("tir,tic->trc", h + mid + lo, v)
        no_lo = np.einsum("tir,tic->trc", h + mid, v)
        no_mid = np.einsum("tir,tic->trc", h + lo, v)
        # fp32 accumulation of the exact products, position by position
        acc = np.zeros((tiles, w.dk, w.dv), np.float32)
        for i in range(m):
            acc = (acc + (wk[:, i, :, None] * v[:, i, None, :]).astype(np.float32)).astype(np.float32)
        e_full, e_acc = _tile_rel(full, exact), _tile_rel(acc.astype(np.float64), exact)
        e_lo, e_mid = _tile_rel(no_lo, exact), _tile_rel(no_mid, exact)
        print("m %d: three terms %.2e, fp32 sums %.2e, without lo %.2e, without mid %.2e, bound %.0e"
              % (m, e_full, e_acc, e_lo, e_mid, FOLD_BOUND))
        assert e_full < 1e-12
        assert e_acc < FOLD_BOUND / 4
        assert e_lo > 1.5 * FOLD_BOUND
        assert e_mid > 100 * FOLD_BOUND
