"""Precision guards for the matrix-core paths, with bounds tighter than the
workload tolerances (2e-3 on outputs, 1e-5 on states), which those paths meet
by a wide margin and which could not see a lost operand term.

Verification of 2-8 drafts, d = 128, bf16.  The four- and eight-draft kernels
form S0^T q on the matrix cores with the fp32 state entering as two exact bf16
terms, hi = bf16(S) and lo = bf16(S - hi), which carry S to about 2^-17 of its
size.  With a large state (std 1) at occupancy 0 the output is almost all
S0^T q.  Bound: per tile max|o_gpu - o_ref| / max|o_ref| <= 2e-5.  On these
inputs the two-term product sits at about 4e-6 and fp32 sums of exact
products at about 5e-7, while a product with the hi term alone (lo dropped)
errs by about 3e-3 (tests/test_precision_model.py computes all three on the
host from the same seeded inputs).

Folds of more than 32 positions, d = 128.  The rank-T update runs on the
matrix cores with its fp32 operand (weighted keys, or the delta rule's
pseudo-values) entering as three bf16 terms hi, mid, lo (about 2^-27).  With a
zero initial state the stored state is the update alone.  Bound: per tile
max|S_gpu - S_ref| / max|S_ref| <= 2e-6, above the fp32 accumulation error of
exact products (about 2e-7) and below what the update gives without its lo
term (about 5e-6) or its mid term (about 2e-3), both computed on the host by
the same model test.
"""

import numpy as np
import pytest
import torch

import synth
import linear_attention_decode_kvbuf_amd as kb
from tests.harness import Run

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

VERIFY_BOUND = 2e-5
FOLD_BOUND = 2e-6


def verify_guard_workload():
    """Verification workload shape (m = 8, gated, bf16, d = 128) with a state
    of std 1; 64 tiles, inputs drawn on the host."""
    return synth.workload(4, B=16, H=4, state_std=1.0)


def fold_guard_workload(rule, m):
    """m buffered tokens folded into a zero state, d = 128, bf16 inputs."""
    return synth.workload(1, B=4, H=2, dk=128, dv=128, m=m, block_size=m, blocks_per_req=2, steps=m + 4,
                          rule=rule, io="bf16", state_std=0.0)


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("tree", [False, True])
def test_verify_state_products_precision(n, tree):
    w = verify_guard_workload()
    run = Run(w, tol_out=VERIFY_BOUND, out_scale="output")
    assert not run.device_gen
    for call in range(3):  # occupancy 0, then wherever the commits leave it
        if tree:
            parent, leaf = synth.draft_tree(w, call, w.B, n)
            run.verify_tree_commit(call, parent, leaf)
        else:
            run.verify_commit(call, n, synth.accepted_lengths(w, call, w.B, n))
    print("n %d tree %s: max output error %.2e (bound %.0e)" % (n, tree, run.max_out, VERIFY_BOUND), flush=True)


@pytest.mark.parametrize("rule", [kb.RULE_LINEAR, kb.RULE_GATED, kb.RULE_DELTA])
@pytest.mark.parametrize("m", [64, 128])
def test_multi_round_fold_precision(rule, m):
    w = fold_guard_workload(rule, m)
    run = Run(w, flush=kb.FLUSH_DEFERRED, tol_state=FOLD_BOUND)
    for t in range(m):
        run.decode(t)
    run.flush()  # the fold of all m positions, compared for every tile at FOLD_BOUND
    assert run.full_state_checks == 1 and run.folds_checked == w.B * w.H
    for t in range(m, m + 4):
        run.decode(t)
    print("rule %d m %d: max state error %.2e (bound %.0e)" % (rule, m, run.max_state, FOLD_BOUND), flush=True)
