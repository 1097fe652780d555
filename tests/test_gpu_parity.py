"""GPU parity: the HIP library (called through its C ABI) against the oracle.

Every test drives seeded synthetic inputs through kvbuf_* and through the
fp64 per-token recurrence, and compares outputs at every step, stored states
after every fold, effective states, and the bookkeeping (block tables,
occupancies, buffered bits) exactly.  Every (request, head) tile is compared,
at the full-size workloads too (their stored states: every tile at the first
and the last fold, a rotating subset at the folds in between).
"""

import numpy as np
import pytest
import torch

import synth
import linear_attention_decode_kvbuf_amd as kb
from tests.harness import Run

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# Tiny workload: fp32, B=2 H=2 d=16 m=4, 32 steps, state from zero.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("flush", [kb.FLUSH_EAGER, kb.FLUSH_DEFERRED])
def test_tiny_every_step(flush):
    w = synth.workload(1)
    _say("tiny workload", w, "flush", flush)
    run = Run(w, flush=flush)
    for t in range(w.steps):
        run.decode(t)
        if flush == kb.FLUSH_DEFERRED:
            run.flush()
        run.check_effective_states()
        run.check_pool()
    assert run.folds_checked == w.B * w.H * (w.steps // w.m)
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("d,io", [(16, "f32"), (64, "bf16"), (128, "bf16"), (128, "f32")])
@pytest.mark.parametrize("m,bs,bpr", [(4, 4, 2), (4, 2, 3), (1, 1, 3), (6, 3, 3)])
def test_small_rules(rule, d, io, m, bs, bpr):
    w = synth.workload(1, B=3, H=2, dk=d, dv=d, m=m, block_size=bs, blocks_per_req=bpr, steps=13,
                       rule=rule, io=io, state_std=0.02)
    _say("small", w)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [1, 3])
@pytest.mark.parametrize("m,bs,bpr,flush", [(8, 1, 64, kb.FLUSH_EAGER), (6, 2, 33, kb.FLUSH_DEFERRED),
                                             (6, 2, 33, kb.FLUSH_EAGER), (64, 8, 8, kb.FLUSH_EAGER)])
def test_long_table_rows(rule, m, bs, bpr, flush):
    """Table rows up to the 64-entry limit: the fold's rotation moves m / bs
    entries of a long row (five requests, so the bookkeeping spans more than
    one workgroup); rows of 66 positions run the chunk kernel (gated rule) or
    the per-channel kernel, eager folds in the launch that follows."""
    w = synth.workload(1, B=5, H=2, dk=16, dv=16, m=m, block_size=bs, blocks_per_req=bpr,
                       steps=2 * m + 3, rule=rule, io="f32", state_std=0.02)
    _say("long rows", w, "flush", flush)
    run = Run(w, flush=flush)
    for t in range(w.steps):
        run.decode(t)
        if flush == kb.FLUSH_DEFERRED and t % 5 == 4:
            run.flush()
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("flush", [kb.FLUSH_EAGER, kb.FLUSH_DEFERRED])
def test_long_folds(rule, io, flush):
    """Folds and materialisations of more than 32 positions at d = 128 (the
    rank-T update on the matrix cores): eager folds of m = 48 where they do
    not fit the decode kernel (per-channel and delta rules, fp32 rows),
    deferred flushes of 48 with a tail behind them, and effective states of
    up to 50 buffered positions."""
    w = synth.workload(1, B=3, H=2, dk=128, dv=128, m=48, block_size=16, blocks_per_req=4, steps=150,
                       rule=rule, io=io, state_std=0.02)
    _say("long folds", w, "flush", flush)
    run = Run(w, flush=flush)
    for t in range(w.steps):
        run.decode(t)
        if flush == kb.FLUSH_DEFERRED and t % 50 == 49:
            run.flush()
        if t % 25 == 24:
            run.check_effective_states()
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2])
@pytest.mark.parametrize("m", [24, 32])
def test_single_round_matrix_core_folds(rule, m):
    """Folds of 17-32 positions at d = 128 through the fold kernel: one
    staging round on the matrix cores, in four-wave workgroups whose decay
    weights come from their second wave.  Deferred flushes of m = 24 / 32
    (a partial and a full round), then eager commits and tree commits that
    fill the buffer."""
    w = synth.workload(1, B=3, H=2, dk=128, dv=128, m=m, block_size=8, blocks_per_req=8, steps=2 * m + 4,
                       rule=rule, io="bf16", state_std=0.02)
    _say("single-round folds", w)
    run = Run(w, flush=kb.FLUSH_DEFERRED)
    for t in range(w.steps):
        run.decode(t)
        if t % m == m - 1:
            run.flush()
            run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    # eager commits: the buffer fills inside kvbuf_commit
    we = synth.workload(1, B=4, H=2, dk=128, dv=128, m=m, block_size=8, blocks_per_req=8, steps=12,
                        rule=rule, io="bf16", state_std=0.02)
    rune = Run(we)
    t = 0
    for call in range(12):
        rune.decode(t)
        t += 1
        rune.verify_commit(call, 8, synth.accepted_lengths(we, call, we.B, 8))
        rune.check_effective_states()
    rune.check_pool()
    rune.check_bookkeeping()
    assert rune.folds_checked > 0
    # eager tree commits: kept rows move after the fold has read them
    runt = Run(we)
    t = 0
    for call in range(12):
        runt.decode(t)
        t += 1
        parent, leaf = synth.draft_tree(we, call, we.B, 8)
        runt.verify_tree_commit(call, parent, leaf)
        runt.check_effective_states()
    runt.check_pool()
    runt.check_bookkeeping()
    assert runt.folds_checked > 0


@pytest.mark.parametrize("rule,d", [(1, 64), (2, 64), (3, 64), (1, 16), (2, 16)])
def test_long_folds_small_dims(rule, d):
    """Folds of 48 positions at d = 64 and 16: several staging rounds of fp32
    rows on the vector ALUs (the matrix-core instances serve d = 128)."""
    w = synth.workload(1, B=3, H=2, dk=d, dv=d, m=48, block_size=16, blocks_per_req=4, steps=110,
                       rule=rule, io="bf16", state_std=0.02)
    _say("long folds small dims", w)
    run = Run(w, flush=kb.FLUSH_DEFERRED)
    for t in range(w.steps):
        run.decode(t)
        if t % 50 == 49:
            run.flush()
        if t % 25 == 24:
            run.check_effective_states()
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_deferred_flush_with_tail(rule):
    """Decode past m before folding: the fold takes the first m tokens and
    leaves the rest buffered in the rotated table."""
    w = synth.workload(1, B=2, H=3, dk=64, dv=64, m=4, block_size=2, blocks_per_req=5, steps=14,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w, flush=kb.FLUSH_DEFERRED)
    t = 0
    for burst in (6, 5, 3):
        for _ in range(burst):
            run.decode(t)
            t += 1
        run.check_effective_states()
        run.flush()
        run.check_effective_states()
        run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_recurrent_m0(rule):
    w = synth.workload(1, B=3, H=4, dk=128, dv=128, m=0, block_size=1, blocks_per_req=1, steps=9,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    st = run.kv.state.detach()
    for j, (b, h) in enumerate(run.sample):
        gpu = st[run.slots[b], h].double().cpu().numpy()
        ref = run.S[j]
        assert np.max(np.abs(gpu - ref)) / np.max(np.abs(ref)) <= 1e-5


@pytest.mark.parametrize("rule,n", [(r, n) for r in (0, 1, 2, 3) for n in (1, 3, 8)])
def test_verify_commit_small(rule, n):
    w = synth.workload(1, B=4, H=2, dk=64, dv=64, m=4, block_size=4, blocks_per_req=4, steps=6,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w)
    t = 0
    for call in range(6):
        run.decode(t)
        t += 1
        acc = synth.accepted_lengths(w, call, w.B, n)
        run.verify_commit(call, n, acc)
        run.check_effective_states()
        run.check_pool()
        run.check_bookkeeping()


@pytest.mark.parametrize("rule,d,io", [(0, 64, "bf16"), (1, 128, "bf16"), (2, 64, "bf16"), (1, 16, "f32"),
                                       (2, 128, "f32"), (3, 128, "bf16"), (3, 16, "f32")])
@pytest.mark.parametrize("n", [1, 5, 8])
def test_tree_verify_commit(rule, d, io, n):
    """Random draft trees: every draft's output is the recurrence over its
    root-to-node path; committing a path moves its rows to consecutive
    positions (pool bits and bookkeeping exact) and, when the buffer fills,
    folds them (states within tolerance)."""
    w = synth.workload(1, B=6, H=2, dk=d, dv=d, m=8, block_size=4, blocks_per_req=5, steps=8,
                       rule=rule, io=io, state_std=0.02)
    _say("tree", w, "n", n)
    run = Run(w)
    t = 0
    for call in range(8):
        run.decode(t)
        t += 1
        parent, leaf = synth.draft_tree(w, call, w.B, n)
        run.verify_tree_commit(call, parent, leaf)
        run.check_effective_states()
        run.check_pool()
        run.check_bookkeeping()


@pytest.mark.parametrize("rule,io", [(1, "bf16"), (2, "bf16"), (0, "f32")])
def test_tree_commit_long_fold(rule, io):
    """Tree commits that fill a buffer of m = 48 at d = 128: the commit's fold
    takes two staging rounds on the matrix cores (bf16 keys: the transposing
    reads; fp32 rows: the plain ones) while the kept drafts move to their
    path positions."""
    w = synth.workload(1, B=3, H=2, dk=128, dv=128, m=48, block_size=16, blocks_per_req=4, steps=60,
                       rule=rule, io=io, state_std=0.02)
    _say("tree long fold", w)
    run = Run(w)
    t = 0
    for call in range(12):
        for _ in range(4):
            run.decode(t)
            t += 1
        parent, leaf = synth.draft_tree(w, call, w.B, 8)
        run.verify_tree_commit(call, parent, leaf)
        run.check_effective_states()
        run.check_pool()
        run.check_bookkeeping()


@pytest.mark.parametrize("rule", [1, 2])
def test_tree_deferred_with_flush_and_stars(rule):
    """Deferred policy: tree commits only append; kvbuf_flush after each call
    folds the first m positions once the buffer holds m (leaving the rest of
    a commit buffered behind them).  Every third call is a star (every draft
    follows the buffer directly), whose paths keep at most one draft."""
    w = synth.workload(1, B=5, H=2, dk=64, dv=64, m=8, block_size=4, blocks_per_req=6, steps=9,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w, flush=kb.FLUSH_DEFERRED)
    n = 6
    for call in range(9):
        parent, leaf = synth.draft_tree(w, call, w.B, n)
        if call % 3 == 2:
            parent[:] = -1
        run.verify_tree_commit(call, parent, leaf)
        run.check_effective_states()
        run.flush()
        run.check_effective_states()
        run.check_pool()
        run.check_bookkeeping()


@pytest.mark.parametrize("rule", [1, 3])
@pytest.mark.parametrize("flush", [kb.FLUSH_EAGER, kb.FLUSH_DEFERRED])
def test_tree_chain_matches_verify(rule, flush):
    """A chain-shaped tree gives kvbuf_verify's outputs, and committing its
    first a drafts leaves the same pools as kvbuf_commit(a)."""
    w = synth.workload(1, B=4, H=2, dk=128, dv=128, m=8, block_size=4, blocks_per_req=4, steps=4,
                       rule=rule, io="bf16", state_std=0.02)
    runs = [Run(w, flush=flush), Run(w, flush=flush)]
    n = 6
    chain = np.tile(np.arange(-1, n - 1, dtype=np.int32), (w.B, 1))
    for call in range(4):
        acc = synth.accepted_lengths(w, call, w.B, n)
        o_chain = runs[0].verify_commit(call, n, acc)
        inp = runs[1].inputs(call, n=n, stream_base=100)
        par = torch.from_numpy(chain).to(runs[1].dev)
        o_tree = runs[1].kv.verify_tree(par, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        runs[1].kv.commit_tree(par, torch.from_numpy(acc - 1).to(runs[1].dev))
        torch.cuda.synchronize()
        # the tree path sums the drafts' gates one by one, the chain path by a
        # parallel scan: equal up to rounding
        torch.testing.assert_close(o_tree, o_chain, rtol=0, atol=1e-5 * float(o_chain.abs().max()))
        for name in ("state", "key", "value", "gate", "block_table", "occupancy", "tile_meta"):
            assert torch.equal(getattr(runs[0].kv, name), getattr(runs[1].kv, name)), name
        if flush == kb.FLUSH_DEFERRED:
            runs[0].flush()
            runs[1].kv.flush()


def test_tree_invalid_parent_or_leaf_skips_the_tile():
    """A parent outside {-1 .. d-1} or a leaf outside {-1 .. n-1} sets the
    draft-range error bit and leaves that request untouched."""
    w = synth.workload(1, B=3, H=2, dk=64, dv=64, m=4, block_size=4, blocks_per_req=3, steps=1,
                       rule=1, io="bf16", state_std=0.02)
    run = Run(w)
    inp = run.inputs(0, n=3, stream_base=200)
    parent = torch.tensor([[-1, 0, 1], [-1, 2, 0], [-1, -1, 0]], dtype=torch.int32, device=run.dev)
    out = torch.full((w.B, 3, w.H, w.dk), 7.0, device=run.dev)
    run.kv.verify_tree(parent, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], out=out)
    torch.cuda.synchronize()
    assert int(run.kv.error.item()) == kb.DEVERR_ACCEPT
    assert torch.all(out[1] == 7.0) and not torch.all(out[0] == 7.0)
    run.kv.error.zero_()
    good = torch.tensor([[-1, 0, 1], [-1, 0, 0], [-1, -1, 0]], dtype=torch.int32, device=run.dev)
    occ0 = run.kv.occupancy.clone()
    run.kv.commit_tree(good, torch.tensor([2, 3, -2], dtype=torch.int32, device=run.dev))
    torch.cuda.synchronize()
    assert int(run.kv.error.item()) == kb.DEVERR_ACCEPT
    occ = run.kv.occupancy
    assert torch.equal(occ[1:], occ0[1:]) and torch.all(occ[0] == occ0[0] + 3)


@pytest.mark.parametrize("rule", [0, 1, 3])
@pytest.mark.parametrize("n", [3, 5, 6, 7])
@pytest.mark.parametrize("tree", [False, True])
def test_verify_partial_query_blocks(rule, n, tree):
    """d = 128 bf16 verifies of 4 or 8 queries per launch with only n of them
    used (the matrix-core path pads the rest with zeros), across folds and
    buffers of every occupancy."""
    w = synth.workload(1, B=5, H=3, dk=128, dv=128, m=8, block_size=4, blocks_per_req=5, steps=10,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w)
    t = 0
    for call in range(7):
        run.decode(t)
        t += 1
        if tree:
            parent, leaf = synth.draft_tree(w, call, w.B, n)
            run.verify_tree_commit(call, parent, leaf)
        else:
            run.verify_commit(call, n, synth.accepted_lengths(w, call, w.B, n))
        run.check_effective_states()
        run.check_pool()
        run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_staggered_occupancies(rule):
    """Commits of different lengths desynchronise the requests' occupancies,
    so one decode launch serves requests at every buffer position and folds
    some of them."""
    w = synth.workload(1, B=8, H=2, dk=128, dv=128, m=8, block_size=4, blocks_per_req=4, steps=20,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w)
    run.verify_commit(0, 7, np.arange(w.B, dtype=np.int32) % 8)
    for t in range(w.steps):
        run.decode(t)
    run.check_effective_states()
    run.check_pool()


@pytest.mark.parametrize("rule,d,io", [(0, 128, "bf16"), (1, 128, "bf16"), (3, 128, "bf16"), (1, 64, "f32"),
                                       (0, 16, "f32"), (3, 16, "f32")])
def test_direct_long_rows(rule, d, io):
    """Buffer-only decode of up to 60 positions (table rows of 64): the
    linear and gated rules on the chunk kernel's direct-to-LDS ring (several
    passes of positions), the per-channel rule on the one-token kernel (several
    rounds of 16 positions through its token wave); every output against the
    recurrence from a zero state, and the pool and bookkeeping exactly."""
    w = synth.workload(1, B=3, H=2, dk=d, dv=d, m=64, block_size=16, blocks_per_req=4, steps=60,
                       rule=rule, io=io, state_std=0.02)
    _say("direct long rows", w)
    run = Run(w, stateless=np.ones(3, bool), flush=kb.FLUSH_DEFERRED)
    for t in range(w.steps):
        run.decode(t, direct=True)
        if t % 20 == 19:
            run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_direct_and_promotion(rule):
    """Buffer-only decode equals the recurrence from a zero state; giving the
    request a zeroed state slot afterwards and folding creates its state."""
    w = synth.workload(1, B=3, H=2, dk=128, dv=128, m=8, block_size=8, blocks_per_req=2, steps=11,
                       rule=rule, io="bf16", state_std=0.02)
    run = Run(w, stateless=np.ones(3, bool), flush=kb.FLUSH_DEFERRED)
    for t in range(w.steps):
        run.decode(t, direct=True)
    run.check_effective_states()
    # promotion: a zeroed slot per request, then a fold of the first m tokens
    slots = np.array([0, 1, 2], np.int32)
    run.kv.state[:3].zero_()
    run.kv.state_slot.copy_(torch.from_numpy(slots))
    run.slots = slots
    for b in range(w.B):
        run.model.requests[b].has_state = True
    run.flush()
    run.check_effective_states()
    for t in range(w.steps, w.steps + 5):
        run.decode(t)
    run.check_effective_states()


def test_mixed_stateful_and_stateless_one_launch():
    w = synth.workload(1, B=6, H=2, dk=128, dv=128, m=4, block_size=4, blocks_per_req=3, steps=10,
                       rule=2, io="bf16", state_std=0.02)
    run = Run(w, stateless=np.array([0, 1, 0, 1, 1, 0], bool))
    for t in range(w.steps):
        run.decode(t)
    run.check_effective_states()
    run.check_pool()


# ---------------------------------------------------------------------------
# Edge cases and device-side checks.
# ---------------------------------------------------------------------------

def test_empty_batch_is_a_no_op():
    kv = kb.KVBuffer(batch=2, heads=2, d=16, m=4, rule=kb.RULE_GATED, io_dtype=kb.F32)
    empty = kb.Batch(0, None, None, None, None)
    z = torch.zeros(1, device="cuda")
    assert kb.kvbuf_decode(kv.layout, kv.pools, empty, z, z, z, z, None, z) == kb.OK
    assert kb.kvbuf_flush(kv.layout, kv.pools, empty) == kb.OK


def _errors(kv):
    torch.cuda.synchronize()
    return int(kv.error.item())


def test_device_errors_skip_the_request():
    """Metadata the kernels find out of range skips the request (all its
    heads, when the caller's row is bad), leaves its row and occupancy as
    they were and sets the error bit; a bad per-head copy skips that head
    only, which kvbuf_check then reports."""
    w = synth.workload(1, B=3, H=2, dk=16, dv=16, m=4, block_size=4, blocks_per_req=2, steps=1,
                       rule=1, io="f32", state_std=0.02)
    run = Run(w)
    kv = run.kv
    before_state = kv.state.clone()
    one = lambda b: torch.tensor([b], dtype=torch.int32, device="cuda")
    # request 1: a block id outside the pool, admitted to every head
    kv.block_table[1, 0] = 10_000
    kv.admit(one(1))
    inp = run.inputs(0)
    out = kv.decode(inp["q"], inp["k"], inp["v"], inp["g"])
    assert _errors(kv) & kb.DEVERR_BLOCK
    assert kv.occupancy.cpu().tolist() == [1, 0, 1]  # request 1 was skipped
    assert kv.tile_meta[:, :, 0].cpu().tolist() == [[1, 1], [0, 0], [1, 1]]
    kv.error.zero_()
    kv.check_meta()
    assert _errors(kv) == 0  # every request's heads agree with it
    # request 0: occupancy at capacity -> overflow, nothing written
    cap = run.kv.capacity
    kv.occupancy[0] = cap
    kv.block_table[1, 0] = run.model.requests[1].table[0]
    kv.admit(torch.tensor([0, 1], dtype=torch.int32, device="cuda"))
    kv.decode(inp["q"], inp["k"], inp["v"], inp["g"], out=out)
    assert _errors(kv) & kb.DEVERR_OVERFLOW
    assert kv.occupancy.cpu().tolist() == [cap, 1, 2]
    kv.error.zero_()
    # a bad copy in one head (head 1 of request 2) skips that tile only: head
    # 0 advances (and with it the request's occupancy), head 1 does not
    kv.tile_meta[2, 1, 1] = -3
    kv.decode(inp["q"], inp["k"], inp["v"], inp["g"], out=out)
    assert _errors(kv) & kb.DEVERR_BLOCK
    assert kv.tile_meta[2, :, 0].cpu().tolist() == [3, 2]
    assert kv.occupancy[2].item() == 3
    kv.error.zero_()
    kv.check_meta()
    assert _errors(kv) == kb.DEVERR_META
    kv.error.zero_()
    # an admit index outside the batch is reported
    kv.admit(one(7))
    assert _errors(kv) == kb.DEVERR_META
    kv.error.zero_()
    # accepted count beyond n
    kv.occupancy[0] = 0
    kv.admit(one(0))
    acc = torch.tensor([0, 5, 0], dtype=torch.int32, device="cuda")
    kv.commit(2, acc)
    assert _errors(kv) & kb.DEVERR_ACCEPT
    # state slot outside the pool (recurrent mode)
    kv0 = kb.KVBuffer(batch=2, heads=2, d=16, m=0, rule=kb.RULE_LINEAR, io_dtype=kb.F32, num_state_slots=2)
    kv0.state_slot[1] = 7
    z = torch.zeros((2, 2, 16), device="cuda")
    kv0.decode(z, z, z)
    assert _errors(kv0) & kb.DEVERR_SLOT
    assert torch.equal(kv.state, before_state)


def test_validation_errors_touch_nothing():
    kv = kb.KVBuffer(batch=2, heads=2, d=16, m=4, rule=kb.RULE_GATED, io_dtype=kb.F32)
    z = torch.zeros((2, 2, 16), device="cuda")
    g = torch.zeros((2, 2), device="cuda")
    assert kb.kvbuf_decode(kv.layout, kv.pools, kv.batch, z, z, z, None, None, z,
                           raise_on_error=False) == kb.EINVAL  # gated rule needs g
    assert kb.kvbuf_verify(kv.layout, kv.pools, kv.batch, 9, z, z, z, g, None, z,
                           raise_on_error=False) == kb.EUNSUPPORTED
    torch.cuda.synchronize()
    assert kv.occupancy.cpu().tolist() == [0, 0]
    kb.kvbuf_decode(kv.layout, kv.pools, kv.batch, z, z, z, g, None, z)
    torch.cuda.synchronize()
    assert kv.occupancy.cpu().tolist() == [1, 1]
    assert kv.tile_meta[:, :, 0].cpu().tolist() == [[1, 1], [1, 1]]


# ---------------------------------------------------------------------------
# Full-size workloads, every tile, in the launch configuration the benchmark
# times (eager fold inside the decode kernel).
# ---------------------------------------------------------------------------

def _full_cycle_checks(run):
    """End of a full-size run whose last step folded every request: every
    tile's stored state, effective state and buffered bits."""
    assert run.check_all_states() == run.w.B * run.w.H
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    assert run.full_state_checks == 2
    _say("max out err %.2e, max state err %.2e, tile states checked %d"
         % (run.max_out, run.max_state, run.folds_checked))


# bf16 outputs: errors beyond the rounding itself (half an ulp, 2^-8 of the
# value), relative to the output magnitude: fp32 sums of exact products stay
# near 1e-6 of it.
TOL_BF16_OUT = 2e-5


@pytest.mark.parametrize("rule,d,io", [(0, 64, "bf16"), (1, 128, "bf16"), (2, 128, "bf16"), (3, 128, "bf16"),
                                       (1, 16, "bf16"), (3, 64, "bf16"), (1, 128, "f32"), (2, 16, "f32")])
def test_bf16_outputs(rule, d, io):
    """Outputs stored as bf16 (layout out_dtype): every output of decode, of
    verify with chains of 1, 4 and 8 drafts (the matrix-core instances among
    them) and of a tree verify is the oracle's output rounded to nearest bf16,
    to within the fp32 error of the sums."""
    w = synth.workload(1, B=5, H=3, dk=d, dv=d, m=8, block_size=4, blocks_per_req=5, steps=8,
                       rule=rule, io=io, state_std=0.5)
    _say("bf16 outputs", w)
    run = Run(w, out_dtype=kb.OUT_BF16, tol_out=TOL_BF16_OUT)
    t = 0
    for call, n in enumerate((1, 4, 8)):
        run.decode(t)
        t += 1
        run.verify_commit(call, n, synth.accepted_lengths(w, call, w.B, n))
    parent, leaf = synth.draft_tree(w, 7, w.B, 5)
    run.verify_tree_commit(7, parent, leaf)
    for _ in range(3):
        run.decode(t)
        t += 1
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    _say("max out err beyond rounding %.2e" % run.max_out)


@pytest.mark.parametrize("rule", [0, 1])
def test_bf16_outputs_one_token_kernel(rule):
    """bf16 outputs of the one-token kernel (d = 128, bf16, above 4096 tiles),
    through a fused fold."""
    w = synth.workload(3, B=130, rule=rule, steps=10)
    _say("bf16 outputs, one-token kernel", w)
    run = Run(w, out_dtype=kb.OUT_BF16, tol_out=TOL_BF16_OUT)
    for t in range(w.steps):
        run.decode(t)
    assert run.folds_checked == w.B * w.H
    _say("max out err beyond rounding %.2e" % run.max_out)


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_bf16_outputs_buffer_only_and_recurrent(rule):
    """bf16 outputs of buffer-only decode (one wave per tile) and of the m = 0
    recurrent kernel and its temporary-state verification."""
    w = synth.workload(1, B=3, H=2, dk=128, dv=128, m=8, block_size=8, blocks_per_req=2, steps=10,
                       rule=rule, io="bf16", state_std=0.5)
    run = Run(w, stateless=np.ones(3, bool), flush=kb.FLUSH_DEFERRED, out_dtype=kb.OUT_BF16,
              tol_out=TOL_BF16_OUT)
    for t in range(w.steps):
        run.decode(t, direct=True)
    run.check_effective_states()
    import oracle

    w0 = synth.workload(1, B=3, H=2, dk=128, dv=128, m=0, block_size=1, blocks_per_req=1, steps=4,
                        rule=rule, io="bf16", state_std=0.5)
    run0 = Run(w0, out_dtype=kb.OUT_BF16, tol_out=TOL_BF16_OUT)
    for t in range(w0.steps):
        run0.decode(t)
    n = 3
    inp = run0.inputs(0, n=n, stream_base=100)
    out, _ = run0.kv.verify_recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    assert out.dtype == torch.bfloat16
    torch.cuda.synchronize()
    q, k, v, g, beta = (run0._sampled(inp[x], drafts=True) for x in ("q", "k", "v", "g", "beta"))
    o_gpu = run0._sampled(out, drafts=True)
    o_ref, _, mag = oracle.recurrent(rule, run0.S, q.transpose(1, 0, 2), k.transpose(1, 0, 2),
                                     v.transpose(1, 0, 2), None if g is None else np.swapaxes(g, 0, 1),
                                     None if beta is None else beta.T, with_magnitude=True)
    from tests.harness import BF16_HALF_ULP, out_err_tiles
    for dd in range(n):
        err = out_err_tiles(o_gpu[:, dd], o_ref[dd], mag[dd], slack=BF16_HALF_ULP)
        assert err <= TOL_BF16_OUT, (dd, err)


@pytest.mark.parametrize("B,m", [(4096, 8), (4097, 8), (4096, 32), (4096, 16)])
def test_decode_kernel_choice_boundary(B, m):
    """One-token decode at d = 128, bf16, one head per request, around the
    launch size at which the chunk kernel stops taking it (4096 tiles, when m
    fits that kernel's first staging pass of 16 positions): each side folds
    in the decode launch, and m = 32 stays on the one-token kernel, whose
    fused fold covers it."""
    w = synth.workload(3, B=B, H=1, m=m, block_size=m, blocks_per_req=2, steps=m + 3)
    _say("kernel choice boundary", w)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    assert run.folds_checked == B
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


@pytest.mark.parametrize("B", [64, 160])
def test_workload2_ungated_batched(B):
    """The ungated workload (B = 64: 2048 tiles, served by the chunk kernel)
    and the same at B = 160 (5120 tiles, above the launch size the chunk
    kernel takes: the one-token kernel)."""
    w = synth.workload(2, B=B)
    _say("workload 2", w)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    _full_cycle_checks(run)


def test_workload3_gated_m8_full():
    w = synth.workload(3)
    _say("workload 3", w)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    _full_cycle_checks(run)


@pytest.mark.parametrize("m", [0, 4, 16, 32])
def test_workload3_gated_sweep(m):
    """The other buffer sizes of the gated workload, 512 steps each (64 to 16
    buffer cycles; m = 0 is the recurrent kernel)."""
    w = synth.workload(3, m=m, block_size=max(m, 1), blocks_per_req=2 if m else 1)
    assert w.steps == 512
    _say("workload 3 m=%d" % m, w)
    run = Run(w)
    for t in range(w.steps):
        run.decode(t)
    if m:
        _full_cycle_checks(run)
    else:  # recurrent: every state is current after every step
        assert run.check_all_states() == w.B * w.H
        _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


@pytest.mark.parametrize("n", [4, 8])
def test_workload4_tree_verify_commit(n):
    """Tree drafts at the verification workload's full size (B=128 H=32
    d=128 m=8), in the launch configuration the benchmark times; every tile
    against the recurrence along each draft's path."""
    w = synth.workload(4)
    _say("workload 4 trees n=%d" % n, w)
    run = Run(w)
    t = 0
    for call in range(8):
        run.decode(t)
        t += 1
        parent, leaf = synth.draft_tree(w, call + 1000 * n, w.B, n)
        run.verify_tree_commit(call, parent, leaf)
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_workload4_verify_commit(n):
    w = synth.workload(4)
    _say("workload 4 n=%d" % n, w)
    run = Run(w)
    t = 0
    for call in range(12):
        run.decode(t)
        t += 1
        acc = synth.accepted_lengths(w, call + 1000 * n, w.B, n)
        run.verify_commit(call, n, acc)
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


@pytest.mark.parametrize("split", [False, True])
def test_workload5_mixed_delta(split):
    """The mixed delta-rule workload: 256 requests with a state, 256 served
    from their buffer alone (retired at the end of a random lifetime and
    replaced).  Either one kvbuf_decode over the whole batch under the eager
    policy (the fold runs in the launch that follows a decode), or -- the
    benchmark's launch configuration -- kvbuf_decode over the requests with a
    state and kvbuf_direct over the others, each on a view of its range,
    under the deferred policy with a kvbuf_flush of the stateful view when
    their buffers fill (every 64 steps: they run in lockstep)."""
    w = synth.workload(5)
    _say("workload 5", w, "split", split)
    stateless = np.zeros(w.B, bool)
    stateless[w.B - w.n_short:] = True
    n_long = w.B - w.n_short
    run = Run(w, stateless=stateless, spare_blocks=64, flush=kb.FLUSH_DEFERRED if split else kb.FLUSH_EAGER)
    short = np.arange(w.B - w.n_short, w.B)
    life = synth.short_lengths(w, 0, len(short))
    age = np.zeros(len(short), np.int64)
    draws = 1
    retired = 0
    for t in range(w.steps):
        run.decode(t, direct_from=n_long if split else None)
        if split and t % w.m == w.m - 1:
            run.flush(upto=n_long)
        age += 1
        for i in np.nonzero(age >= life)[0]:
            run.retire_and_admit(int(short[i]))
            age[i] = 0
            life[i] = synth.short_lengths(w, draws, 1)[0]
            draws += 1
            retired += 1
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    # the long requests fold at the last step: every one of their tiles
    assert run.check_all_states() >= (w.B - w.n_short) * w.H
    _say("retired %d; max out err %.2e, max state err %.2e" % (retired, run.max_out, run.max_state))


# ---------------------------------------------------------------------------
# The verification that the buffered one replaces: recurrent form with one
# temporary state per draft (m = 0), and its commit by state replacement.
# ---------------------------------------------------------------------------

def _tile_rel(a, b):
    a = np.asarray(a, np.float64).reshape(a.shape[0], -1)
    b = np.asarray(b, np.float64).reshape(b.shape[0], -1)
    return np.max(np.abs(a - b), axis=1) / np.maximum(np.max(np.abs(b), axis=1), 1e-30)


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("n,d", [(1, 64), (4, 128), (8, 64), (3, 16)])
def test_verify_recurrent_baseline(rule, n, d):
    import oracle

    w = synth.workload(1, B=5, H=2, dk=d, dv=d, m=0, block_size=1, blocks_per_req=1, steps=3,
                       rule=rule, io="bf16", state_std=0.02)
    _say("recurrent verify", w, "n", n)
    run = Run(w)
    for t in range(2):  # move the states away from their initial values
        run.decode(t)
    inp = run.inputs(0, n=n, stream_base=100)
    out, temp = run.kv.verify_recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    torch.cuda.synchronize()
    assert int(run.kv.error.item()) == 0
    q, k, v, g, beta = (run._sampled(inp[x], drafts=True) for x in ("q", "k", "v", "g", "beta"))
    o_gpu = run._sampled(out, drafts=True)
    tmp = temp.detach()
    for dd in range(n):
        sl = slice(0, dd + 1)
        o_ref, S_ref = oracle.recurrent(rule, run.S, q[:, sl].transpose(1, 0, 2), k[:, sl].transpose(1, 0, 2),
                                        v[:, sl].transpose(1, 0, 2),
                                        None if g is None else np.swapaxes(g[:, sl], 0, 1),
                                        None if beta is None else beta[:, sl].T)
        assert np.max(_tile_rel(o_gpu[:, dd], o_ref[dd])) <= 2e-3, dd
        t_gpu = tmp[dd][run.sb, run.sh].double().cpu().numpy()
        assert np.max(_tile_rel(t_gpu, S_ref)) <= 1e-5, dd
    # commit: the state of a request becomes its last accepted draft's temporary state
    acc = synth.accepted_lengths(w, 0, w.B, n)
    before = run.kv.state.detach().clone()
    run.kv.commit_recurrent(n, torch.from_numpy(acc).to("cuda"), temp)
    torch.cuda.synchronize()
    assert int(run.kv.error.item()) == 0
    after = run.kv.state.detach()
    for b in range(w.B):
        want = before[run.slots[b]] if acc[b] == 0 else tmp[acc[b] - 1, b]
        assert torch.equal(after[run.slots[b]], want), b
    # an accepted count outside [0, n] is reported and changes nothing
    bad = torch.from_numpy(acc).to("cuda")
    bad[0] = n + 1
    snap = run.kv.state.detach().clone()
    run.kv.commit_recurrent(n, bad, temp)
    torch.cuda.synchronize()
    assert int(run.kv.error.item()) & kb.DEVERR_ACCEPT
    assert torch.equal(run.kv.state[run.slots[0]], snap[run.slots[0]])


@pytest.mark.parametrize("rule,m", [(1, 64), (1, 128), (2, 64), (2, 128), (0, 128), (3, 64)])
def test_long_fold_full_size(rule, m):
    """kvbuf_flush of m buffered tokens at B=256 H=32 d=128, bf16, in the
    launch configuration the benchmark times (a block of m per request, pools
    filled on the device): every tile against the recurrence over its m
    buffered tokens -- for the delta rule over its stored pseudo-values,
    which a fold applies as the values of the scalar-gated rule.  (The
    per-channel rule keeps buffers of at most 64 positions.)"""
    import oracle
    from tests.harness import NTHREADS, TOL_STATE, rel_err_tiles

    B, H, d = 256, 32, 128
    dev = torch.device("cuda:0")
    kv = kb.KVBuffer(batch=B, heads=H, d=d, m=m, block_size=m, blocks_per_req=1, num_blocks=B,
                     num_state_slots=B, rule=rule, io_dtype=kb.BF16, flush=kb.FLUSH_DEFERRED, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9100 + 10 * rule + m)
    kv.state.normal_(0.0, 0.02, generator=gen)
    kv.key.normal_(generator=gen)
    kv.value.normal_(generator=gen)
    if kv.gate is not None:
        kv.gate.uniform_(-0.1, 0.0, generator=gen)
    # shuffled slots and blocks, so that tile (b, h) reads slot[b] and block[b]
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(9300 + m)).to(torch.int32)
    kv.state_slot.copy_(perm)
    kv.set_block_table(torch.roll(perm, 7).reshape(B, 1))
    slot = kv.state_slot.cpu().numpy().astype(np.int64)
    block = kv.block_table.cpu().numpy()[:, 0].astype(np.int64)
    # host copies, tile-major: S0 [B*H, d, d], K / V [m, B*H, d], G [m, B*H (, d)]
    S0 = kv.state[torch.from_numpy(slot).to(dev)].reshape(B * H, d, d).cpu().numpy().astype(np.float64)
    tiles = lambda x: x[torch.from_numpy(block).to(dev)].float().movedim(2, 0).reshape(m, B * H, *x.shape[3:])
    K = tiles(kv.key).cpu().numpy()
    V = tiles(kv.value).cpu().numpy()
    G = None if kv.gate is None else tiles(kv.gate).cpu().numpy()
    kv.occupancy.fill_(m)
    kv.admit()
    _say("long fold full size rule %d m %d" % (rule, m))
    kv.flush()
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    assert int(kv.occupancy.abs().sum().item()) == 0
    assert int(kv.tile_meta[:, :, 0].abs().sum().item()) == 0
    assert np.array_equal(kv.block_table.cpu().numpy()[:, 0], block)  # one block per request rotates onto itself
    # the fold of the delta rule is the scalar-gated rule's over pseudo-values
    ref_rule = kb.RULE_GATED if rule == kb.RULE_DELTA else rule
    _, S_ref = oracle.recurrent(ref_rule, S0, np.zeros((m, B * H, d)), K, V, G, nthreads=NTHREADS, inplace=True)
    S_gpu = kv.state[torch.from_numpy(slot).to(dev)].reshape(B * H, d, d).cpu().numpy()
    err = rel_err_tiles(S_gpu, S_ref, axes=(-2, -1))
    _say("max state err over %d tiles %.2e" % (B * H, err))
    assert err <= TOL_STATE, "state error %.3e" % err
