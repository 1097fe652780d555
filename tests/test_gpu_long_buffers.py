"""GPU parity for buffers longer than one 64-position pass.

* Table rows whose capacity is not a multiple of 64 (66 = 33 blocks of 2,
  72 = 9 blocks of 8): decode, verify and a deferred flush touch the positions
  past 64.  The pool row of each buffer position is resolved by a wave of 64
  lanes in passes of 64 positions; a lane permute reads zero from an inactive
  lane, so a last partial pass run with only its live lanes active resolved
  these positions to block 0.  These cases run the corrected resolution.
* Buffer-only decode of L = 128, 256 and 512 tokens in the layout the
  context-length sweep of the benchmark times (blocks of 16, L / 16 per
  request, m = L), then a verify of 4 drafts at the end of the row, then the
  promotion of the requests: a zeroed state slot each and one flush of all L
  buffered tokens (KVBuffer: IO-aware Serving for Linear Attention,
  pith.science page: the abstract serves short contexts from the buffer
  alone; the Figure 5 caption compares the decoding forms over context
  lengths of 16 to 256).  512 positions is the largest capacity the library
  accepts.

Every output is compared with the oracle's recurrence (from a zero state for
buffer-only requests), the pool bits and bookkeeping exactly, stored states
after the promotion fold at 1e-5.
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


@pytest.mark.parametrize("bs,bpr", [(2, 33), (8, 9)])
@pytest.mark.parametrize("rule,d,io", [(1, 16, "f32"), (2, 16, "f32"), (0, 128, "bf16"), (1, 128, "bf16"),
                                       (2, 128, "bf16"), (3, 16, "f32"), (3, 128, "bf16")])
def test_table_row_tail(bs, bpr, rule, d, io):
    """m = 64 in rows of 66 or 72 positions, deferred policy: decode to
    four positions short of the capacity, verify 4 drafts there (positions
    cap-4 .. cap-1), commit 3 / 2 / 1 of them, decode once more (one request
    reaches the capacity), flush (64 positions fold, the tail past 64 stays
    buffered in the rotated table), decode on from the tail."""
    m = 64
    cap = bs * bpr
    w = synth.workload(1, B=3, H=2, dk=d, dv=d, m=m, block_size=bs, blocks_per_req=bpr, steps=cap + 8,
                       rule=rule, io=io, state_std=0.02)
    _say("table row tail", w)
    run = Run(w, flush=kb.FLUSH_DEFERRED)
    t = 0
    for _ in range(cap - 4):
        run.decode(t)
        t += 1
    run.verify_commit(0, 4, np.array([3, 2, 1], np.int32))
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    run.decode(t)
    t += 1
    assert list(run.model.occupancies()) == [cap, cap - 1, cap - 2]
    run.check_effective_states()
    run.check_pool()
    run.flush()
    assert list(run.model.occupancies()) == [cap - m, cap - 1 - m, cap - 2 - m]
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    for _ in range(6):
        run.decode(t)
        t += 1
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()


def _promote(run):
    """Every request gets a zeroed state slot; the next fold creates its state."""
    w = run.w
    slots = np.arange(w.B, dtype=np.int32)
    run.kv.state[: w.B].zero_()
    run.kv.state_slot.copy_(torch.from_numpy(slots))
    run.slots = slots
    run.stateless[:] = False
    for b in range(w.B):
        run.model.requests[b].has_state = True


@pytest.mark.parametrize("L,rule,d,io", [(128, 1, 128, "bf16"), (256, 1, 128, "bf16"), (256, 0, 128, "bf16"),
                                         (128, 0, 16, "f32"), (256, 1, 16, "f32"), (512, 1, 16, "f32"),
                                         (512, 0, 128, "bf16"), (512, 1, 128, "bf16"), (128, 3, 128, "bf16"),
                                         (256, 3, 16, "f32"), (128, 2, 128, "bf16")])
def test_direct_long_buffers_and_promotion(L, rule, d, io):
    w = synth.workload(1, B=3, H=2, dk=d, dv=d, m=L, block_size=16, blocks_per_req=L // 16, steps=L,
                       rule=rule, io=io, state_std=0.02)
    _say("direct long buffer", w)
    run = Run(w, stateless=np.ones(w.B, bool), flush=kb.FLUSH_DEFERRED)
    for t in range(L - 4):
        run.decode(t, direct=True)
        if t % 64 == 63:
            run.check_effective_states()
    # four drafts at the end of the row, all kept: the buffer is full
    run.verify_commit(0, 4, np.full(w.B, 4, np.int32))
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    _promote(run)
    run.flush()  # one fold of all L tokens; stored states checked for every tile
    assert int(run.model.occupancies().max()) == 0
    assert run.check_all_states() == w.B * w.H
    run.check_bookkeeping()
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))


def test_direct_full_size_L256_and_promotion():
    """The buffer-only leg of the context sweep at its full size: B=256 H=32
    d=128, gated, bf16, 256 tokens per request in blocks of 16 (every tile,
    every step), then the promotion fold of all 256 tokens (every tile's
    stored state)."""
    L = 256
    w = synth.workload(3, m=L, block_size=16, blocks_per_req=L // 16, steps=L)
    _say("direct full size", w)
    run = Run(w, stateless=np.ones(w.B, bool), flush=kb.FLUSH_DEFERRED)
    for t in range(L):
        run.decode(t, direct=True)
    run.check_effective_states()
    run.check_pool()
    run.check_bookkeeping()
    _promote(run)
    run.flush()
    assert run.check_all_states() == w.B * w.H
    run.check_bookkeeping()
    _say("max out err %.2e, max state err %.2e" % (run.max_out, run.max_state))
