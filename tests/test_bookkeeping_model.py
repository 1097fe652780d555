"""Pins of the oracle's integer bookkeeping model (CPU only)."""

import random

import pytest

from oracle import BufferModel


def test_two_blocks_rotate_on_fold():
    bm = BufferModel(m=4, block_size=4, blocks_per_req=2)
    bm.add_request([7, 3])
    for t in range(3):
        assert not bm.decode(0, ("tok", t))
    assert bm.occupancies().tolist() == [3]
    assert bm.decode(0, ("tok", 3))  # fourth token fills the buffer: fold
    assert bm.tables().tolist() == [[3, 7]]
    assert bm.occupancies().tolist() == [0]
    # the four tokens sit in block 7 at offsets 0..3 and stay there as dead data
    assert [bm.physical[(7, o)] for o in range(4)] == [("tok", t) for t in range(4)]
    bm.decode(0, ("tok", 4))
    assert bm.physical[(3, 0)] == ("tok", 4)


def test_fold_moves_several_blocks():
    bm = BufferModel(m=8, block_size=4, blocks_per_req=4)
    bm.add_request([10, 11, 12, 13])
    for t in range(8):
        bm.decode(0, t)
    assert bm.tables().tolist() == [[12, 13, 10, 11]]


def test_deferred_fold_keeps_tail_tokens():
    bm = BufferModel(m=4, block_size=4, blocks_per_req=2)
    bm.add_request([0, 1])
    for t in range(6):
        bm.decode(0, t, eager=False)
    assert bm.occupancies().tolist() == [6]
    assert bm.flush(0)
    assert bm.occupancies().tolist() == [2]
    assert bm.buffered_tokens(0) == [4, 5]
    assert not bm.flush(0)


def test_verify_commit_crossing_the_fold():
    bm = BufferModel(m=8, block_size=8, blocks_per_req=2)
    bm.add_request([5, 9])
    for t in range(6):
        bm.decode(0, ("d", t))
    bm.verify(0, [("v", i) for i in range(5)])
    assert bm.occupancies().tolist() == [6]  # verify does not advance
    assert bm.commit(0, 3)  # 6 + 3 = 9 >= 8: fold the first 8
    assert bm.occupancies().tolist() == [1]
    assert bm.tables().tolist() == [[9, 5]]
    assert bm.buffered_tokens(0) == [("v", 2)]


def test_commit_zero_changes_nothing():
    bm = BufferModel(m=8, block_size=8, blocks_per_req=2)
    bm.add_request([1, 2])
    for t in range(5):
        bm.decode(0, t)
    before = (bm.tables().tolist(), bm.occupancies().tolist())
    bm.verify(0, ["x", "y"])
    bm.commit(0, 0)
    assert (bm.tables().tolist(), bm.occupancies().tolist()) == before


def test_stateless_requests_never_fold():
    bm = BufferModel(m=4, block_size=4, blocks_per_req=2)
    bm.add_request([0, 1], has_state=False)
    for t in range(7):
        assert not bm.decode(0, t, stateless=True)
    assert bm.occupancies().tolist() == [7]
    with pytest.raises(IndexError):
        for t in range(2):
            bm.decode(0, t, stateless=True)


def test_random_operations_conserve_blocks_and_bound_occupancy():
    rs = random.Random(7)
    m, bs, bpr, B = 8, 4, 4, 6
    pool = list(range(B * bpr + 5))
    rs.shuffle(pool)
    bm = BufferModel(m=m, block_size=bs, blocks_per_req=bpr)
    for b in range(B):
        bm.add_request(pool[b * bpr:(b + 1) * bpr])
    for step in range(300):
        b = rs.randrange(B)
        if rs.random() < 0.6:
            bm.decode(b, ("t", step))
        else:
            n = rs.randint(1, 8)
            bm.verify(b, [("d", step, i) for i in range(n)])
            bm.commit(b, rs.randint(0, n))
        bm.check_invariants(num_blocks=len(pool))
        assert all(0 <= o < m for o in bm.occupancies())
    owned = sorted(x for row in bm.tables().tolist() for x in row)
    assert owned == sorted(pool[: B * bpr])


def test_commit_path_compacts_the_accepted_drafts():
    """Tree drafts: the accepted root-to-node path moves to consecutive
    positions after the buffered tokens; other drafts stay as dead data."""
    bm = BufferModel(m=8, block_size=4, blocks_per_req=3)
    bm.add_request([4, 0, 2])
    for t in range(3):
        bm.decode(0, ("d", t))
    bm.verify(0, [("v", i) for i in range(6)])  # positions 3 .. 8
    bm.commit_path(0, [1, 3, 5])  # drafts 1, 3, 5 -> positions 3, 4, 5
    assert bm.occupancies().tolist() == [6]
    assert bm.buffered_tokens(0) == [("d", 0), ("d", 1), ("d", 2), ("v", 1), ("v", 3), ("v", 5)]
    assert bm.physical[bm.position(0, 8)] == ("v", 5)  # the source stays as dead data


def test_commit_chain_path_is_commit():
    a = BufferModel(m=4, block_size=2, blocks_per_req=4)
    b = BufferModel(m=4, block_size=2, blocks_per_req=4)
    for bm in (a, b):
        bm.add_request([3, 1, 0, 2])
        bm.decode(0, "x")
        bm.verify(0, ["p", "q", "r", "s"])
    assert a.commit(0, 3) == b.commit_path(0, [0, 1, 2])
    assert a.tables().tolist() == b.tables().tolist()
    assert a.occupancies().tolist() == b.occupancies().tolist()
    assert a.buffered_tokens(0) == b.buffered_tokens(0)
