"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/kvbuf.h declares, mirrors the header's structs, and rejects
bad arguments on the host before any HIP call (no kernel is launched here)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import linear_attention_decode_kvbuf_amd as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvbuf.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kb.LIB_PATH):
        from linear_attention_decode_kvbuf_amd import _build
        _build.build()
    return kb.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvbuf_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(kb.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_struct_sizes_match_header(lib):
    # kvbuf_layout: 11 int32 + 1 float + 1 int32; pools: 4 pointers; batch: int32 (+pad) + 6 pointers
    assert ctypes.sizeof(kb.Layout) == 52
    assert ctypes.sizeof(kb.Pools) == 32
    assert ctypes.sizeof(kb.Batch) == 48


def test_structs_match_a_c_compiler():
    """Sizes and field offsets of the binding's structs against the header
    as a C compiler lays it out."""
    fields = {"kvbuf_layout": kb.Layout, "kvbuf_pools": kb.Pools, "kvbuf_batch": kb.Batch}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "kvbuf.h"', "int main(void) {"]
    for cname, py in fields.items():
        lines.append('printf("%%zu\\n", sizeof(%s));' % cname)
        for f, _ in py._fields_:
            lines.append('printf("%%zu\\n", offsetof(%s, %s));' % (cname, f))
    lines.append("return 0; }")
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "t.c"), os.path.join(tmp, "t")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-x", "c", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", src, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()]
    want = []
    for py in fields.values():
        want.append(ctypes.sizeof(py))
        want += [getattr(py, f).offset for f, _ in py._fields_]
    assert got == want


def test_abi_version_and_strerror(lib):
    assert kb.kvbuf_abi_version() == 5
    for st in (kb.OK, kb.EINVAL, kb.EUNSUPPORTED, kb.ECAPACITY, kb.EHIP):
        assert len(kb.strerror(st)) > 5
    assert "unknown" in kb.strerror(-99)


def _layout(**kw):
    base = dict(num_heads=2, d_k=16, d_v=16, m=4, block_size=4, blocks_per_req=2, num_blocks=4,
                num_state_slots=2, rule=kb.RULE_GATED, io_dtype=kb.F32, flush=kb.FLUSH_EAGER, scale=1.0,
                out_dtype=kb.OUT_F32)
    base.update(kw)
    return kb.Layout(*[base[f] for f, _ in kb.Layout._fields_])


FAKE = 0x1000  # never dereferenced: every case below fails validation first
POOLS = kb.Pools(FAKE, FAKE, FAKE, FAKE)
BATCH = kb.Batch(2, FAKE, FAKE, FAKE, None, FAKE)


def _decode(layout, pools=POOLS, batch=BATCH, q=FAKE, g=FAKE, beta=None):
    return kb.kvbuf_decode(layout, pools, batch, q, FAKE, FAKE, g, beta, FAKE, stream=0,
                           raise_on_error=False)


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=0), kb.EINVAL),
    (dict(d_k=32, d_v=32), kb.EUNSUPPORTED),
    (dict(d_k=128, d_v=64), kb.EUNSUPPORTED),
    (dict(rule=4), kb.EUNSUPPORTED),
    (dict(io_dtype=7), kb.EUNSUPPORTED),
    (dict(flush=5), kb.EINVAL),
    (dict(m=6), kb.ECAPACITY),             # not a multiple of block_size
    (dict(m=12), kb.ECAPACITY),            # beyond capacity 8
    (dict(blocks_per_req=65), kb.ECAPACITY),
    (dict(block_size=16, blocks_per_req=33, m=16, num_blocks=66), kb.ECAPACITY),  # 528 > 512 positions
    (dict(m=-1), kb.EINVAL),
    (dict(scale=float("nan")), kb.EINVAL),
    (dict(out_dtype=2), kb.EINVAL),
    (dict(out_dtype=-1), kb.EINVAL),
])
def test_layout_validation(lib, kw, status):
    assert _decode(_layout(**kw)) == status


def test_null_arguments(lib):
    L = _layout()
    assert kb.kvbuf_decode(None, POOLS, BATCH, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, False) == kb.EINVAL
    assert _decode(L, pools=kb.Pools(FAKE, None, FAKE, FAKE)) == kb.EINVAL
    assert _decode(L, pools=kb.Pools(FAKE, FAKE, FAKE, None)) == kb.EINVAL  # gated rule needs gates
    assert _decode(L, batch=kb.Batch(2, FAKE, None, FAKE, None, FAKE)) == kb.EINVAL
    assert _decode(L, batch=kb.Batch(2, FAKE, FAKE, FAKE, None, None)) == kb.EINVAL  # per-tile copies
    assert _decode(L, batch=kb.Batch(2, FAKE, FAKE, None, None, FAKE)) == kb.EINVAL  # occupancy
    assert _decode(L, batch=kb.Batch(-1, FAKE, FAKE, FAKE, None, FAKE)) == kb.EINVAL
    assert _decode(L, q=None) == kb.EINVAL
    assert _decode(L, g=None) == kb.EINVAL
    assert _decode(_layout(rule=kb.RULE_DELTA), beta=None) == kb.EINVAL


def test_mode_specific_validation(lib):
    L = _layout()
    v = lambda n: kb.kvbuf_verify(L, POOLS, BATCH, n, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, False)
    assert v(0) == kb.EUNSUPPORTED
    assert v(9) == kb.EUNSUPPORTED
    L0 = _layout(m=0)
    assert kb.kvbuf_verify(L0, POOLS, BATCH, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, False) == kb.EUNSUPPORTED
    assert kb.kvbuf_direct(L0, POOLS, BATCH, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, False) == kb.EUNSUPPORTED
    assert kb.kvbuf_commit(L, POOLS, BATCH, 2, None, 0, False) == kb.EINVAL
    assert kb.kvbuf_commit(L, POOLS, BATCH, 9, FAKE, 0, False) == kb.EUNSUPPORTED
    assert kb.kvbuf_materialize(L, POOLS, BATCH, None, 0, False) == kb.EINVAL
    # empty batches and m = 0 flushes enqueue nothing and succeed
    empty = kb.Batch(0, None, None, None, None)
    assert _decode(L, batch=empty) == kb.OK
    assert kb.kvbuf_flush(L0, POOLS, BATCH, 0, False) == kb.OK


def test_recurrent_verification_validation(lib):
    L0 = _layout(m=0)
    vr = lambda L, n, temp=FAKE: kb.kvbuf_verify_recurrent(L, POOLS, BATCH, n, FAKE, FAKE, FAKE, FAKE, None,
                                                           FAKE, temp, 0, False)
    cr = lambda L, n, acc=FAKE, temp=FAKE: kb.kvbuf_commit_recurrent(L, POOLS, BATCH, n, acc, temp, 0, False)
    assert vr(_layout(), 2) == kb.EUNSUPPORTED      # the baseline has no buffer: m = 0 only
    assert vr(L0, 0) == kb.EUNSUPPORTED
    assert vr(L0, 9) == kb.EUNSUPPORTED
    assert vr(L0, 2, temp=None) == kb.EINVAL
    assert cr(_layout(), 2) == kb.EUNSUPPORTED
    assert cr(L0, 2, acc=None) == kb.EINVAL
    assert cr(L0, 2, temp=None) == kb.EINVAL
    assert cr(L0, 9) == kb.EUNSUPPORTED
    empty = kb.Batch(0, None, None, None, None)
    assert kb.kvbuf_verify_recurrent(L0, POOLS, empty, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 0,
                                     False) == kb.OK


def test_channel_rule_validation(lib):
    """The per-channel rule takes the same host checks as the others (it is
    served at every draft count and row length): its gates are required."""
    L = _layout(rule=kb.RULE_CHANNEL)
    assert kb.kvbuf_verify(L, POOLS, BATCH, 9, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, False) == kb.EUNSUPPORTED
    assert kb.kvbuf_verify(L, POOLS, BATCH, 2, FAKE, FAKE, FAKE, None, None, FAKE, 0, False) == kb.EINVAL
    assert _decode(_layout(rule=kb.RULE_CHANNEL, block_size=4, blocks_per_req=17, num_blocks=40), g=None) == kb.EINVAL


def test_tree_entry_validation(lib):
    """Tree drafts need a buffer (m > 0), 1 <= n <= 8 and parent (and leaf)
    arrays."""
    L = _layout()
    vt = lambda L, n, parent=FAKE: kb.kvbuf_verify_tree(L, POOLS, BATCH, n, parent, FAKE, FAKE, FAKE, FAKE, None,
                                                        FAKE, 0, False)
    ct = lambda L, n, parent=FAKE, leaf=FAKE: kb.kvbuf_commit_tree(L, POOLS, BATCH, n, parent, leaf, 0, False)
    assert vt(L, 2, parent=None) == kb.EINVAL
    assert vt(L, 0) == kb.EUNSUPPORTED
    assert vt(L, 9) == kb.EUNSUPPORTED
    assert vt(_layout(m=0), 2) == kb.EUNSUPPORTED
    assert ct(L, 2, parent=None) == kb.EINVAL
    assert ct(L, 2, leaf=None) == kb.EINVAL
    assert ct(L, 0) == kb.EUNSUPPORTED
    assert ct(L, 9) == kb.EUNSUPPORTED
    assert ct(_layout(m=0), 2) == kb.EUNSUPPORTED
    empty = kb.Batch(0, None, None, None, None)
    assert kb.kvbuf_commit_tree(L, POOLS, empty, 2, FAKE, FAKE, 0, False) == kb.OK


def test_metadata_entry_validation(lib):
    """kvbuf_admit needs a buffer (m > 0) and a non-negative count with a
    request list; kvbuf_check needs the error word it reports through."""
    L = _layout()
    assert kb.kvbuf_admit(_layout(m=0), BATCH, None, 0, 0, False) == kb.EUNSUPPORTED
    assert kb.kvbuf_admit(L, BATCH, FAKE, -1, 0, False) == kb.EINVAL
    assert kb.kvbuf_admit(L, kb.Batch(2, FAKE, FAKE, FAKE, None, None), None, 0, 0, False) == kb.EINVAL
    assert kb.kvbuf_admit(L, BATCH, FAKE, 0, 0, False) == kb.OK  # nothing listed: nothing enqueued
    assert kb.kvbuf_check(L, BATCH, 0, False) == kb.EINVAL  # no error word
    empty = kb.Batch(0, None, None, None, None, None)
    assert kb.kvbuf_admit(L, empty, None, 0, 0, False) == kb.OK
    assert kb.kvbuf_check(L, empty, 0, False) == kb.OK
