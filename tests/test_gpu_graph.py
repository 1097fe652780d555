"""The library's calls inside a captured HIP graph.

Every entry point enqueues kernels on the caller's stream and nothing else (no
host synchronisation, allocation or memset), so a serving loop can capture a
buffer cycle once and replay it.  A cycle of decodes followed by a verify and a
commit is captured on one set of pools and replayed several times; between
replays the test does eager work (fresh inputs copied into the captured input
buffers, synchronisations), and after every replay the outputs, the state
pool, the buffer pools and the bookkeeping must equal, bit for bit, those of
the same calls made eagerly on a twin set of pools.
"""

import pytest
import torch

import synth
import linear_attention_decode_kvbuf_amd as kb

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _pools(w, dev):
    kv = kb.KVBuffer(batch=w.B, heads=w.H, d=w.dk, m=w.m, block_size=w.block_size,
                     blocks_per_req=w.blocks_per_req, num_blocks=w.B * w.blocks_per_req, num_state_slots=w.B,
                     rule=w.rule, io_dtype=kb.BF16, flush=kb.FLUSH_EAGER, device=dev)
    kv.set_block_table(synth.block_permutation(w, w.B * w.blocks_per_req).reshape(w.B, w.blocks_per_req))
    kv.state_slot.copy_(torch.from_numpy(synth.slot_permutation(w, w.B)))
    kv.state.copy_(synth.device_initial_state(w, w.B, dev))
    return kv


def _inputs(w, call, dev, n):
    steps = [synth.device_token_inputs(w, 10 * call + t, dev) for t in range(w.m)]
    drafts = synth.device_token_inputs(w, 10 * call + 9, dev, n=n, stream_base=100)
    acc = torch.from_numpy(synth.accepted_lengths(w, call, w.B, n)).to(dev)
    return steps, drafts, acc


def _run(kv, steps, drafts, acc, outs, vout, n):
    for j, r in enumerate(steps):
        kv.decode(r["q"], r["k"], r["v"], r["g"], r["beta"], out=outs[j])
    kv.verify(drafts["q"], drafts["k"], drafts["v"], drafts["g"], drafts["beta"], out=vout)
    kv.commit(n, acc)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_buffer_cycle_replayed_from_a_graph(rule):
    dev = torch.device("cuda")
    w = synth.workload(3, B=24, H=4, m=8, block_size=8, blocks_per_req=3, rule=rule)
    n = 3
    eager, graphed = _pools(w, dev), _pools(w, dev)
    outs_e = torch.zeros((w.m, w.B, w.H, w.dv), device=dev)
    outs_g = torch.zeros_like(outs_e)
    v_e = torch.zeros((w.B, n, w.H, w.dv), device=dev)
    v_g = torch.zeros_like(v_e)

    # the captured graph reads its inputs from these buffers
    st_steps, st_drafts, st_acc = _inputs(w, 0, dev, n)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _run(graphed, st_steps, st_drafts, st_acc, outs_g, v_g, n)
    torch.cuda.synchronize()
    # capture records the launches without running them
    assert int(graphed.occupancy.abs().sum().item()) == 0

    for call in range(1, 5):
        steps, drafts, acc = _inputs(w, call, dev, n)  # eager work between replays
        for j in range(w.m):
            for key, x in steps[j].items():
                if x is not None:
                    st_steps[j][key].copy_(x)
        for key, x in drafts.items():
            if x is not None:
                st_drafts[key].copy_(x)
        st_acc.copy_(acc)
        torch.cuda.synchronize()
        graph.replay()
        _run(eager, steps, drafts, acc, outs_e, v_e, n)
        torch.cuda.synchronize()
        assert int(eager.error.item()) == 0 and int(graphed.error.item()) == 0
        assert torch.equal(outs_g, outs_e), "replay %d: decode outputs" % call
        assert torch.equal(v_g, v_e), "replay %d: verify outputs" % call
        for name in ("state", "key", "value", "gate", "block_table", "occupancy", "tile_meta"):
            a, b = getattr(graphed, name), getattr(eager, name)
            if a is not None:
                assert torch.equal(a, b), "replay %d: %s" % (call, name)
