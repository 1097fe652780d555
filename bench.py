#!/usr/bin/env python3
"""Benchmark of the KVBuffer decode path on one MI355X.

Workload: one scalar-gated linear-attention layer, B=256 requests, H=32 heads,
d_k=d_v=128, buffer m=8 (blocks of 8, two per request, shuffled pool), bf16
q/k/v, fp32 state ~ N(0, 0.02), fold fused into the decode that fills the
buffer.  One "step" is one full buffer cycle: m decode launches over the whole
batch, the last of which folds the buffer into the state (KVBuffer: IO-aware
Serving for Linear Attention, pith.science page, Figure 3 caption: kernel
latency is averaged over a full buffer cycle -- occupancies 0 .. m-1 and the
state update).  Inputs are a ring of 2m pre-generated steps resident in HBM.

Also measured in the same run: the m = 0 recurrent kernel at the same shape
(the figure's normaliser), the variant with a separate flush launch,
compute-free probe kernels streaming the same tiles (the measured ceilings of
the access pattern), the other workloads' legs and the oracle on the host
cores.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published


# Algorithmic bytes per (request, head) tile: 2-byte q/k/v, 4-byte state,
# gates and outputs; `gated` = a gate per token (4 bytes; the linear rule has
# none); `gate` overrides the bytes of one token's gates (4 d_k for the
# per-channel rule).
def _gate(gated, gate):
    return gate if gate is not None else (4 if gated else 0)


def decode_bytes(j, dk, dv, io=2, gated=True, gate=None):
    return (4 * dk * dv                        # state tile read
            + io * (2 * dk + dv)               # q, k, v of the new token
            + io * (dk + dv)                   # append of k, v to the pool
            + io * j * (dk + dv)               # buffered keys and values
            + 4 * dv                           # output
            + _gate(gated, gate) * (j + 2))    # gates: buffered, new, appended


def flush_bytes(m, dk, dv, io=2, gated=True, gate=None):
    return 8 * dk * dv + m * (io * (dk + dv) + _gate(gated, gate))


def recurrent_bytes(dk, dv, io=2, gated=True, gate=None):
    return 8 * dk * dv + io * (2 * dk + dv) + 4 * dv + _gate(gated, gate)


def cycle_bytes_fused(m, dk, dv, io=2, gated=True, gate=None):
    """Decodes at occupancy 0 .. m-1 plus one state write (the fold reads the
    state and the buffered tokens the last decode already reads)."""
    return sum(decode_bytes(j, dk, dv, io, gated, gate) for j in range(m)) + 4 * dk * dv


def cycle_bytes_separate(m, dk, dv, io=2, gated=True, gate=None):
    return (sum(decode_bytes(j, dk, dv, io, gated, gate) for j in range(m))
            + flush_bytes(m, dk, dv, io, gated, gate))


def _traffic_file(m):
    return os.path.join(ROOT, "profiles", "traffic_decode_kernel_B256_H32_d128_m%d.txt" % m)


def _kernel_source_digest():
    import hashlib

    h = hashlib.sha256()
    for name in ("decode.hip", "device_common.hpp", "kvbuf_internal.hpp"):
        with open(os.path.join(ROOT, "linear_attention_decode_kvbuf_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(m, launches_per_cycle):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy kernel's reading), if measured for the
    current kernel source; else None."""
    path = _traffic_file(m)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_digest") != _kernel_source_digest():
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_kv(kb, synth, torch, w, flush, device):
    kv = kb.KVBuffer(batch=w.B, heads=w.H, d=w.dk, m=w.m, block_size=max(w.block_size, 1),
                     blocks_per_req=w.blocks_per_req, num_blocks=max(w.B * w.blocks_per_req, 1),
                     num_state_slots=w.B, rule=w.rule, io_dtype=kb.BF16, flush=flush, device=device)
    if w.m > 0:
        perm = synth.block_permutation(w, w.B * w.blocks_per_req)
        kv.set_block_table(perm.reshape(w.B, w.blocks_per_req))
    kv.state_slot.copy_(torch.from_numpy(synth.slot_permutation(w, w.B)))
    kv.state.copy_(synth.device_initial_state(w, w.B, device))
    return kv


def make_ring(synth, w, device, size):
    return [synth.device_token_inputs(w, t, device) for t in range(size)]


def time_loop(torch, fn, cycles, warmup, events=False):
    """Wall time of ``cycles`` calls of fn after ``warmup`` untimed ones; with
    events=True also the time between HIP events recorded on the current
    stream (the one the kernels are launched on) around the same region."""
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(cycles):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if events:
        return wall, e0.elapsed_time(e1) * 1e-3
    return wall


def per_launch_ms(torch, launches, reps, median=False):
    """Duration (ms) of each launch in ``launches`` (a list of callables
    issued back to back), from HIP events recorded on the stream the kernels
    run on, over ``reps`` repetitions: the mean, or the median."""
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record(stream)
        for i, fn in enumerate(launches):
            fn()
            evs[r][i + 1].record(stream)
    torch.cuda.synchronize()
    times = [[evs[r][i].elapsed_time(evs[r][i + 1]) for r in range(reps)] for i in range(len(launches))]
    if median:
        return [sorted(t)[len(t) // 2] for t in times]
    return [sum(t) / reps for t in times]


def cpu_baseline(synth, oracle, np, torch, w, ring, max_tiles=None, min_seconds=10.0, max_passes=64):
    """The oracle (fp64 per-token recurrence) over consecutive tokens of the
    same workload on the host's cores; returns tokens/s in the metric's unit
    (tokens of all B requests per second, scaled from the sampled tiles).
    Each pass takes the next m tokens of the input ring, starting from the
    state the previous pass left, until at least min_seconds have elapsed."""
    ncores = len(os.sched_getaffinity(0))
    tiles = w.B * w.H if max_tiles is None else min(max_tiles, w.B * w.H)
    steps = w.m
    n = len(ring)
    q = np.stack([r["q"].reshape(-1, w.dk)[:tiles].float().cpu().numpy() for r in ring])
    k = np.stack([r["k"].reshape(-1, w.dk)[:tiles].float().cpu().numpy() for r in ring])
    v = np.stack([r["v"].reshape(-1, w.dv)[:tiles].float().cpu().numpy() for r in ring])
    g = np.stack([r["g"].reshape(-1)[:tiles].cpu().numpy() for r in ring])
    S0 = synth.device_initial_state(w, w.B, torch.device("cuda")).reshape(
        -1, w.dk, w.dv)[:tiles].double().cpu().numpy()
    used = oracle.threads_used(ncores)

    def run(ntiles, nthreads, seconds):
        S, passes, spent = S0[:ntiles], 0, 0.0
        while passes < max_passes and (passes == 0 or spent < seconds):
            idx = [(passes * steps + j) % n for j in range(steps)]
            t0 = time.perf_counter()
            _, S = oracle.recurrent(1, S, q[idx, :ntiles], k[idx, :ntiles], v[idx, :ntiles],
                                    g=g[idx, :ntiles], nthreads=nthreads)
            spent += time.perf_counter() - t0
            passes += 1
        return passes, spent

    passes, dt = run(tiles, ncores, min_seconds)
    # the same on one thread, over the first 1/16 of the tiles
    t1 = max(1, tiles // 16)
    passes1, dt1 = run(t1, 1, min_seconds / 5)
    return {
        "value": tiles * steps * passes / dt / w.H,  # a token of one request = H tiles
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "sample": "fp64 recurrent oracle (C, OpenMP over tiles), %d passes of %d consecutive tokens over %d "
                  "of the %d (request, head) tiles of the same workload, %.1f s" % (
                      passes, steps, tiles, w.B * w.H, dt),
        "one_thread": {"value": t1 * steps * passes1 / dt1 / w.H, "unit": "tokens/s",
                       "sample": "%d passes of %d tokens over %d tiles, %.1f s" % (passes1, steps, t1, dt1)},
    }


def cycle_leg(kb, synth, torch, dev, w, cycles, warmup):
    """Full buffer cycles (eager policy, fold fused into the filling decode)
    of workload w, or decode steps of the recurrent kernel when w.m = 0.
    Returns tokens/s, time per cycle, algorithmic HBM GB/s and bytes per
    token (all H tiles of a request)."""
    gated = w.rule != 0
    gate = 4 * w.dk if w.rule == 3 else None  # per-channel rule: d_k gates per token
    m = max(w.m, 1)
    kv = build_kv(kb, synth, torch, w, kb.FLUSH_EAGER, dev)
    ring = make_ring(synth, w, dev, 2 * m)
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)

    def cycle(i):
        for j in range(m):
            r = ring[(i * m + j) % len(ring)]
            kv.decode(r["q"], r["k"], r["v"], r["g"] if gated else None, out=out)

    wall = time_loop(torch, cycle, cycles, warmup)
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    del kv
    tiles = w.B * w.H
    per_tile = (cycle_bytes_fused(w.m, w.dk, w.dv, gated=gated, gate=gate) if w.m > 0
                else recurrent_bytes(w.dk, w.dv, gated=gated, gate=gate))
    cyc_s = wall / cycles
    return {"m": w.m, "tokens_per_s": w.B * m / cyc_s, "ms_per_cycle": cyc_s * 1e3,
            "hbm_gbps": per_tile * tiles / cyc_s / 1e9,
            "hbm_frac_of_peak": per_tile * tiles / cyc_s / 1e9 / PEAK_HBM_GBPS,
            "bytes_per_token": per_tile * w.H / m}


def separate_cycle_leg(kb, synth, torch, dev, w, cycles, warmup):
    """Full buffer cycles under the deferred policy: m decode launches that
    only append, then one kvbuf_flush launch folding the m tokens."""
    m = w.m
    kv = build_kv(kb, synth, torch, w, kb.FLUSH_DEFERRED, dev)
    ring = make_ring(synth, w, dev, 2 * m)
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)

    def cycle(i):
        for j in range(m):
            r = ring[(i * m + j) % len(ring)]
            kv.decode(r["q"], r["k"], r["v"], r["g"], out=out)
        kv.flush()

    wall = time_loop(torch, cycle, cycles, warmup)
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    del kv
    tiles = w.B * w.H
    per_tile = cycle_bytes_separate(m, w.dk, w.dv)
    cyc_s = wall / cycles
    return {"m": m, "tokens_per_s": w.B * m / cyc_s, "ms_per_cycle": cyc_s * 1e3,
            "hbm_gbps": per_tile * tiles / cyc_s / 1e9,
            "hbm_frac_of_peak": per_tile * tiles / cyc_s / 1e9 / PEAK_HBM_GBPS,
            "bytes_per_token": per_tile * w.H / m}


def ceilings_leg(torch, dev):
    """What the memory system gives the decode path's access pattern, measured
    with compute-free probe kernels (libkvbuf_probe.so) at the metric shape:
    8192 fp32 tiles of 128 x 128 at shuffled slots, one 256-thread workgroup
    per tile, 16 non-temporal 128-bit loads per thread issued at once.
      read                  the state read alone
      read_write_1k         + 1 KiB written per tile (a decode's output row and
                            appended key and value)
      read_write_back       the tile read and written back in place (a fold)
      read_write_1k_read_24k  + 24 KiB more read per tile (a delta-rule decode's
                            buffered rows at occupancy 32)
      fold_m64, fold_m128   the tile read and written back plus 32 / 64 KiB
                            more read per tile (a flush of 64 / 128 bf16 key
                            and value rows)
    Each figure is the median of 20 launches: algorithmic bytes / duration."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_decode_kvbuf_amd", "libkvbuf_probe.so"))
    P, i32 = ctypes.c_void_p, ctypes.c_int
    lib.kvbuf_probe_stream.argtypes = [P, P, i32, i32, i32, P, i32, P, i32, P]
    lib.kvbuf_probe_stream.restype = i32
    d, ntiles = 128, 256 * 32
    tile = 4 * d * d
    tiles = torch.empty((ntiles, d, d), dtype=torch.float32, device=dev).normal_()
    slot = torch.randperm(ntiles, generator=torch.Generator().manual_seed(5)).to(torch.int32).to(dev)
    extra = 1024
    side = torch.zeros(ntiles * extra // 4, dtype=torch.float32, device=dev)
    side2 = torch.ones(ntiles * 65536 // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, kind, extra2 in (("read", 0, 0), ("read_write_1k", 1, 0), ("read_write_back", 2, 0),
                               ("read_write_1k_read_24k", 3, 24704), ("fold_m64", 4, 32768),
                               ("fold_m128", 4, 65536)):
        nbytes = tile * (2 if kind in (2, 4) else 1) + (extra if kind in (1, 3) else 0) + extra2

        def launch():
            rc = lib.kvbuf_probe_stream(tiles.data_ptr(), slot.data_ptr(), ntiles, d, kind, side.data_ptr(),
                                        extra if kind in (1, 3) else 0, side2.data_ptr(), extra2, stream)
            assert rc == 0, rc
        for _ in range(3):
            launch()
        ms = per_launch_ms(torch, [launch], 20, median=True)[0]
        out[name] = {"us": ms * 1e3, "gbps": nbytes * ntiles / (ms * 1e-3) / 1e9,
                     "frac_of_peak": nbytes * ntiles / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    torch.cuda.synchronize()
    del tiles, side, side2
    return out


def sweep_leg(kb, synth, torch, dev, args):
    """The Figure 3 protocol over buffer sizes m = 4, 8, 16, 32 of the metric
    workload (blocks of m, two per request): per-token latency averaged over a
    full buffer cycle -- decodes at occupancies 0 .. m-1 plus the state update
    -- normalised by the recurrent (m = 0) kernel's per-token latency, with
    the update fused into the decode that fills the buffer and as a separate
    flush launch (the pages time the update as its own step)."""
    w0 = synth.workload(3, m=0, block_size=1, blocks_per_req=1)
    rec = cycle_leg(kb, synth, torch, dev, w0, max(5, args.steps), max(2, args.warmup))
    rec_tok = rec["ms_per_cycle"] / w0.B  # one decode step per "cycle" at m = 0
    out = {"m0": rec}
    for m in (4, 8, 16, 32):
        w = synth.workload(3, m=m)
        cycles = max(5, args.steps * 8 // m)
        warm = max(2, args.warmup * 8 // m)
        fused = cycle_leg(kb, synth, torch, dev, w, cycles, warm)
        sep = separate_cycle_leg(kb, synth, torch, dev, w, cycles, warm)
        for leg in (fused, sep):
            leg["normalized_latency_vs_m0"] = (leg["ms_per_cycle"] / (m * w.B)) / rec_tok
        out["m%d" % m] = {"fused": fused, "separate_flush": sep}
    return out


def linear_leg(kb, synth, torch, dev, args):
    """Linear rule (no gates), B=64 H=32 d=128: buffered m=8 against the
    recurrent m=0 kernel at the same shape."""
    w = synth.workload(2)
    buf = cycle_leg(kb, synth, torch, dev, w, args.steps, args.warmup)
    rec = cycle_leg(kb, synth, torch, dev, synth.workload(2, m=0, blocks_per_req=1), args.steps, args.warmup)
    return {"m8": buf, "m0": rec, "speedup_vs_m0": buf["tokens_per_s"] / rec["tokens_per_s"]}


def channel_leg(kb, synth, torch, dev, args):
    """Per-channel gates (one log-gate per key channel) at the metric shape:
    buffered m = 8 against the recurrent m = 0 kernel of the same rule."""
    buf = cycle_leg(kb, synth, torch, dev, synth.workload(3, rule=3), args.steps, args.warmup)
    rec = cycle_leg(kb, synth, torch, dev, synth.workload(3, rule=3, m=0, blocks_per_req=1),
                    args.steps, args.warmup)
    return {"m8": buf, "m0": rec, "speedup_vs_m0": buf["tokens_per_s"] / rec["tokens_per_s"]}


def head_share_leg(kb, synth, torch, dev, args):
    """One GPU's share when the 32 heads are split over 8 GPUs: B=256 H=4
    (1024 tiles, 4 workgroups per CU), m=8, fold fused."""
    w = synth.workload(3, H=4)
    return cycle_leg(kb, synth, torch, dev, w, args.steps, args.warmup)


def context_leg(kb, synth, torch, dev, args):
    """A request's first L tokens, L = 16 .. 256, served three ways at the
    metric shape (B=256 H=32 d=128, gated): recurrent (m = 0: the state is
    read and written every token), chunkwise (m = 8, fold fused) and
    buffer-only (kvbuf_direct with a buffer of capacity >= L: no state at
    all).  Then the promotion of the buffer-only requests: a zeroed state
    slot and one kvbuf_flush folding all L buffered tokens (the page's
    Figure 5 compares the three decoding forms over context lengths 16-256;
    the abstract: short contexts are served from the buffer alone)."""
    out = {}
    reps = 3
    for L in (16, 32, 64, 128, 256):
        w = synth.workload(3, steps=L)
        ring = make_ring(synth, w, dev, 16)
        obuf = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)

        def run(kv, direct):
            fn = kv.direct if direct else kv.decode
            for t in range(L):
                r = ring[t % len(ring)]
                fn(r["q"], r["k"], r["v"], r["g"], out=obuf)

        res = {}
        for name, wl, direct in (("recurrent", synth.workload(3, m=0, blocks_per_req=1), False),
                                 ("chunkwise_m8", synth.workload(3, m=8), False),
                                 ("buffer_only", synth.workload(3, m=L, block_size=min(L, 16),
                                                                blocks_per_req=max(L // 16, 1)), True)):
            kv = build_kv(kb, synth, torch, wl, kb.FLUSH_EAGER, dev)
            if direct:
                kv.state_slot.fill_(-1)
            times = []
            for _ in range(reps):
                if wl.m > 0:  # (the recurrent form keeps no buffer)
                    kv.occupancy.zero_()
                    kv.admit()
                torch.cuda.synchronize()
                stream = torch.cuda.current_stream()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(kv, direct)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            assert int(kv.error.item()) == 0
            res[name] = {"ms_per_token_step": min(times) / L}
            if direct:
                # promotion: every request gets a zeroed slot, then one fold of
                # its L tokens.  m = capacity, so the fold's table rotation is
                # the identity and the same buffer can be promoted again: the
                # second promotion is timed.
                kv.state_slot.copy_(torch.from_numpy(synth.slot_permutation(w, w.B)).to(dev))
                pt = []
                for _ in range(2):
                    kv.occupancy.fill_(L)
                    kv.admit()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record(torch.cuda.current_stream())
                    kv.state.zero_()
                    kv.flush()
                    e1.record(torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    assert int(kv.error.item()) == 0
                    assert int(kv.occupancy.max().item()) == 0
                    pt.append(e0.elapsed_time(e1))
                res[name]["promotion_ms"] = pt[-1]
            del kv
        rec = res["recurrent"]["ms_per_token_step"]
        for v in res.values():
            v["normalized_to_recurrent"] = v["ms_per_token_step"] / rec
        out["L%d" % L] = res
    return out


def verify_leg(kb, synth, torch, dev, args):
    """B=128 H=32 d=128 m=8 gated: per n, one kvbuf_verify of n drafts then
    one kvbuf_commit of the accepted prefixes (the fold, when a commit fills
    the buffer, runs inside the commit)."""
    w = synth.workload(4)
    tiles = w.B * w.H
    out = {}
    for n in (1, 2, 4, 8):
        kv = build_kv(kb, synth, torch, w, kb.FLUSH_EAGER, dev)
        drafts = [synth.device_token_inputs(w, c, dev, n=n, stream_base=100) for c in range(4)]
        accs = [torch.from_numpy(synth.accepted_lengths(w, c, w.B, n)).to(dev) for c in range(4)]
        obuf = torch.empty((w.B, n, w.H, w.dv), dtype=torch.float32, device=dev)

        def call(c):
            d = drafts[c % 4]
            return [lambda: kv.verify(d["q"], d["k"], d["v"], d["g"], out=obuf),
                    lambda: kv.commit(n, accs[c % 4])]

        for c in range(10):
            for f in call(c):
                f()
        launches = []
        for c in range(8):
            launches += call(c)
        per = per_launch_ms(torch, launches, 20)
        torch.cuda.synchronize()
        assert int(kv.error.item()) == 0
        ver = sum(per[0::2]) / 8
        com = sum(per[1::2]) / 8
        accepted = float(sum(int(a.sum()) for a in accs[:4]) / 4)
        # one state read serves all n drafts
        vbytes = tiles * (4 * w.dk * w.dv + 2 * n * (2 * w.dk + w.dv) + 4 * n * w.dv)
        res = {"verify_ms": ver, "commit_ms": com,
               "verify_hbm_gbps": vbytes / (ver * 1e-3) / 1e9,
               "verify_frac_of_peak": vbytes / (ver * 1e-3) / 1e9 / PEAK_HBM_GBPS,
               "accepted_tokens_per_s": accepted / ((ver + com) * 1e-3)}
        res["tree"] = tree_verify(kb, synth, torch, kv, w, n, drafts, obuf, vbytes)
        del kv
        res["recurrent_baseline"] = verify_baseline(kb, synth, torch, dev, w, n, drafts, accs)
        # state memory per request: KVBuffer keeps one state and a buffer of
        # capacity block_size * blocks_per_req; the baseline keeps the state
        # and one temporary state per draft (Figure 2 caption)
        s_bytes = w.H * 4 * w.dk * w.dv
        cap = w.block_size * w.blocks_per_req
        kvb = s_bytes + w.H * cap * (2 * (w.dk + w.dv) + 4)
        base = (1 + n) * s_bytes
        res["state_memory_per_request_bytes"] = {"kvbuffer": kvb, "recurrent_temporaries": base,
                                                 "requests_ratio": base / kvb}
        out["n%d" % n] = res
    return out


def tree_verify(kb, synth, torch, kv, w, n, drafts, obuf, vbytes):
    """The same drafts arranged as random trees (kvbuf_verify_tree: each draft
    attends to its ancestors only, decays along its path), then
    kvbuf_commit_tree of a random root-to-leaf path per request."""
    dev = obuf.device
    trees = [synth.draft_tree(w, c, w.B, n) for c in range(4)]
    par = [torch.from_numpy(p).to(dev) for p, _ in trees]
    leaf = [torch.from_numpy(lf).to(dev) for _, lf in trees]

    def depth(p, d):
        k = 0
        while d >= 0:
            k, d = k + 1, int(p[d])
        return k

    kept = [sum(depth(p[b], int(lf[b])) for b in range(w.B)) for p, lf in trees]

    def call(c):
        d = drafts[c % 4]
        return [lambda: kv.verify_tree(par[c % 4], d["q"], d["k"], d["v"], d["g"], out=obuf),
                lambda: kv.commit_tree(par[c % 4], leaf[c % 4])]

    for c in range(4):
        for f in call(c):
            f()
    launches = []
    for c in range(8):
        launches += call(c)
    per = per_launch_ms(torch, launches, 20)
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    ver = sum(per[0::2]) / 8
    com = sum(per[1::2]) / 8
    accepted = sum(kept) / 4
    return {"verify_ms": ver, "commit_ms": com, "verify_hbm_gbps": vbytes / (ver * 1e-3) / 1e9,
            "verify_frac_of_peak": vbytes / (ver * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "accepted_tokens_per_s": accepted / ((ver + com) * 1e-3)}


def verify_baseline(kb, synth, torch, dev, w, n, drafts, accs):
    """The verification KVBuffer replaces: recurrent form with a temporary
    state per draft (m = 0), then the commit that copies the last accepted
    draft's temporary state into the request's slot."""
    w0 = synth.workload(4, m=0, blocks_per_req=1)
    kv = build_kv(kb, synth, torch, w0, kb.FLUSH_EAGER, dev)
    temp = torch.empty((n, w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    obuf = torch.empty((w.B, n, w.H, w.dv), dtype=torch.float32, device=dev)

    def call(c):
        d = drafts[c % 4]
        return [lambda: kv.verify_recurrent(d["q"], d["k"], d["v"], d["g"], out=obuf, temp=temp),
                lambda: kv.commit_recurrent(n, accs[c % 4], temp)]

    for c in range(4):
        for f in call(c):
            f()
    launches = []
    for c in range(8):
        launches += call(c)
    per = per_launch_ms(torch, launches, 10)
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    del kv, temp
    ver = sum(per[0::2]) / 8
    com = sum(per[1::2]) / 8
    tiles = w.B * w.H
    vbytes = tiles * (4 * w.dk * w.dv * (1 + n) + 2 * n * (2 * w.dk + w.dv) + 4 * n * (w.dv + 1))
    accepted = float(sum(int(a.sum()) for a in accs[:4]) / 4)
    return {"verify_ms": ver, "commit_ms": com, "verify_hbm_gbps": vbytes / (ver * 1e-3) / 1e9,
            "verify_frac_of_peak": vbytes / (ver * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "accepted_tokens_per_s": accepted / ((ver + com) * 1e-3)}


def long_fold_leg(kb, synth, torch, dev, args):
    """kvbuf_flush of m = 32, 64, 128 buffered tokens at B=256 H=32 d=128
    (deferred policy, scalar-gated and delta rules): one state read and write
    plus the m rows per tile; folds of more than 16 positions run their rank-m
    update on the matrix cores."""
    out = {}
    for rule, name in ((kb.RULE_GATED, "gated"), (kb.RULE_DELTA, "delta")):
        for m in (32, 64, 128):
            w = synth.workload(3, m=m, block_size=m, blocks_per_req=1, rule=rule)
            kv = kb.KVBuffer(batch=w.B, heads=w.H, d=w.dk, m=m, block_size=m, blocks_per_req=1, num_blocks=w.B,
                             num_state_slots=w.B, rule=rule, io_dtype=kb.BF16, flush=kb.FLUSH_DEFERRED,
                             device=dev)
            kv.state.normal_(0.0, 0.02)
            kv.key.normal_()
            kv.value.normal_()
            kv.gate.uniform_(-0.1, 0.0)

            def fill():
                kv.occupancy.fill_(m)
                kv.admit()

            launches = []
            for _ in range(4):
                launches += [fill, kv.flush]
            for f in launches:
                f()
            per = per_launch_ms(torch, launches, 5)
            torch.cuda.synchronize()
            assert int(kv.error.item()) == 0
            ms = sum(per[1::2]) / 4
            xb = 4 * w.dv if rule == kb.RULE_DELTA else 2 * w.dv  # pseudo-values are fp32
            tile_bytes = 8 * w.dk * w.dv + m * (2 * w.dk + xb + 4)
            gbps = tile_bytes * w.B * w.H / (ms * 1e-3) / 1e9
            out["%s_m%d" % (name, m)] = {"flush_ms": ms, "hbm_gbps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS,
                                         "algorithmic_bytes_per_launch": tile_bytes * w.B * w.H}
            del kv
    return out


def copy_leg(torch, dev):
    """A 1 GiB device-to-device copy, repeated: it reads 1 GiB and writes
    1 GiB per dispatch, so the HBM counters' readings for it (rocprofv3
    FETCH_SIZE, WRITE_SIZE) give the factors that turn their readings for the
    library's kernels into bytes."""
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "ms": ms, "gbps": 8 * n / (ms * 1e-3) / 1e9}


def delta_decode_bytes(j, dk, dv, stateful):
    """Algorithmic bytes of one delta-rule decode of a tile at occupancy j:
    state read (requests with a state), q / k / v in (bf16), log-gate and
    step size in, j buffered rows read (bf16 key, fp32 pseudo-value, fp32
    log-gate), the new row appended, the output written (fp32)."""
    row = 2 * dk + 4 * dv + 4
    return (4 * dk * dv if stateful else 0) + 2 * (2 * dk + dv) + 8 + row * (j + 1) + 4 * dv


def delta_fold_bytes(m, dk, dv):
    """A fold of m delta-rule rows: state read and write plus the m rows."""
    return 8 * dk * dv + m * (2 * dk + 4 * dv + 4)


def delta_leg(kb, synth, torch, dev, args):
    """Gated delta rule, B=512 (256 requests with a state, 256 served from the
    buffer alone), H=32 d=128 m=64, over a full 64-step cycle.  A step is
    kvbuf_decode over the requests with a state (the chunk kernel) and
    kvbuf_direct over the buffer-only ones (one wave per tile), each on a view
    of its request range.  The requests with a state flush under the deferred
    policy: every request starts the cycle empty, so at step t all tiles are
    at occupancy t, and the last step ends with one kvbuf_flush of the 64
    buffered tokens of every request with a state."""
    w = synth.workload(5)
    kv = kb.KVBuffer(batch=w.B, heads=w.H, d=w.dk, m=w.m, block_size=w.block_size,
                     blocks_per_req=w.blocks_per_req, num_blocks=w.B * w.blocks_per_req,
                     num_state_slots=w.B - w.n_short, rule=kb.RULE_DELTA, io_dtype=kb.BF16,
                     flush=kb.FLUSH_DEFERRED, device=dev)
    perm = synth.block_permutation(w, w.B * w.blocks_per_req)
    kv.set_block_table(perm.reshape(w.B, w.blocks_per_req))
    slots = torch.full((w.B,), -1, dtype=torch.int32)
    slots[: w.B - w.n_short] = torch.arange(w.B - w.n_short, dtype=torch.int32)
    kv.state_slot.copy_(slots)
    kv.state.copy_(synth.device_initial_state(w, w.B - w.n_short, dev))
    ring = [synth.device_token_inputs(w, t, dev) for t in range(8)]
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)
    # requests with a state: kvbuf_decode on a view of their range; the
    # buffer-only ones: kvbuf_direct on a view of theirs
    s = w.B - w.n_short
    long_kv, short_kv = kv.view(0, s), kv.view(s, w.n_short)

    def step(r, last):
        part = lambda a, z: [None if r[x] is None else r[x][a:z] for x in ("q", "k", "v", "g", "beta")]
        lo, hi, out_lo, out_hi = part(0, s), part(s, w.B), out[:s], out[s:]
        if last:  # the deferred flush of the requests with a state, whose buffers are now full
            return lambda: (long_kv.decode(*lo, out=out_lo), short_kv.direct(*hi, out=out_hi), long_kv.flush())
        return lambda: (long_kv.decode(*lo, out=out_lo), short_kv.direct(*hi, out=out_hi))

    fns = [step(ring[t % 8], t == w.m - 1) for t in range(w.m)]
    for f in fns:  # one warm cycle
        f()
    per = [0.0] * w.m
    reps = 3
    for _ in range(reps):
        # every request starts the cycle empty: the stateful ones folded at
        # its last step, the buffer-only ones are restarted (capacity 128)
        kv.occupancy.zero_()
        kv.admit()
        per = [a + b / reps for a, b in zip(per, per_launch_ms(torch, fns, 1))]
    torch.cuda.synchronize()
    assert int(kv.error.item()) == 0
    cyc = sum(per)
    n_long = (w.B - w.n_short) * w.H
    n_short = w.n_short * w.H
    step_bytes = [n_long * delta_decode_bytes(t, w.dk, w.dv, True) + n_short * delta_decode_bytes(t, w.dk, w.dv, False)
                  for t in range(w.m)]
    step_bytes[-1] += n_long * delta_fold_bytes(w.m, w.dk, w.dv)
    cyc_bytes = sum(step_bytes)
    gbps = cyc_bytes / (cyc * 1e-3) / 1e9
    step_gbps = [b / (t * 1e-3) / 1e9 for b, t in zip(step_bytes, per)]
    return {"cycle_ms": cyc, "tokens_per_s": w.B * w.m / (cyc * 1e-3),
            "decode_step_ms_mean": cyc / w.m, "fold_step_ms": per[-1],
            "step_ms": [round(x, 4) for x in per],
            "algorithmic_bytes_per_cycle": cyc_bytes, "hbm_gbps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS,
            "step_frac_of_peak": [round(x / PEAK_HBM_GBPS, 3) for x in step_gbps]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed buffer cycles")
    ap.add_argument("--warmup", type=int, default=20, help="untimed buffer cycles")
    ap.add_argument("--m", type=int, default=8, help="buffer size")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--no-extras", action="store_true", help="skip the m=0 / separate-flush / copy legs")
    ap.add_argument("--only", choices=["fused", "recurrent", "separate", "ceilings", "copy", "verify", "delta", "sweep",
                                       "linear", "heads4", "context", "channel", "longfold"], default=None,
                    help="run one leg only (for profiling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode path has no cross-GPU step, and what is "
              "measured is one GPU's kernel (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import linear_attention_decode_kvbuf_amd as kb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = args.m
    w = synth.workload(3, m=m, block_size=m, blocks_per_req=2)
    tiles = w.B * w.H
    ring = make_ring(synth, w, dev, 2 * m)
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)
    result = {}

    def decode_fn(kv, t):
        r = ring[t % len(ring)]
        return lambda: kv.decode(r["q"], r["k"], r["v"], r["g"], out=out)

    # ---- headline: fused fold, one step = one buffer cycle ----------------
    if args.only in (None, "fused"):
        kv = build_kv(kb, synth, torch, w, kb.FLUSH_EAGER, dev)

        def cycle(i):
            for j in range(m):
                decode_fn(kv, i * m + j)()

        wall, ev = time_loop(torch, cycle, args.steps, args.warmup, events=True)
        ms_per_step = wall / args.steps * 1e3
        tok_s = w.B * m * args.steps / wall
        # each decode call is one decode_kernel launch: the average launch
        # duration is the event time of the timed region over its launches
        avg_launch_ms = ev * 1e3 / (args.steps * m)
        # per-occupancy durations, medians over the cycles, one event pair per
        # launch (each adds an event record to the launch it brackets)
        reps = max(10, min(args.steps, 50))
        per = per_launch_ms(torch, [decode_fn(kv, j) for j in range(m)], reps, median=True)
        torch.cuda.synchronize()
        assert int(kv.error.item()) == 0
        cyc_bytes = cycle_bytes_fused(m, w.dk, w.dv) * tiles
        achieved = cyc_bytes / m / (avg_launch_ms * 1e-3) / 1e9
        traffic = read_traffic(m, m)
        result.update(
            value=tok_s, ms_per_step=ms_per_step,
            hbm_gbps=cyc_bytes / (wall / args.steps) / 1e9,
            hbm_frac_of_peak=cyc_bytes / (wall / args.steps) / 1e9 / PEAK_HBM_GBPS,
            bytes_per_token=cyc_bytes / m / w.B,
            per_occupancy_ms=[round(x, 5) for x in per],
            roofline={"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                      "kernel": "decode_kernel (one-token decode; the last launch of a cycle folds)",
                      "avg_launch_ms": avg_launch_ms,
                      "algorithmic_bytes_per_launch": cyc_bytes / m},
        )
        del kv

    # ---- m = 0 recurrent kernel at the same shape -------------------------
    if not args.no_extras and args.only in (None, "recurrent"):
        w0 = synth.workload(3, m=0, block_size=1, blocks_per_req=1)
        kv0 = build_kv(kb, synth, torch, w0, kb.FLUSH_EAGER, dev)
        wall0, ev0 = time_loop(torch, lambda i: [decode_fn(kv0, i * m + j)() for j in range(m)],
                               args.steps, args.warmup, events=True)
        avg0 = ev0 * 1e3 / (args.steps * m)
        b0 = recurrent_bytes(w.dk, w.dv) * tiles
        result["m0_recurrent"] = {
            "tokens_per_s": w.B * m * args.steps / wall0,
            "ms_per_token_step": wall0 / (args.steps * m) * 1e3,
            "avg_launch_ms": avg0,
            "hbm_gbps": b0 / (avg0 * 1e-3) / 1e9,
            "bytes_per_token": b0 / w.B,
        }
        del kv0

    # ---- separate flush launch (deferred policy) --------------------------
    if not args.no_extras and args.only in (None, "separate"):
        kvd = build_kv(kb, synth, torch, w, kb.FLUSH_DEFERRED, dev)

        def cycle_d(i):
            for j in range(m):
                decode_fn(kvd, i * m + j)()
            kvd.flush()

        walld = time_loop(torch, cycle_d, args.steps, args.warmup)
        perd = per_launch_ms(torch, [decode_fn(kvd, j) for j in range(m)] + [kvd.flush], 20)
        torch.cuda.synchronize()
        assert int(kvd.error.item()) == 0
        bd = cycle_bytes_separate(m, w.dk, w.dv) * tiles
        result["separate_flush"] = {
            "tokens_per_s": w.B * m * args.steps / walld,
            "ms_per_cycle": walld / args.steps * 1e3,
            "decode_avg_launch_ms": sum(perd[:m]) / m,
            "flush_launch_ms": perd[m],
            "flush_hbm_gbps": flush_bytes(m, w.dk, w.dv) * tiles / (perd[m] * 1e-3) / 1e9,
            "hbm_gbps": bd / (walld / args.steps) / 1e9,
            "bytes_per_token": bd / m / w.B,
        }
        del kvd

    # ---- memory-system ceilings of the access pattern (probe kernels) -------
    if not args.no_extras and args.only in (None, "ceilings"):
        result["memory_ceilings"] = ceilings_leg(torch, dev)
        if "roofline" in result:
            # a compute-free stream of the cycle's traffic: m - 1 launches that
            # read the tile and write about 1 KiB, one that writes it back
            c = result["memory_ceilings"]
            t_cycle = ((m - 1) * c["read_write_1k"]["us"] + c["read_write_back"]["us"] + c["read_write_1k"]["us"]
                       - c["read"]["us"]) * 1e-6
            ceil = cycle_bytes_fused(m, w.dk, w.dv) * tiles / t_cycle / 1e9
            result["roofline"]["measured_ceiling_gbps"] = ceil
            result["roofline"]["frac_of_measured_ceiling"] = result["roofline"]["achieved"] / ceil

    # ---- counter calibration: a device copy of known size (only on request) -
    if args.only == "copy":
        result["copy_calibration"] = copy_leg(torch, dev)

    # ---- speculative verification: n drafts, then commit a ~ U{0..n} -------
    if not args.no_extras and args.only in (None, "verify"):
        result["verify"] = verify_leg(kb, synth, torch, dev, args)

    # ---- gated delta rule, half stateful / half buffer-only, m = 64 --------
    if not args.no_extras and args.only in (None, "delta"):
        result["delta_mixed"] = delta_leg(kb, synth, torch, dev, args)

    # ---- buffer-size sweep, linear rule at B=64, one GPU's head share ---------
    if not args.no_extras and args.only in (None, "sweep"):
        result["m_sweep"] = sweep_leg(kb, synth, torch, dev, args)
    if not args.no_extras and args.only in (None, "linear"):
        result["linear_B64"] = linear_leg(kb, synth, torch, dev, args)
    if not args.no_extras and args.only in (None, "heads4"):
        result["head_share_H4"] = head_share_leg(kb, synth, torch, dev, args)
    if not args.no_extras and args.only in (None, "context"):
        result["context_sweep"] = context_leg(kb, synth, torch, dev, args)
    if not args.no_extras and args.only in (None, "channel"):
        result["channel_gates"] = channel_leg(kb, synth, torch, dev, args)
    if not args.no_extras and args.only in (None, "longfold"):
        result["long_folds"] = long_fold_leg(kb, synth, torch, dev, args)
        if "memory_ceilings" in result:
            # the compute-free stream of a flush's traffic (tile read and
            # written back, the buffered rows read): its time over the flush's
            for key, probe in (("gated_m64", "fold_m64"), ("gated_m128", "fold_m128")):
                lf, c = result["long_folds"][key], result["memory_ceilings"][probe]
                lf["measured_ceiling_us"] = c["us"]
                lf["frac_of_measured_ceiling"] = c["us"] / (lf["flush_ms"] * 1e3)

    if args.only not in (None, "fused"):
        print(json.dumps(result))
        return

    cpu = None
    if not args.no_cpu:
        import oracle

        cpu = cpu_baseline(synth, oracle, np, torch, w, ring)

    line = {
        "metric": "decode tokens/s + achieved HBM GB/s (%% peak), B=256 H=32 d=128 m=%d" % m,
        "value": result["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "KVBuffer decode cycle: scalar-gated linear attention, B=256 H=32 d_k=d_v=128, "
                        "m=%d (blocks of %d, 2 per request, shuffled pool), bf16 q/k/v, fp32 state and "
                        "accumulation, fold fused into the filling decode; step = one buffer cycle "
                        "(%d decode launches)" % (m, m, m),
            "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "m": m, "io": "bf16",
        },
        "hbm_gbps": result["hbm_gbps"],
        "hbm_frac_of_peak": result["hbm_frac_of_peak"],
        "bytes_per_token": result["bytes_per_token"],
        "roofline": result["roofline"],
        "cpu_baseline": cpu,
    }
    for key in ("per_occupancy_ms", "m0_recurrent", "separate_flush", "memory_ceilings", "verify",
                "delta_mixed", "m_sweep", "linear_B64", "head_share_H4", "context_sweep", "channel_gates",
                "long_folds"):
        if key in result:
            line[key] = result[key]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
