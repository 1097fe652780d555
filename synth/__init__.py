"""Seeded synthetic inputs for the KVBuffer decode path.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds none of the method's arithmetic: it only draws numbers, rounds them to
the storage precision and describes the workloads' shapes.  Every array is
produced on the host with numpy's PCG64 from a seed tuple
(workload id, step, stream), so both sides of a comparison receive identical
bits.

Workloads (the pages evaluate end-to-end serving of trained models; these
synthetic tensors stand in for them with a head shape of H = 32, d = 128):

  1  tiny ungated, fp32 inputs, B=2 H=2 d=16 m=4, 32 steps, state starts at 0
  2  ungated, bf16 q/k/v, B=64 H=32 d=128 m=8, 256 steps, state ~ N(0, 0.02)
  3  scalar-gated sweep, B=256 H=32 d=128, m in {0,4,8,16,32}, 512 steps
  4  speculative verify, B=128 H=32 d=128 m=8, n in {1,2,4,8} drafts
  5  gated delta rule, B=512 (256 stateful + 256 buffer-only), m=64, 256 steps
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# Stream ids of the seed tuple.
Q, K, V, G, BETA, ACCEPT, LENGTHS, STATE, PERM, SLOTS, TREE = range(1, 12)


def rng(workload: int, step: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(workload), int(step), int(stream)])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as
    float32 holding bf16-representable values.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of bf16-representable float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    ident: int
    B: int
    H: int
    dk: int
    dv: int
    m: int
    block_size: int
    blocks_per_req: int
    steps: int
    rule: int  # 0 ungated, 1 scalar gate, 2 gated delta rule
    io: str  # "f32" or "bf16"
    state_std: float  # 0 -> state starts at zero
    n_drafts: int = 0
    n_short: int = 0  # requests served from the buffer alone (workload 5)

    @property
    def capacity(self) -> int:
        return self.block_size * self.blocks_per_req

    @property
    def tiles(self) -> int:
        return self.B * self.H


WORKLOADS = {
    1: Workload(1, B=2, H=2, dk=16, dv=16, m=4, block_size=4, blocks_per_req=2, steps=32,
                rule=0, io="f32", state_std=0.0),
    2: Workload(2, B=64, H=32, dk=128, dv=128, m=8, block_size=8, blocks_per_req=2, steps=256,
                rule=0, io="bf16", state_std=0.02),
    3: Workload(3, B=256, H=32, dk=128, dv=128, m=8, block_size=8, blocks_per_req=2, steps=512,
                rule=1, io="bf16", state_std=0.02),
    4: Workload(4, B=128, H=32, dk=128, dv=128, m=8, block_size=8, blocks_per_req=2, steps=64,
                rule=1, io="bf16", state_std=0.02, n_drafts=8),
    5: Workload(5, B=512, H=32, dk=128, dv=128, m=64, block_size=64, blocks_per_req=2, steps=256,
                rule=2, io="bf16", state_std=0.02, n_short=256),
}


def workload(ident: int, **overrides) -> Workload:
    """A workload by id, with any field overridden (smaller B, another m, ...).
    Changing m also sets the block size to m (two blocks per request)."""
    w = WORKLOADS[ident]
    if "m" in overrides and "block_size" not in overrides:
        overrides["block_size"] = max(int(overrides["m"]), 1)
    return replace(w, **overrides)


def _store(x: np.ndarray, io: str) -> np.ndarray:
    return bf16_round(x) if io == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def token_inputs(w: Workload, step: int, B: int | None = None, n: int | None = None, stream_base: int = 0):
    """Inputs of one decode step (n is None: shapes [B, H, d]) or of one verify
    call with n drafts (shapes [B, n, H, d]).  Returns float32 arrays
    q, k, v (storage-rounded), g and beta ([B, H] or [B, n, H]; None when the
    rule does not use them).  k is L2-normalised over d_k before rounding."""
    B = w.B if B is None else B
    lead = (B,) if n is None else (B, n)
    s = stream_base
    q = rng(w.ident, step, Q + s).standard_normal(lead + (w.H, w.dk), dtype=np.float32)
    k = rng(w.ident, step, K + s).standard_normal(lead + (w.H, w.dk), dtype=np.float32)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32))
    v = rng(w.ident, step, V + s).standard_normal(lead + (w.H, w.dv), dtype=np.float32)
    g = beta = None
    if w.rule >= 1:
        gshape = lead + (w.H, w.dk) if w.rule == 3 else lead + (w.H,)  # rule 3: one gate per key channel
        g = rng(w.ident, step, G + s).uniform(-0.1, 0.0, size=gshape).astype(np.float32)
    if w.rule == 2:
        beta = rng(w.ident, step, BETA + s).uniform(0.0, 1.0, size=lead + (w.H,)).astype(np.float32)
    return dict(q=_store(q, w.io), k=_store(k, w.io), v=_store(v, w.io), g=g, beta=beta)


def initial_state(w: Workload, nslots: int | None = None) -> np.ndarray:
    """fp32 state pool [nslots, H, dk, dv]: zeros, or N(0, std) (std = 0.02)."""
    nslots = w.B if nslots is None else nslots
    shape = (nslots, w.H, w.dk, w.dv)
    if w.state_std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    x = rng(w.ident, 0, STATE).standard_normal(shape, dtype=np.float32)
    x *= np.float32(w.state_std)
    return x


def block_permutation(w: Workload, num_blocks: int) -> np.ndarray:
    """A seeded shuffle of the block ids 0 .. num_blocks-1 (the free list)."""
    return rng(w.ident, 0, PERM).permutation(num_blocks).astype(np.int32)


def slot_permutation(w: Workload, nslots: int) -> np.ndarray:
    """A seeded shuffle of the state-slot ids 0 .. nslots-1."""
    return rng(w.ident, 0, SLOTS).permutation(nslots).astype(np.int32)


def accepted_lengths(w: Workload, call: int, B: int, n: int) -> np.ndarray:
    """Accepted-prefix lengths a ~ U{0..n}, one per request, for one verify call."""
    return rng(w.ident, call, ACCEPT).integers(0, n + 1, size=B).astype(np.int32)


def draft_tree(w: Workload, call: int, B: int, n: int):
    """A random tree of n drafts per request for one verify call and the leaf
    whose root-to-leaf path is accepted: parent[b][d] ~ U{-1 .. d-1} (-1 = the
    draft follows the buffer), leaf[b] ~ U{-1 .. n-1} (-1 = none kept).
    Returns (parent [B, n], leaf [B]) int32."""
    r = rng(w.ident, call, TREE)
    parent = np.floor(r.random((B, n)) * (np.arange(n) + 1)).astype(np.int32) - 1
    leaf = r.integers(-1, n, size=B).astype(np.int32)
    return parent, leaf


def short_lengths(w: Workload, draw: int, count: int) -> np.ndarray:
    """Lifetimes L ~ U{1..m} of buffer-only (short-context) requests."""
    return rng(w.ident, draw, LENGTHS).integers(1, w.m + 1, size=count).astype(np.int32)


# ---------------------------------------------------------------------------
# Device-side generation for the full-size workloads.  Same recipe (normal
# q, k, v; k L2-normalised in fp32 then rounded; uniform gates and step
# sizes), drawn with torch's seeded generator on the GPU so that hundreds of
# steps of a 256-request batch need no host round trip.  Consumers that need
# the values on the host (the oracle) copy them back from these tensors.
# ---------------------------------------------------------------------------

def _torch_gen(device, workload: int, step: int, stream: int):
    import torch

    seed = int(np.random.SeedSequence([int(workload), int(step), int(stream)]).generate_state(1)[0])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def device_token_inputs(w: Workload, step: int, device, B: int | None = None, n: int | None = None,
                        stream_base: int = 0):
    """As ``token_inputs`` but drawn on ``device``; q, k, v in the storage dtype
    (bf16 or fp32), g and beta fp32 (or None)."""
    import torch

    B = w.B if B is None else B
    lead = (B,) if n is None else (B, n)
    s = stream_base
    io = torch.bfloat16 if w.io == "bf16" else torch.float32
    f = dict(device=device, dtype=torch.float32)
    q = torch.randn(lead + (w.H, w.dk), generator=_torch_gen(device, w.ident, step, Q + s), **f)
    k = torch.randn(lead + (w.H, w.dk), generator=_torch_gen(device, w.ident, step, K + s), **f)
    k = k / torch.sqrt(torch.sum(k * k, dim=-1, keepdim=True))
    v = torch.randn(lead + (w.H, w.dv), generator=_torch_gen(device, w.ident, step, V + s), **f)
    g = beta = None
    if w.rule >= 1:
        gshape = lead + (w.H, w.dk) if w.rule == 3 else lead + (w.H,)  # rule 3: one gate per key channel
        g = -0.1 * torch.rand(gshape, generator=_torch_gen(device, w.ident, step, G + s), **f)
    if w.rule == 2:
        beta = torch.rand(lead + (w.H,), generator=_torch_gen(device, w.ident, step, BETA + s), **f)
    return dict(q=q.to(io), k=k.to(io), v=v.to(io), g=g, beta=beta)


def device_initial_state(w: Workload, nslots: int, device):
    """fp32 state pool [nslots, H, dk, dv] ~ N(0, state_std), drawn on ``device``."""
    import torch

    shape = (nslots, w.H, w.dk, w.dv)
    if w.state_std == 0.0:
        return torch.zeros(shape, dtype=torch.float32, device=device)
    x = torch.randn(shape, generator=_torch_gen(device, w.ident, 0, STATE), dtype=torch.float32, device=device)
    return x.mul_(w.state_std)
