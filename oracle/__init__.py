"""The oracle: a plain, slow, obviously correct CPU model of the KVBuffer decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and imports nothing from it; the GPU library never imports
this package.

Two parts:

* ``recurrent`` -- the per-token recurrent form of linear attention in fp64
  (``recurrence.c``): the state is updated at every token and the output is read
  from the updated state.  This is what the method must reproduce exactly up to
  rounding (KVBuffer: IO-aware Serving for Linear Attention, pith.science page,
  "What would settle it": identical token sequences through the recurrent and
  the buffered form must agree).  Every GPU output and state is compared with it.

* ``BufferModel`` -- integer bookkeeping of the key/value buffer: where each
  token's key, value and gate land in the block pool, how the per-request block
  table rotates when the buffered tokens are folded into the state, and the
  occupancy counter (same page, Figure 1 caption: buffer memory comes in
  fixed-size blocks, two per request in the figure, and a full buffer is
  folded into the state, which goes back to its slot; Figure 2 caption: drafts
  occupy buffer positions as well).

Where the pages leave a point open (they give no equation, no layout and no
API), the plainest reading that the rest of the pages support is taken, and the
function that depends on it says which.

Functions whose results have a pin (a test that checks them against closed
forms, exact rational arithmetic or invariants): ``recurrent`` for all four
rules, ``BufferModel`` (conservation, rotation, occupancy range).  Nothing here
is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recurrence.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

RULE_LINEAR = 0  # S_t = S_{t-1} + k v^T
RULE_GATED = 1  # S_t = exp(g) S_{t-1} + k v^T
RULE_DELTA = 2  # S_t = exp(g) (I - beta k k^T) S_{t-1} + beta k v^T
RULE_CHANNEL = 3  # S_t = diag(exp(g)) S_{t-1} + k v^T, g over the d_k key channels


def build(force: bool = True) -> str:
    """Compile recurrence.c into liboracle.so with gcc (fp64, OpenMP over tiles)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_recurrent.argtypes = [
            ctypes.c_int, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
        ]
        lib.oracle_recurrent.restype = ctypes.c_int
        lib.oracle_threads_used.argtypes = [ctypes.c_int]
        lib.oracle_threads_used.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(rule, S0, q, k, v, g=None, beta=None, scale=1.0, nthreads=1, inplace=False,
              with_magnitude=False):
    """Per-token recurrence over ``nsteps`` tokens for ``ntiles`` independent tiles.

    Arguments (any float dtype; widened exactly to fp64):
      S0   [ntiles, dk, dv]    state before the first token (not modified unless ``inplace``)
      q, k [nsteps, ntiles, dk]
      v    [nsteps, ntiles, dv]
      g    [nsteps, ntiles]    log-gate, gamma = exp(g) (rules 1 and 2);
           [nsteps, ntiles, dk] one log-gate per key channel (rule 3)
      beta [nsteps, ntiles]    delta-rule step size (rule 2)
    Returns (out [nsteps, ntiles, dv], S [ntiles, dk, dv]): every token's output
    o_t = S_t^T (scale q_t) and the state after the last token, both fp64.
    With ``inplace`` S0 must be a C-contiguous float64 array; it is advanced in
    place and returned as S (no copy of a large state).  ``nthreads`` spreads
    the independent tiles over OpenMP threads; each tile's arithmetic is the
    same at any thread count.
    With ``with_magnitude`` a third array [nsteps, ntiles, dv] is returned:
    |S_t|^T |scale q_t|, each output computed from the absolute values of its
    terms -- the size of the product that defines o_t, which bounds what
    rounding in any summation order can do to it (a near-cancelling output
    is small next to it).
    """
    if inplace:
        if not (isinstance(S0, np.ndarray) and S0.dtype == np.float64 and S0.flags.c_contiguous):
            raise ValueError("oracle: inplace needs a C-contiguous float64 state")
        S = S0
    else:
        S = _f64(S0).copy()
    if S.ndim != 3:
        raise ValueError("oracle: S0 must be [ntiles, dk, dv]")
    ntiles, dk, dv = S.shape
    q = _f64(q)
    nsteps = q.shape[0]
    q = _f64(q, (nsteps, ntiles, dk))
    k = _f64(k, (nsteps, ntiles, dk))
    v = _f64(v, (nsteps, ntiles, dv))
    if rule == 3:
        g = _f64(g, (nsteps, ntiles, dk))
    else:
        g = _f64(g, (nsteps, ntiles)) if rule >= 1 else None
    beta = _f64(beta, (nsteps, ntiles)) if rule == 2 else None
    out = np.zeros((nsteps, ntiles, dv), dtype=np.float64)
    mag = np.zeros((nsteps, ntiles, dv), dtype=np.float64) if with_magnitude else None
    rc = _load().oracle_recurrent(int(rule), ntiles, nsteps, dk, dv, float(scale), _ptr(S),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(out),
                                  _ptr(mag), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_recurrent rejected its arguments")
    if with_magnitude:
        return out, S, mag
    return out, S


def threads_used(n: int) -> int:
    """Threads an OpenMP region of the oracle gets when asked for ``n``."""
    return int(_load().oracle_threads_used(int(n)))


# ----------------------------------------------------------------------------
# Bookkeeping model (integers only).
# ----------------------------------------------------------------------------

@dataclass
class _Request:
    table: list  # block ids, logical order
    occupancy: int = 0
    has_state: bool = True


@dataclass
class BufferModel:
    """Integer model of the buffer bookkeeping for a batch of requests.

    Logical buffer position p of request b lives in block ``table[b][p // bs]``
    at offset ``p % bs``.  Tokens are appended at p = occupancy.  Folding the
    buffer into the state (a "flush"; Figure 1 caption: a full buffer is folded
    into the state) consumes the first m positions,
    moves the m / bs blocks that held them to the back of the table and lowers
    the occupancy by m; tokens already buffered beyond position m keep their
    physical place and become positions 0, 1, ...

    ``physical`` records which token last wrote each (block, offset); the GPU
    pool must hold exactly that token's bits there (rejected drafts and flushed
    tokens stay as dead data -- nothing is cleared).
    """

    m: int
    block_size: int
    blocks_per_req: int
    requests: list = field(default_factory=list)
    physical: dict = field(default_factory=dict)  # (block, offset) -> token id

    @property
    def capacity(self) -> int:
        return self.block_size * self.blocks_per_req

    def add_request(self, table, occupancy=0, has_state=True):
        if len(table) != self.blocks_per_req:
            raise ValueError("table length must equal blocks_per_req")
        self.requests.append(_Request(list(table), occupancy, has_state))
        return len(self.requests) - 1

    def replace_request(self, b, table, occupancy=0, has_state=True):
        self.requests[b] = _Request(list(table), occupancy, has_state)

    def position(self, b, p):
        r = self.requests[b]
        if not 0 <= p < self.capacity:
            raise IndexError("buffer position %d outside capacity %d" % (p, self.capacity))
        return r.table[p // self.block_size], p % self.block_size

    def _write(self, b, p, token):
        self.physical[self.position(b, p)] = token

    def flush(self, b) -> bool:
        """Fold the first m buffered tokens into the state if the buffer is full."""
        r = self.requests[b]
        if self.m <= 0 or not r.has_state or r.occupancy < self.m:
            return False
        nb = self.m // self.block_size
        r.table = r.table[nb:] + r.table[:nb]
        r.occupancy -= self.m
        return True

    def decode(self, b, token, eager=True, stateless=False) -> bool:
        """Append one token; with ``eager`` fold the buffer as soon as it is full.
        Returns whether a flush happened.  ``stateless`` requests never fold."""
        r = self.requests[b]
        self._write(b, r.occupancy, token)
        r.occupancy += 1
        if eager and not stateless:
            return self.flush(b)
        return False

    def verify(self, b, tokens):
        """Buffer draft tokens at positions occupancy, occupancy+1, ... without
        advancing the occupancy (Figure 2 caption: the drafts' keys and values
        are buffered, no temporary state is kept)."""
        r = self.requests[b]
        for i, t in enumerate(tokens):
            self._write(b, r.occupancy + i, t)

    def commit(self, b, accepted, eager=True) -> bool:
        """Keep the first ``accepted`` drafts: the occupancy advances over them."""
        r = self.requests[b]
        r.occupancy += int(accepted)
        if r.occupancy > self.capacity:
            raise IndexError("commit beyond buffer capacity")
        if eager:
            return self.flush(b)
        return False

    def commit_path(self, b, path, eager=True) -> bool:
        """Tree drafts: keep the drafts on one root-to-node path (indices into
        the verified drafts, in path order).  Draft path[k] moves from
        position occupancy + path[k] to occupancy + k, then the occupancy
        advances over the path (a chain tree with path [0 .. a-1] is
        ``commit(b, a)``).  The pages' reference list includes tree
        speculative decoding; the accepted path is what the request keeps."""
        r = self.requests[b]
        moved = [self.physical.get(self.position(b, r.occupancy + d)) for d in path]
        for k, tok in enumerate(moved):
            self._write(b, r.occupancy + k, tok)
        return self.commit(b, len(path), eager)

    def buffered_tokens(self, b):
        """Token ids at logical positions 0 .. occupancy-1 of request b."""
        r = self.requests[b]
        return [self.physical.get(self.position(b, p)) for p in range(r.occupancy)]

    def tables(self):
        return np.array([r.table for r in self.requests], dtype=np.int32)

    def occupancies(self):
        return np.array([r.occupancy for r in self.requests], dtype=np.int32)

    def check_invariants(self, num_blocks=None):
        """Every block belongs to at most one request; occupancy within range."""
        seen = {}
        for b, r in enumerate(self.requests):
            for blk in r.table:
                if blk in seen:
                    raise AssertionError("block %d owned by requests %d and %d" % (blk, seen[blk], b))
                if num_blocks is not None and not 0 <= blk < num_blocks:
                    raise AssertionError("block id %d outside the pool" % blk)
                seen[blk] = b
            if not 0 <= r.occupancy <= self.capacity:
                raise AssertionError("occupancy %d of request %d out of range" % (r.occupancy, b))
