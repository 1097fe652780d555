"""KVBuffer linear-attention decode on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libkvbuf.so`` (C ABI declared in ``include/kvbuf.h``).
The functions ``kvbuf_decode``, ``kvbuf_flush``, ``kvbuf_verify``,
``kvbuf_commit``, ``kvbuf_direct`` and ``kvbuf_materialize`` only marshal
arguments: every step of the decode path runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: without the built library every call raises.

``KVBuffer`` owns the pools and per-request metadata of one layer as torch
tensors and calls the entry points with them.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvbuf.so")

RULE_LINEAR, RULE_GATED, RULE_DELTA, RULE_CHANNEL = 0, 1, 2, 3
BF16, F32 = 0, 1
FLUSH_EAGER, FLUSH_DEFERRED = 0, 1
OUT_F32, OUT_BF16 = 0, 1

OK, EINVAL, EUNSUPPORTED, ECAPACITY, EHIP = 0, -1, -2, -3, -4
DEVERR_BLOCK, DEVERR_SLOT, DEVERR_OVERFLOW, DEVERR_ACCEPT, DEVERR_META = 1, 2, 4, 8, 16

EXPORTED = ("kvbuf_decode", "kvbuf_flush", "kvbuf_verify", "kvbuf_commit", "kvbuf_direct",
            "kvbuf_verify_tree", "kvbuf_commit_tree", "kvbuf_verify_recurrent", "kvbuf_commit_recurrent",
            "kvbuf_materialize", "kvbuf_admit", "kvbuf_check", "kvbuf_strerror", "kvbuf_abi_version")


class Layout(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("m", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("blocks_per_req", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_state_slots", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flush", ctypes.c_int32), ("scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32)]


class Pools(ctypes.Structure):
    _fields_ = [("state", ctypes.c_void_p), ("key", ctypes.c_void_p), ("value", ctypes.c_void_p),
                ("gate", ctypes.c_void_p)]


class Batch(ctypes.Structure):
    _fields_ = [("size", ctypes.c_int32), ("state_slot", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("occupancy", ctypes.c_void_p),
                ("error", ctypes.c_void_p), ("tile_meta", ctypes.c_void_p)]


class KVBufError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, strerror(status), status))


_lib = None


def load():
    """The loaded library.  Raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libkvbuf.so is not built (expected at %s); run "
                "`python -m linear_attention_decode_kvbuf_amd._build` or __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L, PO, B = ctypes.POINTER(Layout), ctypes.POINTER(Pools), ctypes.POINTER(Batch)
        i32 = ctypes.c_int32
        lib.kvbuf_decode.argtypes = [L, PO, B, P, P, P, P, P, P, P]
        lib.kvbuf_direct.argtypes = [L, PO, B, P, P, P, P, P, P, P]
        lib.kvbuf_verify.argtypes = [L, PO, B, i32, P, P, P, P, P, P, P]
        lib.kvbuf_flush.argtypes = [L, PO, B, P]
        lib.kvbuf_commit.argtypes = [L, PO, B, i32, P, P]
        lib.kvbuf_materialize.argtypes = [L, PO, B, P, P]
        lib.kvbuf_verify_tree.argtypes = [L, PO, B, i32, P, P, P, P, P, P, P, P]
        lib.kvbuf_commit_tree.argtypes = [L, PO, B, i32, P, P, P]
        lib.kvbuf_verify_recurrent.argtypes = [L, PO, B, i32, P, P, P, P, P, P, P, P]
        lib.kvbuf_commit_recurrent.argtypes = [L, PO, B, i32, P, P, P]
        lib.kvbuf_admit.argtypes = [L, B, P, i32, P]
        lib.kvbuf_check.argtypes = [L, B, P]
        for name in ("kvbuf_decode", "kvbuf_direct", "kvbuf_verify", "kvbuf_flush",
                     "kvbuf_commit", "kvbuf_materialize", "kvbuf_verify_tree", "kvbuf_commit_tree",
                     "kvbuf_verify_recurrent", "kvbuf_commit_recurrent", "kvbuf_admit", "kvbuf_check"):
            getattr(lib, name).restype = ctypes.c_int
        lib.kvbuf_strerror.argtypes = [ctypes.c_int]
        lib.kvbuf_strerror.restype = ctypes.c_char_p
        lib.kvbuf_abi_version.argtypes = []
        lib.kvbuf_abi_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return load().kvbuf_strerror(int(status)).decode()


def _ptr(x):
    """Device (or host) address of a tensor, an int address, or NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, what, raise_on_error):
    if raise_on_error and status != OK:
        raise KVBufError(status, what)
    return status


def _ref(s):
    return None if s is None else ctypes.byref(s)


def kvbuf_decode(layout, pools, batch, q, k, v, g, beta, out, stream=None, raise_on_error=True):
    st = load().kvbuf_decode(_ref(layout), _ref(pools), _ref(batch), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta), _ptr(out), _stream(stream))
    return _check(st, "kvbuf_decode", raise_on_error)


def kvbuf_direct(layout, pools, batch, q, k, v, g, beta, out, stream=None, raise_on_error=True):
    st = load().kvbuf_direct(_ref(layout), _ref(pools), _ref(batch), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta), _ptr(out), _stream(stream))
    return _check(st, "kvbuf_direct", raise_on_error)


def kvbuf_verify(layout, pools, batch, n, q, k, v, g, beta, out, stream=None, raise_on_error=True):
    st = load().kvbuf_verify(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(g), _ptr(beta), _ptr(out), _stream(stream))
    return _check(st, "kvbuf_verify", raise_on_error)


def kvbuf_flush(layout, pools, batch, stream=None, raise_on_error=True):
    st = load().kvbuf_flush(_ref(layout), _ref(pools), _ref(batch), _stream(stream))
    return _check(st, "kvbuf_flush", raise_on_error)


def kvbuf_commit(layout, pools, batch, n, accepted, stream=None, raise_on_error=True):
    st = load().kvbuf_commit(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(accepted),
                             _stream(stream))
    return _check(st, "kvbuf_commit", raise_on_error)


def kvbuf_materialize(layout, pools, batch, states, stream=None, raise_on_error=True):
    st = load().kvbuf_materialize(_ref(layout), _ref(pools), _ref(batch), _ptr(states),
                                  _stream(stream))
    return _check(st, "kvbuf_materialize", raise_on_error)


def kvbuf_verify_tree(layout, pools, batch, n, parent, q, k, v, g, beta, out, stream=None, raise_on_error=True):
    st = load().kvbuf_verify_tree(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(parent), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(out), _stream(stream))
    return _check(st, "kvbuf_verify_tree", raise_on_error)


def kvbuf_commit_tree(layout, pools, batch, n, parent, leaf, stream=None, raise_on_error=True):
    st = load().kvbuf_commit_tree(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(parent), _ptr(leaf),
                                  _stream(stream))
    return _check(st, "kvbuf_commit_tree", raise_on_error)


def kvbuf_verify_recurrent(layout, pools, batch, n, q, k, v, g, beta, out, temp, stream=None,
                           raise_on_error=True):
    st = load().kvbuf_verify_recurrent(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(g), _ptr(beta), _ptr(out), _ptr(temp),
                                       _stream(stream))
    return _check(st, "kvbuf_verify_recurrent", raise_on_error)


def kvbuf_commit_recurrent(layout, pools, batch, n, accepted, temp, stream=None, raise_on_error=True):
    st = load().kvbuf_commit_recurrent(_ref(layout), _ref(pools), _ref(batch), int(n), _ptr(accepted),
                                       _ptr(temp), _stream(stream))
    return _check(st, "kvbuf_commit_recurrent", raise_on_error)


def kvbuf_admit(layout, batch, requests, count, stream=None, raise_on_error=True):
    st = load().kvbuf_admit(_ref(layout), _ref(batch), _ptr(requests), int(count), _stream(stream))
    return _check(st, "kvbuf_admit", raise_on_error)


def kvbuf_check(layout, batch, stream=None, raise_on_error=True):
    st = load().kvbuf_check(_ref(layout), _ref(batch), _stream(stream))
    return _check(st, "kvbuf_check", raise_on_error)


def kvbuf_abi_version() -> int:
    return int(load().kvbuf_abi_version())


class KVBuffer:
    """Pools and per-request metadata of one linear-attention layer, as torch
    tensors on ``device``, with the library's entry points bound to them.

    state      [num_state_slots, H, d_k, d_v] fp32
    key        [num_blocks, H, block_size, d_k] io dtype
    value      [num_blocks, H, block_size, d_v] io dtype (fp32 for the delta rule)
    gate       [num_blocks, H, block_size] fp32 (None for the linear rule;
               [num_blocks, H, block_size, d_k] for the per-channel rule)
    state_slot [B] int32
    block_table [B, blocks_per_req] int32, occupancy [B] int32: each request's
               row and occupancy, kept current by the library; after writing a
               request's row / occupancy, call ``admit`` for it
    tile_meta  [B, H, 1 + blocks_per_req] int32: the library's per-head copies
    error      [1] int32
    """

    def __init__(self, *, batch, heads, d, m, block_size=None, blocks_per_req=2, num_blocks=None,
                 num_state_slots=None, rule=RULE_GATED, io_dtype=BF16, flush=FLUSH_EAGER,
                 scale=1.0, out_dtype=OUT_F32, device="cuda"):
        import torch

        load()
        self.torch = torch
        block_size = block_size if block_size is not None else max(m, 1)
        num_blocks = num_blocks if num_blocks is not None else batch * blocks_per_req
        num_state_slots = num_state_slots if num_state_slots is not None else batch
        self.layout = Layout(heads, d, d, m, block_size, blocks_per_req, num_blocks,
                             num_state_slots, rule, io_dtype, flush, float(scale), out_dtype)
        self.B, self.H, self.d, self.m = batch, heads, d, m
        self.rule, self.io_dtype = rule, io_dtype
        io = torch.bfloat16 if io_dtype == BF16 else torch.float32
        self.io_torch = io
        self.out_torch = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
        dev = torch.device(device)
        self.state = torch.zeros((max(num_state_slots, 1), heads, d, d), dtype=torch.float32, device=dev)
        if m > 0:
            self.key = torch.zeros((num_blocks, heads, block_size, d), dtype=io, device=dev)
            vdt = torch.float32 if rule == RULE_DELTA else io
            self.value = torch.zeros((num_blocks, heads, block_size, d), dtype=vdt, device=dev)
            gshape = (num_blocks, heads, block_size, d) if rule == RULE_CHANNEL else (num_blocks, heads, block_size)
            self.gate = torch.zeros(gshape, dtype=torch.float32, device=dev) if rule != RULE_LINEAR else None
        else:
            self.key = self.value = self.gate = None
        i32 = torch.int32
        self.state_slot = torch.arange(batch, dtype=i32, device=dev) % max(num_state_slots, 1)
        self.block_table = torch.empty((batch, blocks_per_req), dtype=i32, device=dev)
        self.occupancy = torch.zeros(batch, dtype=i32, device=dev)
        self.tile_meta = torch.zeros((batch, heads, 1 + blocks_per_req), dtype=i32, device=dev)
        self.error = torch.zeros(1, dtype=i32, device=dev)
        self._refresh()
        self.set_block_table(torch.arange(batch * blocks_per_req, dtype=i32).reshape(
            batch, blocks_per_req) % max(num_blocks, 1))

    def _refresh(self):
        self.pools = Pools(_ptr(self.state), _ptr(self.key), _ptr(self.value), _ptr(self.gate))
        self.batch = Batch(self.B, _ptr(self.state_slot), _ptr(self.block_table), _ptr(self.occupancy),
                           _ptr(self.error), _ptr(self.tile_meta))

    def view(self, start, count):
        """Requests start .. start+count-1 as a batch of their own: the same
        pools, the metadata rows of those requests (views, so calls on the
        view advance this object's metadata).  Two views over disjoint
        request ranges may be called one after the other on a stream, e.g.
        kvbuf_decode for requests with a state and kvbuf_direct for those
        served from their buffer alone."""
        import copy

        if not (0 <= start and count >= 0 and start + count <= self.B):
            raise ValueError("request range %d + %d outside the batch of %d" % (start, count, self.B))
        v = copy.copy(self)
        v.B = count
        v.state_slot = self.state_slot[start:start + count]
        v.block_table = self.block_table[start:start + count]
        v.occupancy = self.occupancy[start:start + count]
        v.tile_meta = self.tile_meta[start:start + count]
        v._refresh()
        return v

    def set_block_table(self, table, occupancy=None):
        """Every request's table row <- table [B, blocks_per_req] (and its
        occupancy, when given), then kvbuf_admit for all of them."""
        t = self.torch.as_tensor(table, dtype=self.torch.int32).to(self.block_table.device)
        self.block_table.copy_(t.reshape(self.B, -1))
        if occupancy is not None:
            self.occupancy.copy_(self.torch.as_tensor(occupancy, dtype=self.torch.int32).to(self.occupancy.device))
        if self.m > 0:
            self.admit()

    def admit(self, requests=None, stream=None):
        """kvbuf_admit: the per-head copies of the listed requests (a [k]
        int32 device tensor of indices; None = every request) <- their
        block_table rows and occupancies."""
        if requests is None:
            kvbuf_admit(self.layout, self.batch, None, 0, stream)
        else:
            self._need(requests, "requests", (requests.numel(),), self.torch.int32)
            kvbuf_admit(self.layout, self.batch, requests, requests.numel(), stream)

    def check_meta(self, stream=None):
        """kvbuf_check: sets DEVERR_META in ``error`` if any request's per-head
        copies disagree with its row or occupancy."""
        kvbuf_check(self.layout, self.batch, stream)

    @property
    def capacity(self):
        return self.layout.block_size * self.layout.blocks_per_req

    # ---- argument checks: the library reads raw pointers, so a tensor of the
    # wrong dtype, shape, layout or device would be reinterpreted or read out
    # of bounds; these raise ValueError before anything is enqueued.
    def _need(self, x, name, shape, dtype):
        if not isinstance(x, self.torch.Tensor):
            raise ValueError("%s must be a tensor" % name)
        if x.device != self.state.device:
            raise ValueError("%s is on %s; the pools are on %s" % (name, x.device, self.state.device))
        if x.dtype != dtype:
            raise ValueError("%s has dtype %s, expected %s" % (name, x.dtype, dtype))
        if tuple(x.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
        if not x.is_contiguous():
            raise ValueError("%s must be contiguous" % name)

    def _tokens(self, lead, q, k, v, g, beta, out):
        """Checks q, k, v [*lead, H, d] (io dtype), g / beta [*lead, H] fp32
        (g [*lead, H, d] for the per-channel rule) and out [*lead, H, d] (the
        layout's output dtype); allocates out when it is None."""
        H, d, f32 = self.H, self.d, self.torch.float32
        for name, x in (("q", q), ("k", k), ("v", v)):
            self._need(x, name, lead + (H, d), self.io_torch)
        if self.rule == RULE_LINEAR:
            g = None  # unused by the rule
        else:
            gshape = lead + (H, d) if self.rule == RULE_CHANNEL else lead + (H,)
            self._need(g, "g", gshape, f32)
        if self.rule == RULE_DELTA:
            self._need(beta, "beta", lead + (H,), f32)
        else:
            beta = None
        if out is None:
            out = self.torch.empty(lead + (H, d), dtype=self.out_torch, device=self.state.device)
        self._need(out, "out", lead + (H, d), self.out_torch)
        return g, beta, out

    def _drafts(self, q):
        if not isinstance(q, self.torch.Tensor) or q.dim() != 4:
            raise ValueError("drafts are [B, n, H, d] tensors")
        return int(q.shape[1])

    def _ints(self, x, name, shape):
        self._need(x, name, shape, self.torch.int32)

    def decode(self, q, k, v, g=None, beta=None, out=None, stream=None):
        g, beta, out = self._tokens((self.B,), q, k, v, g, beta, out)
        kvbuf_decode(self.layout, self.pools, self.batch, q, k, v, g, beta, out, stream)
        return out

    def direct(self, q, k, v, g=None, beta=None, out=None, stream=None):
        g, beta, out = self._tokens((self.B,), q, k, v, g, beta, out)
        kvbuf_direct(self.layout, self.pools, self.batch, q, k, v, g, beta, out, stream)
        return out

    def verify(self, q, k, v, g=None, beta=None, out=None, stream=None):
        n = self._drafts(q)
        g, beta, out = self._tokens((self.B, n), q, k, v, g, beta, out)
        kvbuf_verify(self.layout, self.pools, self.batch, n, q, k, v, g, beta, out, stream)
        return out

    def commit(self, n, accepted, stream=None):
        self._ints(accepted, "accepted", (self.B,))
        kvbuf_commit(self.layout, self.pools, self.batch, n, accepted, stream)

    def verify_tree(self, parent, q, k, v, g=None, beta=None, out=None, stream=None):
        """Tree drafts: parent [B, n] int32 on the device (-1 = follows the buffer)."""
        n = self._drafts(q)
        self._ints(parent, "parent", (self.B, n))
        g, beta, out = self._tokens((self.B, n), q, k, v, g, beta, out)
        kvbuf_verify_tree(self.layout, self.pools, self.batch, n, parent, q, k, v, g, beta, out, stream)
        return out

    def commit_tree(self, parent, leaf, stream=None):
        """Keep the path from the root to leaf [B] int32 (-1 = none) of the last tree verify."""
        if not isinstance(parent, self.torch.Tensor) or parent.dim() != 2:
            raise ValueError("parent is a [B, n] tensor")
        self._ints(parent, "parent", (self.B, parent.shape[1]))
        self._ints(leaf, "leaf", (self.B,))
        kvbuf_commit_tree(self.layout, self.pools, self.batch, parent.shape[1], parent, leaf, stream)

    def verify_recurrent(self, q, k, v, g=None, beta=None, out=None, temp=None, stream=None):
        """Temporary-state verification (m = 0 only): returns (out, temp)."""
        n = self._drafts(q)
        g, beta, out = self._tokens((self.B, n), q, k, v, g, beta, out)
        if temp is None:
            temp = self.torch.empty((n, self.B, self.H, self.d, self.d), dtype=self.torch.float32,
                                    device=self.state.device)
        self._need(temp, "temp", (n, self.B, self.H, self.d, self.d), self.torch.float32)
        kvbuf_verify_recurrent(self.layout, self.pools, self.batch, n, q, k, v, g, beta, out, temp, stream)
        return out, temp

    def commit_recurrent(self, n, accepted, temp, stream=None):
        self._ints(accepted, "accepted", (self.B,))
        self._need(temp, "temp", (n, self.B, self.H, self.d, self.d), self.torch.float32)
        kvbuf_commit_recurrent(self.layout, self.pools, self.batch, n, accepted, temp, stream)

    def flush(self, stream=None):
        kvbuf_flush(self.layout, self.pools, self.batch, stream)

    def materialize(self, out=None, stream=None):
        if out is None:
            out = self.torch.empty((self.B, self.H, self.d, self.d), dtype=self.torch.float32,
                                   device=self.state.device)
        self._need(out, "out", (self.B, self.H, self.d, self.d), self.torch.float32)
        kvbuf_materialize(self.layout, self.pools, self.batch, out, stream)
        return out
