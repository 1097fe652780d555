"""Drives a workload through the HIP library (through its C ABI) and through
the oracle side by side, and compares them.

Tolerances (the method must reproduce the recurrence exactly up to rounding;
the GPU accumulates in fp32 from bf16 or fp32 inputs):
  outputs  per tile  max|o_gpu - o_ref| / max(|S_t|^T |q_t|)  <= 2e-3
  states   per tile  max|S_gpu - S_ref| / max|S_ref|          <= 1e-5 after every fold
  block tables, occupancies and buffered key / value / gate bits: exact.
An output's error is measured against the size of the product that defines
it, |S_t|^T |scale q_t| (the oracle computes it beside the output): a sum
accumulated in fp32 carries rounding of the order of its terms' magnitudes,
so an output that nearly cancels (a single buffered token whose q . k is 1e-7
while its products are of order 1, as happens among thousands of tiles) has
no relative accuracy in any summation order.  ``out_scale="output"`` measures
against max|o_ref| instead (for inputs built so that no output cancels).

By default every (request, head) tile is compared, at every size: outputs at
every step, effective states where a test asks for them, and the stored state
of every tile that folds -- all of them at the first fold of a run and at
``check_all_states``, a rotating subset of ``state_sample`` tiles at the folds
in between (a full-size state pool is half a GiB to copy per check).  The
oracle's state of every compared tile is kept in fp64 and advanced in place,
its tiles spread over the host's cores.
"""

from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import synth
import linear_attention_decode_kvbuf_amd as kb

TOL_OUT = 2e-3
TOL_STATE = 1e-5
NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def rel_err_tiles(gpu, ref, axes, chunk=1024, den=None, slack=0.0):
    """max over tiles of max|gpu - ref| / max|den| (den = ref unless given;
    reduction over ``axes``), in chunks of the leading axis so that full-size
    states are never widened whole.  With ``slack`` each element's error is
    counted beyond slack |ref| (the rounding of a narrower output type)."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    if gpu.shape != ref.shape:
        raise ValueError("compared shapes differ: %s vs %s" % (gpu.shape, ref.shape))
    if gpu.size == 0:
        return 0.0
    if gpu.ndim == 0:
        gpu, ref = gpu[None], ref[None]
    worst = 0.0
    for i in range(0, gpu.shape[0], chunk):
        g = np.asarray(gpu[i:i + chunk], np.float64)
        r = np.asarray(ref[i:i + chunk], np.float64)
        d = r if den is None else np.asarray(den[i:i + chunk], np.float64)
        num = np.max(np.maximum(np.abs(g - r) - slack * np.abs(r), 0.0), axis=axes)
        worst = max(worst, float(np.max(num / np.maximum(np.max(np.abs(d), axis=axes), 1e-30))))
    return worst


def all_tiles(w):
    """Every (b, h) tile, request-major."""
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def _np(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy()
    return np.asarray(x, np.float32)


def recurrence(rule, S, q, k, v, g, beta):
    """The oracle over [steps, tiles, ...] inputs, advancing S (fp64) in place.
    Returns the outputs and their magnitudes |S_t|^T |q_t|."""
    out, _, mag = oracle.recurrent(rule, S, q, k, v, g, beta, nthreads=NTHREADS, inplace=True,
                                   with_magnitude=True)
    return out, mag


# bf16 outputs: rounding to nearest moves an element by at most half an ulp,
# 2^-8 of its size (8 significant bits)
BF16_HALF_ULP = 2.0 ** -8


def out_err_tiles(gpu, ref, mag, out_scale="magnitude", slack=0.0):
    """max over tiles of max|gpu - ref| / max(scale): the output magnitude, or
    max|ref| with out_scale="output"; errors counted beyond slack |ref|."""
    return rel_err_tiles(gpu, ref, axes=-1, den=(mag if out_scale == "magnitude" else None), slack=slack)


class Run:
    def __init__(self, w, *, flush=kb.FLUSH_EAGER, sample=None, device_gen=None, spare_blocks=3,
                 stateless=None, check_every_step=None, state_sample=64, tol_out=TOL_OUT, tol_state=TOL_STATE,
                 out_scale="magnitude", out_dtype=kb.OUT_F32):
        self.w = w
        self.out_scale = out_scale
        self.tol_out = tol_out
        self.tol_state = tol_state
        self.dev = torch.device("cuda")
        self.flush_policy = flush
        self.device_gen = device_gen if device_gen is not None else w.B * w.H > 256
        self.check_every_step = check_every_step if check_every_step is not None else w.B * w.H <= 64
        B, H, d = w.B, w.H, w.dk
        bpr = w.blocks_per_req
        nb = B * bpr + spare_blocks if w.m > 0 else 1
        nslots = B + 1
        self.kv = kb.KVBuffer(batch=B, heads=H, d=d, m=w.m, block_size=w.block_size if w.m > 0 else 1,
                              blocks_per_req=bpr, num_blocks=nb, num_state_slots=nslots, rule=w.rule,
                              io_dtype=kb.BF16 if w.io == "bf16" else kb.F32, flush=flush,
                              out_dtype=out_dtype)
        # bf16 outputs are compared beyond their own rounding
        self.out_slack = BF16_HALF_ULP if out_dtype == kb.OUT_BF16 else 0.0
        if w.m > 0:
            perm = synth.block_permutation(w, nb)
            self.free = list(perm[B * bpr:])
            table = perm[: B * bpr].reshape(B, bpr)
        else:  # recurrent mode: no buffer
            self.free = []
            table = np.zeros((B, bpr), np.int32)
        slots = synth.slot_permutation(w, nslots)[:B].copy()
        self.stateless = np.zeros(B, bool) if stateless is None else np.asarray(stateless, bool)
        slots[self.stateless] = -1
        self.slots = slots
        self.kv.set_block_table(table)
        self.kv.state_slot.copy_(torch.from_numpy(slots))
        if self.device_gen:
            self.kv.state.copy_(synth.device_initial_state(w, nslots, self.dev))
        else:
            self.kv.state.copy_(torch.from_numpy(synth.initial_state(w, nslots)))
        torch.cuda.synchronize()

        self.model = oracle.BufferModel(w.m, w.block_size, bpr)
        for b in range(B):
            self.model.add_request(table[b], 0, has_state=not self.stateless[b])

        self.sample = list(sample) if sample is not None else all_tiles(w)
        self.all = self.sample == all_tiles(w)
        self.sb_np = np.array([b for b, _ in self.sample], np.int64)
        self.sh_np = np.array([h for _, h in self.sample], np.int64)
        self.sb = torch.from_numpy(self.sb_np).to(self.dev)
        self.sh = torch.from_numpy(self.sh_np).to(self.dev)
        # per request: the indices j of its sampled tiles (a slice when every tile is compared)
        self.rows_of = {}
        if self.all:
            for b in range(B):
                self.rows_of[b] = slice(b * H, (b + 1) * H)
        else:
            for j, b in enumerate(self.sb_np):
                self.rows_of.setdefault(int(b), []).append(j)
            self.rows_of = {b: np.array(js, np.int64) for b, js in self.rows_of.items()}
        self.S = np.ascontiguousarray(self._stored_states(np.arange(len(self.sample))).astype(np.float64))
        self.tokens = {}  # token id -> (k, v, g) rows of its request's sampled tiles, for the pool check
        self.calls = 0
        self.max_out = 0.0
        self.max_state = 0.0
        self.folds_checked = 0
        self.full_state_checks = 0
        self.state_sample = state_sample
        self._rotor = 0

    # ---------------------------------------------------------------- inputs
    def inputs(self, step, n=None, stream_base=0):
        if self.device_gen:
            return synth.device_token_inputs(self.w, step, self.dev, n=n, stream_base=stream_base)
        inp = synth.token_inputs(self.w, step, n=n, stream_base=stream_base)
        io = torch.bfloat16 if self.w.io == "bf16" else torch.float32
        out = {}
        for key, x in inp.items():
            if x is None:
                out[key] = None
            elif key in ("q", "k", "v"):
                out[key] = torch.from_numpy(x).to(self.dev).to(io)
            else:
                out[key] = torch.from_numpy(x).to(self.dev)
        return out

    def _sampled(self, x, drafts=False):
        """[ns, (n,) ...] float32 host copy of the sampled tiles of a [B, (n,) H, ...] tensor."""
        if x is None:
            return None
        if self.all:
            B, H = self.w.B, self.w.H
            if drafts:
                x = x.transpose(1, 2)  # [B, H, n, ...]
                return _np(x.reshape((B * H,) + tuple(x.shape[2:])))
            return _np(x.reshape((B * H,) + tuple(x.shape[2:])))
        if drafts:
            return _np(x[self.sb, :, self.sh])
        return _np(x[self.sb, self.sh])

    def _stored_states(self, js):
        """fp32 host copy of the stored state of sampled tiles js (zeros without a slot)."""
        js = np.asarray(js, np.int64)
        b = self.sb_np[js]
        slot = self.slots[b]
        st = self.kv.state.detach()
        got = st[torch.from_numpy(np.maximum(slot, 0)).to(self.dev), torch.from_numpy(self.sh_np[js]).to(self.dev)]
        got = got.cpu().numpy()
        got[slot < 0] = 0.0
        return got

    # ---------------------------------------------------------------- steps
    def decode(self, t, direct=False, direct_from=None):
        """One decode step of every request: kvbuf_decode, or kvbuf_direct
        with ``direct``; with ``direct_from`` = s, kvbuf_decode on a view of
        requests 0 .. s-1 and kvbuf_direct on a view of s .. B-1."""
        w = self.w
        inp = self.inputs(t)
        if direct_from is not None:
            s = direct_from
            part = lambda x, a, z: None if x is None else x[a:z]
            out = torch.empty((w.B, w.H, w.dv), dtype=self.kv.out_torch, device=self.dev)
            for view, fn, a, z in ((self.kv.view(0, s), "decode", 0, s), (self.kv.view(s, w.B - s), "direct", s, w.B)):
                if z > a:
                    getattr(view, fn)(*(part(inp[x], a, z) for x in ("q", "k", "v", "g", "beta")), out=out[a:z])
        elif direct:
            out = self.kv.direct(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        else:
            out = self.kv.decode(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        folded = set()
        if w.m > 0:
            eager = self.flush_policy == kb.FLUSH_EAGER
            for b in range(w.B):
                served_direct = direct or (direct_from is not None and b >= direct_from)
                if self.model.decode(b, ("d", t, b), eager=eager, stateless=served_direct or self.stateless[b]):
                    folded.add(b)
        q, k, v, g, beta = (self._sampled(inp[x]) for x in ("q", "k", "v", "g", "beta"))
        self._remember(lambda b: ("d", t, b), k, v, g)
        o_ref, mag = recurrence(w.rule, self.S, q[None], k[None], v[None],
                                None if g is None else g[None], None if beta is None else beta[None])
        o_gpu = self._sampled(out)
        err = out_err_tiles(o_gpu, o_ref[0], mag[0], self.out_scale, self.out_slack)
        self.max_out = max(self.max_out, err)
        assert err <= self.tol_out, "step %d: output error %.3e" % (t, err)
        self._after(folded)
        return out

    def flush(self, upto=None):
        """kvbuf_flush over the batch, or over a view of requests 0 .. upto-1."""
        (self.kv if upto is None else self.kv.view(0, upto)).flush()
        folded = {b for b in range(self.w.B if upto is None else upto) if self.model.flush(b)}
        self._after(folded)

    def verify_commit(self, call, n, accepted):
        """One verify of n drafts per request, then commit ``accepted`` [B].
        Draft d's reference output is the recurrence over drafts 0 .. d from the
        current state; the state after commit is the recurrence over the
        accepted prefix."""
        w = self.w
        inp = self.inputs(call, n=n, stream_base=100)
        out = self.kv.verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        for b in range(w.B):
            self.model.verify(b, [("v", call, b, d) for d in range(n)])
        q, k, v, g, beta = (self._sampled(inp[x], drafts=True) for x in ("q", "k", "v", "g", "beta"))
        o_gpu = self._sampled(out, drafts=True)  # [ns, n, d]
        for dd in range(n):
            self._remember(lambda b: ("v", call, b, dd), k[:, dd], v[:, dd], None if g is None else g[:, dd])
        acc_tile = np.asarray(accepted, np.int64)[self.sb_np]
        S_tmp = self.S.copy()
        for dd in range(n):
            col = lambda x: None if x is None else x[:, dd][None]
            o_ref, mag = recurrence(w.rule, S_tmp, col(q), col(k), col(v), col(g), col(beta))
            err = out_err_tiles(o_gpu[:, dd], o_ref[0], mag[0], self.out_scale, self.out_slack)
            self.max_out = max(self.max_out, err)
            assert err <= self.tol_out, "verify %d draft %d: output error %.3e" % (call, dd, err)
            keep = acc_tile == dd + 1
            self.S[keep] = S_tmp[keep]
        del S_tmp
        acc = torch.from_numpy(np.asarray(accepted, np.int32)).to(self.dev)
        self.kv.commit(n, acc)
        eager = self.flush_policy == kb.FLUSH_EAGER
        folded = {b for b in range(w.B) if self.model.commit(b, int(accepted[b]), eager=eager)}
        self._after(folded)
        return out

    def _along_paths(self, paths, q, k, v, g, beta, S):
        """The recurrence along each sampled tile's path of drafts (paths[b]:
        draft indices of request b, root first), advancing S in place.  Shorter
        paths are padded at the front with identity steps (zero key, value,
        gate and step size leave every rule's state unchanged exactly).
        Returns the output of each tile's last path step and its magnitude,
        or None."""
        L = max((len(p) for p in paths.values()), default=0)
        if L == 0:
            return None
        ns = len(self.sample)
        idx = np.full((L, ns), -1, np.int64)
        for b, p in paths.items():
            if p and b in self.rows_of:
                idx[L - len(p):, self.rows_of[b]] = np.asarray(p, np.int64)[:, None]
        live = idx >= 0
        col = np.arange(ns)[None, :]

        def gather(x):
            if x is None:
                return None
            y = x[col, np.maximum(idx, 0)]  # [L, ns, ...]
            y[~live] = 0.0
            return y

        o, mag = recurrence(self.w.rule, S, gather(q), gather(k), gather(v), gather(g), gather(beta))
        return o[-1], mag[-1]

    def verify_tree_commit(self, call, parent, leaf):
        """One tree verify (parent [B, n]) per request, then keep the path from
        the root to leaf[b].  Each draft's reference output is the recurrence
        run over its root-to-node path."""
        w = self.w
        n = parent.shape[1]
        inp = self.inputs(call, n=n, stream_base=200)
        par = torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(self.dev)
        out = self.kv.verify_tree(par, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        for b in range(w.B):
            self.model.verify(b, [("t", call, b, d) for d in range(n)])
        q, k, v, g, beta = (self._sampled(inp[x], drafts=True) for x in ("q", "k", "v", "g", "beta"))
        o_gpu = self._sampled(out, drafts=True)  # [ns, n, d]
        for dd in range(n):
            self._remember(lambda b: ("t", call, b, dd), k[:, dd], v[:, dd], None if g is None else g[:, dd])

        def path_to(b, d):
            path = []
            while d >= 0:
                path.append(d)
                d = int(parent[b][d])
            return path[::-1]

        for dd in range(n):
            o_ref, mag = self._along_paths({b: path_to(b, dd) for b in range(w.B)}, q, k, v, g, beta,
                                           self.S.copy())
            err = out_err_tiles(o_gpu[:, dd], o_ref, mag, self.out_scale, self.out_slack)
            self.max_out = max(self.max_out, err)
            assert err <= self.tol_out, "tree verify %d draft %d: output error %.3e" % (call, dd, err)
        self._along_paths({b: path_to(b, int(leaf[b])) for b in range(w.B)}, q, k, v, g, beta, self.S)
        lf = torch.from_numpy(np.ascontiguousarray(leaf, np.int32)).to(self.dev)
        self.kv.commit_tree(par, lf)
        eager = self.flush_policy == kb.FLUSH_EAGER
        folded = {b for b in range(w.B) if self.model.commit_path(b, path_to(b, int(leaf[b])), eager=eager)}
        self._after(folded)
        return out

    def retire_and_admit(self, b):
        """Request b ends; a new buffer-only request takes its batch entry with
        fresh blocks from the free list (the old ones go to its end)."""
        bpr = self.w.blocks_per_req
        old = self.model.requests[b].table
        new = [self.free.pop(0) for _ in range(bpr)]
        self.free.extend(old)
        self.model.replace_request(b, new, 0, has_state=False)
        self.kv.block_table[b].copy_(torch.tensor(new, dtype=torch.int32))
        self.kv.occupancy[b] = 0
        self.kv.admit(torch.tensor([b], dtype=torch.int32, device=self.dev))
        if b in self.rows_of:
            self.S[self.rows_of[b]] = 0.0

    # ---------------------------------------------------------------- checks
    def _remember(self, tid_of, k, v, g):
        """Keeps, per request, its sampled tiles' rows of one token's key,
        value (not for the delta rule, whose pool holds pseudo-values) and gate."""
        keep_v = self.w.rule != kb.RULE_DELTA
        for b, rows in self.rows_of.items():
            self.tokens[tid_of(b)] = (k[rows], v[rows] if keep_v else None, None if g is None else g[rows])
        self.calls += 1
        if self.calls % 16 == 0:  # forget tokens no pool position holds any more
            live = set(self.model.physical.values())
            for tid in [t for t in self.tokens if t not in live]:
                del self.tokens[tid]

    def _after(self, folded):
        # The stored state equals the recurrence's state when the fold used up
        # every buffered token; otherwise tokens past m are still buffered and
        # only the effective state (check_effective_states) is comparable.
        if folded:
            f = np.zeros(self.w.B, bool)
            f[list(folded)] = True
            empty = self.model.occupancies() == 0
            js = np.nonzero((f & empty)[self.sb_np])[0]
            if js.size:
                if self.full_state_checks == 0:
                    self.check_states(js)
                    self.full_state_checks += 1
                else:
                    self.check_states(self._rotate(js))
        if self.check_every_step or folded:
            self.check_bookkeeping()

    def _rotate(self, js):
        if js.size <= self.state_sample:
            return js
        start = (self._rotor * self.state_sample) % js.size
        self._rotor += 1
        return np.take(js, np.arange(start, start + self.state_sample), mode="wrap")

    def check_states(self, js):
        """Stored states of sampled tiles js against the oracle."""
        js = np.asarray(js, np.int64)
        gpu = self._stored_states(js)
        err = rel_err_tiles(gpu, self.S[js], axes=(-2, -1))
        self.max_state = max(self.max_state, err)
        self.folds_checked += js.size
        assert err <= self.tol_state, "stored state error %.3e" % err

    def check_all_states(self):
        """Stored state of every compared tile whose buffer is empty (its last
        fold used every buffered token, or it has not buffered any)."""
        empty = (self.model.occupancies() == 0)[self.sb_np]
        js = np.nonzero(empty & (self.slots[self.sb_np] >= 0))[0]
        if js.size:
            self.check_states(js)
            self.full_state_checks += 1
        return js.size

    def check_effective_states(self):
        """kvbuf_materialize against the oracle state of every sampled tile."""
        eff = self.kv.materialize()
        if self.all:
            gpu = eff.reshape(-1, self.w.dk, self.w.dv).cpu().numpy()
        else:
            gpu = eff[self.sb, self.sh].cpu().numpy()
        del eff
        err = rel_err_tiles(gpu, self.S, axes=(-2, -1))
        assert err <= self.tol_state, "materialized state error %.3e" % err
        return err

    def check_bookkeeping(self):
        if self.w.m == 0:
            return
        torch.cuda.synchronize()
        assert int(self.kv.error.item()) == 0, "device error flags %d" % int(self.kv.error.item())
        # each request's table row and occupancy, and every head's copy of them
        np.testing.assert_array_equal(self.kv.block_table.cpu().numpy(), self.model.tables())
        np.testing.assert_array_equal(self.kv.occupancy.cpu().numpy(), self.model.occupancies())
        tm = self.kv.tile_meta.cpu().numpy()
        np.testing.assert_array_equal(tm[:, :, 0], np.broadcast_to(self.model.occupancies()[:, None], tm.shape[:2]))
        np.testing.assert_array_equal(tm[:, :, 1:], np.broadcast_to(self.model.tables()[:, None, :], tm[:, :, 1:].shape))

    def check_pool(self):
        """Buffered keys, gates and (linear / gated rules) values of the sampled
        tiles are the inputs' bits."""
        bf16 = self.w.io == "bf16"

        def host_bits(x, io_plane):
            if x is None:
                return None
            x = x.detach()
            if io_plane and bf16:
                return x.view(torch.int16).cpu().numpy().view(np.uint16)
            return x.float().view(torch.int32).cpu().numpy().view(np.uint32)

        def ref_bits(x, io_plane):
            b = np.ascontiguousarray(x, np.float32).view(np.uint32)
            return (b >> 16).astype(np.uint16) if (io_plane and bf16) else b

        key = host_bits(self.kv.key, True)
        value = None if self.w.rule == kb.RULE_DELTA else host_bits(self.kv.value, True)
        gate = host_bits(self.kv.gate, False)
        for b, rows in self.rows_of.items():
            toks = self.model.buffered_tokens(b)
            if not toks:
                continue
            heads = self.sh_np[rows]
            pos = [self.model.position(b, p) for p in range(len(toks))]
            blk = np.array([p[0] for p in pos], np.int64)[:, None]
            off = np.array([p[1] for p in pos], np.int64)[:, None]
            hh = heads[None, :]
            kref = np.stack([self.tokens[t][0] for t in toks])  # [P, nh, d]
            np.testing.assert_array_equal(key[blk, hh, off], ref_bits(kref, True), err_msg="key bits, request %d" % b)
            if value is not None:
                vref = np.stack([self.tokens[t][1] for t in toks])
                np.testing.assert_array_equal(value[blk, hh, off], ref_bits(vref, True),
                                              err_msg="value bits, request %d" % b)
            if gate is not None:  # one gate, or one per key channel
                gref = np.stack([self.tokens[t][2] for t in toks])
                np.testing.assert_array_equal(gate[blk, hh, off], ref_bits(gref, False),
                                              err_msg="gate bits, request %d" % b)
