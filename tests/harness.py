"""Drives a workload through the HIP library (through its C ABI) and through
the oracle side by side, and compares them.

Tolerances (the method must reproduce the recurrence exactly up to rounding;
the GPU accumulates in fp32 from bf16 or fp32 inputs):
  outputs  per tile  max|o_gpu - o_ref| / max|o_ref|  <= 2e-3
  states   per tile  max|S_gpu - S_ref| / max|S_ref|  <= 1e-5 after every fold
  block tables, occupancies and buffered key / gate bits: exact.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import linear_attention_decode_kvbuf_amd as kb

TOL_OUT = 2e-3
TOL_STATE = 1e-5


def rel_err_tiles(gpu, ref, axes):
    """max over tiles of max|gpu - ref| / max|ref| (reduction over ``axes``)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(gpu - ref), axis=axes)
    den = np.maximum(np.max(np.abs(ref), axis=axes), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0


def default_sample(w, count=24, seed=0):
    """(b, h) tiles to compare: all of them for tiny batches, else a spread."""
    if w.B * w.H <= 64:
        return [(b, h) for b in range(w.B) for h in range(w.H)]
    rs = np.random.default_rng(seed)
    bs = np.unique(np.concatenate([[0, w.B - 1], rs.integers(0, w.B, count)]))[:count]
    return [(int(b), int(rs.integers(0, w.H))) for b in bs]


def _np(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy()
    return np.asarray(x, np.float32)


class Run:
    def __init__(self, w, *, flush=kb.FLUSH_EAGER, sample=None, device_gen=None, spare_blocks=3,
                 stateless=None, check_every_step=None):
        self.w = w
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
                              io_dtype=kb.BF16 if w.io == "bf16" else kb.F32, flush=flush)
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

        self.sample = sample if sample is not None else default_sample(w)
        self.sb = torch.tensor([b for b, _ in self.sample], device=self.dev, dtype=torch.long)
        self.sh = torch.tensor([h for _, h in self.sample], device=self.dev, dtype=torch.long)
        st = self.kv.state.detach()
        S = []
        for b, h in self.sample:
            S.append(np.zeros((w.dk, w.dv)) if slots[b] < 0 else st[slots[b], h].double().cpu().numpy())
        self.S = np.stack(S)  # oracle state of every sampled tile, fp64
        self.tokens = {}  # (token id, sample index) -> (k bits, g) for the pool check
        self.max_out = 0.0
        self.max_state = 0.0
        self.folds_checked = 0

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
        """[ns, ...] host copy of the sampled tiles of a [B, (n,) H, ...] tensor."""
        if x is None:
            return None
        if drafts:
            return _np(x[self.sb, :, self.sh])
        return _np(x[self.sb, self.sh])

    # ---------------------------------------------------------------- steps
    def decode(self, t, direct=False):
        w = self.w
        inp = self.inputs(t)
        if direct:
            out = self.kv.direct(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        else:
            out = self.kv.decode(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        folded = set()
        if w.m > 0:
            eager = self.flush_policy == kb.FLUSH_EAGER
            for b in range(w.B):
                if self.model.decode(b, ("d", t, b), eager=eager, stateless=direct or self.stateless[b]):
                    folded.add(b)
        q, k, v, g, beta = (self._sampled(inp[x]) for x in ("q", "k", "v", "g", "beta"))
        self._remember([("d", t, b) for b, _ in self.sample], k, v, g)
        o_ref, self.S = oracle.recurrent(w.rule, self.S, q[None], k[None], v[None],
                                         None if g is None else g[None],
                                         None if beta is None else beta[None])
        o_gpu = self._sampled(out)
        err = rel_err_tiles(o_gpu, o_ref[0], axes=-1)
        self.max_out = max(self.max_out, err)
        assert err <= TOL_OUT, "step %d: output error %.3e" % (t, err)
        self._after(folded)
        return out

    def flush(self):
        self.kv.flush()
        folded = {b for b in range(self.w.B) if self.model.flush(b)}
        self._after(folded)

    def verify_commit(self, call, n, accepted):
        """One verify of n drafts per request, then commit ``accepted`` [B]."""
        w = self.w
        inp = self.inputs(call, n=n, stream_base=100)
        out = self.kv.verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        for b in range(w.B):
            self.model.verify(b, [("v", call, b, d) for d in range(n)])
        q, k, v, g, beta = (self._sampled(inp[x], drafts=True) for x in ("q", "k", "v", "g", "beta"))
        o_gpu = self._sampled(out, drafts=True)  # [ns, n, d]
        for j, (b, h) in enumerate(self.sample):
            for dd in range(n):
                self.tokens[(("v", call, b, dd), j)] = (k[j, dd].copy(), v[j, dd].copy(),
                                                        None if g is None else np.array(g[j, dd], np.float32))
            tr = lambda x: None if x is None else np.swapaxes(x[j:j + 1], 0, 1)  # [n, 1, ...]
            o_ref, _ = oracle.recurrent(w.rule, self.S[j:j + 1], tr(q), tr(k), tr(v), tr(g), tr(beta))
            err = rel_err_tiles(o_gpu[j], o_ref[:, 0], axes=-1)
            self.max_out = max(self.max_out, err)
            assert err <= TOL_OUT, "verify %d tile %s: output error %.3e" % (call, (b, h), err)
            a = int(accepted[b])
            if a:
                _, S1 = oracle.recurrent(w.rule, self.S[j:j + 1], tr(q)[:a], tr(k)[:a], tr(v)[:a],
                                         None if g is None else tr(g)[:a],
                                         None if beta is None else tr(beta)[:a])
                self.S[j] = S1[0]
        acc = torch.from_numpy(np.asarray(accepted, np.int32)).to(self.dev)
        self.kv.commit(n, acc)
        eager = self.flush_policy == kb.FLUSH_EAGER
        folded = {b for b in range(w.B) if self.model.commit(b, int(accepted[b]), eager=eager)}
        self._after(folded)
        return out

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

        def path_to(b, d):
            path = []
            while d >= 0:
                path.append(d)
                d = int(parent[b][d])
            return path[::-1]

        for j, (b, h) in enumerate(self.sample):
            for dd in range(n):
                self.tokens[(("t", call, b, dd), j)] = (k[j, dd].copy(), v[j, dd].copy(),
                                                        None if g is None else np.array(g[j, dd], np.float32))
            sel = lambda x, path: None if x is None else np.swapaxes(x[j:j + 1, path], 0, 1)  # [len, 1, ...]
            for dd in range(n):
                path = path_to(b, dd)
                o_ref, _ = oracle.recurrent(w.rule, self.S[j:j + 1], sel(q, path), sel(k, path), sel(v, path),
                                            sel(g, path), sel(beta, path))
                err = rel_err_tiles(o_gpu[j, dd][None], o_ref[-1], axes=-1)
                self.max_out = max(self.max_out, err)
                assert err <= TOL_OUT, "tree verify %d tile %s draft %d: output error %.3e" % (call, (b, h), dd, err)
            path = path_to(b, int(leaf[b]))
            if path:
                _, S1 = oracle.recurrent(w.rule, self.S[j:j + 1], sel(q, path), sel(k, path), sel(v, path),
                                         sel(g, path), sel(beta, path))
                self.S[j] = S1[0]
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
        self.kv.block_table[b].copy_(torch.tensor(new, dtype=torch.int32))  # every head
        self.kv.occupancy[b] = 0
        for j, (bb, _) in enumerate(self.sample):
            if bb == b:
                self.S[j] = 0.0

    # ---------------------------------------------------------------- checks
    def _remember(self, tids, k, v, g):
        for j, tid in enumerate(tids):
            self.tokens[(tid, j)] = (k[j].copy(), v[j].copy(), None if g is None else np.array(g[j], np.float32))

    def _after(self, folded):
        # The stored state equals the recurrence's state when the fold used up
        # every buffered token; otherwise tokens past m are still buffered and
        # only the effective state (check_effective_states) is comparable.
        sampled_folds = [j for j, (b, _) in enumerate(self.sample)
                         if b in folded and self.model.requests[b].occupancy == 0]
        if sampled_folds:
            self.check_states(sampled_folds)
        if self.check_every_step or folded:
            self.check_bookkeeping()

    def check_states(self, js):
        st = self.kv.state.detach()
        for j in js:
            b, h = self.sample[j]
            gpu = st[self.slots[b], h].double().cpu().numpy()
            err = rel_err_tiles(gpu[None], self.S[j][None], axes=(-2, -1))
            self.max_state = max(self.max_state, err)
            self.folds_checked += 1
            assert err <= TOL_STATE, "state of tile %s: error %.3e" % ((b, h), err)

    def check_effective_states(self):
        """kvbuf_materialize against the oracle state of every sampled tile."""
        eff = self.kv.materialize()
        gpu = eff[self.sb, self.sh].double().cpu().numpy()
        err = rel_err_tiles(gpu, self.S, axes=(-2, -1))
        assert err <= TOL_STATE, "materialized state error %.3e" % err
        return err

    def check_bookkeeping(self):
        if self.w.m == 0:
            return
        torch.cuda.synchronize()
        assert int(self.kv.error.item()) == 0, "device error flags %d" % int(self.kv.error.item())
        # every head's copy of the table and occupancy equals the model's
        bt = self.kv.block_table.cpu().numpy()
        occ = self.kv.occupancy.cpu().numpy()
        np.testing.assert_array_equal(bt, np.broadcast_to(self.model.tables()[:, None, :], bt.shape))
        np.testing.assert_array_equal(occ, np.broadcast_to(self.model.occupancies()[:, None], occ.shape))

    def check_pool(self):
        """Buffered keys, gates and (linear / gated rules) values of the sampled
        tiles are the inputs' bits."""
        key = self.kv.key.detach()
        value = None if self.w.rule == 2 else self.kv.value.detach()
        gate = None if self.kv.gate is None else self.kv.gate.detach()
        bits = lambda x: np.asarray(x, np.float32).view(np.uint32)
        for j, (b, h) in enumerate(self.sample):
            toks = self.model.buffered_tokens(b)
            for p, tid in enumerate(toks):
                blk, off = self.model.position(b, p)
                kref, vref, gref = self.tokens[(tid, j)]
                np.testing.assert_array_equal(bits(key[blk, h, off].float().cpu().numpy()), bits(kref))
                if value is not None:
                    np.testing.assert_array_equal(bits(value[blk, h, off].float().cpu().numpy()), bits(vref))
                if gate is not None:  # one gate, or one per key channel
                    np.testing.assert_array_equal(bits(gate[blk, h, off].cpu().numpy()), bits(gref))
