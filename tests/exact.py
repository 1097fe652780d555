"""Exact rational arithmetic (fractions.Fraction) for tiny cases.

Two independent evaluations of the same token sequence:

* ``exact_recurrent`` -- the per-token recurrence with the rule-2 projection
  formed as an explicit d_k x d_k matrix (I - beta k k^T);
* ``ExactKVBuffer`` -- the buffered method: the state is only rewritten when m
  tokens are buffered; outputs come from the state at the last fold plus a
  causal, decay-weighted sum over the buffered tokens (and, for the delta
  rule, pseudo-values u computed token by token); drafts are verified in
  parallel from the buffer without temporary states.

The buffered form follows from the recurrence by unrolling it since the last
fold (pith.science page, "Load-bearing premise": reordering the state updates
into chunks must not change results).  With gamma_s the per-token decay and
W(t, i) = gamma_{i+1} ... gamma_t (the product over the tokens after i, up to t):

  S_t = W(t, -1) S_0 + sum_{i<=t} W(t, i) k_i x_i^T
  o_t = W(t, -1) S_0^T q_t + sum_{i<=t} W(t, i) (q_t . k_i) x_i

where x_i = v_i for rules 0 and 1 and, for the delta rule,
  x_t = u_t = beta_t (v_t - W(t, -1) S_0^T k_t - sum_{i<t} W(t, i) (k_i . k_t) u_i).
For rule 3 (one decay per key channel) gamma_s and W(t, i) are vectors over
the d_k channels and act on the rows: W(t, -1) S_0 scales row r by W(t, -1)[r],
and W(t, i) (q_t . k_i) becomes sum_r q_t[r] W(t, i)[r] k_i[r].

Both are pure Python and only meant for d <= 4 and a few dozen tokens.
"""

from fractions import Fraction as F


def zeros(r, c):
    return [[F(0) for _ in range(c)] for _ in range(r)]


def matT_vec(S, x):
    """S^T x for S [r][c], x [r] -> [c]."""
    return [sum((S[r][c] * x[r] for r in range(len(S))), F(0)) for c in range(len(S[0]))]


def dot(a, b):
    return sum((x * y for x, y in zip(a, b)), F(0))


def exact_recurrent(rule, S0, q, k, v, gam, beta, scale=F(1)):
    """Token-by-token recurrence.  q/k/v are lists of vectors, gam/beta lists of
    scalars (gam = 1 and beta unused for rule 0; for rule 3 gam[t] is a vector
    over the key channels).  Returns (outputs, states)."""
    S = [row[:] for row in S0]
    dk, dv = len(S), len(S[0])
    outs, states = [], []
    for t in range(len(q)):
        g = gam[t] if rule >= 1 else F(1)
        if rule == 2:
            b = beta[t]
            P = [[(F(1) if r == s else F(0)) - b * k[t][r] * k[t][s] for s in range(dk)] for r in range(dk)]
            PS = [[sum((P[r][s] * S[s][c] for s in range(dk)), F(0)) for c in range(dv)] for r in range(dk)]
            S = [[g * PS[r][c] + b * k[t][r] * v[t][c] for c in range(dv)] for r in range(dk)]
        elif rule == 3:
            S = [[g[r] * S[r][c] + k[t][r] * v[t][c] for c in range(dv)] for r in range(dk)]
        else:
            S = [[g * S[r][c] + k[t][r] * v[t][c] for c in range(dv)] for r in range(dk)]
        outs.append(matT_vec(S, [scale * x for x in q[t]]))
        states.append([row[:] for row in S])
    return outs, states


class ExactKVBuffer:
    """One tile of the buffered method in exact arithmetic."""

    def __init__(self, rule, S0, m, scale=F(1)):
        self.rule, self.m, self.scale = rule, m, scale
        self.S = [row[:] for row in S0]  # state at the last fold
        self.buf = []  # buffered tokens since the last fold: (k, x, gamma)

    def _weights(self, gammas):
        """W(t, i) for the token list: decay[i] = product of gammas after i up to the
        last token; decay_s = product of all of them (the weight of S_0).  For
        rule 3 every gamma and every weight is a vector over the key channels."""
        n = len(gammas)
        if self.rule == 3:
            dk = len(self.S)
            after = [[F(1)] * dk for _ in range(n)]
            acc = [F(1)] * dk
            for i in range(n - 1, -1, -1):
                after[i] = acc[:]
                acc = [a * g for a, g in zip(acc, gammas[i])]
            return after, acc
        after = [F(1)] * n
        acc = F(1)
        for i in range(n - 1, -1, -1):
            after[i] = acc
            acc *= gammas[i]
        return after, acc

    def _pseudo_value(self, kt, vt, gt, bt, prev):
        """x_t for a new token given the tokens before it (``prev``) since the fold."""
        if self.rule != 2:
            return list(vt)
        gammas = [p[2] for p in prev] + [gt]
        after, w0 = self._weights(gammas)
        Sk = matT_vec(self.S, kt)
        u = [vt[c] - w0 * Sk[c] for c in range(len(vt))]
        for i, (ki, xi, _) in enumerate(prev):
            s = after[i] * dot(ki, kt)
            u = [u[c] - s * xi[c] for c in range(len(u))]
        return [bt * x for x in u]

    def _output(self, qt, toks):
        gammas = [p[2] for p in toks]
        after, w0 = self._weights(gammas)
        qs = [self.scale * x for x in qt]
        if self.rule == 3:
            o = matT_vec(self.S, [w * x for w, x in zip(w0, qs)])
            for i, (ki, xi, _) in enumerate(toks):
                s = sum((a * x * y for a, x, y in zip(after[i], qs, ki)), F(0))
                o = [o[c] + s * xi[c] for c in range(len(o))]
            return o
        o = [w0 * x for x in matT_vec(self.S, qs)]
        for i, (ki, xi, _) in enumerate(toks):
            s = after[i] * dot(qs, ki)
            o = [o[c] + s * xi[c] for c in range(len(o))]
        return o

    def effective_state(self):
        gammas = [p[2] for p in self.buf]
        after, w0 = self._weights(gammas)
        if self.rule == 3:
            S = [[w0[r] * x for x in row] for r, row in enumerate(self.S)]
            for i, (ki, xi, _) in enumerate(self.buf):
                for r in range(len(S)):
                    for c in range(len(S[0])):
                        S[r][c] += after[i][r] * ki[r] * xi[c]
            return S
        S = [[w0 * x for x in row] for row in self.S]
        for i, (ki, xi, _) in enumerate(self.buf):
            for r in range(len(S)):
                for c in range(len(S[0])):
                    S[r][c] += after[i] * ki[r] * xi[c]
        return S

    def fold(self):
        """Fold the first m buffered tokens into the state."""
        head, tail = self.buf[: self.m], self.buf[self.m:]
        self.buf = head
        self.S = self.effective_state()
        self.buf = tail

    def decode(self, qt, kt, vt, gt=F(1), bt=F(0)):
        x = self._pseudo_value(kt, vt, gt, bt, self.buf)
        self.buf.append((list(kt), x, gt))
        o = self._output(qt, self.buf)
        if self.m > 0 and len(self.buf) >= self.m:
            self.fold()
        return o

    def verify(self, qs, ks, vs, gs, bs):
        """Outputs of n drafts, each attending to the buffer and the drafts before it."""
        drafts = []
        outs = []
        for d in range(len(qs)):
            x = self._pseudo_value(ks[d], vs[d], gs[d], bs[d], self.buf + drafts)
            drafts.append((list(ks[d]), x, gs[d]))
            outs.append(self._output(qs[d], self.buf + drafts))
        self._drafts = drafts
        return outs

    def verify_tree(self, qs, ks, vs, gs, bs, parent):
        """Tree drafts: draft d attends to the buffer, its ancestors (parent[d],
        parent[parent[d]], ... up to -1 = the buffer) and itself, with the
        decay accumulated along that path."""
        drafts, outs = [], []
        for d in range(len(qs)):
            anc, a = [], parent[d]
            while a >= 0:
                anc.append(a)
                a = parent[a]
            prev = self.buf + [drafts[a] for a in reversed(anc)]
            x = self._pseudo_value(ks[d], vs[d], gs[d], bs[d], prev)
            drafts.append((list(ks[d]), x, gs[d]))
            outs.append(self._output(qs[d], prev + [drafts[d]]))
        self._drafts = drafts
        return outs

    def commit_path(self, path):
        self.buf.extend(self._drafts[d] for d in path)
        self._drafts = []
        if self.m > 0 and len(self.buf) >= self.m:
            self.fold()

    def commit(self, accepted):
        self.buf.extend(self._drafts[:accepted])
        self._drafts = []
        if self.m > 0 and len(self.buf) >= self.m:
            self.fold()
