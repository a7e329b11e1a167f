"""Draft head driver and draft selection (TEST INFRASTRUCTURE ONLY).

The pages' speculative decoding (page 5, bs178.com llamAmpere article, "为什么
它真能这么快" point 四) lets the model's own draft head propose three tokens
that the target then checks with the min(1, p/q) rule, and it shrinks only
the draft head's output projection to a list of 65,536 ids; the target keeps
the full vocabulary.  This module mirrors, on the oracle model, the order in
which the library feeds the draft head; the arithmetic of one draft step is
or_draft_step in aw4_oracle.c.

Readings where the pages are silent:
  - the draft head's cache gets one entry per committed position r whose next
    token x_{r+1} is known, built from (target hidden h_r, x_{r+1}); prefill
    feeds every prompt position, a verify pass leaves its accepted positions
    pending until the next draft call, a plain decode step feeds nothing;
  - a draft call first commits the pending entries and the entry of the last
    committed position with t0 (the token the target runs next); drafts 2..k
    come from the draft head's own output hidden and previous draft, in cache
    entries that are not committed;
  - temperature 0: the draft is the mapped id with the largest score (lowest
    id on ties); temperature T > 0: q = softmax(scores / T) over the mapped ids
    (zero elsewhere) and the draft is drawn by inverse CDF in ascending-id
    order with one uniform per draft.
"""
import numpy as np

from .accept import accept, inverse_cdf, softmax_t


def select(z, temperature, u):
    """index into the ascending map and the draft distribution over the map
    (None at temperature 0)"""
    if temperature == 0:
        return int(np.argmax(z)), None
    q = softmax_t(z, temperature)
    return inverse_cdf(q, u), q


class DraftDriver:
    """An oracle.Model with a draft head, plus the pending entries of the draft
    head's cache and the hidden state of the last committed position."""

    def __init__(self, model):
        self.m = model
        self.map = model.draft_map()
        self.pending = []        # (hidden, next token) of committed positions not yet fed
        self.last = None         # hidden of the last committed position

    def _feed(self, token, h):
        out = self.m.draft_step(int(token), h, 0)
        self.m.set_dpos(self.m.dpos + 1)
        return out

    def decode(self, token):
        x, logits, am = self.m.decode_token(int(token))
        self.pending, self.last = [], x
        return x, logits, am

    def prefill(self, tokens):
        out = None
        for i, t in enumerate(tokens):
            out = self.m.decode_token(int(t))
            if i + 1 < len(tokens):
                self._feed(tokens[i + 1], out[0])
        self.pending, self.last = [], out[0]
        return out

    def verify(self, tokens, q, u, temperature):
        """accept.verify on the target, keeping the hidden states of the
        committed positions -> (emitted, accepted, logits)"""
        snap = self.m.snapshot()
        logits = np.stack([self.m.decode_token(int(t))[1] for t in tokens])
        out, a = accept(logits, list(tokens[1:]), q, u, temperature)
        self.m.restore(snap)
        xs = [self.m.decode_token(int(t))[0] for t in tokens[:a + 1]]
        self.pending = [(xs[i], int(tokens[i + 1])) for i in range(a)]
        self.last = xs[a]
        return out, a, logits

    def draft(self, t0, k, temperature=0.0, u=None, force=None):
        """-> (k drafts, q [k][vocab] or None, mapped scores [k][draft_vocab]);
        force (optional): the tokens fed to drafts 2..k instead of this
        driver's own earlier drafts (teacher forcing for comparisons)"""
        if self.last is None:
            raise ValueError("no committed hidden state to draft from")
        for h, t in self.pending:
            self._feed(t, h)
        x, z = self._feed(t0, self.last)
        self.pending, self.last = [], None
        V = self.m.shape.vocab
        drafts, qs, zs = [], [], []
        for j in range(k):
            if j > 0:
                x, z = self.m.draft_step(drafts[-1] if force is None else force[j - 1], x, j - 1)
            i, qm = select(z, temperature, None if u is None else u[j])
            drafts.append(int(self.map[i]))
            zs.append(z)
            if qm is not None:
                qf = np.zeros(V)
                qf[self.map] = qm
                qs.append(qf)
        return drafts, (np.stack(qs) if qs else None), np.stack(zs)
