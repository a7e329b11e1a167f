"""Draft verification by rejection sampling (TEST INFRASTRUCTURE ONLY).

The rule the pages give for speculative decoding with a built-in draft head
(page 5, bs178.com llamAmpere article, "为什么它真能这么快" point 四): each
draft token is kept with probability min(1, p/q), p the target model's
probability of that token and q the draft head's; the result has exactly the
target distribution.  The older rule the same passage mentions, keeping a draft
only when it equals the target's top choice, is the temperature-0 case here.

Readings where the pages are silent: p_j = softmax(L_j / T); strict "<" against the uniform;
on the first rejection one token is drawn from max(0, p_j - q_j) renormalised
(from p_j if that is all zero) by inverse CDF in index order with the last
uniform; if every draft is kept a bonus token is drawn from p_k the same way.
"""
import numpy as np


def softmax_t(logits, T):
    z = np.asarray(logits, np.float64) / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def inverse_cdf(weights, u):
    """smallest index r with sum(weights[:r+1]) > u * sum(weights)"""
    w = np.asarray(weights, np.float64)
    c = np.cumsum(w)
    r = int(np.searchsorted(c, u * c[-1], side="right"))
    # skip zero-weight entries that a u = 0 draw could land on
    while w[min(r, len(w) - 1)] == 0 and r < len(w) - 1:
        r += 1
    return min(r, len(w) - 1)


def accept(logits, drafts, q, u, temperature):
    """logits: [k+1][V] target logits at the k+1 verified positions (row j is
    the distribution of the token after position j); drafts: k draft ids;
    q: [k][V] draft probabilities; u: k+1 uniforms in [0, 1).
    Returns (emitted tokens, number of drafts accepted)."""
    k = len(drafts)
    out = []
    if temperature == 0:
        for j in range(k):
            t = int(np.argmax(logits[j]))
            if drafts[j] == t:
                out.append(t)
            else:
                out.append(t)
                return out, j
        out.append(int(np.argmax(logits[k])))
        return out, k
    for j in range(k):
        p = softmax_t(logits[j], temperature)
        d = int(drafts[j])
        qd = float(q[j][d])
        # a draft the draft distribution gives probability 0 is rejected
        ratio = p[d] / qd if qd > 0 else 0.0
        if u[j] < min(1.0, ratio):
            out.append(d)
            continue
        resid = np.maximum(p - np.asarray(q[j], np.float64), 0.0)
        if resid.sum() <= 0:
            resid = p
        out.append(inverse_cdf(resid, u[k]))
        return out, j
    out.append(inverse_cdf(softmax_t(logits[k], temperature), u[k]))
    return out, k


def verify(model, tokens, q, u, temperature):
    """Oracle of draft verification on an oracle.Model: run tokens [t0, d1..dk]
    from the model's state, apply the acceptance rule, then restore the state
    and commit t0 .. d_a (the accepted prefix).  Returns (emitted, accepted,
    logits [k+1][V])."""
    snap = model.snapshot()
    logits = []
    for t in tokens:
        _, L, _ = model.decode_token(int(t))
        logits.append(L)
    logits = np.stack(logits)
    out, a = accept(logits, list(tokens[1:]), q, u, temperature)
    model.restore(snap)
    for t in tokens[:a + 1]:
        model.decode_token(int(t))
    return out, a, logits
