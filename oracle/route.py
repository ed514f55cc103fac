"""Expert routing: top-k of E routed experts per token, and the grouped table.

What the pages fix: each MoE layer sends a token to 8 of 512 routed experts
plus one always-on shared expert [card §background; news §where the speed comes
from; ic §three scalpels].  Verifying 4 draft tokens at once can touch up to 32
distinct experts, and that activation -- not attention -- is what a verify
round costs [card §method #3].

Readings where the pages are silent (stated, not derived from them):
  * selection is on the float32 logits, ordered by (logit descending, expert
    index ascending); +0.0 and -0.0 compare equal, so the index decides;
  * the weights are the softmax over all E logits renormalised over the k
    selected experts (equal to a softmax over the k selected logits);
  * no group limit, no expert bias, routed scaling factor 1;
  * the grouped table lists the distinct selected experts in ascending id, each
    with the set of tokens that chose it and their weights, followed by the
    shared expert serving every token with weight 1;
  * for many tokens (a prefill chunk, a long verify window) the same grouping
    is kept as one token list per expert, tokens ascending, the shared
    expert's list (every token) last [card §method #3: each active expert is
    read once for all the tokens it serves].

Parity status: pinned (tests/test_oracle_route.py) by the invariant that the
selection equals the first k entries of a stable full sort done by a library
routine (numpy lexsort) on random and tie-heavy logits, by k = E, by the
softmax-over-selected closed form (scipy), by sum(w) = 1 and k = 1 -> w = 1, and
by a hand-worked tie fixture under tests/golden/.  expert_groups is pinned
against dispatch_table (same membership, for M <= 32), by its counting
invariants (every token in exactly k routed lists and the shared one), and by
a hand-worked fixture under tests/golden/.  The router logits are pinned
by a hand-worked 3 x 2 example, one-hot activations selecting one column of the
router matrix per expert (orientation), x = 0, and linearity in x.
"""

import numpy as np


def router_logits(w_router, x):
    """Router logits, the step before the selection [card §background: the
    router picks 8 of 512 experts from the token's hidden state]: logits[m, e]
    = sum_k x[m, k] W_router[e, k] in float64 (products of bf16 values are
    exact there), no bias.

    w_router [E][H] and x [M][H] bf16-exact values; returns float64 [M][E].
    """
    w = np.asarray(w_router, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return x @ w.T


def route_topk(logits, k):
    """Top-k routing of each token.

    logits  float32 [M][E]
    returns ids int32 [M][k] in selection order, weights float64 [M][k]
    """
    logits = np.asarray(logits, dtype=np.float32)
    m_tokens, n_exp = logits.shape
    assert 1 <= k <= n_exp
    ids = np.zeros((m_tokens, k), dtype=np.int32)
    w = np.zeros((m_tokens, k), dtype=np.float64)
    for m in range(m_tokens):
        row = [float(v) for v in logits[m]]            # exact float32 -> float64
        # Python's sort is stable; the key makes larger logits first and, for
        # equal logits (including +0.0 == -0.0), the smaller index first.
        order = sorted(range(n_exp), key=lambda i: (-row[i], i))
        sel = order[:k]
        ids[m] = sel
        top = max(row)
        p = np.array([np.exp(v - top) for v in row])   # softmax over all E
        p = p / p.sum()
        chosen = np.array([p[i] for i in sel])
        w[m] = chosen / chosen.sum()                   # renormalise over the k
    return ids, w


def dispatch_table(ids, w, n_experts):
    """Group the routing of M tokens by expert.

    Returns (experts, masks, weights):
      experts int32 [S]   distinct selected expert ids ascending, then n_experts
                          standing for the shared expert
      masks   uint32 [S]  bit m set when token m is served by that expert
      weights float64 [S][M]  weight of token m for that expert, 0 when unserved
    S = (number of distinct selected experts) + 1.
    """
    ids = np.asarray(ids)
    m_tokens, k = ids.shape
    distinct = sorted(set(int(e) for e in ids.flatten()))
    experts, masks, weights = [], [], []
    for e in distinct:
        mask = 0
        wt = np.zeros(m_tokens, dtype=np.float64)
        for m in range(m_tokens):
            for j in range(k):
                if int(ids[m, j]) == e:
                    mask |= 1 << m
                    wt[m] = w[m, j]
        experts.append(e)
        masks.append(mask)
        weights.append(wt)
    experts.append(n_experts)                           # shared expert
    masks.append((1 << m_tokens) - 1)
    weights.append(np.ones(m_tokens, dtype=np.float64))
    return (np.array(experts, dtype=np.int32), np.array(masks, dtype=np.uint32),
            np.array(weights, dtype=np.float64))


def expert_groups(ids, n_experts):
    """Token lists of the E routed experts and the shared expert.

    ids  int [T][k], the k distinct experts of each token
    returns a list of n_experts + 1 int64 arrays: entry e holds, ascending, the
    tokens t with e among ids[t]; entry n_experts (the shared expert) holds
    every token.  len(entry) is the number of rows expert e multiplies.
    """
    ids = np.asarray(ids)
    t_tokens = ids.shape[0]
    lists = [[] for _ in range(n_experts)]
    for t in range(t_tokens):
        for e in ids[t]:
            lists[int(e)].append(t)
    groups = [np.array(sorted(lst), dtype=np.int64) for lst in lists]
    groups.append(np.arange(t_tokens, dtype=np.int64))
    return groups
