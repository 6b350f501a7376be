"""fp64 CPU oracle for stochastic tree verification at temperature T > 0 --
test infrastructure only.

Nothing in the product path may import, call or execute this module: only
the test suite, the smoke check and the CPU-baseline leg of the benchmark use
it.  It shares no code with the HIP path.

Sources:

* "SpecPV: Improving Self-Speculative Decoding for Long-Context Generation
  via Partial Verification" (paperlayer.ai summary), Sec. 2 "Related Work":
  speculative sampling (Leviathan et al.) is equivalent to sampling from the
  target; SpecInfer verifies a tree of candidates.  App. D and App. E: runs
  at temperatures 0.6, 0.7 and 1.0.
* "SpecBlock: Block-Iterative Speculative Decoding with Dynamic Tree
  Drafting" (paperlayer.ai summary), Sec. 4: evaluation at temperature 0 and
  1.0.
* Random numbers: Philox-4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written from its
  published round function and constants.

Readings (listed in the design notes):

* Node u's target distribution is p_u = softmax(logits_u / T) over the whole
  vocabulary, optionally filtered (SpecPV App. D: Qwen3 thinking mode samples
  at T = 0.6 with top-p 0.95 and top-k 20; App. E: T = 0.7 and 1.0 with
  top-k off and top-p 0.9).  Filters, in this order:
  - top-k (k > 0): token x is kept iff fewer than k tokens have a strictly
    larger logit (tokens tied with the k-th largest are all kept);
  - top-p (p < 1): among the tokens top-k kept, with their probabilities
    renormalised, x is kept iff the tokens with a strictly larger logit hold
    less than p of that mass (so the most likely token is always kept);
  - the kept tokens' probabilities are renormalised to sum to 1.
* The pages give no draft distributions, so a draft token is a point mass:
  at an accepted node u the children are tried in ascending node index;
  child c with token x is accepted with probability p_u(x) / R, R the
  probability mass not yet rejected at u (R starts at 1; a rejected token's
  mass leaves R, and a token already rejected at u has probability 0).  The
  first accepted child becomes the next node.
* When no child is accepted the walk ends and the bonus token is drawn from
  the residual: p_u without the rejected tokens, renormalised by R, by
  inverse CDF in vocabulary order.
* Uniforms: the first 64-bit word of Philox-4x64-10 with key (seed0, seed1)
  and counter (step, sequence, node, slot), slot = the child's rank among its
  siblings for an acceptance test and 2^64 - 1 for the bonus draw; the
  uniform is (word >> 40) * 2^-24, exact in fp32 and fp64.
* A draft token outside [0, V) is never accepted and removes nothing.  If
  the residual holds no probability (all of it rejected, possible only
  through rounding), the bonus is the lowest-index most probable token.
"""

from __future__ import annotations

import numpy as np

from .tree_verify import OracleInputError, bf16_to_f64

__all__ = ["philox4x64_10", "uniform", "BONUS_SLOT", "target_probs", "stochastic_accept"]

_MASK = (1 << 64) - 1
_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157   # Philox-4x64 multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B   # key schedule (Weyl) increments
BONUS_SLOT = _MASK


def philox4x64_10(counter, key):
    """Philox-4x64-10 block: four 64-bit counter words and two key words in,
    four 64-bit words out.  Each round multiplies words 0 and 2 by the two
    constants (full 128-bit products), and the new state is
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the
    key is bumped by the Weyl constants between rounds."""
    c = [int(x) & _MASK for x in counter]
    k0, k1 = (int(x) & _MASK for x in key)
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & _MASK, (p0 >> 64) ^ c[3] ^ k1, p0 & _MASK]
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return c


def uniform(key, step: int, seq: int, node: int, slot: int) -> float:
    """The uniform in [0, 1) of one decision: 24 high bits of the first word."""
    w = philox4x64_10((step, seq, node, slot), key)[0]
    return (w >> 40) * 2.0 ** -24


def _row_f64(row) -> np.ndarray:
    r = np.asarray(row)
    return bf16_to_f64(r) if r.dtype == np.uint16 else r.astype(np.float64)


def target_probs(row, temperature: float, top_k: int = 0, top_p: float = 1.0) -> np.ndarray:
    """softmax(logits / T) in fp64, then the top-k and top-p filters of the
    module notes (top_k = 0 and top_p = 1 leave it unfiltered)."""
    if not temperature > 0:
        raise OracleInputError("temperature must be positive")
    if top_k < 0 or not 0.0 < top_p <= 1.0:
        raise OracleInputError("top_k must be >= 0 and top_p in (0, 1]")
    l = _row_f64(row)
    z = l / float(temperature)
    if not np.all(np.isfinite(z)):
        raise OracleInputError("non-finite logits")
    e = np.exp(z - z.max())
    p = e / e.sum()
    keep = np.ones(p.shape, dtype=bool)
    if top_k > 0:
        # number of tokens with a strictly larger logit, for every token
        keep &= _count_above(l) < top_k
    if top_p < 1.0:
        q = np.where(keep, p, 0.0)
        q = q / q.sum()
        mass_above = _mass_above(l, q)
        keep &= mass_above < top_p
    f = np.where(keep, p, 0.0)
    return f / f.sum()


def _count_above(l):
    """For each entry, how many entries are strictly larger (via a sort)."""
    s = np.sort(l)
    return l.size - np.searchsorted(s, l, side="right")


def _mass_above(l, q):
    """For each entry, the total of q over entries with a strictly larger l."""
    order = np.argsort(-l, kind="stable")
    ls, qs = l[order], q[order]
    out = np.empty_like(q)
    run = 0.0
    i = 0
    while i < ls.size:
        j = i
        while j < ls.size and ls[j] == ls[i]:
            j += 1
        out[order[i:j]] = run          # mass strictly above this value
        run += qs[i:j].sum()
        i = j
    return out


def _walk(probs_of, parents_row, draft_row, vocab, key, step, seq, decide=None):
    n = len(parents_row)
    children = [[] for _ in range(n)]
    for j in range(1, n):
        children[int(parents_row[j])].append(j)
    u, path, events = 0, [0], []
    while True:
        p = probs_of(u)
        rest, removed, nxt = 1.0, set(), None
        for rank, c in enumerate(children[u]):
            x = int(draft_row[c])
            valid = 0 <= x < vocab and x not in removed
            px = float(p[x]) if valid else 0.0
            unif = uniform(key, step, seq, u, rank)
            ok = unif * rest < px
            if decide is not None:
                ok = decide(("child", u, c, unif, rest, px), ok)
            events.append(("child", u, c, unif, rest, px, ok))
            if ok:
                nxt = c
                break
            rest -= px
            if valid:
                removed.add(x)
        if nxt is None:
            unif = uniform(key, step, seq, u, BONUS_SLOT)
            resid = p.copy()
            for x in removed:
                resid[x] = 0.0
            target = unif * rest
            cum = np.cumsum(resid)
            hits = np.nonzero(cum > target)[0]
            if hits.size:
                y = int(hits[0])
            else:
                pos = np.nonzero(resid > 0)[0]
                y = int(pos[-1]) if pos.size else int(np.argmax(p))
            events.append(("bonus", u, y, unif, rest, target))
            return len(path) - 1, path, y, events
        path.append(nxt)
        u = nxt


def stochastic_accept(logits, parents, draft_tokens, temperature: float, key, step: int = 0,
                      return_events: bool = False, decide=None, top_k: int = 0,
                      top_p: float = 1.0):
    """Stochastic verification of a draft tree (see the module notes).

    logits [B][N][V] (bf16 as uint16 bit patterns, or fp32); parents and
    draft_tokens int [B][N].  Returns (accept_len [B], accept_path [B][N]
    root first and -1 padded, bonus [B]); with ``return_events`` also the
    per-sequence list of decisions.  ``decide(event, ok)`` may override an
    acceptance decision (used to follow another implementation's choice where
    a uniform lies within rounding distance of its threshold).  ``top_k`` /
    ``top_p`` filter every node's distribution (module notes).
    """
    lg = np.asarray(logits)
    par = np.asarray(parents)
    dr = np.asarray(draft_tokens)
    bsz, n, vocab = lg.shape
    alen = np.zeros(bsz, dtype=np.int32)
    path = np.full((bsz, n), -1, dtype=np.int32)
    bonus = np.zeros(bsz, dtype=np.int32)
    all_events = []
    for b in range(bsz):
        if par[b, 0] != -1 or any(not 0 <= int(par[b, j]) < j for j in range(1, n)):
            raise OracleInputError("malformed parent array")
        cache = {}

        def probs_of(u, b=b, cache=cache):
            if u not in cache:
                cache[u] = target_probs(lg[b, u], temperature, top_k, top_p)
            return cache[u]
        a, pth, y, ev = _walk(probs_of, par[b], dr[b], vocab, key, step, b,
                              None if decide is None else (lambda e, ok, b=b: decide(b, e, ok)))
        alen[b] = a
        path[b, :len(pth)] = pth
        bonus[b] = y
        all_events.append(ev)
    if return_events:
        return alen, path, bonus, all_events
    return alen, path, bonus
