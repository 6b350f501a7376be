"""Plain CPU oracle for SpecPV's partial-verification buffer and rectifying
full verification -- test infrastructure only.

Nothing in the product path may import, call or execute this module: only
the test suite, the smoke check and the CPU-baseline leg of the benchmark use
it.  It shares no code with the HIP path or its host-side policy.

Source: "SpecPV: Improving Self-Speculative Decoding for Long-Context
Generation via Partial Verification" (paperlayer.ai summary of arXiv
2512.02337v2):

* Sec. 3.3 "Rectified with Full Verification": tokens accepted by partial
  verification are only partially verified; periodically a full verification
  re-checks them, with those tokens prepended to the new candidates, over the
  full KV, and the partial cache is rebuilt.  Partial verification starts
  after a full verification has set up its cache; overflowing the partial
  cache's buffer triggers the full verification.
* App. C "Ablation Study": the buffer is sized as one verification step's
  tokens plus 20; App. D "Generation Settings": buffer size 20.

Readings (listed in the design notes):

* The buffer holds the current step's candidates plus the partially verified
  tokens, capacity n_nodes + buffer_size.  A step is run as a full
  (rectifying) verification when more than buffer_size partially verified
  tokens are waiting, i.e. when the next step's candidates would not fit.
* The rectifying tree is the partially verified tokens, oldest first, as a
  chain, followed by the current root (the last emitted token, whose K/V is
  not in the cache) and the new draft tree under it.  Its node 0 is the first
  partially verified token: it was emitted by the last full verification
  (its bonus token), so it is certain and plays the root's role.  Every later
  chain token must again match the target's greedy choice at its parent.
* The rectifying step attends to the fully verified prefix only (full mode)
  and commits at the fully verified length, replacing the partially verified
  rows; afterwards the whole new prefix counts as fully verified.
"""

from __future__ import annotations

import numpy as np

from .tree_verify import OracleInputError

__all__ = ["needs_rectification", "rectify_tree", "first_chain_mismatch"]


def needs_rectification(n_partial: int, buffer_size: int) -> bool:
    """True when the waiting partially verified tokens exceed the buffer
    (App. C / App. D: capacity = step tokens + buffer_size)."""
    if n_partial < 0 or buffer_size < 0:
        raise OracleInputError("negative buffer counts")
    return n_partial > buffer_size


def rectify_tree(buffer_tokens, root_token: int, parents, draft_tokens):
    """Tree of a rectifying full verification (SpecPV Sec. 3.3).

    buffer_tokens: the L >= 1 partially verified tokens, oldest first (the
      first is the last full verification's bonus token).
    root_token: the current root (last emitted token).
    parents, draft_tokens: the new draft tree, node 0 = the current root.
    Returns (parents_out, tokens_out) with L + len(parents) nodes: a chain
    0 <- 1 <- ... <- L (node L = current root) and the draft tree's node j >= 1
    at L + j with parent L + parents[j].  tokens_out[i] is the token of node
    i (entry 0 is not compared by acceptance).
    """
    buf = [int(x) for x in buffer_tokens]
    par = [int(x) for x in parents]
    if not buf:
        raise OracleInputError("a rectifying tree needs at least one buffered token")
    if not par or par[0] != -1 or any(not 0 <= par[j] < j for j in range(1, len(par))):
        raise OracleInputError("draft tree is not topologically ordered")
    ln = len(buf)
    parents_out = [-1] + list(range(0, ln))            # chain nodes 1..L
    tokens_out = buf + [int(root_token)]
    for j in range(1, len(par)):
        parents_out.append(ln + par[j])
        tokens_out.append(int(draft_tokens[j]))
    return np.asarray(parents_out, dtype=np.int32), np.asarray(tokens_out, dtype=np.int32)


def first_chain_mismatch(chain_tokens, greedy_next) -> int:
    """Number of chain tokens after the first that survive re-verification:
    token k (k >= 1) survives iff every token before it survived and it
    equals the target's greedy choice after token k-1 (greedy_next[k-1])."""
    n = 0
    for k in range(1, len(chain_tokens)):
        if int(chain_tokens[k]) != int(greedy_next[k - 1]):
            break
        n += 1
    return n
