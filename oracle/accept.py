"""Greedy acceptance along a verified draft tree and the KV commit of the accepted path
(test infrastructure only).

The pages decode at batch one with greedy sampling: the draft proposes a 16-token tree, one
verify step of the target model scores every node, and the accepted tokens are kept
(alphasignal.ai, "Draft and verify share one graph"; orcarouter.ai, "what the number is and
isn't": 16 verified, 6.6 accepted on average).  They print no rule; the plain greedy rule is
taken: from the root, follow the child whose drafted token equals the target's greedy token
at the current node (the lowest-index such child), until no child matches; the target's token
at the last accepted node is the bonus token.  Node i's K/V row sits at slot ctx + i during
verification; committing moves the accepted nodes' rows to positions ctx + depth, in order.
"""
from __future__ import annotations

import numpy as np


def tree_accept(parent, draft, target):
    """parent[T] (parent[0] = -1, parent[i] < i), draft[T] (token of each node; node 0 is the
    root, the last accepted token), target[T] (the target model's greedy token after each node).
    Returns (path, bonus): the accepted nodes root-first, and the token after the last one."""
    parent = [int(p) for p in parent]
    T = len(parent)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(1, T):                       # children in index order
            if parent[c] == cur and int(draft[c]) == int(target[cur]):
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return path, int(target[cur])


def kv_commit(k_cache, v_cache, ctx: int, path):
    """Copies of the caches with row ctx + path[j] moved to row ctx + j for every j (the other
    rows unchanged)."""
    k, v = k_cache.copy(), v_cache.copy()
    src = [ctx + int(p) for p in path]
    k[ctx:ctx + len(path)] = k_cache[src]
    v[ctx:ctx + len(path)] = v_cache[src]
    return k, v
