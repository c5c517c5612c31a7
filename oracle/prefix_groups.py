"""Shared-prefix detection for cascade decode: group a batch's sequences by
the longest prefixes their block tables share.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes
----------------
The Tokasaurus page ("dynamic prefix identification and exploration")
detects shared prefixes in an engine where sequences start and finish all
the time by running a greedy depth-first search before each forward pass,
one that repeatedly finds the longest shared prefix it can.  Blocks of a
shared prefix are stored once and named by every table that shares it (the
shared blocks of the SwiftLLM page, section 3.1), so two sequences share
their first d pages exactly when their first d table entries are equal.

Readings (the page gives no more than that sentence):

* the search runs over a trie of the tables' page ids: node (d, path) holds
  the sequences whose first d entries are that path; a sequence reaches
  depth d only if d * block_size < its context length (a cascade prefix
  must be shorter than every member's context);
* "the longest shared prefix" is taken literally: each round takes the
  deepest node that still holds at least ``min_group`` (at least 2)
  sequences not yet grouped and is at least ``min_pages`` pages deep (ties:
  the node with more such sequences, then the node created first when the
  tables are inserted sequence by sequence, i.e. table order), makes those
  sequences a group with prefix d * block_size, and removes them from every
  node; rounds stop when no node qualifies;
* the sequences left over form one last group with prefix 0;
* the output orders sequences group by group (groups in the order they were
  found, members by their original index), which is the contiguous layout
  ``pa_prefix_cascade`` takes.

Pins (tests/test_prefix_groups_pins.py): the known groups of a shuffled
shared-prefix batch are recovered; a hand-worked nested batch (two
sequences sharing 100 pages inside 26 sharing 10) gives the deep pair
first, where ranking by pages saved would take all 26 at 10 pages; a second
implementation that groups by page-id tuples at every depth (no trie)
agrees on random nested layouts; every group's members share their first
prefix pages and are longer than the prefix; prefix depths never increase
from one group to the next; planted mistakes (prefix allowed to reach the
context length, ranking by pages saved, ties broken the other way, members
not removed) are each caught.
"""

from __future__ import annotations

import numpy as np


def _max_depth(L: int, block_size: int) -> int:
    """Deepest prefix (in pages) sequence of length L can share: d * BS < L."""
    return max(0, (int(L) - 1) // block_size)


def _rank(depth: int, count: int, node: int):
    """Order of candidates: deeper, then more ungrouped members, then created
    first (table order)."""
    return (depth, count, -node)


def _remove(count, path):
    """A grouped sequence no longer counts at any node on its path."""
    for n in path:
        count[n] -= 1


def detect_prefix_groups(block_tables, context_lens, block_size: int, min_group: int = 2, min_pages: int = 1):
    """Returns (order [S], group_offsets [NG+1], prefix_lens [NG]) as int32
    arrays: positions group_offsets[g] .. group_offsets[g+1]-1 of ``order``
    are the original indices of group g's members, which share their first
    prefix_lens[g] / block_size table entries."""
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = len(ctx)
    # trie: node 0 is the root; children keyed by (parent, page id); node ids
    # in creation order (sequence by sequence, depth by depth)
    child = {}
    depth = [0]
    members = [[]]
    paths = []
    for s in range(S):
        dmax = _max_depth(ctx[s], block_size)
        node = 0
        path = []
        for d in range(dmax):
            key = (node, int(bt[s, d]))
            if key not in child:
                child[key] = len(depth)
                depth.append(d + 1)
                members.append([])
            node = child[key]
            members[node].append(s)
            path.append(node)
        paths.append(path)
    count = [len(m) for m in members]
    assigned = np.zeros(S, dtype=bool)
    order, offsets, prefix = [], [0], []
    while True:
        best, best_key = -1, None
        for n in range(1, len(depth)):
            if count[n] < max(2, min_group) or depth[n] < min_pages:
                continue
            key = _rank(depth[n], count[n], n)
            if best_key is None or key > best_key:
                best, best_key = n, key
        if best < 0:
            break
        group = [s for s in members[best] if not assigned[s]]
        if not group:  # a node's count always equals its unassigned members
            raise RuntimeError("prefix detection: chosen node has no remaining members")
        for s in group:
            assigned[s] = True
            _remove(count, paths[s])
        order.extend(group)
        offsets.append(len(order))
        prefix.append(depth[best] * block_size)
    rest = [s for s in range(S) if not assigned[s]]
    if rest:
        order.extend(rest)
        offsets.append(len(order))
        prefix.append(0)
    return (np.array(order, dtype=np.int32), np.array(offsets, dtype=np.int32),
            np.array(prefix, dtype=np.int32))
