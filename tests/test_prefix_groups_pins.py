"""Pins for shared-prefix detection: a known answer, a second implementation
by a different route (page-id tuples at every depth, no trie), invariants
of the output, and planted mistakes."""

import numpy as np
import pytest

import oracle
from oracle import prefix_groups as opg
from workloads import cascade_layout


def nested_tables(rng, S=40, block_size=16):
    """Block tables with nested shared prefixes: a random tree of page runs
    (each run its own pages), every sequence a random path down it plus
    private pages; context lengths end somewhere in the last page.  Some
    sequences share nothing.  Returns (tables, context_lens)."""
    next_page = [1]

    def run(n):
        r = list(range(next_page[0], next_page[0] + n))
        next_page[0] += n
        return r

    roots = []
    for _ in range(int(rng.integers(2, 5))):
        node = {"pages": run(int(rng.integers(1, 6))), "kids": []}
        for _ in range(int(rng.integers(0, 4))):
            kid = {"pages": run(int(rng.integers(1, 5))), "kids": []}
            for _ in range(int(rng.integers(0, 3))):
                kid["kids"].append({"pages": run(int(rng.integers(1, 4))), "kids": []})
            node["kids"].append(kid)
        roots.append(node)
    rows, ctx = [], []
    for _ in range(S):
        pages = []
        if rng.random() < 0.85:
            node = roots[int(rng.integers(len(roots)))]
            while True:
                pages += node["pages"]
                if not node["kids"] or rng.random() < 0.3:
                    break
                node = node["kids"][int(rng.integers(len(node["kids"])))]
        pages += run(int(rng.integers(0, 4)))
        if not pages:
            pages = run(1)
        rows.append(pages)
        # anywhere in the last page (a prefix as long as the whole context is
        # then possible for sequences without private pages: the oracle must
        # not take it)
        ctx.append((len(pages) - 1) * block_size + int(rng.integers(1, block_size + 1)))
    mb = max(len(r) for r in rows)
    bt = np.full((S, mb), -1, dtype=np.int32)
    for s, r in enumerate(rows):
        bt[s, : len(r)] = r
    return bt, np.array(ctx, dtype=np.int32)


def tuple_route(bt, ctx, block_size, min_group=2, min_pages=1):
    """The same greedy rounds without a trie: at every depth d the remaining
    sequences that reach d are bucketed by their first d page ids; the
    deepest bucket with enough members wins, ties to the one with more
    members, then to the one whose first holder (over all sequences) comes
    first."""
    S = len(ctx)
    dmax = [max(0, (int(L) - 1) // block_size) for L in ctx]
    first_holder = {}
    for s in range(S):
        for d in range(1, dmax[s] + 1):
            first_holder.setdefault(tuple(int(x) for x in bt[s, :d]), s)
    assigned = set()
    order, offsets, prefix = [], [0], []
    while True:
        best = None
        for d in range(max(1, min_pages), max(dmax, default=0) + 1):
            buckets = {}
            for s in range(S):
                if s in assigned or dmax[s] < d:
                    continue
                buckets.setdefault(tuple(int(x) for x in bt[s, :d]), []).append(s)
            for key, mem in buckets.items():
                if len(mem) < max(2, min_group):
                    continue
                cand = (d, len(mem), -first_holder[key])
                if best is None or cand > best[0]:
                    best = (cand, mem, d)
        if best is None:
            break
        _, mem, d = best
        assigned.update(mem)
        order += mem
        offsets.append(len(order))
        prefix.append(d * block_size)
    rest = [s for s in range(S) if s not in assigned]
    if rest:
        order += rest
        offsets.append(len(order))
        prefix.append(0)
    return np.array(order), np.array(offsets), np.array(prefix)


def pin_known_groups():
    """16 groups x 8 members over a 128-token prefix, shuffled: the groups
    come back with their prefix, nothing else is grouped."""
    lay = cascade_layout(num_groups=16, seqs_per_group=8, prefix_len=128, suffix_lo=1, suffix_hi=40, num_q_heads=8,
                         num_kv_heads=2, head_dim=64, dtype="f32", seed=3)
    perm = np.random.default_rng(5).permutation(lay.num_seqs)
    bt, ctx = lay.block_tables[perm], lay.context_lens[perm]
    order, offs, pref = oracle.detect_prefix_groups(bt, ctx, 16)
    fails = []
    if len(pref) != 16 or not (pref == 128).all():
        fails.append(f"groups {len(pref)}, prefixes {sorted(set(pref.tolist()))}")
    truth = {}
    for g in range(16):
        for s in range(lay.group_seq_offsets[g], lay.group_seq_offsets[g + 1]):
            truth[s] = g
    for g in range(len(pref)):
        orig = {truth[int(perm[i])] for i in order[offs[g] : offs[g + 1]]}
        if len(orig) != 1 or offs[g + 1] - offs[g] != 8:
            fails.append(f"group {g} mixes true groups {orig}")
    return fails


def pin_longest_first():
    """Worked by hand: sequences 0 and 1 share 100 pages; all 26 sequences
    share the first 10 of them.  The longest shared prefix is the pair's:
    group {0, 1} at 100 pages first, then the other 24 at 10 pages.  (Ranked
    by pages saved, d * (n - 1), the 26 at 10 pages would win: 250 > 99.)"""
    bs = 16
    common = list(range(1, 11))
    deep = common + list(range(11, 101))
    rows, nxt = [], 1000
    for s in range(26):
        pages = (deep if s < 2 else common) + [nxt]
        nxt += 1
        rows.append(pages)
    mb = max(len(r) for r in rows)
    bt = np.full((26, mb), -1, dtype=np.int32)
    for s, r in enumerate(rows):
        bt[s, : len(r)] = r
    ctx = np.array([len(r) * bs - 3 for r in rows], dtype=np.int32)
    order, offs, pref = oracle.detect_prefix_groups(bt, ctx, bs)
    fails = []
    if order.tolist() != list(range(26)):
        fails.append(f"order {order.tolist()}")
    if offs.tolist() != [0, 2, 26]:
        fails.append(f"offsets {offs.tolist()}")
    if pref.tolist() != [100 * bs, 10 * bs]:
        fails.append(f"prefix lengths {pref.tolist()}")
    # min_group 3: the pair no longer qualifies, all 26 share 10 pages
    order, offs, pref = oracle.detect_prefix_groups(bt, ctx, bs, 3)
    if offs.tolist() != [0, 26] or pref.tolist() != [10 * bs]:
        fails.append(f"min_group 3: offsets {offs.tolist()} prefixes {pref.tolist()}")
    # ties: equal depth, more members first; equal members, table order
    bt2 = np.array([[7, 1], [5, 2], [5, 3], [7, 4], [5, 6], [9, 8], [9, 10]], dtype=np.int32)
    ctx2 = np.full(7, 2 * bs, dtype=np.int32)
    order, offs, pref = oracle.detect_prefix_groups(bt2, ctx2, bs)
    if order.tolist() != [1, 2, 4, 0, 3, 5, 6] or offs.tolist() != [0, 3, 5, 7] or pref.tolist() != [bs] * 3:
        fails.append(f"ties: {order.tolist()} {offs.tolist()} {pref.tolist()}")
    return fails


def pin_tuple_route():
    fails = []
    for seed in range(12):
        rng = np.random.default_rng(seed)
        bt, ctx = nested_tables(rng)
        for mg, mp in ((2, 1), (3, 1), (2, 2)):
            got = oracle.detect_prefix_groups(bt, ctx, 16, mg, mp)
            want = tuple_route(bt, ctx, 16, mg, mp)
            if not all(np.array_equal(a, b) for a, b in zip(got, want)):
                fails.append(f"seed {seed} min_group {mg} min_pages {mp}")
    return fails


def pin_invariants():
    fails = []
    for seed in range(12, 24):
        rng = np.random.default_rng(seed)
        bt, ctx = nested_tables(rng, S=60)
        order, offs, pref = oracle.detect_prefix_groups(bt, ctx, 16)
        if sorted(order.tolist()) != list(range(len(ctx))):
            fails.append(f"seed {seed}: order is not a permutation")
        depths = []
        for g in range(len(pref)):
            mem = order[offs[g] : offs[g + 1]]
            P = int(pref[g]) // 16
            if P and not (bt[mem, :P] == bt[mem[0], :P]).all():
                fails.append(f"seed {seed} group {g}: members do not share the prefix pages")
            if not (ctx[mem] > pref[g]).all():
                fails.append(f"seed {seed} group {g}: prefix not shorter than a member")
            if P:
                depths.append(P)
        if any(b > a for a, b in zip(depths, depths[1:])):
            fails.append(f"seed {seed}: prefix depths increase from one group to the next")
        if (pref[:-1] == 0).any():
            fails.append(f"seed {seed}: a prefix-0 group before the last")
    # the output is a valid cascade grouping for the table checker
    rng = np.random.default_rng(99)
    bt, ctx = nested_tables(rng, S=50)
    order, offs, pref = oracle.detect_prefix_groups(bt, ctx, 16)
    probs = oracle.check_block_tables(bt[order], ctx[order], int(bt.max()) + 1, 16, offs, pref)
    # pages shared outside a declared prefix (e.g. two sequences sharing one
    # page that no group was formed for) are not the detector's concern;
    # everything about the groups themselves must hold
    probs = [p for p in probs if "also used elsewhere" not in p]
    if probs:
        fails.append(f"table checker: {probs[:3]}")
    return fails


ALL_PINS = [pin_known_groups, pin_longest_first, pin_tuple_route, pin_invariants]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    fails = pin()
    assert not fails, fails[:5]


PLANTED = {
    "prefix may reach the context length": ("_max_depth", lambda L, bs: max(0, int(L) // bs)),
    "ranked by pages saved": ("_rank", lambda depth, count, node: (depth * (count - 1), depth, -node)),
    "ties to fewer members": ("_rank", lambda depth, count, node: (depth, -count, -node)),
    "ties to the later node": ("_rank", lambda depth, count, node: (depth, count, node)),
    "members not removed": ("_remove", lambda count, path: None),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, bad = PLANTED[name]
    monkeypatch.setattr(opg, attr, bad)

    def noticed(pin):
        try:
            return bool(pin())
        except Exception:  # a broken oracle that fails outright is noticed too
            return True

    assert any(noticed(p) for p in ALL_PINS), f"no pin noticed: {name}"
