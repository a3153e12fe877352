"""Independent small models used to pin the oracle (pure Python, tiny inputs).

Nothing here is imported by the oracle or by the GPU library.  Each model
states one property of the method in a different way from the oracle's own
code, so that a slip in the oracle (a wrong sort key, a transposed
assignment, a dropped refresh) disagrees with at least one of them.
"""

from __future__ import annotations

import itertools
from collections import OrderedDict


class TextbookLRU:
    """A capacity-C LRU cache of tokens kept in numbered slots.

    Hit: the token becomes most recently used.  Miss: if a slot is free the
    lowest-numbered free slot is used, otherwise the least recently used token
    is evicted and its slot reused.  This is the classic policy the pages name
    ("copy one row into the LRU slot"), for one access at a time.
    """

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.order: OrderedDict[int, int] = OrderedDict()  # token -> slot, LRU first

    def access(self, token: int):
        if token in self.order:
            self.order.move_to_end(token)
            return "hit", self.order[token], None
        if len(self.order) < self.capacity:
            used = set(self.order.values())
            slot = min(q for q in range(self.capacity) if q not in used)
            evicted = None
        else:
            evicted, slot = self.order.popitem(last=False)
        self.order[token] = slot
        return "miss", slot, evicted


def declarative_solutions(hit_slots: set, misses: list, slots: list, stamp_of: dict):
    """Every assignment of ``misses`` to slots that satisfies the resolver's
    declarative conditions, found by exhaustive enumeration of all partial
    injective maps from misses to non-hit slots.

    Conditions (pre-call state; ``slots`` = the usable slots):
      * assigned slots are distinct and none of them is a hit slot;
      * as many misses as possible get a slot: min(#misses, #non-hit slots);
      * a miss never overflows while a larger miss gets a slot;
      * no unassigned non-hit slot is less recently used than an assigned one,
        recency ordered by (stamp, slot);
      * a smaller miss never gets a more recently used slot than a larger one.
    Returns a list of dicts token -> slot (overflowing tokens are absent).
    """
    free = [q for q in slots if q not in hit_slots]
    key = lambda q: (stamp_of[q], q)
    sols = []
    for k in range(len(misses) + 1):
        for subset in itertools.combinations(misses, k):
            for chosen in itertools.permutations(free, k):
                assign = dict(zip(subset, chosen))
                if k != min(len(misses), len(free)):
                    continue
                if any(m not in assign and any(m < s for s in assign) for m in misses):
                    continue
                rest = [q for q in free if q not in chosen]
                if rest and chosen and max(key(q) for q in chosen) > min(key(q) for q in rest):
                    continue
                if any(key(assign[a]) > key(assign[b])
                       for a, b in itertools.permutations(assign, 2) if a < b):
                    continue
                sols.append(assign)
    return sols


def sequential_resolve(tokens, ctx, page, bt, hbt, hot_blocks, tok, stp, stamp,
                       pool_blocks=None, host_blocks=None):
    """The resolver restated as a sequential process over one list.

    Classify each entry; refresh every hit; then walk the distinct misses from
    the smallest token up and hand each the least recently used slot that has
    not been touched in this call.  Returns (rows, new_tok, new_stp, copies)
    with copies = [(host_row, pool_row)].
    """
    C = len(tok)
    pool_blocks = pool_blocks if pool_blocks is not None else 1 << 40
    host_blocks = host_blocks if host_blocks is not None else 1 << 40
    tok, stp = list(tok), list(stp)
    usable = [0 <= hot_blocks[q // page] < pool_blocks for q in range(C)]

    def hot_row(q):
        return hot_blocks[q // page] * page + q % page

    def cls(t):
        if t == -1:
            return "pad", -1
        if t < 0 or t >= ctx or t // page >= len(bt):
            return "invalid", -3
        b = bt[t // page]
        if b >= 0:
            return ("resident", b * page + t % page) if b < pool_blocks else ("invalid", -3)
        return "nonres", None

    touched = [False] * C
    result = {}
    nonres = sorted({t for t in tokens if cls(t)[0] == "nonres"})
    pending = []
    for t in nonres:
        q = next((q for q in range(C) if usable[q] and tok[q] == t), None)
        if q is not None:
            touched[q] = True
            stp[q] = stamp
            result[t] = hot_row(q)
        elif 0 <= hbt[t // page] < host_blocks:
            pending.append(t)
        else:
            result[t] = -3
    # hits are taken first; then misses in ascending order, one LRU slot each
    copies = []
    old_stp = list(stp)
    for t in pending:
        cands = [q for q in range(C) if usable[q] and not touched[q]]
        if not cands:
            result[t] = -2
            continue
        q = min(cands, key=lambda q: (old_stp[q], q))
        touched[q] = True
        tok[q] = t
        stp[q] = stamp
        copies.append((hbt[t // page] * page + t % page, hot_row(q)))
        result[t] = hot_row(q)
    rows = []
    for t in tokens:
        c, r = cls(t)
        rows.append(result[t] if c == "nonres" else r)
    return rows, tok, stp, copies
