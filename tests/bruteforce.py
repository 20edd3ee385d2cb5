"""Independent brute-force simulator for tiny traces (no sort keys).

It keeps an explicit recency list of the C LRU slots, least recently used
first.  A step takes the victims from the front of the list, skipping slots
the step referenced; afterwards every slot the step referenced or filled moves
to the back in ascending slot order (they all share the newest stamp, so the
slot number breaks the tie).  This is a different formulation from the
oracle's "sort the unreferenced slots by (last_use, slot)"; agreement of the
two on every tiny trace pins the oracle's victim order.

Resident-window rows (last R positions, ring slot C + p mod R) and padding
(-1) follow the same readings as the oracle.  Plain Python, tiny inputs only.
"""
from __future__ import annotations


class BruteStream:
    def __init__(self, C: int, R: int):
        self.C, self.R = C, R
        self.recency = list(range(C))          # front = least recently used
        self.where = {}                        # position -> slot
        self.held = [None] * C                 # slot -> position

    def resolve(self, sel, ctx):
        for p in sel:
            if p < -1 or p >= ctx:
                return None
        pos = [p for p in sel if p >= 0]
        if len(set(pos)) != len(pos) or len(sel) > self.C:
            return None
        out = [None] * len(sel)
        touched = set()
        misses = []
        for i, p in enumerate(sel):
            if p == -1:
                out[i] = -1
            elif self.R > 0 and p >= ctx - self.R:
                out[i] = self.C + p % self.R
            elif p in self.where:
                out[i] = self.where[p]
                touched.add(self.where[p])
            else:
                misses.append(i)
        candidates = [s for s in self.recency if s not in touched]
        log = []
        for j, i in enumerate(misses):
            s = candidates[j]
            old = self.held[s]
            log.append((s, -1 if old is None else old))
            if old is not None:
                del self.where[old]
            self.where[sel[i]] = s
            self.held[s] = sel[i]
            touched.add(s)
            out[i] = s
        self.recency = [s for s in self.recency if s not in touched] + sorted(touched)
        return out, log

    def resolve_multi(self, queries, ctx):
        """Several queries' selections in one step, entry by entry: the first
        entry of a position classifies it (resident, hit, or a new miss in
        the order first met); later entries of the same position reuse its
        slot.  Victims as in `resolve`.  Returns (out per query, log,
        (n_pad, n_res, n_hit, n_miss)) over the Q*k entries, with each
        distinct position counted once and the rest counted as padding."""
        width = sum(len(q) for q in queries)
        for q in queries:
            for p in q:
                if p < -1 or p >= ctx:
                    return None
        if width > self.C:
            return None
        slot_of, touched, pending = {}, set(), []
        n_res = n_hit = 0
        for q in queries:
            for p in q:
                if p == -1 or p in slot_of or p in pending:
                    continue
                if self.R > 0 and p >= ctx - self.R:
                    slot_of[p] = self.C + p % self.R
                    n_res += 1
                elif p in self.where:
                    slot_of[p] = self.where[p]
                    touched.add(self.where[p])
                    n_hit += 1
                else:
                    pending.append(p)
        candidates = [s for s in self.recency if s not in touched]
        log = []
        for j, p in enumerate(pending):
            s = candidates[j]
            old = self.held[s]
            log.append((s, -1 if old is None else old))
            if old is not None:
                del self.where[old]
            self.where[p] = s
            self.held[s] = p
            touched.add(s)
            slot_of[p] = s
        self.recency = [s for s in self.recency if s not in touched] + sorted(touched)
        out = [[-1 if p == -1 else slot_of[p] for p in q] for q in queries]
        n_distinct = len(slot_of)
        return out, log, (width - n_distinct, n_res, n_hit, len(pending))

    def slot2pos(self):
        return [-1 if p is None else p for p in self.held]


def brute_topk(scores, ctx: int, k: int):
    """Top-k by exhaustive search over position subsets (tiny ctx only), as a
    different formulation from the oracle's sort: the chosen set has the
    largest score vector (sorted descending, compared lexicographically),
    and among sets with that vector the smallest sorted position list.
    Returns ascending positions padded with -1 to k."""
    import itertools
    m = min(k, ctx)
    best = None
    for subset in itertools.combinations(range(ctx), m):
        key = (tuple(sorted((float(scores[i]) for i in subset), reverse=True)),
               tuple(-i for i in subset))
        if best is None or key > best[0]:
            best = (key, subset)
    chosen = list(best[1]) if best else []
    return chosen + [-1] * (k - len(chosen))
