"""Reuse-or-restore bookkeeping of the AKV server, as a plain model.  (Oracle: test
infrastructure only.)

[P1] "AKV serving system" (§4.2, App. A.1.2, Fig. 8) and its request-flow diagram;
[P2] §3.4 / Fig. 5 and the serving-flow section.  What the pages fix:
  * KV may be shared between requests only where the token history AND the cache-op
    history agree; a drop node records where and which entries were removed, a repos
    opens a branch whose keys sit at new positions (a new position version);
  * a resident row at the position the request needs is copied unchanged; a row of the
    same history at another position is converted by rotating the key;
  * physical storage is released only when no running computation or restore uses
    it; dropped entries are evicted before those of finished requests; an evicted
    entry keeps its place in the tree, so what was built after it stays reachable;
    each position version is evicted on its own;
  * a state whose KV is gone is rebuilt with one segment-batch prefill.

This model has no tree: every stored row is keyed by the full canonical history up to
and including its token (a tuple of items) plus its position, and every query is
answered by scanning plain dictionaries.

Readings where the pages leave a step open (the library implements the same ones):
  C1 Canonical history.  Items are ('t', token id) per appended token, ('d', ranges)
     for the logical indices a boundary actually removes (drops of tokens no longer
     active are no-ops, drops at one boundary are merged), and ('r',) for a repos
     that changes a position or the next position (a repos that changes nothing is
     not an event).
  C2 "Finished request" entries are the final states of completed requests whose
     history is not a strict prefix of another completed request's history (the
     latest round of each conversation).  A version (history key, position) is held
     if such a final state holds that token at that position; every other unlocked
     version counts as dropped and is evicted first.  Within a class the least
     recently used goes first (one clock tick per call), then the lower slot.
  C3 Restore start.  Tokens from s on are recomputed, s being the largest index in
     [0, T] such that every key that a query at or after s sees, and every token of
     the final state below s, has a resident version.  s = T means nothing is
     recomputed.
  C4 Preferred version per token: the one at the needed position (the final
     position for tokens of the final state, else the append position), else the
     most recently used, then the lowest position.
  C5 Locks: a slot handed out by match(lock=True) or alloc is locked once per hand-
     out; unlock releases one lock; an allocated slot that never received a version
     returns to the free list when its last lock goes.
"""
from __future__ import annotations

from .opseq import APPEND, DROP, REPOS
from .replay import NEVER, replay_tokens


class CacheError(ValueError):
    pass


def _ranges(idx):
    out = []
    for j in sorted(idx):
        if out and out[-1][1] == j:
            out[-1][1] = j + 1
        else:
            out.append([j, j + 1])
    return tuple((a, b) for a, b in out)


def history(tok, ops):
    """Canonical item list (C1) and the replay facts the model needs.

    Returns dict(items, tok_item (index of each token's item), tok_pos, tok_drop,
    final (active tokens ascending), final_pos, p_next)."""
    tok = [int(x) for x in tok]
    T = len(tok)
    items, tok_item = [], []
    active, pos = [], {}
    p_next = t = 0
    tok_pos, tok_drop = [0] * T, [NEVER] * T
    pending = set()

    def flush():
        if pending:
            items.append(("d", _ranges(pending)))
            pending.clear()

    for op in ops:
        kind = op[0]
        if kind == APPEND:
            if op[1] < 0:
                raise CacheError("negative append")
            if op[1] > 0:               # an empty append is not a boundary
                flush()
            for _ in range(op[1]):
                if t >= T:
                    raise CacheError("ops append more tokens than given")
                tok_pos[t] = pos[t] = p_next
                p_next += 1
                active.append(t)
                tok_item.append(len(items))
                items.append(("t", tok[t]))
                t += 1
        elif kind == DROP:
            a, b = op[1], op[2]
            if a < 0 or b < a or b > t:
                raise CacheError("drop range not yet appended")
            gone = [j for j in active if a <= j < b]
            for j in gone:
                tok_drop[j] = t
                del pos[j]
            active = [j for j in active if not a <= j < b]
            pending.update(gone)
        elif kind == REPOS:
            if p_next != len(active) or any(pos[j] != r for r, j in enumerate(active)):
                flush()
                for r, j in enumerate(active):
                    pos[j] = r
                p_next = len(active)
                items.append(("r",))
        else:
            raise CacheError("unknown op kind")
    flush()
    if t != T:
        raise CacheError("ops append fewer tokens than given")
    return dict(items=tuple(items), tok_item=tok_item, tok_pos=tok_pos, tok_drop=tok_drop,
                final=list(active), final_pos=[pos[j] for j in active], p_next=p_next)


def token_keys(h):
    """History key of every token: the item tuple up to and including its append."""
    return [h["items"][:k + 1] for k in h["tok_item"]]


def restore_start(tok_ops_visible, final, resident):
    """C3 by brute force: tok_ops_visible[i] = keys token i attends to (itself
    included); final = final active tokens; resident[j] = token j has a version."""
    T = len(tok_ops_visible)
    best = 0
    for s in range(T + 1):
        need = {j for j in final if j < s}
        for i in range(s, T):
            need.update(j for j in tok_ops_visible[i] if j < s)
        if all(resident[j] for j in need):
            best = s
    return best


class CacheModel:
    """Slots 0..n_slots-1 of a KV pool and the rows they hold."""

    def __init__(self, n_slots):
        if n_slots < 1:
            raise CacheError("n_slots must be positive")
        self.n_slots = n_slots
        self.free = set(range(n_slots))
        self.lock = [0] * n_slots
        self.row = [None] * n_slots          # (key, pos) held by the slot, or None
        self.last = [0] * n_slots            # clock of the last touch
        self.by_row = {}                     # (key, pos) -> slot
        self.prefixes = set()                # every item prefix ever inserted
        self.marks = {}                      # history items -> frozenset of (key, pos)
        self.clock = 0

    # -- C2 -----------------------------------------------------------------
    def _frontier_states(self):
        hs = list(self.marks)
        out = []
        for h in hs:
            if not any(len(g) > len(h) and g[:len(h)] == h for g in hs):
                out.append(self.marks[h])
        return out

    def _evict_order(self):
        held = set().union(*self._frontier_states()) if self.marks else set()
        cand = [s for s in range(self.n_slots) if self.row[s] is not None and self.lock[s] == 0]
        return sorted(cand, key=lambda s: (self.row[s] in held, self.last[s], s))

    # -- API ----------------------------------------------------------------
    def match(self, tok, ops, lock=False):
        """Returns (slot[T], pos[T], info) following C3-C5; slot -1 = no version."""
        self.clock += 1
        h = history(tok, ops)
        keys = token_keys(h)
        T = len(keys)
        n_matched = 0
        while n_matched < T and keys[n_matched] in self.prefixes:
            n_matched += 1
        fpos = dict(zip(h["final"], h["final_pos"]))
        slot, pos = [-1] * T, [-1] * T
        for i, k in enumerate(keys):
            vers = [(p, s) for (kk, p), s in self.by_row.items() if kk == k]
            if not vers:
                continue
            want = fpos.get(i, h["tok_pos"][i])
            exact = [v for v in vers if v[0] == want]
            p, s = exact[0] if exact else min(vers, key=lambda v: (-self.last[v[1]], v[0]))
            slot[i], pos[i] = s, p
        for s in slot:
            if s >= 0:
                self.last[s] = self.clock
                if lock:
                    self.lock[s] += 1
        records, _ = replay_tokens(ops)
        vis = [[j for j, _ in rec[1]] for rec in records]
        s0 = restore_start(vis, h["final"], [s >= 0 for s in slot])
        info = dict(n_tokens=T, n_matched=n_matched, n_resident=sum(s >= 0 for s in slot),
                    restore_from=s0, n_final=len(h["final"]), p_next=h["p_next"])
        return slot, pos, info

    def alloc(self, n):
        self.clock += 1
        if n < 0:
            raise CacheError("negative count")
        order = self._evict_order()
        if n > len(self.free) + len(order):
            raise CacheError("no space: locked rows fill the pool")
        out = sorted(self.free)[:n]
        for s in out:
            self.free.discard(s)
        for s in order[:n - len(out)]:
            del self.by_row[self.row[s]]
            self.row[s] = None
            out.append(s)
        for s in out:
            self.lock[s] = 1
            self.last[s] = self.clock
        return out

    def insert(self, tok, ops, ver_token, ver_pos, ver_slot):
        self.clock += 1
        h = history(tok, ops)
        keys = token_keys(h)
        new = {}
        for i, p, s in zip(ver_token, ver_pos, ver_slot):
            if not 0 <= i < len(keys) or not 0 <= s < self.n_slots or p < 0:
                raise CacheError("version out of range")
            if self.row[s] is not None or self.lock[s] == 0 or s in new.values():
                raise CacheError("slot is not an allocated empty slot")
            r = (keys[i], int(p))
            if r in self.by_row or r in new:
                raise CacheError("version already resident")
            new[r] = s
        for r, s in new.items():
            self.row[s] = r
            self.by_row[r] = s
            self.last[s] = self.clock
        items = h["items"]
        for m in range(1, len(items) + 1):
            self.prefixes.add(items[:m])
        self.marks[items] = frozenset((keys[j], p) for j, p in zip(h["final"], h["final_pos"]))

    def unlock(self, slots):
        count = {}
        for s in slots:
            count[s] = count.get(s, 0) + 1
        for s, c in count.items():
            if not 0 <= s < self.n_slots or self.lock[s] < c:
                raise CacheError("slot is not locked")
        for s in slots:
            self.lock[s] -= 1
            if self.lock[s] == 0 and self.row[s] is None:
                self.free.add(s)

    def stats(self):
        return dict(n_free=len(self.free), n_resident=len(self.by_row),
                    n_locked=sum(1 for x in self.lock if x > 0), n_marks=len(self.marks),
                    n_frontier=len(self._frontier_states()))
