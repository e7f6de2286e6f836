"""Operational semantics of append / drop / repos.  (Oracle: test infrastructure only.)

[P1] "three cache operations" (§3.3) and [P2] §1:
  * append: a new token's KV joins the active cache, C <- [C; C_{t+1}]; the
    new token is computed against the current active cache like ordinary
    inference;
  * drop(P): C <- C \\ {C_i : i in P}; the remaining entries keep their
    values, positions and logical tokens, nothing is recomputed;
  * repos: the remaining keys get positions 0..r-1 in logical order and the
    next append uses position r.
[P1] "three cache operations" (§3.4): from an empty cache, the op sequence
determines the cache state.

Two replays of the same semantics:
  replay_tokens  -- one token at a time, returning every query's visible
                    (token, position) list: the literal definition, for tiny
                    inputs only;
  replay_events  -- the same walk recording only events (append positions,
                    the boundary at which each token is dropped, the active
                    list after each repos), for inputs of any size.
"""
from __future__ import annotations

import numpy as np

from .opseq import APPEND, DROP, REPOS

NEVER = np.iinfo(np.int32).max


def replay_tokens(ops):
    """Return (records, final) where records[i] = (pos_i, [(j, pos_j), ...]) lists
    the keys token i attends to (itself included) with their positions at
    that moment, and final = (active tokens, their positions, p_next)."""
    active = []
    pos = {}
    p_next = 0
    t = 0
    records = []
    for op in ops:
        if op[0] == APPEND:
            for _ in range(op[1]):
                i = t
                t += 1
                pos[i] = p_next
                p_next += 1
                active.append(i)
                records.append((pos[i], [(j, pos[j]) for j in active]))
        elif op[0] == DROP:
            a, b = op[1], op[2]
            if b > t:
                raise ValueError("drop of a token not yet appended")
            active = [j for j in active if not (a <= j < b)]
        elif op[0] == REPOS:
            for r, j in enumerate(active):
                pos[j] = r
            p_next = len(active)
        else:
            raise ValueError(op)
    return records, (list(active), [pos[j] for j in active], p_next)


class Events:
    """Result of replay_events.

    tok_pos[i]   position of token i when it was appended
    tok_drop[i]  token index of the boundary at which i was dropped (NEVER if not)
    boundaries   sorted token indices at which a DROP or REPOS op happened
    epochs       list of (tok_begin, tok_end, ver_src) for every stretch
                 between repos ops that appends at least one token; ver_src is
                 the active list just after the opening repos (empty for the
                 first stretch); version row v of it sits at position v
    final        (active tokens, positions, p_next) after the last op
    visible_pairs  sum over tokens of the number of keys each one attends to
    """

    def __init__(self, T):
        self.T = T
        self.tok_pos = np.zeros(T, np.int64)
        self.tok_drop = np.full(T, NEVER, np.int64)
        self.boundaries = []
        self.epochs = []
        self.final = None
        self.visible_pairs = 0

    def epoch_of_token(self):
        e = np.full(self.T, -1, np.int64)
        for k, (tb, te, _) in enumerate(self.epochs):
            e[tb:te] = k
        return e


def replay_events(ops):
    T = sum(op[1] for op in ops if op[0] == APPEND)
    ev = Events(T)
    active = []                 # ascending logical indices
    pos = {}                    # current position of active tokens
    p_next = 0
    t = 0
    ep_begin, ep_src = 0, []
    bset = set()
    for op in ops:
        if op[0] == APPEND:
            n = op[1]
            a0 = len(active)
            ev.tok_pos[t:t + n] = p_next + np.arange(n)
            for m in range(n):
                pos[t + m] = p_next + m
            # token t+m sees the a0 keys already active plus m+1 of its own
            ev.visible_pairs += n * a0 + n * (n + 1) // 2
            active.extend(range(t, t + n))
            t += n
            p_next += n
        elif op[0] == DROP:
            a, b = op[1], op[2]
            if b > t:
                raise ValueError("drop of a token not yet appended")
            keep = []
            for j in active:
                if a <= j < b:
                    ev.tok_drop[j] = t
                    del pos[j]
                else:
                    keep.append(j)
            active = keep
            bset.add(t)
        elif op[0] == REPOS:
            if t > ep_begin:
                ev.epochs.append((ep_begin, t, np.asarray(ep_src, np.int64)))
            for r, j in enumerate(active):
                pos[j] = r
            p_next = len(active)
            ep_begin, ep_src = t, list(active)
            bset.add(t)
        else:
            raise ValueError(op)
    if t > ep_begin:
        ev.epochs.append((ep_begin, t, np.asarray(ep_src, np.int64)))
    ev.boundaries = sorted(bset)
    ev.final = (np.asarray(active, np.int64), np.asarray([pos[j] for j in active], np.int64), p_next)
    return ev
