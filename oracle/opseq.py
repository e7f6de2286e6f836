"""Message-level cache ops -> canonical op list.  (Oracle: test infrastructure only.)

[P1] "AKV serving system" (§4, Fig. 6): the agent sends the whole message
list (each message is an implicit append) plus optional `drop` and
`reposition` fields in operate-after form: drop {k: [j...]} removes the KV of
messages j once message k has been appended; reposition [k] renumbers the
remaining keys after message k.  At one boundary drop is applied before repos.
[P2] §4 restates this for the pinned README (drop_message / reposition,
0-based message indices, drop first, every message still sent).

Canonical form chosen here (a reading; the pages do not fix it):
  for k = 0..M-1:  APPEND(n_k);
                   one DROP(a, b) per distinct non-empty target j of drop[k],
                   ascending j, with [a, b) the token range of message j;
                   REPOS once if k occurs in reposition.
Invalid: k or j outside [0, M), or j > k (dropping a message not yet sent).
Dropping an already dropped message is allowed (set difference: no effect).
"""
from __future__ import annotations

APPEND, DROP, REPOS = 0, 1, 2


class OpSequenceError(ValueError):
    pass


def canonical_ops(msg_len, drop=None, reposition=None):
    """Return a list of tuples (APPEND, n) | (DROP, a, b) | (REPOS,)."""
    msg_len = [int(n) for n in msg_len]
    M = len(msg_len)
    drop = {} if drop is None else drop
    reposition = [] if reposition is None else list(reposition)
    if any(n < 0 for n in msg_len):
        raise OpSequenceError("negative message length")
    starts = [0] * M
    for k in range(1, M):
        starts[k] = starts[k - 1] + msg_len[k - 1]
    targets = {}
    for k, js in drop.items():
        k = int(k)
        if not 0 <= k < M:
            raise OpSequenceError(f"drop after message {k}: no such message")
        for j in js:
            j = int(j)
            if not 0 <= j < M:
                raise OpSequenceError(f"drop target {j}: no such message")
            if j > k:
                raise OpSequenceError(f"drop target {j} comes after message {k}")
            targets.setdefault(k, set()).add(j)
    rset = set()
    for k in reposition:
        k = int(k)
        if not 0 <= k < M:
            raise OpSequenceError(f"reposition after message {k}: no such message")
        rset.add(k)
    ops = []
    for k in range(M):
        ops.append((APPEND, msg_len[k]))
        for j in sorted(targets.get(k, ())):
            if msg_len[j] > 0:
                ops.append((DROP, starts[j], starts[j] + msg_len[j]))
        if k in rset:
            ops.append((REPOS,))
    return ops
