"""Pins for the cache-index model in oracle/cache_index.py.  CPU only.

Each check ties the model to something outside it:
  * the history-dependence counter-example of the pages (review §3.4 / Fig. 5,
    explainer Fig. 5): the three op orders and which rows they may share;
  * the definition of what a row's KV depends on: in any attention stack, token i's
    keys and values are a function of its token, its position and the (KV, position)
    pairs it attended to, so two rows are interchangeable when that recursive
    description is equal.  Histories with equal keys must have equal descriptions;
  * the eviction order the review states (dropped before finished, never a row in
    use, emptied rows keep what follows reachable), on hand-built pools;
  * the restore start on a hand-worked case and against the visibility rule.
"""
import random

import pytest

import oracle
from oracle import APPEND, DROP, REPOS
from oracle.cache_index import CacheError, CacheModel, history, restore_start, token_keys


def _ident(tok, ops):
    """Recursive description of every token's KV: (token id, position, frozenset of
    (description, position) over the other keys it attended to)."""
    records, _ = oracle.replay_tokens(ops)
    ids = []
    for i, (p, vis) in enumerate(records):
        ids.append((tok[i], p, frozenset((ids[j], pj) for j, pj in vis if j != i)))
    return ids


def _fig5(a=3, b=4, c=5):
    A, B, C = list(range(100, 100 + a)), list(range(200, 200 + b)), list(range(300, 300 + c))
    return {
        1: (A + B + C, oracle.canonical_ops([a, b, c], {2: [0]})),   # read A,B; compute C; drop A
        2: (A + B + C, oracle.canonical_ops([a, b, c], {1: [0]})),   # read A,B; drop A; compute C
        3: (B + C, oracle.canonical_ops([b, c])),                    # start at B; append C
    }


def _insert_all(m, tok, ops):
    """Store every token at its append position (what a full prefill computes)."""
    h = history(tok, ops)
    slots = m.alloc(len(tok))
    m.insert(tok, ops, list(range(len(tok))), h["tok_pos"], slots)
    m.unlock(slots)
    return slots


# ------------------------------------------------------------------ Fig. 5

def test_fig5_descriptions_follow_the_example():
    a, b, c = 3, 4, 5
    P = _fig5(a, b, c)
    I = {k: _ident(*v) for k, v in P.items()}
    B = {1: I[1][a:a + b], 2: I[2][a:a + b], 3: I[3][:b]}
    C = {1: I[1][a + b:], 2: I[2][a + b:], 3: I[3][b:]}
    assert B[1] == B[2] and B[1] != B[3]
    assert C[1] != C[2] and C[1] != C[3] and C[2] != C[3]


def test_fig5_sharing_in_the_model():
    a, b, c = 3, 4, 5
    P = _fig5(a, b, c)
    m = CacheModel(64)
    _insert_all(m, *P[1])
    slot, pos, info = m.match(*P[2])
    # path 2 shares A and B (same history up to B) but not C (A was dropped first)
    assert all(s >= 0 for s in slot[:a + b]) and all(s < 0 for s in slot[a + b:])
    assert info["n_matched"] == a + b
    assert info["restore_from"] == a + b
    # path 3 starts at B: a separate branch, nothing shared
    slot, pos, info = m.match(*P[3])
    assert all(s < 0 for s in slot) and info["n_matched"] == 0 and info["restore_from"] == 0
    # path 1 again: every row resident, nothing to recompute
    slot, pos, info = m.match(*P[1])
    assert all(s >= 0 for s in slot) and info["restore_from"] == a + b + c


# ------------------------------------------------------------------ keys vs descriptions

def _random_history(rng, tok_pool):
    n_msg = rng.randint(1, 5)
    lens = [rng.randint(0, 3) for _ in range(n_msg)]
    drop = {}
    for k in range(n_msg):
        if rng.random() < 0.4:
            drop[k] = rng.sample(range(k + 1), rng.randint(1, k + 1))
    repos = [k for k in range(n_msg) if rng.random() < 0.3]
    ops = oracle.canonical_ops(lens, drop, repos)
    T = sum(lens)
    return tok_pool[:T], ops


def test_equal_keys_mean_equal_descriptions():
    rng = random.Random(7)
    pool = [rng.randint(0, 2) for _ in range(20)]      # few ids: many coincidences
    hs = [_random_history(rng, pool) for _ in range(300)]
    seen = {}
    shared = 0
    for tok, ops in hs:
        keys, ids = token_keys(history(tok, ops)), _ident(tok, ops)
        for k, d in zip(keys, ids):
            if k in seen:
                assert seen[k] == d
                shared += 1
            seen[k] = d
    assert shared > 100


def test_canonical_form_drops_no_op_events():
    tok = [5, 6, 7, 8]
    base = [(APPEND, 2), (DROP, 0, 1), (APPEND, 2)]
    same = [
        [(APPEND, 2), (DROP, 0, 1), (DROP, 0, 1), (APPEND, 2)],           # repeated drop
        [(APPEND, 2), (DROP, 0, 1), (DROP, 1, 1), (APPEND, 2)],           # empty drop
        [(REPOS,), (APPEND, 2), (DROP, 0, 1), (APPEND, 2)],               # repos at start
        [(APPEND, 1), (REPOS,), (APPEND, 1), (DROP, 0, 1), (APPEND, 2)],  # repos with no gap
    ]
    kb, ib = token_keys(history(tok, base)), _ident(tok, base)
    for ops in same:
        assert token_keys(history(tok, ops)) == kb
        assert _ident(tok, ops) == ib
    split = [(APPEND, 3), (DROP, 0, 1), (APPEND, 0), (DROP, 1, 2), (APPEND, 1)]
    merged = [(APPEND, 3), (DROP, 0, 2), (APPEND, 1)]
    assert token_keys(history(tok, split)) == token_keys(history(tok, merged))
    assert _ident(tok, split) == _ident(tok, merged)
    # a repos after a drop moves positions: a real event
    moved = [(APPEND, 2), (DROP, 0, 1), (REPOS,), (APPEND, 2)]
    assert token_keys(history(tok, moved))[2] != kb[2]
    assert _ident(tok, moved)[2] != ib[2]


# ------------------------------------------------------------------ restore start

def test_restore_start_hand_worked():
    # 6 tokens in messages [0,2) [2,4) [4,6); message 0 (tokens 0, 1) is dropped after
    # message 1, i.e. at token 4: queries 0..3 see tokens 0, 1; queries 4, 5 do not
    tok = list(range(6))
    ops = oracle.canonical_ops([2, 2, 2], {1: [0]})
    records, final = oracle.replay_tokens(ops)
    vis = [[j for j, _ in r[1]] for r in records]
    # nothing resident -> restore everything
    assert restore_start(vis, final[0], [False] * 6) == 0
    # only token 0 missing: no query from 4 on sees it and it is not in the final state
    # {2..5}, so nothing is recomputed (s = 6)
    res = [False, True, True, True, True, True]
    assert restore_start(vis, final[0], res) == 6
    # token 3 missing (never dropped): every s > 3 needs it
    res = [True, True, True, False, True, True]
    assert restore_start(vis, final[0], res) == 3
    # token 1 missing: only starts s in (1, 4) need it, so again s = 6; with token 4
    # missing as well s = 6 and s = 5 fail (final state), s = 4 needs only 2, 3 below it
    res = [True, False, True, True, True, True]
    assert restore_start(vis, final[0], res) == 6
    res = [True, False, True, True, False, True]
    assert restore_start(vis, final[0], res) == 4


def test_restore_start_interval_form():
    """Largest s outside every (j, D_j) of a missing j equals the brute force."""
    rng = random.Random(3)
    for _ in range(200):
        tok, ops = _random_history(rng, list(range(20)))
        h = history(tok, ops)
        T = len(tok)
        records, final = oracle.replay_tokens(ops)
        vis = [[j for j, _ in r[1]] for r in records]
        res = [rng.random() < 0.6 for _ in range(T)]
        s = T
        while any(not res[j] and j < s < h["tok_drop"][j] for j in range(T)):
            s -= 1
        assert restore_start(vis, final[0], res) == s


# ------------------------------------------------------------------ eviction

def test_dropped_rows_go_before_finished_rows():
    m = CacheModel(8)
    tok = [1, 2, 3, 4]
    ops = oracle.canonical_ops([2, 2], {1: [0]})          # tokens 0, 1 dropped at the end
    slots = _insert_all(m, tok, ops)                        # slots 0..3
    # touch the dropped rows later than the held ones
    m.match(tok[:2], oracle.canonical_ops([2]))
    got = m.alloc(6)                                        # 4 free + 2 evicted
    assert got[:4] == [4, 5, 6, 7]
    assert sorted(got[4:]) == [slots[0], slots[1]]          # dropped despite newer use


def test_rows_in_use_are_never_evicted():
    m = CacheModel(4)
    tok = [1, 2, 3, 4]
    ops = oracle.canonical_ops([4])
    h = history(tok, ops)
    slots = m.alloc(4)
    m.insert(tok, ops, [0, 1, 2, 3], h["tok_pos"], slots)   # still locked
    with pytest.raises(CacheError):
        m.alloc(1)
    m.unlock(slots[:1])
    assert m.alloc(1) == [slots[0]]


def test_evicted_rows_keep_later_rows_reachable():
    a, b, c = 3, 4, 5
    P = _fig5(a, b, c)
    m = CacheModel(a + b + c)
    _insert_all(m, *P[1])
    # a new unrelated request needs 3 rows: the dropped A rows are the ones to go
    got = m.alloc(3)
    assert sorted(got) == list(range(a))
    slot, pos, info = m.match(*P[1])
    assert all(s < 0 for s in slot[:a]) and all(s >= 0 for s in slot[a:])
    assert info["n_matched"] == a + b + c
    # path 1's final state (B, C) is all resident: reuse without any prefill
    assert info["restore_from"] == a + b + c
    # path 2 would need C computed with A dropped earlier: A is gone, B is there, C was
    # never stored under that history -> recompute C only
    slot, pos, info = m.match(*P[2])
    assert info["restore_from"] == a + b


def test_a_later_round_retires_the_earlier_final_state():
    m = CacheModel(16)
    r1 = ([1, 2, 3, 4], oracle.canonical_ops([2, 2]))
    r2 = ([1, 2, 3, 4, 5, 6], oracle.canonical_ops([2, 2, 2], {2: [0]}))
    s1 = _insert_all(m, *r1)
    h2 = history(*r2)
    s2 = m.alloc(2)
    m.insert(*r2, [4, 5], h2["tok_pos"][4:], s2)
    m.unlock(s2)
    # tokens 0, 1 are held by round 1's final state only; round 2 supersedes it
    assert m.alloc(10) == list(range(6, 16))
    assert sorted(m.alloc(2)) == sorted(s1[:2])


def test_versions_are_preferred_at_the_needed_position():
    m = CacheModel(16)
    tok = [1, 2, 3, 4, 5]
    ops = oracle.canonical_ops([2, 3], {1: [0]}, [1])       # drop message 0, then repos
    h = history(tok, ops)
    assert h["final"] == [2, 3, 4] and h["final_pos"] == [0, 1, 2]
    s = m.alloc(5 + 3)
    # base rows at append positions and the final versions at 0..2
    m.insert(tok, ops, [0, 1, 2, 3, 4, 2, 3, 4], h["tok_pos"] + [0, 1, 2], s)
    slot, pos, info = m.match(tok, ops)
    assert pos == [0, 1, 0, 1, 2] and slot[2:] == s[5:]
    # without the repos the append positions are the ones needed
    ops2 = oracle.canonical_ops([2, 3], {1: [0]})
    slot, pos, info = m.match(tok, ops2)
    assert info["n_matched"] == 5
    assert pos == [0, 1, 2, 3, 4]


def test_bad_calls_are_rejected():
    m = CacheModel(4)
    tok = [1, 2]
    ops = oracle.canonical_ops([2])
    with pytest.raises(CacheError):
        m.insert(tok, ops, [0], [0], [0])                  # slot not allocated
    s = m.alloc(2)
    with pytest.raises(CacheError):
        m.insert(tok, ops, [0, 0], [0, 0], s)               # same version twice
    with pytest.raises(CacheError):
        m.unlock([3])
    with pytest.raises(CacheError):
        history([1], [(DROP, 0, 1)])                         # drop before append
    m.insert(tok, ops, [0], [0], s[:1])
    with pytest.raises(CacheError):
        m.unlock([s[0], s[0]])                               # locked once only
