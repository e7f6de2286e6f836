"""KV cache index (akv_cache_*) against the plain model in oracle/cache_index.py.  CPU only
(host code of libakv).

Synthetic multi-request streams in the shape of the pages' workloads (agents that
share a system prompt and task prefix, alternate reasoning and tool messages, drop
old tool responses on a rolling window, reposition past a position threshold, and
fork into branches that drop at different times, as in the history-dependence
example) drive both sides through the same calls; every output (slots, positions,
match summary, allocated slots and their order, statistics, errors) must agree
exactly.
"""
import random

import numpy as np
import pytest

import oracle
from oracle.cache_index import CacheError, CacheModel, history
from segmented_attention_seq_amd import akv


def _pair(n_slots):
    return akv.CacheIndex(n_slots), CacheModel(n_slots)


def _same_match(lib, mod, tok, ops, lock):
    s1, p1, i1 = lib.match(tok, akv.ops_array(ops), lock)
    s2, p2, i2 = mod.match(tok, ops, lock)
    assert s1.tolist() == s2 and p1.tolist() == p2 and i1 == i2
    return s2, p2, i2


def _same_stats(lib, mod):
    a, b = lib.stats(), mod.stats()
    for k in ("n_free", "n_resident", "n_locked", "n_marks", "n_frontier"):
        assert a[k] == b[k], k


def _both_fail(f_lib, f_mod):
    with pytest.raises(akv.AkvError):
        f_lib()
    with pytest.raises(CacheError):
        f_mod()


class Agent:
    """One conversation: messages, rolling tool drop, repos past a threshold."""

    def __init__(self, rng, prefix, keep, repos_at, vocab):
        self.rng, self.keep, self.repos_at, self.vocab = rng, keep, repos_at, vocab
        self.msgs = [list(m) for m in prefix]
        self.tools = []                     # message indices of tool responses
        self.drop, self.repos = {}, []

    def fork(self):
        a = Agent(self.rng, [], self.keep, self.repos_at, self.vocab)
        a.msgs = [list(m) for m in self.msgs]
        a.tools = list(self.tools)
        a.drop = {k: list(v) for k, v in self.drop.items()}
        a.repos = list(self.repos)
        return a

    def step(self, late_drop=False):
        r = self.rng
        self.msgs.append([r.randrange(self.vocab) for _ in range(r.randint(1, 4))])   # reasoning
        self.msgs.append([r.randrange(self.vocab) for _ in range(r.randint(2, 7))])   # tool
        k = len(self.msgs) - 1
        self.tools.append(k)
        if len(self.tools) > self.keep:
            victim = self.tools[-self.keep - 1]
            at = k - 1 if late_drop and k - 1 > victim else k   # the fork drops a message earlier
            self.drop.setdefault(at, []).append(victim)
        ops = self.ops()
        if history(self.tokens(), ops)["p_next"] >= self.repos_at:
            self.repos.append(k)

    def tokens(self):
        return [t for m in self.msgs for t in m]

    def ops(self):
        return oracle.canonical_ops([len(m) for m in self.msgs], self.drop, sorted(set(self.repos)))


def _serve(lib, mod, tok, ops, in_flight, rng):
    """One request through both sides: match(lock), alloc the missing needed
    versions, insert them, keep the locks in flight for a while."""
    slot, pos, info = _same_match(lib, mod, tok, ops, True)
    h = history(tok, ops)
    want = list(h["tok_pos"])
    for j, p in zip(h["final"], h["final_pos"]):
        want[j] = p
    fin = set(h["final"])
    need = [i for i in range(len(tok))
            if (i >= info["restore_from"] or i in fin) and pos[i] != want[i]]
    locked = [s for s in slot if s >= 0]
    try:
        got = lib.alloc(len(need)).tolist()
    except akv.AkvError as e:
        assert e.status == akv.ENOSPACE
        with pytest.raises(CacheError):
            mod.alloc(len(need))
        lib.unlock(locked)
        mod.unlock(locked)
        return "full"
    assert got == mod.alloc(len(need))
    vt, vp = need, [want[i] for i in need]
    lib.insert(tok, akv.ops_array(ops), vt, vp, got)
    mod.insert(tok, ops, vt, vp, got)
    in_flight.append(locked + got)
    while in_flight and (len(in_flight) > 2 or rng.random() < 0.5):
        done = in_flight.pop(0)
        lib.unlock(done)
        mod.unlock(done)
    _same_stats(lib, mod)
    return "reuse" if info["restore_from"] == len(tok) else "restore"


@pytest.mark.parametrize("seed,n_slots", [(1, 400), (2, 160), (3, 90)])
def test_agent_streams_match_model(seed, n_slots):
    rng = random.Random(seed)
    lib, mod = _pair(n_slots)
    system = [[rng.randrange(50) for _ in range(6)]]
    agents = [Agent(rng, system + [[rng.randrange(50) for _ in range(rng.randint(2, 5))]],
                    keep=2, repos_at=40, vocab=12) for _ in range(3)]
    in_flight, seen = [], {"reuse": 0, "restore": 0, "full": 0}
    for rnd in range(14):
        for a in list(agents):
            a.step()
            seen[_serve(lib, mod, a.tokens(), a.ops(), in_flight, rng)] += 1
            if rng.random() < 0.15 and len(agents) < 6:        # a branch with other drop timing
                b = a.fork()
                b.step(late_drop=True)
                agents.append(b)
                seen[_serve(lib, mod, b.tokens(), b.ops(), in_flight, rng)] += 1
            if rng.random() < 0.2:                              # the same request again
                seen[_serve(lib, mod, a.tokens(), a.ops(), in_flight, rng)] += 1
    while in_flight:
        done = in_flight.pop(0)
        lib.unlock(done)
        mod.unlock(done)
    _same_stats(lib, mod)
    print(f"[cache streams seed={seed} slots={n_slots}] {seen} stats={lib.stats()}")
    assert seen["restore"] > 0 and seen["reuse"] > 0


def test_fig5_paths_in_the_index():
    """Review §3.4 / Fig. 5: paths 1 and 2 share A and B but not C; path 3 shares
    nothing; repeated path 1 is a pure reuse."""
    a, b, c = 3, 4, 5
    A, B, C = list(range(100, 103)), list(range(200, 204)), list(range(300, 305))
    P = {1: (A + B + C, oracle.canonical_ops([a, b, c], {2: [0]})),
         2: (A + B + C, oracle.canonical_ops([a, b, c], {1: [0]})),
         3: (B + C, oracle.canonical_ops([b, c]))}
    lib, mod = _pair(32)
    tok, ops = P[1]
    h = history(tok, ops)
    s = lib.alloc(12).tolist()
    assert s == mod.alloc(12)
    lib.insert(tok, akv.ops_array(ops), list(range(12)), h["tok_pos"], s)
    mod.insert(tok, ops, list(range(12)), h["tok_pos"], s)
    slot, _, info = _same_match(lib, mod, *P[2], False)
    assert info["n_matched"] == a + b and info["restore_from"] == a + b
    slot, _, info = _same_match(lib, mod, *P[3], False)
    assert info["n_matched"] == 0 and max(slot) == -1
    slot, _, info = _same_match(lib, mod, *P[1], False)
    assert info["restore_from"] == a + b + c
    _same_stats(lib, mod)


def test_node_split_keeps_marks_and_versions():
    """A later history that diverges inside a stored run splits the tree node; rows
    and the completed-request state on both sides of the cut stay as they were."""
    lib, mod = _pair(64)
    long = (list(range(10)), oracle.canonical_ops([4, 6]))
    short = (list(range(4)) + [99, 98], oracle.canonical_ops([4, 2]))
    mid = (list(range(7)), oracle.canonical_ops([4, 3]))
    for tok, ops in (long, short, mid):
        _serve(lib, mod, tok, ops, [], random.Random(0))
    for tok, ops in (long, short, mid):
        slot, _, info = _same_match(lib, mod, tok, ops, False)
        assert info["restore_from"] == len(tok) and min(slot) >= 0
    _same_stats(lib, mod)
    assert lib.stats()["n_frontier"] == 2          # "mid" is a prefix of "long"


def test_empty_and_degenerate_requests():
    lib, mod = _pair(8)
    # no tokens at all
    _same_match(lib, mod, [], [], False)
    # only drops and repos of nothing
    _same_match(lib, mod, [], [(oracle.REPOS,)], False)
    # every token dropped at the end: nothing is needed from the cache
    tok, ops = [1, 2, 3], oracle.canonical_ops([3], {0: [0]})
    slot, _, info = _same_match(lib, mod, tok, ops, False)
    assert info["restore_from"] == 3 and info["n_final"] == 0
    # zero-size alloc and unlock
    assert lib.alloc(0).size == 0 and mod.alloc(0) == []
    lib.unlock([])
    mod.unlock([])
    _same_stats(lib, mod)


def test_bad_calls_rejected_on_both_sides():
    lib, mod = _pair(4)
    tok, ops = [1, 2], oracle.canonical_ops([2])
    A = akv.ops_array(ops)
    _both_fail(lambda: lib.insert(tok, A, [0], [0], [0]), lambda: mod.insert(tok, ops, [0], [0], [0]))
    s = lib.alloc(2).tolist()
    assert s == mod.alloc(2)
    _both_fail(lambda: lib.insert(tok, A, [0, 0], [0, 0], s), lambda: mod.insert(tok, ops, [0, 0], [0, 0], s))
    _both_fail(lambda: lib.insert(tok, A, [2], [0], s[:1]), lambda: mod.insert(tok, ops, [2], [0], s[:1]))
    _both_fail(lambda: lib.unlock([3]), lambda: mod.unlock([3]))
    _both_fail(lambda: lib.match([1], akv.ops_array([(oracle.DROP, 0, 1)]), False),
               lambda: mod.match([1], [(oracle.DROP, 0, 1)], False))
    _both_fail(lambda: lib.match([1, 2, 3], A, False), lambda: mod.match([1, 2, 3], ops, False))
    lib.insert(tok, A, [0], [0], s[:1])
    mod.insert(tok, ops, [0], [0], s[:1])
    _both_fail(lambda: lib.unlock([s[0], s[0]]), lambda: mod.unlock([s[0], s[0]]))
    _both_fail(lambda: lib.alloc(3), lambda: mod.alloc(3))     # 2 free, 2 locked
    with pytest.raises(akv.AkvError):
        akv.CacheIndex(0)
    _same_stats(lib, mod)


def test_large_history_match_is_fast():
    """A 48k-token history (the restore workload's shape) through insert and match."""
    import time
    from segmented_attention_seq_amd import workload
    tr = workload.config_trajectory(2)
    ops = akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition)
    T = int(sum(tr.msg_len))
    tok = np.random.default_rng(0).integers(0, 32000, T).astype(np.int32)
    lib = akv.CacheIndex(2 * T)
    t0 = time.perf_counter()
    slot, pos, info = lib.match(tok, ops)
    t1 = time.perf_counter()
    assert info["n_matched"] == 0 and info["restore_from"] == 0
    plan = akv.build_visibility(ops).tables()
    s = lib.alloc(T)
    lib.insert(tok, ops, np.arange(T), plan["tok_pos"], s)
    t2 = time.perf_counter()
    slot, pos, info = lib.match(tok, ops)
    t3 = time.perf_counter()
    assert info["n_matched"] == T and info["n_resident"] == T and info["restore_from"] == T
    print(f"[cache 48k] match(empty) {1e3 * (t1 - t0):.1f} ms, insert {1e3 * (t2 - t1):.1f} ms, "
          f"match(hit) {1e3 * (t3 - t2):.1f} ms")
    assert t3 - t2 < 2.0
