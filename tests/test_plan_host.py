"""Host side of libakv (no GPU needed): exported symbols, op canonicalisation and
every plan table, bit-exact against the CPU oracle."""
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from segmented_attention_seq_amd import akv, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "akv.h")).read()
    declared = set(re.findall(r"\b(akv_\w+)\s*\(", hdr))
    assert declared == set(akv.EXPORTED)
    nm = subprocess.run(["nm", "-D", "--defined-only", akv.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (akv_\w+)$", nm, re.M))
    missing = declared - exported
    assert not missing, missing
    assert "gfx950" in akv.version()


def _tuples(ops):
    out = []
    for o in ops:
        k = int(o["kind"])
        out.append((k, int(o["a"])) if k == akv.OP_APPEND else
                   (k, int(o["a"]), int(o["b"])) if k == akv.OP_DROP else (k,))
    return out


@st.composite
def requests(draw, max_msgs=7, max_len=9):
    M = draw(st.integers(1, max_msgs))
    lens = draw(st.lists(st.integers(0, max_len), min_size=M, max_size=M))
    drop = {}
    for k in range(M):
        tg = draw(st.lists(st.integers(0, k), max_size=3))
        if tg:
            drop[k] = tg
    repos = draw(st.lists(st.integers(0, M - 1), max_size=4))
    return lens, drop, repos


@settings(max_examples=300, deadline=None)
@given(requests())
def test_ops_from_messages_matches_oracle(req):
    lens, drop, repos = req
    assert _tuples(akv.ops_from_messages(lens, drop, repos)) == oracle.canonical_ops(lens, drop, repos)


@pytest.mark.parametrize("bad,status", [
    (dict(drop={3: [0]}), akv.EOPSEQ), (dict(drop={1: [2]}), akv.EOPSEQ),
    (dict(drop={0: [-1]}), akv.EOPSEQ), (dict(reposition=[5]), akv.EOPSEQ),
    (dict(lens=[2, -1, 2]), akv.EINVAL),
])
def test_invalid_requests(bad, status):
    with pytest.raises(akv.AkvError) as e:
        akv.ops_from_messages(bad.get("lens", [2, 2, 2]), bad.get("drop"), bad.get("reposition", ()))
    assert e.value.status == status


def test_invalid_op_lists():
    for ops in ([(akv.OP_APPEND, -1)], [(akv.OP_APPEND, 3), (akv.OP_DROP, 1, 5)],
                [(7, 0)], [(akv.OP_APPEND, 3), (akv.OP_DROP, 2, 1)]):
        with pytest.raises(akv.AkvError) as e:
            akv.build_visibility(ops)
        assert e.value.status == akv.EOPSEQ
    with pytest.raises(akv.AkvError) as e:
        akv.build_visibility([(akv.OP_APPEND, 3)], bq=0)
    assert e.value.status == akv.EINVAL


def _compare(lens, drop, repos, bq, bk, tiles="full", rng=None):
    ops_o = oracle.canonical_ops(lens, drop, repos)
    plan = akv.build_visibility(akv.ops_from_messages(lens, drop, repos), bq, bk)
    t = plan.tables()
    ev = oracle.replay_events(ops_o)
    o = oracle.plan_tables(ev=ev, bq=bq, bk=bk, with_tiles=(tiles == "full"))
    info = plan.info
    assert info["n_tokens"] == ev.T
    for name in ("tok_pos", "tok_drop", "segments", "epochs", "versions", "final_tok", "final_pos"):
        assert np.array_equal(t[name], o[name].astype(np.int32).reshape(t[name].shape)), name
    assert info["p_next"] == o["p_next"]
    assert info["visible_pairs"] == o["visible_pairs"]
    # runs of version rows with one shift (to - from), restarting at every stretch
    ver = o["versions"].reshape(-1, 3)
    shift = ver[:, 2] - ver[:, 1]
    starts = (ver[:, 2] == 0) | np.r_[True, shift[1:] != shift[:-1]] if ver.size else np.zeros(0, bool)
    assert np.array_equal(t["ver_run"], np.cumsum(starts) - 1)
    assert np.array_equal(t["run_delta"], shift[starts])
    assert info["n_runs"] == int(starts.sum())
    n_items = info["n_items"]
    order = t["item_order"]
    assert sorted(order.tolist()) == list(range(n_items))
    cnt = np.diff(t["tile_ptr"])
    # stretch by stretch (longest item first, ties by index), items longest first inside
    st = t["items"].reshape(-1, 2)[:, 0]
    longest = {}
    for i in range(n_items):
        longest[st[i]] = max(longest.get(st[i], 0), cnt[i])
    key = sorted(range(n_items), key=lambda i: (-longest[st[i]], st[i], -cnt[i], i))
    assert order.tolist() == key
    kt, cls = t["tiles"] >> 2, t["tiles"] & 3
    assert info["n_full"] == int((cls == akv.TILE_FULL).sum())
    assert info["n_partial"] == int((cls == akv.TILE_PARTIAL).sum())
    if tiles == "full":
        assert np.array_equal(t["items"], o["items"].astype(np.int32))
        assert np.array_equal(t["tile_ptr"], o["tile_ptr"].astype(np.int32))
        assert np.array_equal(kt, o["tile_k"]) and np.array_equal(cls, o["tile_cls"])
    else:
        # spot checks against the explicit mask: whole lists of sampled items,
        # and sampled absent (EMPTY) tiles
        for n in rng.choice(n_items, size=min(n_items, 40), replace=False):
            e, qt = t["items"][n]
            a, b = t["tile_ptr"][n], t["tile_ptr"][n + 1]
            tb, te, src = ev.epochs[e]
            nk = -(-src.size // bk) + -(-(te - tb) // bk)
            present = dict(zip(kt[a:b].tolist(), cls[a:b].tolist()))
            for k in rng.choice(nk, size=min(nk, 60), replace=False).tolist() + list(present)[:20]:
                assert present.get(k, 0) == oracle.tile_class_of(ev, e, qt, k, bq, bk), (n, k)
    return plan


@settings(max_examples=300, deadline=None)
@given(requests(), st.sampled_from([(1, 1), (2, 3), (4, 4), (3, 2), (64, 64)]))
def test_tables_match_oracle_random(req, tiles):
    lens, drop, repos = req
    _compare(lens, drop, repos, *tiles)


@settings(max_examples=60, deadline=None)
@given(requests(max_msgs=12, max_len=150), st.sampled_from([(16, 16), (64, 64), (32, 16), (128, 64), (256, 64)]))
def test_tables_match_oracle_longer(req, tiles):
    lens, drop, repos = req
    _compare(lens, drop, repos, *tiles)


@pytest.mark.parametrize("bq,bk", [(64, 64), (16, 16), (8, 32)])
def test_tables_tiny_request_example(bq, bk):
    tr = workload.config_trajectory(1)
    plan = _compare(tr.msg_len, tr.drop, tr.reposition, bq, bk)
    assert plan.info["visible_pairs"] == 2600
    assert plan.info["p_next"] == 40


def test_tables_48k_workload():
    tr = workload.config_trajectory(2)
    plan = _compare(tr.msg_len, tr.drop, tr.reposition, 64, 64)
    assert plan.info["n_segments"] == 8 and plan.info["n_versions"] == 0


@pytest.mark.parametrize("bq", [128, 256, 512])
def test_tables_48k_workload_large_query_tiles(bq):
    """Query tiles of 128, 256 and 512 tokens (the plans the attention takes for 4,
    2 and 1 query heads per kv head): items, tile lists and classes against the
    oracle on sampled items."""
    tr = workload.config_trajectory(2)
    plan = _compare(tr.msg_len, tr.drop, tr.reposition, bq, 64, tiles="sampled", rng=np.random.default_rng(bq))
    assert plan.info["n_items"] == sum(-(-(e[1] - e[0]) // bq) for e in plan.tables()["epochs"])


@pytest.mark.parametrize("cfg", [3, 4])
def test_tables_large_workloads_sampled(cfg):
    tr = workload.config_trajectory(cfg)
    plan = _compare(tr.msg_len, tr.drop, tr.reposition, 64, 64, tiles="sampled",
                    rng=np.random.default_rng(cfg))
    if cfg == 3:
        assert plan.info["n_epochs"] == 7
    else:
        assert plan.info["n_epochs"] == 200 and plan.info["n_segments"] == 200


def test_empty_and_degenerate():
    p = akv.build_visibility([])
    assert p.info["n_tokens"] == 0 and p.info["n_items"] == 0
    p = akv.build_visibility([(akv.OP_APPEND, 0), (akv.OP_REPOS,), (akv.OP_APPEND, 1)])
    assert p.info["n_tokens"] == 1 and p.info["visible_pairs"] == 1
    # drop everything then append: the new token sees only itself
    lens, drop = [5, 3], {0: [0]}
    _compare(lens, drop, [0], 4, 4)


@pytest.mark.parametrize("cfg,parts,n_edge", [(2, 1, 32), (3, 3, 352), (4, 4, 800)])
def test_full_size_parity_parts_cover_every_boundary_row(cfg, parts, n_edge):
    """The parts of the full-size GPU parity check (tests/test_gpu_parity.py) cover
    every boundary-adjacent row and every seeded row of the workload exactly once."""
    from tests.gpu_helpers import SEEDED_ROWS, edge_rows, full_size_rows
    tr = workload.config_trajectory(cfg)
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    t, T = plan.tables(), tr.n_tokens
    got = [full_size_rows(t, T, cfg, p, parts) for p in range(parts)]
    edges = edge_rows(t, T)
    seeded = np.unique(np.random.default_rng(cfg).integers(0, T, SEEDED_ROWS[cfg]))
    assert edges.size == n_edge
    assert np.array_equal(np.concatenate([g[1] for g in got]), edges)
    assert np.array_equal(np.concatenate([g[2] for g in got]), seeded)
    assert np.array_equal(np.concatenate([g[0] for g in got]), np.union1d(edges, seeded))


def test_attention_bq_choice():
    """The plan query tile the bf16 attention runs fastest with: 64 for 8 query heads
    per kv head, 64 * 8 / group for groups of 1, 2 and 4 (eight waves take the
    group's query heads over 8 / group 64-token parts), 64 otherwise."""
    assert akv.attention_bq(64, 8) == 64
    assert akv.attention_bq(32, 8) == 128 and akv.attention_bq(12, 3) == 128
    assert akv.attention_bq(16, 8) == 256 and akv.attention_bq(8, 8) == 512
    assert akv.attention_bq(24, 8) == 64 and akv.attention_bq(3, 2) == 64 and akv.attention_bq(0, 8) == 64
