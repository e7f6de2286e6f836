"""Cache index + reuse path + decode on the GPU, over a real KV pool.

Review, AKV serving system (§4.2, App. A.1.2, Fig. 8) and the request flow: a request
is matched in the index; rows held at the needed position are used as they are,
rows of the same history at another position are converted by key rotation
(akv_kv_reuse), tokens from the restore start on are computed afresh (here: the
RoPE-apply form of akv_rope_repos on the token's raw row, standing in for the
prefill), new rows go into slots the index hands out (evicting under pressure),
and decode reads the request's final state straight from the pool by slot.

Each raw K/V row is drawn from a seed derived from the token's full history key, so a
row shared across different histories, a wrong position, or a slot that was evicted
and reused would change the decode output by O(0.1); the bound is the decode tests'
2e-2 (bf16 storage, with up to two roundings of a converted key).
"""
import random
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.cache_index import history, token_keys
from segmented_attention_seq_amd import akv, workload
from tests.gpu_helpers import dev_tensor, host_f64
from tests.test_cache_index import Agent

pytestmark = pytest.mark.gpu

HQ, HKV, D = 8, 2, 64
BASE = workload.ROPE_BASE


def _raw_rows(key):
    rng = np.random.default_rng(zlib.crc32(repr(key).encode()))
    k = workload.f32_to_bf16_bits(rng.standard_normal((HKV, D)).astype(np.float32))
    v = workload.f32_to_bf16_bits(rng.standard_normal((HKV, D)).astype(np.float32))
    return k, v


def _dint(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


class Server:
    def __init__(self, n_slots):
        self.idx = akv.CacheIndex(n_slots)
        self.k = torch.full((n_slots, HKV, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.v = torch.full_like(self.k, float("nan"))
        self.counts = {"reused": 0, "converted": 0, "computed": 0, "requests": 0, "full": 0}

    def serve(self, tok, ops_list, rng):
        ops = akv.ops_array(ops_list)
        T = len(tok)
        slot, pos, info = self.idx.match(tok, ops, lock=True)
        tabs = akv.build_visibility(ops).tables()
        fin, fpos = tabs["final_tok"].astype(np.int64), tabs["final_pos"].astype(np.int64)
        want = tabs["tok_pos"].astype(np.int64).copy()
        want[fin] = fpos
        s0 = info["restore_from"]
        assert np.all(slot[fin[fin < s0]] >= 0), "final-state token below the restore start is not resident"
        fset = set(fin.tolist())
        need = [i for i in range(T) if (i >= s0 or i in fset) and pos[i] != want[i]]
        locked = slot[slot >= 0]
        try:
            new = self.idx.alloc(len(need))
        except akv.AkvError as e:
            assert e.status == akv.ENOSPACE
            self.idx.unlock(locked)
            self.counts["full"] += 1
            return None
        keys = token_keys(history(tok, ops_list))
        conv = [n for n, i in enumerate(need) if slot[i] >= 0]
        comp = [n for n, i in enumerate(need) if slot[i] < 0]
        if need:
            k_new = torch.empty((len(need), HKV, D), dtype=torch.bfloat16, device="cuda")
            v_new = torch.empty_like(k_new)
            if conv:
                ii = [need[n] for n in conv]
                kc, vc = torch.empty_like(k_new[:len(conv)]), torch.empty_like(k_new[:len(conv)])
                akv.kv_reuse(kc, vc, self.k, self.v, _dint(slot[ii]), _dint(pos[ii]), _dint(want[ii]), BASE)
                k_new[conv], v_new[conv] = kc, vc
            if comp:
                ii = [need[n] for n in comp]
                rows = [_raw_rows(keys[i]) for i in ii]
                kr = dev_tensor(np.stack([r[0] for r in rows]), True)
                vr = dev_tensor(np.stack([r[1] for r in rows]), True)
                kc = torch.empty_like(kr)
                akv.rope_repos(kc, kr, _dint(want[ii]), _dint(np.zeros(len(ii))), None, BASE)
                k_new[comp], v_new[comp] = kc, vr
            dst = torch.from_numpy(new.astype(np.int64)).cuda()
            self.k[dst], self.v[dst] = k_new, v_new
        self.idx.insert(tok, ops, need, want[need], new)
        # the final state straight from the pool
        where = slot.copy()
        where[need] = new
        indices = where[fin]
        assert np.all(indices >= 0)
        q_bits = workload.f32_to_bf16_bits(np.random.default_rng(rng.randrange(1 << 30))
                                           .standard_normal((1, HQ, D)).astype(np.float32))
        out = torch.empty((1, HQ, D), dtype=torch.bfloat16, device="cuda")
        akv.decode_attention(dev_tensor(q_bits, True), self.k, self.v, _dint([0, len(fin)]), _dint(indices),
                             len(fin), out)
        torch.cuda.synchronize()
        raw = [_raw_rows(keys[j]) for j in fin]
        k_ref = oracle.rope(np.stack([workload.bf16_bits_to_f32(r[0]) for r in raw]).astype(np.float64),
                            fpos, BASE)
        v_ref = np.stack([workload.bf16_bits_to_f32(r[1]) for r in raw]).astype(np.float64)
        q_ref = workload.bf16_bits_to_f32(q_bits).astype(np.float64)
        o_ref, _ = oracle.decode(q_ref, k_ref, v_ref, np.array([0, len(fin)]))
        err = np.abs(host_f64(out) - o_ref).max()
        assert err <= 2e-2, (err, info)
        self.idx.unlock(np.concatenate([locked, new]).astype(np.int32))
        self.counts["requests"] += 1
        self.counts["reused"] += int(np.sum(pos[fin] == want[fin]))
        self.counts["converted"] += len(conv)
        self.counts["computed"] += len(comp)
        return err


@pytest.mark.parametrize("seed,n_slots", [(11, 600), (12, 150)])
def test_agent_streams_through_pool(seed, n_slots):
    rng = random.Random(seed)
    srv = Server(n_slots)
    system = [[rng.randrange(50) for _ in range(6)]]
    agents = [Agent(rng, system + [[rng.randrange(50) for _ in range(rng.randint(2, 5))]],
                    keep=2, repos_at=30, vocab=12) for _ in range(3)]
    worst = 0.0
    for rnd in range(10):
        for a in list(agents):
            a.step()
            e = srv.serve(a.tokens(), a.ops(), rng)
            worst = max(worst, e or 0.0)
            if rng.random() < 0.2 and len(agents) < 5:
                b = a.fork()
                b.step(late_drop=True)
                agents.append(b)
                e = srv.serve(b.tokens(), b.ops(), rng)
                worst = max(worst, e or 0.0)
    print(f"[cache+pool seed={seed} slots={n_slots}] {srv.counts} worst max-abs {worst:.3e} "
          f"stats={srv.idx.stats()}")
    assert srv.counts["requests"] > 10 and srv.counts["converted"] > 0 and srv.counts["reused"] > 0


def test_fig5_paths_through_pool():
    """Paths 1, 2 and 3 of the history-dependence example served one after another:
    path 2 reuses A and B from path 1 and computes C, path 3 computes everything."""
    srv = Server(64)
    A, B, C = [1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11, 12]
    rng = random.Random(0)
    srv.serve(A + B + C, oracle.canonical_ops([3, 4, 5], {2: [0]}), rng)
    before = dict(srv.counts)
    srv.serve(A + B + C, oracle.canonical_ops([3, 4, 5], {1: [0]}), rng)
    assert srv.counts["computed"] - before["computed"] == 5
    before = dict(srv.counts)
    srv.serve(B + C, oracle.canonical_ops([4, 5]), rng)
    assert srv.counts["computed"] - before["computed"] == 9
