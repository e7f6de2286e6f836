"""Seeded synthetic inputs for the AKV restore / repos / decode path.

This module is the only code shared by the CPU oracle's tests and the GPU
path.  It holds none of the method's arithmetic: it draws message lengths,
decides which cache operations the agent harness sends (the tool-response
rolling drop and the repos trigger are the harness's policy, not the server's
computation), and draws Gaussian Q/K/V tensors, rounded to bfloat16 with
round-to-nearest-even on the raw bits.

Sources (page "Cache Engineering for Agents", jaehun.me review):
  * rolling drop keeps every reasoning message and the 12 most recent tool
    responses (section "what to keep", Fig. 2 / App. A.4.3);
  * the repos threshold equals the model's Standard summarisation threshold,
    96k tokens (section "results", §5.1);
  * requests are message lists; cache ops use the operate-after syntax
    (section "AKV serving system", Fig. 6).
Workload shapes (rounds, 200-800 token reasoning, 1k-4k token tool responses,
64/8 GQA heads, d=64) are the synthetic stand-in for the agent trajectories
(BrowseComp-Plus, SWE-Verified) measured on the pages; no dataset item is used.
"""
from __future__ import annotations

import dataclasses
import json
from typing import Dict, List, Optional

import numpy as np

USER_LEN = 256
ASSIST_RANGE = (200, 801)     # integers(lo, hi) upper bound exclusive
TOOL_RANGE = (1000, 4001)
KEEP_TOOLS = 12
REPOS_THRESHOLD = 96_000
ROPE_BASE = 150000.0
BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass
class Trajectory:
    """A request as the agent sends it: message lengths plus cache ops.

    drop[k] lists the messages whose KV is dropped once message k has been
    appended; reposition lists the messages after which the remaining keys
    are renumbered.  Indices are 0-based message indices.
    """
    msg_len: List[int]
    roles: List[str]
    drop: Dict[int, List[int]]
    reposition: List[int]
    name: str = ""

    @property
    def n_tokens(self) -> int:
        return int(sum(self.msg_len))

    def drop_pairs(self):
        """Flattened (after, target) pairs in ascending `after` order."""
        after, target = [], []
        for k in sorted(self.drop):
            for j in self.drop[k]:
                after.append(k)
                target.append(j)
        return np.asarray(after, np.int32), np.asarray(target, np.int32)

    def to_json(self) -> str:
        return json.dumps({"name": self.name, "msg_len": self.msg_len, "roles": self.roles,
                           "drop": {str(k): v for k, v in self.drop.items()},
                           "reposition": self.reposition})

    @staticmethod
    def from_json(s: str) -> "Trajectory":
        o = json.loads(s)
        return Trajectory(list(o["msg_len"]), list(o["roles"]),
                          {int(k): list(v) for k, v in o["drop"].items()},
                          list(o["reposition"]), o.get("name", ""))


# ----------------------------------------------------------------------------
# bfloat16 helpers (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) -> uint16 bits.
    Inputs here are finite Gaussian draws; NaN/Inf are not special-cased."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Trajectories
# ----------------------------------------------------------------------------

def _largest_remainder(lengths: List[int], total: int) -> List[int]:
    """Scale lengths by one factor so they sum to `total` exactly.
    Floor each scaled length, then hand the remaining units to the largest
    fractional parts (ties to the lower index).  Every message keeps >= 1."""
    lengths = np.asarray(lengths, dtype=np.float64)
    exact = lengths * (total / lengths.sum())
    base = np.maximum(np.floor(exact).astype(np.int64), 1)
    rem = total - int(base.sum())
    frac = exact - np.floor(exact)
    order = sorted(range(len(lengths)), key=lambda i: (-frac[i], i))
    i = 0
    while rem > 0:
        base[order[i % len(order)]] += 1
        rem -= 1
        i += 1
    while rem < 0:  # only if the >=1 floor pushed us over
        j = int(np.argmax(base))
        base[j] -= 1
        rem += 1
    return [int(v) for v in base]


def agent_trajectory(rounds: int, seed: int, total: Optional[int] = None,
                     keep: int = KEEP_TOOLS, repos: str = "none",
                     repos_threshold: int = REPOS_THRESHOLD,
                     user_len: int = USER_LEN, assist_range=ASSIST_RANGE,
                     tool_range=TOOL_RANGE, name: str = "") -> Trajectory:
    """User message, then `rounds` x (assistant reasoning, tool response).

    keep:   after tool message of round r completes, drop the tool message of
            round r-keep (rolling drop; reasoning is never dropped).
    repos:  "none"; "every" (after every tool message); or "threshold" --
            after a round's drop, repos when the harness's next position
            index has reached `repos_threshold`.  The harness tracks that
            index itself: it grows by each appended message and, after a
            repos, restarts at the number of tokens it has not dropped.
    """
    rng = np.random.default_rng(seed)
    lens = [user_len]
    roles = ["user"]
    for _ in range(rounds):
        lens.append(int(rng.integers(*assist_range)))
        roles.append("assistant")
        lens.append(int(rng.integers(*tool_range)))
        roles.append("tool")
    if total is not None:
        lens = _largest_remainder(lens, total)
    drop: Dict[int, List[int]] = {}
    reposition: List[int] = []
    kept = 0          # tokens of messages not dropped (harness bookkeeping)
    next_index = 0    # harness's view of the next position index
    dropped = set()
    for k, n in enumerate(lens):
        kept += n
        next_index += n
        if roles[k] != "tool":
            continue
        r = (k - 2) // 2
        if keep is not None and r >= keep:
            tgt = 2 + 2 * (r - keep)
            drop[k] = [tgt]
            dropped.add(tgt)
            kept -= lens[tgt]
        fire = (repos == "every") or (repos == "threshold" and next_index >= repos_threshold)
        if fire:
            reposition.append(k)
            next_index = kept
    return Trajectory(lens, roles, drop, reposition, name)


def config_trajectory(cfg: int) -> Trajectory:
    """The four prefill workloads (tiny worked example, 48k, ~300k/96k-window, 192k)."""
    if cfg == 1:
        # The pages' request example: user 16, assistant 24, tool 40 tokens,
        # drop {1:[0], 2:[1]}, reposition [2].
        return Trajectory([16, 24, 40], ["user", "assistant", "tool"],
                          {1: [0], 2: [1]}, [2], "tiny")
    if cfg == 2:
        return agent_trajectory(20, 1000 + cfg, total=48_000, name="48k-20rounds-keep12")
    if cfg == 3:
        return agent_trajectory(100, 1000 + cfg, total=None, repos="threshold",
                                name="100rounds-keep12-repos96k")
    if cfg == 4:
        return agent_trajectory(200, 1000 + cfg, total=192_000, repos="every",
                                name="192k-200rounds-keep12-repos-every-round")
    raise ValueError(cfg)


CONFIG_HEADS = {1: (1, 1, 64), 2: (64, 8, 64), 3: (64, 8, 64), 4: (64, 8, 64), 5: (64, 8, 64)}


# ----------------------------------------------------------------------------
# Tensors
# ----------------------------------------------------------------------------

def _normal_rows(rng, rows: int, width: int, bf16: bool, chunk_rows: int = 1 << 14):
    """Draw rows x width standard normals (float32) in row chunks; return bf16 bits
    (uint16) or float32.  Chunking does not change the stream."""
    out = np.empty((rows, width), np.uint16 if bf16 else np.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, width), dtype=np.float32)
        out[r0:r1] = f32_to_bf16_bits(x) if bf16 else x
    return out


def prefill_tensors(T: int, hq: int, hkv: int, d: int, seed: int, bf16: bool = True):
    """Raw (un-rotated) Q [T,hq,d], K [T,hkv,d], V [T,hkv,d], drawn in that order."""
    rng = np.random.default_rng(seed)
    q = _normal_rows(rng, T, hq * d, bf16).reshape(T, hq, d)
    k = _normal_rows(rng, T, hkv * d, bf16).reshape(T, hkv, d)
    v = _normal_rows(rng, T, hkv * d, bf16).reshape(T, hkv, d)
    return q, k, v


def config_prefill(cfg: int):
    traj = config_trajectory(cfg)
    hq, hkv, d = CONFIG_HEADS[cfg]
    q, k, v = prefill_tensors(traj.n_tokens, hq, hkv, d, seed=cfg, bf16=(cfg != 1))
    return traj, q, k, v


# ----------------------------------------------------------------------------
# Decode / batched-repos workload
# ----------------------------------------------------------------------------

def survivor_trajectory(n_active: int, seed: int, keep: int = KEEP_TOOLS):
    """Grow an agent trajectory (rolling drop) until exactly `n_active` tokens
    survive; the last appended message is cut short to land on the count.
    Returns (message lengths, ascending surviving logical token indices)."""
    rng = np.random.default_rng(seed)
    lens: List[int] = []
    alive: List[bool] = []

    def survivors():
        return sum(n for n, a in zip(lens, alive) if a)

    def append(n):
        have = survivors()
        if have + n >= n_active:
            lens.append(n_active - have)
            alive.append(True)
            return True
        lens.append(n)
        alive.append(True)
        return False

    done = append(min(USER_LEN, n_active))
    r = 0
    while not done:
        if append(int(rng.integers(*ASSIST_RANGE))):
            break
        if append(int(rng.integers(*TOOL_RANGE))):
            break
        if r >= keep:
            alive[2 + 2 * (r - keep)] = False
        r += 1
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    surv = np.concatenate([np.zeros(0, np.int64)] + [np.arange(s, s + n, dtype=np.int64)
                                                     for s, n, a in zip(starts, lens, alive) if a and n > 0])
    assert surv.size == n_active
    return lens, surv


@dataclasses.dataclass
class DecodeBatch:
    """Batch of single-token decode requests over a shared slot pool.

    Request b owns pool slots [base_b, base_b + T_b + 1): its logical tokens,
    then the new token's own slot.  Its gathered list is its surviving tokens'
    slots (ascending, with holes where messages were dropped) followed by the
    own slot.  Only gathered slots hold data (k_rows/v_rows, in gather order);
    every other pool slot is a hole.
    """
    hq: int
    hkv: int
    d: int
    q: np.ndarray          # [B, hq, d]
    k_rows: np.ndarray     # [sum n, hkv, d]
    v_rows: np.ndarray     # [sum n, hkv, d]
    indptr: np.ndarray     # int32 [B+1]
    indices: np.ndarray    # int32 [sum n]  pool slots
    pool_slots: int
    bf16: bool


def decode_batch(batch: int = 14, lo: int = 32_000, hi: int = 96_001, seed: int = 1005,
                 hq: int = 64, hkv: int = 8, d: int = 64, bf16: bool = True,
                 shuffle_slots: bool = False) -> DecodeBatch:
    n = np.random.default_rng(seed).integers(lo, hi, size=batch)
    indptr = np.zeros(batch + 1, np.int64)
    idx = []
    base = 0
    for b in range(batch):
        lens, surv = survivor_trajectory(int(n[b]) - 1, 2000 + b)
        T_b = int(sum(lens))
        idx.append(np.concatenate([base + surv, [base + T_b]]))
        indptr[b + 1] = indptr[b] + surv.size + 1
        base += T_b + 1
    indices = np.concatenate(idx)
    if shuffle_slots:
        perm = np.random.default_rng(seed + 7).permutation(base)
        indices = perm[indices]
    rng = np.random.default_rng(seed + 1)
    q = _normal_rows(rng, batch, hq * d, bf16).reshape(batch, hq, d)
    total = int(indptr[-1])
    k_rows = _normal_rows(rng, total, hkv * d, bf16).reshape(total, hkv, d)
    v_rows = _normal_rows(rng, total, hkv * d, bf16).reshape(total, hkv, d)
    return DecodeBatch(hq, hkv, d, q, k_rows, v_rows, indptr.astype(np.int32),
                       indices.astype(np.int32), base, bf16)


@dataclasses.dataclass
class ReposBatch:
    """Batched repos of the surviving keys of one trajectory.

    Key n lives in pool slot `slots[n]` (= its logical index; the pool has the
    trajectory's T slots, the rest are holes) at position pos_from[n] (its
    logical index: no earlier repos) and moves to pos_to[n] = n.
    """
    hkv: int
    d: int
    k_rows: np.ndarray     # [n, hkv, d] values at the gathered slots
    slots: np.ndarray      # int32 [n]
    pos_from: np.ndarray   # int32 [n]
    pos_to: np.ndarray     # int32 [n]
    pool_slots: int
    bf16: bool


def repos_batch(n_keys: int = 96_000, seed: int = 3005, hkv: int = 8, d: int = 64,
                bf16: bool = True) -> ReposBatch:
    lens, surv = survivor_trajectory(n_keys, seed)
    rng = np.random.default_rng(seed + 1)
    k_rows = _normal_rows(rng, n_keys, hkv * d, bf16).reshape(n_keys, hkv, d)
    return ReposBatch(hkv, d, k_rows, surv.astype(np.int32), surv.astype(np.int32),
                      np.arange(n_keys, dtype=np.int32), int(sum(lens)), bf16)
