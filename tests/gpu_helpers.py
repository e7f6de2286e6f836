"""Helpers for the GPU parity tests: host arrays <-> device tensors, sampled rows."""
import os

import numpy as np
import torch

from segmented_attention_seq_amd import workload


def dev_tensor(a: np.ndarray, bf16: bool):
    """uint16 bf16 bits or float32 array -> CUDA tensor."""
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def host_bf16_bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(a: np.ndarray, bf16: bool) -> np.ndarray:
    return workload.bf16_bits_to_f32(a).astype(np.float64) if bf16 else a.astype(np.float64)


def edge_rows(plan_tables, T, edge=2):
    """Every row within `edge` rows of a segment boundary (both sides) and the first
    and last row of every repos stretch, ascending."""
    rows = set()
    for a, b, _ in plan_tables["segments"]:
        for x in range(a, min(b, a + edge)):
            rows.add(int(x))
        for x in range(max(a, b - edge), b):
            rows.add(int(x))
    for tb, te, _, _ in plan_tables["epochs"]:
        rows.update({int(tb), int(te - 1)})
    return np.array(sorted(r for r in rows if 0 <= r < T), np.int64)


def boundary_rows(plan_tables, T, rng, n_random, edge=2):
    """Rows next to every segment / stretch boundary plus seeded random rows."""
    rows = set(edge_rows(plan_tables, T, edge).tolist())
    rows.update(int(x) for x in rng.integers(0, T, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < T))


SEEDED_ROWS = {2: 192, 3: 1024, 4: 1024}   # seeded random rows drawn per full-size workload


def full_size_rows(plan_tables, T, cfg, part, parts, edge=2):
    """Rows one part of a full-size parity check covers: the stretches of the
    workload are split into `parts` consecutive ranges; a part takes every edge row
    (edge_rows) and every seeded row (SEEDED_ROWS[cfg] draws from
    default_rng(cfg)) inside its range.  Returns (rows, edge rows in the part,
    seeded rows in the part, (first stretch, last stretch + 1))."""
    ep = plan_tables["epochs"]
    s0, s1 = part * len(ep) // parts, (part + 1) * len(ep) // parts
    lo, hi = int(ep[s0][0]), int(ep[s1 - 1][1])
    edges = edge_rows(plan_tables, T, edge)
    seeded = np.unique(np.random.default_rng(cfg).integers(0, T, SEEDED_ROWS[cfg]))
    e_part = edges[(edges >= lo) & (edges < hi)]
    s_part = seeded[(seeded >= lo) & (seeded < hi)]
    return np.union1d(e_part, s_part), e_part, s_part, (s0, s1)


def oracle_threads():
    """Threads for the oracle's pool: the host's share of cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


class Bf16Rows:
    """Read-only view of a bf16-bits array that decodes rows to float64 on indexing
    (lets the oracle read a few rows of a multi-GB input)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return workload.bf16_bits_to_f32(self.bits[idx]).astype(np.float64)


def dev_int(a) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
