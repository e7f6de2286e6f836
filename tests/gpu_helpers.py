"""Helpers for the GPU parity tests: host arrays <-> device tensors, sampled rows."""
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


def boundary_rows(plan_tables, T, rng, n_random, edge=2):
    """Rows next to every segment / stretch boundary plus seeded random rows."""
    rows = set()
    for a, b, _ in plan_tables["segments"]:
        for x in range(a, min(b, a + edge)):
            rows.add(int(x))
        for x in range(max(a, b - edge), b):
            rows.add(int(x))
    for tb, te, _, _ in plan_tables["epochs"]:
        rows.update({int(tb), int(te - 1)})
    rows.update(int(x) for x in rng.integers(0, T, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < T))


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
