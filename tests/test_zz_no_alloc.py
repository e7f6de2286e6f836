"""The decode entry point that allocates nothing (akv_decode_attention_noalloc)
against akv_decode_attention on the same inputs, through the C ABI: the same
kernels, so the results must agree bit for bit; two calls in a row, the second
with a smaller batch, so the second reads scratch left by the first."""
import numpy as np
import pytest
import torch

from segmented_attention_seq_amd import akv, workload
from tests.gpu_helpers import dev_int, dev_tensor, nan_like

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _inputs(batch, lo, hi, seed):
    db = workload.decode_batch(batch=batch, lo=lo, hi=hi, seed=seed)
    pool_k = nan_like((db.pool_slots, db.hkv, db.d), torch.bfloat16)
    pool_v = nan_like((db.pool_slots, db.hkv, db.d), torch.bfloat16)
    idx = torch.from_numpy(db.indices.astype(np.int64)).cuda()
    pool_k[idx] = dev_tensor(db.k_rows, True)
    pool_v[idx] = dev_tensor(db.v_rows, True)
    return (dev_tensor(db.q, True), pool_k, pool_v, dev_int(db.indptr), dev_int(db.indices),
            int(np.diff(db.indptr).max()))


def test_noalloc_decode_matches_workspace_decode_twice():
    for batch, lo, hi, seed in ((9, 2000, 30000, 141), (3, 100, 5000, 142)):
        q, pk, pv, indptr, indices, max_n = _inputs(batch, lo, hi, seed)
        B, hq, d = q.shape
        ref = nan_like((B, hq, d), torch.bfloat16)
        ref_l = nan_like((B, hq), torch.float32)
        akv.decode_attention(q, pk, pv, indptr, indices, max_n, ref, ref_l)
        got = nan_like((B, hq, d), torch.bfloat16)
        got_l = nan_like((B, hq), torch.float32)
        akv.decode_attention_noalloc(q, pk, pv, indptr, indices, max_n, got, got_l)
        torch.cuda.synchronize()
        print(f"[noalloc decode batch={batch}] keys={int(indptr[-1].item())}", flush=True)
        assert not torch.isnan(ref).any().item()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(got_l, ref_l)


def test_noalloc_decode_rejects_oversized_batch():
    # (256 + batch) * hq * 66 floats must fit the fixed 16 MiB scratch: 1000 x 64 does not
    B, hq = 1000, 64
    q = torch.zeros((B, hq, 64), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    indptr = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    indices = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, hq, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(akv.AkvError) as e:
        akv.decode_attention_noalloc(q, pool, pool, indptr, indices, 1, out)
    assert e.value.status == akv.EINVAL
