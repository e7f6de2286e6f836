"""GPU parity: every libakv kernel against the CPU oracle on the same seeded inputs.

Tolerances (written here; each follows from the roundings of the kernel's arithmetic):
  bf16 attention / decode outputs  max-abs 2e-2
  fp32 attention                   max-abs 1e-5 (also lse)
  fp32 repos / RoPE                max-abs 1e-5
  bf16 repos / RoPE                <= 1 bf16 ulp of the exact value + 1e-6 x |pair| (fp32
                                   evaluation), and rounding disagreements with the exactly
                                   rounded value rare (round-to-nearest-even)
  bf16 versions (two roundings)    |err| <= 2^-7 * |rotated pair|; values bit-exact
Output buffers start as NaN so unwritten rows fail.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from segmented_attention_seq_amd import akv, workload
from threadpoolctl import threadpool_limits

from tests.gpu_helpers import (Bf16Rows, as_f64, boundary_rows, dev_int, dev_tensor, full_size_rows,
                               host_bf16_bits, host_f64, nan_like, oracle_threads)

pytestmark = pytest.mark.gpu
BASE = workload.ROPE_BASE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[gpu] {torch.cuda.get_device_name(0)} lib={akv.lib_path()}", flush=True)


def _ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _bf16_rot_bound(exact, layout=akv.ROPE_HALF):
    """One bf16 ulp of the exact element plus the float32 evaluation error of the
    rotation (angle ~3e-7 rad after fp64 reduction, products ~1e-7), which scales
    with the norm of the element's pair, not with the element itself: an element
    that cancels to ~0 cannot be within one of its own tiny ulps."""
    if layout == akv.ROPE_HALF:
        h = exact.shape[-1] // 2
        pn = np.sqrt(exact[..., :h] ** 2 + exact[..., h:] ** 2)
        pn = np.concatenate([pn, pn], axis=-1)
    else:
        pn = np.sqrt(exact[..., 0::2] ** 2 + exact[..., 1::2] ** 2)
        pn = np.repeat(pn, 2, axis=-1)
    return _ulp_bf16(exact) + 1e-6 * pn


# ---------------------------------------------------------------- RoPE / repos

@pytest.mark.parametrize("layout", [akv.ROPE_HALF, akv.ROPE_INTERLEAVED])
def test_repos_fp32_large_shifts(layout):
    rng = np.random.default_rng(11)
    rows, n, H, d = 5000, 3000, 8, 64
    k = rng.standard_normal((rows, H, d)).astype(np.float32)
    g = rng.integers(0, rows, n).astype(np.int32)
    pf = rng.integers(0, 1 << 20, n).astype(np.int32)
    pt = rng.integers(0, 1 << 20, n).astype(np.int32)
    out = nan_like((n, H, d), torch.float32)
    akv.rope_repos(out, dev_tensor(k, False), dev_int(pt), dev_int(pf),
                   dev_int(g), BASE, layout)
    ref = oracle.repos(k[g], pf, pt, BASE, layout)
    err = np.abs(host_f64(out) - ref).max()
    print(f"[repos fp32 layout={layout}] max-abs {err:.2e}")
    assert err <= 1e-5


# Head dims 16-128 run one thread per (row, head, 8-pair chunk) with the angles
# shared by cross-lane shuffle among groups of 8 heads; other dims (48 here) walk all
# heads per thread.  Head counts that are not multiples of 8 leave idle lanes in the
# last head group.
@pytest.mark.parametrize("d,H", [(16, 3), (32, 8), (48, 5), (64, 1), (64, 12), (128, 9)])
@pytest.mark.parametrize("layout", [akv.ROPE_HALF, akv.ROPE_INTERLEAVED])
def test_repos_fp32_head_dims_and_counts(d, H, layout):
    rng = np.random.default_rng(1000 + d + H)
    rows, n = 700, 513
    k = rng.standard_normal((rows, H, d)).astype(np.float32)
    g = rng.integers(0, rows, n).astype(np.int32)
    pf = rng.integers(0, 1 << 20, n).astype(np.int32)
    pt = rng.integers(0, 1 << 20, n).astype(np.int32)
    out = nan_like((n, H, d), torch.float32)
    akv.rope_repos(out, dev_tensor(k, False), dev_int(pt), dev_int(pf), dev_int(g), BASE, layout)
    ref = oracle.repos(k[g], pf, pt, BASE, layout)
    err = np.abs(host_f64(out) - ref).max()
    print(f"[repos fp32 d={d} H={H} layout={layout}] max-abs {err:.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("n", [1, 2, 3, 257])
def test_repos_writes_exactly_its_rows(n):
    """Rows are handled in groups of two; a group past the last row must store
    nothing: the output is a view into a larger buffer whose tail stays untouched."""
    rng = np.random.default_rng(40 + n)
    H, d = 8, 64
    k = rng.standard_normal((300, H, d)).astype(np.float32)
    g = rng.integers(0, 300, n).astype(np.int32)
    pf = rng.integers(0, 5000, n).astype(np.int32)
    pt = rng.integers(0, 5000, n).astype(np.int32)
    full = nan_like((n + 4, H, d), torch.float32)
    akv.rope_repos(full[:n], dev_tensor(k, False), dev_int(pt), dev_int(pf), dev_int(g), BASE)
    ref = oracle.repos(k[g], pf, pt, BASE)
    got = host_f64(full)
    assert np.abs(got[:n] - ref).max() <= 1e-5
    assert np.isnan(got[n:]).all()


def test_repos_bf16_one_ulp_and_rne():
    rng = np.random.default_rng(12)
    n, H, d = 4000, 8, 64
    kb = workload.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
    pf = rng.integers(0, 200_000, n).astype(np.int32)
    pt = rng.integers(0, 100_000, n).astype(np.int32)
    out = nan_like((n, H, d), torch.bfloat16)
    akv.rope_repos(out, dev_tensor(kb, True), dev_int(pt), dev_int(pf))
    exact = oracle.repos(as_f64(kb, True), pf, pt, BASE)
    ref_bits = oracle.f64_to_bf16_bits(exact)
    got = host_f64(out)
    assert np.all(np.abs(got - exact) <= _bf16_rot_bound(exact))
    mism = np.mean(host_bf16_bits(out) != ref_bits)
    print(f"[repos bf16] rounding disagreements {mism:.4%}")
    assert mism < 0.01


@pytest.mark.parametrize("bf16", [False, True])
def test_kv_reuse_copies_and_converts_positions(bf16):
    """Reuse path of a cache hit (review, serving system, extended radix tree:
    same position index -> reuse as is, different -> convert by key rotation):
    gathered keys are rotated to their new positions and values copied bit for bit;
    rows whose position is unchanged come out bit-identical."""
    rng = np.random.default_rng(31 + bf16)
    rows, n, H, d = 6000, 4000, 8, 64
    k = rng.standard_normal((rows, H, d)).astype(np.float32)
    v = rng.standard_normal((rows, H, d)).astype(np.float32)
    if bf16:
        k, v = workload.f32_to_bf16_bits(k), workload.f32_to_bf16_bits(v)
    g = rng.permutation(rows)[:n].astype(np.int32)
    pf = rng.integers(0, 150_000, n).astype(np.int32)
    pt = rng.integers(0, 150_000, n).astype(np.int32)
    same = rng.random(n) < 0.25
    pt[same] = pf[same]                      # a quarter of the rows keep their position
    dt = torch.bfloat16 if bf16 else torch.float32
    ko, vo = nan_like((n, H, d), dt), nan_like((n, H, d), dt)
    kp, vp = dev_tensor(k, bf16), dev_tensor(v, bf16)
    akv.kv_reuse(ko, vo, kp, vp, dev_int(g), dev_int(pf), dev_int(pt), BASE)
    torch.cuda.synchronize()
    exact = oracle.repos(as_f64(k, bf16)[g], pf, pt, BASE)
    got = host_f64(ko)
    if bf16:
        assert np.all(np.abs(got - exact) <= _bf16_rot_bound(exact))
        assert np.array_equal(host_bf16_bits(vo), v[g])
        assert np.array_equal(host_bf16_bits(ko)[same], k[g][same])
    else:
        assert np.abs(got - exact).max() <= 1e-5
        assert np.array_equal(vo.cpu().numpy(), v[g])
        assert np.array_equal(ko.cpu().numpy()[same], k[g][same])


def test_kv_reuse_rejects_bad_arguments():
    x = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(akv.AkvError):
        akv.kv_reuse(x, x.clone(), x, x.clone(), idx, idx, idx)   # k_out aliases k_pool


@pytest.mark.parametrize("bf16", [True, False])
def test_rope_apply_and_versions(bf16):
    tr = workload.agent_trajectory(4, seed=21, total=900, keep=2, repos="every",
                                   user_len=50, assist_range=(20, 90), tool_range=(60, 200))
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    t = plan.tables()
    T, H, d = tr.n_tokens, 8, 64
    _, k, v = workload.prefill_tensors(T, 1, H, d, seed=22, bf16=bf16)
    kd, vd = dev_tensor(k, bf16), dev_tensor(v, bf16)
    kr = torch.empty_like(kd)
    akv.rope_apply(plan, kr, kd)
    kexact = oracle.rope(as_f64(k, bf16), t["tok_pos"], BASE)
    nv = plan.info["n_versions"]
    assert nv > 0
    kv, vv = nan_like((nv, H, d), kd.dtype), nan_like((nv, H, d), kd.dtype)
    akv.build_kv_versions(plan, kr, vd, kv, vv)
    src, to = t["versions"][:, 0], t["versions"][:, 2]
    vexact = oracle.rope(as_f64(k, bf16)[src], to, BASE)
    if bf16:
        assert np.all(np.abs(host_f64(kr) - kexact) <= _bf16_rot_bound(kexact))
        # versions round twice (append position, then the repos shift)
        pair = np.sqrt(vexact[..., :32] ** 2 + vexact[..., 32:] ** 2)
        bound = 2.0 ** -7 * np.concatenate([pair, pair], axis=-1) + 1e-30
        assert np.all(np.abs(host_f64(kv) - vexact) <= bound)
        assert np.array_equal(host_bf16_bits(vv), v[src])
    else:
        assert np.abs(host_f64(kr) - kexact).max() <= 1e-5
        assert np.abs(host_f64(kv) - vexact).max() <= 1e-5
        assert np.array_equal(vv.cpu().numpy(), v[src])


def test_repos_workload_96k_keys():
    """Batched repos of 96,000 surviving keys (gathered from a pool with NaN holes)."""
    for bf16 in (True, False):
        rb = workload.repos_batch(bf16=bf16)
        dt = torch.bfloat16 if bf16 else torch.float32
        pool = nan_like((rb.pool_slots, rb.hkv, rb.d), dt)
        pool[torch.from_numpy(rb.slots.astype(np.int64)).cuda()] = dev_tensor(rb.k_rows, bf16)
        out = nan_like((rb.slots.size, rb.hkv, rb.d), dt)
        akv.rope_repos(out, pool, dev_int(rb.pos_to), dev_int(rb.pos_from),
                       dev_int(rb.slots))
        exact = oracle.repos(as_f64(rb.k_rows, bf16), rb.pos_from, rb.pos_to, BASE)
        got = host_f64(out)
        if bf16:
            assert np.all(np.abs(got - exact) <= _bf16_rot_bound(exact))
        else:
            err = np.abs(got - exact).max()
            print(f"[repos 96k fp32] max-abs {err:.2e}")
            assert err <= 1e-5


# ---------------------------------------------------------------- segment attention

def _run_restore(tr, hq, hkv, d, bf16, seed, layout=akv.ROPE_HALF, lse=True, bq=64):
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition), bq=bq)
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, hkv, d, seed=seed, bf16=bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    T = tr.n_tokens
    bufs = {"out": nan_like((T, hq, d), dt), "lse": nan_like((T, hq), torch.float32)}
    out, l = akv.restore(plan, dev_tensor(q, bf16), dev_tensor(k, bf16), dev_tensor(v, bf16),
                         BASE, layout, with_lse=lse, bufs=bufs)
    torch.cuda.synchronize()
    return plan, (q, k, v), out, l


def _check_rows(tr, qkv, out, lse, bf16, rows=None, layout=akv.ROPE_HALF, tol=None):
    q, k, v = qkv
    ops = oracle.canonical_ops(tr.msg_len, tr.drop, tr.reposition)
    view = (lambda a: Bf16Rows(a)) if bf16 else (lambda a: a)
    sel = np.arange(tr.n_tokens) if rows is None else np.asarray(rows, np.int64)
    with threadpool_limits(1):   # the oracle's own pool spreads heads and key blocks
        o_ref, l_ref = oracle.segment_attention(view(q), view(k), view(v), ops, base=BASE, layout=layout,
                                                rows=sel, compact=True, threads=oracle_threads())
    idx = torch.from_numpy(sel).cuda()
    got = host_f64(out[idx])
    err = np.abs(got - o_ref).max()
    lerr = np.abs(host_f64(lse[idx]) - l_ref).max()
    tol = tol if tol is not None else (2e-2 if bf16 else 1e-5)
    print(f"[attn {tr.name or 'traj'} bf16={bf16} rows={sel.size}] max-abs {err:.3e} lse {lerr:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol
    assert lerr <= (2e-2 if bf16 else 1e-5)


# The restore path rotates the raw queries inside the attention (akv.restore default);
# the separate RoPE-apply of Q into a rotated copy is the other form.  Both must meet
# the oracle, and the fused form rounds Q to bf16 once instead of twice, so its error
# is no larger (a small margin covers summation-order noise).
@pytest.mark.parametrize("bf16,hq,hkv,layout", [(True, 64, 8, akv.ROPE_HALF), (True, 16, 4, akv.ROPE_INTERLEAVED),
                                                (False, 4, 2, akv.ROPE_HALF), (False, 6, 2, akv.ROPE_INTERLEAVED)])
def test_query_rotation_inside_attention(bf16, hq, hkv, layout):
    tr = workload.agent_trajectory(4, seed=61, total=1400, keep=2, repos="every", user_len=40,
                                   assist_range=(20, 120), tool_range=(80, 300))
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, hkv, 64, seed=62, bf16=bf16)
    ops = oracle.canonical_ops(tr.msg_len, tr.drop, tr.reposition)
    view = (lambda a: Bf16Rows(a)) if bf16 else (lambda a: a)
    o_ref, l_ref = oracle.segment_attention(view(q), view(k), view(v), ops, base=BASE, layout=layout)
    errs = {}
    for fuse in (True, False):
        out, lse = akv.restore(plan, dev_tensor(q, bf16), dev_tensor(k, bf16), dev_tensor(v, bf16), BASE, layout,
                               with_lse=True, fuse_q=fuse)
        torch.cuda.synchronize()
        errs[fuse] = (np.abs(host_f64(out) - o_ref).max(), np.abs(host_f64(lse) - l_ref).max())
    print(f"[q rotation in attention bf16={bf16} layout={layout}] fused {errs[True]} separate {errs[False]}")
    tol = 2e-2 if bf16 else 1e-5
    for e, le in errs.values():
        assert e <= tol and le <= tol
    assert errs[True][0] <= errs[False][0] * 1.25 + (1e-4 if bf16 else 1e-7)


def test_tiny_request_example_fp32():
    tr = workload.config_trajectory(1)
    plan, qkv, out, lse = _run_restore(tr, 1, 1, 64, bf16=False, seed=1)
    _check_rows(tr, qkv, out, lse, bf16=False)


@pytest.mark.parametrize("seed", [31, 32, 33])
def test_random_small_fp32(seed):
    tr = workload.agent_trajectory(5, seed=seed, total=700, keep=2, repos="every" if seed % 2 else "none",
                                   user_len=30, assist_range=(10, 60), tool_range=(40, 150))
    plan, qkv, out, lse = _run_restore(tr, 4, 2, 64, bf16=False, seed=seed)
    _check_rows(tr, qkv, out, lse, bf16=False)


SMALL = [
    # rounds, total, keep, repos, hq, hkv
    (3, 1500, 1, "every", 64, 8),
    (6, 2300, 2, "none", 64, 8),
    (8, 3100, 3, "every", 16, 4),
    (5, 1234, 1, "every", 8, 8),
    (4, 999, 2, "every", 16, 8),
    (4, 2000, 1, "every", 32, 8),   # 4 query heads per kv head: two kv heads per workgroup
    (5, 1600, 2, "every", 12, 3),   # 4 per kv head with an odd kv head count: one-wave-per-head kernel
    (3, 1200, 1, "every", 128, 16),  # 8 per kv head over 16 kv heads
    (3, 900, 2, "every", 8, 1),      # 8 query heads over a single kv head
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_random_small_bf16(case):
    rounds, total, keep, repos, hq, hkv = SMALL[case]
    tr = workload.agent_trajectory(rounds, seed=40 + case, total=total, keep=keep, repos=repos,
                                   user_len=64, assist_range=(30, 200), tool_range=(100, 500),
                                   name=f"small{case}")
    plan, qkv, out, lse = _run_restore(tr, hq, hkv, 64, bf16=True, seed=50 + case)
    _check_rows(tr, qkv, out, lse, bf16=True)


def test_interleaved_layout_bf16():
    tr = workload.agent_trajectory(3, seed=61, total=800, keep=1, repos="every", user_len=40,
                                   assist_range=(30, 100), tool_range=(100, 300))
    plan, qkv, out, lse = _run_restore(tr, 16, 2, 64, bf16=True, seed=62, layout=akv.ROPE_INTERLEAVED)
    _check_rows(tr, qkv, out, lse, bf16=True, layout=akv.ROPE_INTERLEAVED)


EDGE = {
    "single-token-messages": workload.Trajectory([1] * 9, ["x"] * 9, {3: [0, 1], 6: [2, 4]}, [3, 6, 8]),
    "drop-everything": workload.Trajectory([70, 5, 80], ["x"] * 3, {0: [0], 1: [1]}, [1]),
    "zero-length-and-repeats": workload.Trajectory([65, 0, 0, 130, 1], ["x"] * 5,
                                                   {1: [0, 0], 2: [1], 3: [0]}, [1, 2, 2, 3]),
    "final-boundary-only": workload.Trajectory([100, 29], ["x"] * 2, {1: [0, 1]}, [1]),
    "no-ops": workload.Trajectory([129, 64, 63], ["x"] * 3, {}, []),
}


@pytest.mark.parametrize("hq,bq", [(16, 64), (8, 64), (4, 256), (2, 512)])
@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases_bf16(name, hq, bq):
    tr = EDGE[name]
    tr.name = name
    plan, qkv, out, lse = _run_restore(tr, hq, 2, 64, bf16=True, seed=71, bq=bq)
    _check_rows(tr, qkv, out, lse, bf16=True)


@pytest.mark.parametrize("repos", [False, True])
def test_short_items_every_tile_count(repos):
    """Work items of 1 to 8 key tiles on the 8-head kernel, so that each one starts
    and ends its tile ring differently (the prologue's copies, copies past the
    last tile, the final waits): eight 64-token query tiles of one stretch, or a
    repos after the first 256 tokens, whose version rows give a second stretch
    with PARTIAL and ragged tiles.  Every row is checked, and the fused staging
    equals the version buffers bit for bit."""
    lens, rp = ([512], []) if not repos else ([256, 256], [0])
    tr = workload.Trajectory(lens, ["x"] * len(lens), {}, rp, name=f"short-items-{repos}")
    q, k, v = workload.prefill_tensors(tr.n_tokens, 16, 2, 64, seed=81)
    plan, ((o0, l0), (o1, l1)) = _restore_both(tr, q, k, v, 16, 2)
    counts = set(np.diff(plan.tables()["tile_ptr"]).tolist())
    assert set(range(1, 5)) <= counts and (repos or set(range(1, 9)) <= counts)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    _check_rows(tr, (q, k, v), o0, l0, bf16=True)


@pytest.mark.parametrize("repos", [False, True])
def test_two_kv_heads_per_workgroup_every_tile_count(repos):
    """4 query heads per kv head run the ping-pong kernel with two kv heads per
    workgroup (each slot of the tile ring holds both heads' tiles): work items of 1
    to 8 key tiles, with and without version rows, every row checked."""
    lens, rp = ([512], []) if not repos else ([256, 256], [0])
    tr = workload.Trajectory(lens, ["x"] * len(lens), {}, rp, name=f"two-heads-{repos}")
    plan, qkv, out, lse = _run_restore(tr, 8, 2, 64, bf16=True, seed=83)
    counts = set(np.diff(plan.tables()["tile_ptr"]).tolist())
    assert set(range(1, 5)) <= counts and (repos or set(range(1, 9)) <= counts)
    _check_rows(tr, qkv, out, lse, bf16=True)


# (query heads, kv heads, plan bq): 4, 2 and 1 query heads per kv head with query
# tiles of 64 * 8 / group tokens, cut into 8 / group parts of the ping-pong kernel
PARTS = [(8, 2, 128), (4, 2, 256), (2, 2, 512), (32, 8, 128), (16, 8, 256), (8, 8, 512), (12, 3, 128), (32, 16, 256)]


@pytest.mark.parametrize("hq,hkv,bq", PARTS[:3])
@pytest.mark.parametrize("repos", [False, True])
def test_query_tile_parts_every_tile_count(repos, hq, hkv, bq):
    """Query tiles of 128, 256 or 512 tokens cut into 64-token parts, one part per
    wave group: work items of many tile counts, parts past a ragged item end, PARTIAL
    tiles that are EMPTY for some parts, every row checked."""
    lens, rp = ([1100], []) if not repos else ([530, 610], [0])
    tr = workload.Trajectory(lens, ["x"] * len(lens), {}, rp, name=f"parts-{bq}-{repos}")
    plan, qkv, out, lse = _run_restore(tr, hq, hkv, 64, bf16=True, seed=84, bq=bq)
    assert plan.info["bq"] == bq
    _check_rows(tr, qkv, out, lse, bf16=True)


@pytest.mark.parametrize("hq,hkv,bq", PARTS)
def test_query_tile_parts_random_plans(hq, hkv, bq):
    tr = workload.agent_trajectory(5, seed=90 + bq + hq, total=2100, keep=1, repos="every" if hq % 3 else "none",
                                   user_len=64, assist_range=(30, 200), tool_range=(100, 500),
                                   name=f"parts-rand-{hq}-{hkv}-{bq}")
    plan, qkv, out, lse = _run_restore(tr, hq, hkv, 64, bf16=True, seed=91, bq=bq)
    _check_rows(tr, qkv, out, lse, bf16=True)


def test_empty_plan_and_unsupported():
    plan = akv.build_visibility([])
    x = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    akv.segment_attention(plan, torch.empty((0, 64, 64), dtype=torch.bfloat16, device="cuda"), x, x, None,
                          None, torch.empty((0, 64, 64), dtype=torch.bfloat16, device="cuda"))
    p16 = akv.build_visibility([(akv.OP_APPEND, 10)], bq=16, bk=16)
    q = torch.zeros((10, 8, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((10, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(akv.AkvError) as e:
        akv.segment_attention(p16, q, kv, kv, None, None, torch.empty_like(q))
    assert e.value.status == akv.EUNSUPPORTED
    p = akv.build_visibility([(akv.OP_APPEND, 10)])
    q3 = torch.zeros((10, 3, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(akv.AkvError) as e:
        akv.segment_attention(p, q3, kv, kv, None, None, torch.empty_like(q3))
    assert e.value.status == akv.EUNSUPPORTED
    # query tiles of 64 * 8 / group tokens only: not 128 for 8 or 2 query heads per kv head
    p128 = akv.build_visibility([(akv.OP_APPEND, 10)], bq=128)
    for heads in (8, 2):
        qh = torch.zeros((10, heads, 64), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(akv.AkvError) as e:
            akv.segment_attention(p128, qh, kv, kv, None, None, torch.empty_like(qh))
        assert e.value.status == akv.EUNSUPPORTED


def test_deterministic():
    tr = workload.agent_trajectory(3, seed=81, total=1500, keep=1, repos="every", user_len=64,
                                   assist_range=(30, 200), tool_range=(100, 500))
    _, _, a, la = _run_restore(tr, 64, 8, 64, bf16=True, seed=82)
    _, _, b, lb = _run_restore(tr, 64, 8, 64, bf16=True, seed=82)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@functools.lru_cache(maxsize=1)
def _workload(cfg):
    return workload.config_prefill(cfg)


@functools.lru_cache(maxsize=1)
def _restored(cfg):
    """The full-size restore of workload cfg in the launch bench.py times (raw
    queries rotated inside the attention), outputs NaN-initialised."""
    tr, q, k, v = _workload(cfg)
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    T, hq, d = q.shape
    bufs = {"out": nan_like((T, hq, d), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
    out, lse = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                           with_lse=True, bufs=bufs)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    return tr, (q, k, v), plan.tables(), out, lse


# (workload, part, parts): the stretches of a workload are split into `parts`
# consecutive ranges so each test's oracle work stays bounded; together the parts
# check every row next to a segment or stretch boundary (32, 352 and 800 rows) and
# the seeded rows (tests/test_plan_host.py checks the cover).
FULL_SIZE_PARTS = [(2, 0, 1), (3, 0, 3), (3, 1, 3), (3, 2, 3), (4, 0, 4), (4, 1, 4), (4, 2, 4), (4, 3, 4)]


@pytest.mark.parametrize("cfg,part,parts", FULL_SIZE_PARTS)
def test_workloads_full_size_boundary_and_seeded_rows(cfg, part, parts):
    """The three prefill workloads at full size: the oracle checks every row within
    two rows of a segment boundary (a dropped entry must stay visible to the
    segments that used it and be hidden from later ones), the first and last row of
    every repos stretch, and seeded random rows; this part covers a range of
    stretches."""
    tr, qkv, tables, out, lse = _restored(cfg)
    T = tr.n_tokens
    rows, e_part, s_part, (s0, s1) = full_size_rows(tables, T, cfg, part, parts)
    print(f"[cfg{cfg} part {part + 1}/{parts}] T={T} stretches {s0}..{s1 - 1}: {e_part.size} boundary rows, "
          f"{s_part.size} seeded rows", flush=True)
    assert e_part.size > 0
    _check_rows(tr, qkv, out, lse, bf16=True, rows=rows)
    if part == 0:
        # bench.py's own call passes no lse: the same output bit for bit
        q, k, v = qkv
        plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
        o2, l2 = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                             bufs={"out": nan_like(tuple(out.shape), torch.bfloat16)})
        torch.cuda.synchronize()
        assert l2 is None and torch.equal(out.view(torch.int16), o2.view(torch.int16))
        del o2


# (query heads, kv heads, plan bq, fused version rows, bf16): one case per kernel form
NO_LSE = [(16, 2, 64, False, True), (16, 2, 64, True, True), (8, 2, 64, False, True), (8, 2, 128, False, True),
          (8, 2, 128, True, True), (4, 2, 64, False, True), (2, 2, 512, True, True), (12, 3, 64, False, True),
          (16, 2, 64, False, False)]


@pytest.mark.parametrize("hq,hkv,bq,fused,bf16", NO_LSE)
def test_output_without_lse_is_the_same(hq, hkv, bq, fused, bf16):
    """Without an lse buffer (the way bench.py calls the attention) every kernel form
    writes the same output bit for bit as with one."""
    tr = workload.agent_trajectory(4, seed=141, total=1700, keep=1, repos="every", user_len=50,
                                   assist_range=(20, 200), tool_range=(60, 400), name="no-lse")
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition), bq=bq)
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, hkv, 64, seed=142, bf16=bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    res = []
    for with_lse in (True, False):
        bufs = {"out": nan_like((tr.n_tokens, hq, 64), dt), "lse": nan_like((tr.n_tokens, hq), torch.float32)}
        out, lse = akv.restore(plan, dev_tensor(q, bf16), dev_tensor(k, bf16), dev_tensor(v, bf16), BASE,
                               with_lse=with_lse, bufs=bufs, fused_versions=fused)
        torch.cuda.synchronize()
        res.append((out, lse, bufs["lse"]))
    (o1, l1, _), (o2, l2, lb2) = res
    assert plan.info["n_versions"] > 0 and l2 is None
    assert torch.equal(o1.view(torch.int32 if not bf16 else torch.int16), o2.view(torch.int32 if not bf16 else torch.int16))
    assert torch.isnan(lb2).all()   # the lse buffer the call was not given stays untouched
    _check_rows(tr, (q, k, v), o1, l1, bf16=bf16)


# ---------------------------------------------------------------- fused version rows

def _restore_both(tr, q, k, v, hq, hkv, layout=akv.ROPE_HALF, bq=64):
    """The same restore with version buffers and with version rows rotated while
    key tiles are staged."""
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition), bq=bq)
    T = tr.n_tokens
    res = []
    for fused in (False, True):
        bufs = {"out": nan_like((T, hq, 64), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
        out, lse = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE, layout,
                               with_lse=True, bufs=bufs, fused_versions=fused)
        torch.cuda.synchronize()
        res.append((out, lse))
    return plan, res


@pytest.mark.parametrize("seed,layout,keep", [(171, akv.ROPE_HALF, 1), (172, akv.ROPE_INTERLEAVED, 2),
                                              (173, akv.ROPE_HALF, 3), (174, akv.ROPE_HALF, 0)])
def test_fused_versions_equal_version_buffers(seed, layout, keep):
    """Version rows rotated at staging time equal the version-buffer path bit for
    bit (the same rotation arithmetic, the same attention), on trajectories with a
    repos after every round, rolling drops (PARTIAL tiles) and ragged tails; and
    both meet the oracle."""
    tr = workload.agent_trajectory(5, seed=seed, total=2600, keep=keep, repos="every", user_len=50,
                                   assist_range=(20, 200), tool_range=(60, 500), name=f"fused{seed}")
    q, k, v = workload.prefill_tensors(tr.n_tokens, 16, 2, 64, seed=seed + 1)
    plan, ((o0, l0), (o1, l1)) = _restore_both(tr, q, k, v, 16, 2, layout)
    assert plan.info["n_versions"] > 0 and plan.info["n_runs"] > 1
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)
    _check_rows(tr, (q, k, v), o1, l1, bf16=True, layout=layout)


@pytest.mark.parametrize("hq,hkv,bq,layout", [(8, 2, 128, akv.ROPE_HALF), (4, 2, 256, akv.ROPE_INTERLEAVED),
                                             (2, 2, 512, akv.ROPE_HALF), (12, 3, 128, akv.ROPE_HALF)])
def test_fused_versions_query_tile_parts(hq, hkv, bq, layout):
    """4, 2 and 1 query heads per kv head over query-tile parts with version rows
    rotated at staging time: bit for bit the version-buffer path, and the oracle."""
    tr = workload.agent_trajectory(5, seed=175 + hq, total=2300, keep=2, repos="every", user_len=50,
                                   assist_range=(20, 200), tool_range=(60, 500), name=f"fused-parts{bq}")
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, hkv, 64, seed=176 + hq)
    plan, ((o0, l0), (o1, l1)) = _restore_both(tr, q, k, v, hq, hkv, layout, bq=bq)
    assert plan.info["n_versions"] > 0 and plan.info["n_runs"] > 1
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)
    _check_rows(tr, (q, k, v), o1, l1, bf16=True, layout=layout)


@pytest.mark.parametrize("cfg", [3, 4])
def test_fused_versions_workloads_full_size(cfg):
    """The 300k (7 repos stretches) and 192k (200 stretches) restores with version
    rows rotated at staging time: the whole output equals the version-buffer path's
    bit for bit (that path is checked on every boundary row in
    test_workloads_full_size_boundary_and_seeded_rows), and the first stretch range
    with version rows is checked against the oracle directly."""
    tr, qkv, tables, out_ref, lse_ref = _restored(cfg)
    q, k, v = qkv
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    T, hq, d = q.shape
    bufs = {"out": nan_like((T, hq, d), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
    out, lse = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                           with_lse=True, bufs=bufs, fused_versions=True)
    torch.cuda.synchronize()
    print(f"[cfg{cfg} fused] version rows {plan.info['n_versions']}, runs {plan.info['n_runs']}", flush=True)
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
    parts = {3: 3, 4: 4}[cfg]
    rows, e_part, s_part, _ = full_size_rows(tables, T, cfg, 1, parts)
    _check_rows(tr, qkv, out, lse, bf16=True, rows=rows)


def test_fused_versions_rejects_unsupported():
    tr = workload.agent_trajectory(2, seed=181, total=400, keep=1, repos="every", user_len=20,
                                   assist_range=(20, 60), tool_range=(40, 120))
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition))
    q, k, v = workload.prefill_tensors(tr.n_tokens, 8, 2, 64, seed=182)
    out = nan_like((tr.n_tokens, 8, 64), torch.bfloat16)
    with pytest.raises(akv.AkvError) as e:   # 4 query heads per kv head with 64-token query tiles
        akv.segment_attention_fused(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), out)
    assert e.value.status == akv.EUNSUPPORTED
    q8 = workload.prefill_tensors(tr.n_tokens, 16, 2, 64, seed=183)[0]
    out8 = nan_like((tr.n_tokens, 16, 64), torch.bfloat16)
    assert akv.rot_table_bytes(plan, 64) == plan.info["n_runs"] * 32 * 8 > 0
    short = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(akv.AkvError) as e:
        akv.segment_attention_fused(plan, dev_tensor(q8, True), dev_tensor(k, True), dev_tensor(v, True), out8,
                                    ws=short)
    assert e.value.status == akv.EINVAL


@pytest.mark.parametrize("hq,bq", [(32, 64), (16, 64), (8, 64), (32, 128), (16, 256), (8, 512)])
def test_48k_workload_smaller_head_groups_sampled(hq, bq):
    """The 48k restore with 4, 2 and 1 query heads per kv head at full size, checked
    on boundary and seeded rows: with 64-token query tiles (two kv heads per
    ping-pong workgroup for 4, else the one-wave-per-head kernel) and with query
    tiles of 64 * 8 / group tokens in parts."""
    tr = workload.config_trajectory(2)
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, 8, 64, seed=300 + hq)
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition), bq=bq)
    T = tr.n_tokens
    bufs = {"out": nan_like((T, hq, 64), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
    out, lse = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                           with_lse=True, bufs=bufs)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    rows = boundary_rows(plan.tables(), T, np.random.default_rng(hq), 48, edge=1)
    _check_rows(tr, (q, k, v), out, lse, bf16=True, rows=rows)

# ---------------------------------------------------------------- decode

def _decode_case(batch, lo, hi, seed, hq=64, hkv=8, shuffle=False):
    db = workload.decode_batch(batch=batch, lo=lo, hi=hi, seed=seed, hq=hq, hkv=hkv, shuffle_slots=shuffle)
    pool_k = nan_like((db.pool_slots, hkv, db.d), torch.bfloat16)
    pool_v = nan_like((db.pool_slots, hkv, db.d), torch.bfloat16)
    idx = torch.from_numpy(db.indices.astype(np.int64)).cuda()
    pool_k[idx] = dev_tensor(db.k_rows, True)
    pool_v[idx] = dev_tensor(db.v_rows, True)
    out = nan_like((batch, hq, db.d), torch.bfloat16)
    lse = nan_like((batch, hq), torch.float32)
    max_n = int(np.diff(db.indptr).max())
    akv.decode_attention(dev_tensor(db.q, True), pool_k, pool_v, dev_int(db.indptr),
                         dev_int(db.indices), max_n, out, lse)
    # without lse (bench.py's call): the same output bit for bit
    out2 = nan_like((batch, hq, db.d), torch.bfloat16)
    akv.decode_attention(dev_tensor(db.q, True), pool_k, pool_v, dev_int(db.indptr),
                         dev_int(db.indices), max_n, out2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    o_ref, l_ref = oracle.decode(Bf16Rows(db.q)[:], Bf16Rows(db.k_rows), Bf16Rows(db.v_rows), db.indptr)
    err = np.abs(host_f64(out) - o_ref).max()
    lerr = np.abs(host_f64(lse) - l_ref).max()
    print(f"[decode batch={batch} n=[{lo},{hi}) hq={hq}/{hkv} shuffle={shuffle}] max-abs {err:.3e} lse {lerr:.3e}")
    assert err <= 2e-2 and lerr <= 2e-2


@pytest.mark.parametrize("args", [(5, 1, 40, 91, 64, 8), (7, 900, 5000, 92, 64, 8),
                                  (3, 2000, 3000, 93, 16, 4), (4, 1, 3000, 94, 8, 8)])
def test_decode_small(args):
    b, lo, hi, seed, hq, hkv = args
    _decode_case(b, lo, hi, seed, hq, hkv)


# The split kernel cuts all gathered keys of the batch into 256 equal ranges: more
# requests than ranges (several requests per range), fewer keys than ranges (most
# ranges empty), one request spread over every range (256 partials to merge), more
# than 8 kv heads (two head groups per range), and more requests than threads in a
# workgroup (512 with 8 kv heads, 128 with 2), so a range's first request is found
# past the bounds read with N.
@pytest.mark.parametrize("args", [(300, 1, 40, 95, 64, 8), (2, 1, 4, 96, 8, 8), (1, 9000, 9001, 97, 64, 8),
                                  (3, 100, 2000, 98, 32, 16), (700, 1, 40, 99, 64, 8), (300, 1, 60, 100, 16, 2)])
def test_decode_balanced_split_edges(args):
    batch, lo, hi, seed, hq, hkv = args
    _decode_case(batch, lo, hi, seed, hq=hq, hkv=hkv)


def test_decode_zero_key_requests_are_nan():
    """Requests with no keys (first, middle, last) get NaN outputs and -inf lse; the
    other requests of the same batch still match the oracle."""
    db = workload.decode_batch(batch=4, lo=300, hi=4000, seed=131)
    lens = np.diff(db.indptr)
    keep = [0, 2]                 # requests that keep their keys; 1 is emptied, and
    # empty requests are added before the first and after the last
    new_len = [0, lens[0], 0, lens[2], 0]
    srcs = [None, 0, None, 2, None]
    idx = np.concatenate([db.indices[db.indptr[b]:db.indptr[b + 1]] for b in keep])
    indptr = np.concatenate([[0], np.cumsum(new_len)]).astype(np.int32)
    q = np.stack([db.q[b if b is not None else 1] for b in srcs])
    pool_k = nan_like((db.pool_slots, db.hkv, db.d), torch.bfloat16)
    pool_v = nan_like((db.pool_slots, db.hkv, db.d), torch.bfloat16)
    all_idx = torch.from_numpy(db.indices.astype(np.int64)).cuda()
    pool_k[all_idx] = dev_tensor(db.k_rows, True)
    pool_v[all_idx] = dev_tensor(db.v_rows, True)
    B = len(new_len)
    out = torch.zeros((B, db.hq, db.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, db.hq), dtype=torch.float32, device="cuda")
    akv.decode_attention(dev_tensor(q, True), pool_k, pool_v, dev_int(indptr), dev_int(idx),
                         int(max(new_len)), out, lse)
    torch.cuda.synchronize()
    o, l = host_f64(out), host_f64(lse)
    for b in (0, 2, 4):
        assert np.isnan(o[b]).all() and np.isneginf(l[b]).all(), b
    rows = lambda a, b: a[db.indptr[b]:db.indptr[b + 1]]  # noqa: E731
    for b, src in ((1, 0), (3, 2)):
        o_ref, l_ref = oracle.decode(Bf16Rows(db.q[src:src + 1])[:], Bf16Rows(rows(db.k_rows, src)),
                                     Bf16Rows(rows(db.v_rows, src)), np.array([0, lens[src]]))
        err = np.abs(o[b] - o_ref[0]).max()
        print(f"[decode zero-key batch, request {b}] max-abs {err:.3e}")
        assert err <= 2e-2 and np.abs(l[b] - l_ref[0]).max() <= 2e-2


def test_decode_workload_batch14():
    _decode_case(14, 32_000, 96_001, 1005)


def test_decode_workload_shuffled_slots():
    _decode_case(6, 32_000, 96_001, 1006, shuffle=True)


def test_decode_equals_last_prefill_row():
    """Decode of the next token = the last row of a restore over the extended sequence."""
    tr = workload.agent_trajectory(4, seed=101, total=2000, keep=2, repos="every", user_len=64,
                                   assist_range=(30, 200), tool_range=(100, 500))
    ext = workload.Trajectory(tr.msg_len + [1], tr.roles + ["x"], tr.drop, tr.reposition)
    plan, (q, k, v), out, _ = _run_restore(ext, 64, 8, 64, bf16=True, seed=102)
    T = ext.n_tokens
    # decode inputs: rotated q of the new token and the final state's keys, from the GPU restore
    ops = akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition)
    p0 = akv.build_visibility(ops)
    t0 = p0.tables()
    act = t0["final_tok"]
    pos_all = np.concatenate([t0["final_pos"], [p0.info["p_next"]]]).astype(np.int32)
    rows = np.concatenate([act, [T - 1]]).astype(np.int32)
    kd, qd = dev_tensor(k, True), dev_tensor(q, True)
    kfin = torch.empty((rows.size, 8, 64), dtype=torch.bfloat16, device="cuda")
    akv.rope_repos(kfin, kd, dev_int(pos_all), None, dev_int(rows))
    qn = torch.empty((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    akv.rope_repos(qn, qd, dev_int(np.array([p0.info["p_next"]], np.int32)), None,
                   dev_int(np.array([T - 1], np.int32)))
    vfin = dev_tensor(v, True)[torch.from_numpy(rows.astype(np.int64)).cuda()].contiguous()
    o = torch.empty((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    akv.decode_attention(qn, kfin, vfin, torch.tensor([0, rows.size], dtype=torch.int32, device="cuda"),
                         torch.arange(rows.size, dtype=torch.int32, device="cuda"), rows.size, o)
    assert (o[0].float() - out[T - 1].float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("hq,hkv,bq", [(16, 2, 64), (8, 2, 64), (4, 2, 64), (2, 2, 64),
                                       (8, 2, 128), (4, 2, 256), (2, 2, 512)])
@pytest.mark.parametrize("offset", [300.0, -300.0, 600.0, 1000.0])
def test_score_jumps_past_running_max_bf16(offset, hq, hkv, bq):
    """Scores of a block of keys shifted by a common offset C/8 (C/8 * log2 e in the
    kernels' log2 units): +C on the later half of the keys (scores jump far above
    those of earlier tiles) or -C on the first third (early scores far below later
    ones).  In log2 units the shifts are 54 (C = 300), 108 (C = 600) and 180
    (C = 1000).  The ping-pong kernel's fast pass (8 query heads per kv head; 4 with
    two kv heads per workgroup; 4, 2 or 1 over query-tile parts) keeps the exponent
    offset at 0: at -300 every column sum of the early tiles falls under 2^-40, at
    +600 the sums exceed the 2^100 the fast pass accepts and at +1000 exp2 overflows
    float32 to inf, so the work item is redone with the rescaling softmax.  The
    one-wave-per-head kernels (1 and 2 query heads per kv head with 64-token query
    tiles) rescale a tile whenever its column sums leave [2^-40, 2^40], which every
    offset here triggers.  The offset rides on the
    lowest-frequency RoPE pair (i = 31, which turns ~1e-5 rad per position, so it
    is position independent here) with q = 1 on that dimension, so it shifts whole
    blocks of scores without sharpening the softmax within them."""
    tr = workload.agent_trajectory(3, seed=111, total=1400, keep=1, repos="every", user_len=64,
                                   assist_range=(30, 200), tool_range=(100, 500), name=f"jump{offset}")
    plan = akv.build_visibility(akv.ops_from_messages(tr.msg_len, tr.drop, tr.reposition), bq=bq)
    q, k, v = workload.prefill_tensors(tr.n_tokens, hq, hkv, 64, seed=112)
    qf, kf = workload.bf16_bits_to_f32(q), workload.bf16_bits_to_f32(k)
    T = tr.n_tokens
    qf[:, :, 31], qf[:, :, 63] = 1.0, 0.0
    kf[:, :, 31], kf[:, :, 63] = 0.0, 0.0
    if offset > 0:
        kf[T // 2:, :, 31] = offset
    else:
        kf[: T // 3, :, 31] = offset
    q, k = workload.f32_to_bf16_bits(qf), workload.f32_to_bf16_bits(kf)
    bufs = {"out": nan_like((T, hq, 64), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
    out, lse = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                           with_lse=True, bufs=bufs)
    torch.cuda.synchronize()
    ops = oracle.canonical_ops(tr.msg_len, tr.drop, tr.reposition)
    o_ref, l_ref = oracle.segment_attention(Bf16Rows(q), Bf16Rows(k), Bf16Rows(v), ops, base=BASE)
    err = np.abs(host_f64(out) - o_ref).max()
    # lse carries the offset (|lse| up to ~130); the query's one rounding to bf16 of
    # q * scale * log2(e) scales every score by 1 +- 2^-9, so the bound is relative
    lerr = np.abs(host_f64(lse) - l_ref).max()
    lbound = 2e-2 + 2.0 ** -8 * np.abs(l_ref).max()
    print(f"[attn jump offset={offset} hq/hkv={hq}/{hkv} bq={bq}] max-abs {err:.3e} lse {lerr:.3e} (bound {lbound:.3f})")
    assert np.isfinite(host_f64(out)).all()
    assert err <= 2e-2 and lerr <= lbound
    if hq == 8 * hkv or bq * (hq // hkv) == 512:
        # the fused kernel (version rows rotated at staging) redoes the same items
        # and its redo pass rotates them again: bit for bit the version-buffer path
        assert plan.info["n_versions"] > 0
        bufs = {"out": nan_like((T, hq, 64), torch.bfloat16), "lse": nan_like((T, hq), torch.float32)}
        out_f, lse_f = akv.restore(plan, dev_tensor(q, True), dev_tensor(k, True), dev_tensor(v, True), BASE,
                                   with_lse=True, bufs=bufs, fused_versions=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_f.view(torch.int16))
        assert torch.equal(lse, lse_f)
