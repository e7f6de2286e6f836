"""Benchmark of the AKV restore hot path on one MI355X.

One step = one pass over every stage of the path on synthetic agent inputs:
  A1  host: operate-after request -> canonical ops -> restore plan; upload
  A2  RoPE-apply of the raw Q and K to their append positions
  A3  KV versions of every repos stretch (rotated keys + copied values)
  A4  segment-batch attention (bf16 MFMA)
  A5  batched repos of 96,000 surviving keys (gathered, p -> q)
  A6  decode: 14 requests x 1 query over 32k-96k gathered active keys each
The restore stages run on the ~300k-token, 100-round trajectory with tool-response
rolling drop (keep 12) and a repos whenever the next position reaches the 96k
window (7 repos stretches, 384,931 version rows; 64/8 GQA heads, d = 64, bf16,
RoPE base 150000), the largest restore workload that fits one GPU, unless
--config picks another.  The host builds each step's plan while the GPU runs the
previous step, and uploads it on a copy stream into one of two device buffers.

Prints one JSON line.  `value` = algorithmic attention FLOP of the restore
(4 * d * Hq * visible pairs) per step / wall time per step (all stages included).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segment-attn restore TFLOP/s (% MFMA peak); repos+decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
ATTN_SRCS = [os.path.join(ROOT, "segmented_attention_seq_amd", "csrc", f)
             for f in ("attention.hip", "internal.h", "rope_angle.h", "plan.cpp")]
TRAFFIC_FILES = {2: os.path.join(ROOT, "profiles", "segment_attention_48k_traffic.md"),
                 3: os.path.join(ROOT, "profiles", "segment_attention_300k_traffic.md"),
                 4: os.path.join(ROOT, "profiles", "segment_attention_192k_traffic.md")}


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4],
                    help="restore workload: 2 = 48k/20 rounds, 3 = ~300k/100 rounds with 96k repos "
                         "window, 4 = 192k/200 rounds with repos every round")
    ap.add_argument("--hq", type=int, default=64, choices=[8, 16, 32, 64],
                    help="query heads of the restore (8 kv heads): 64 is the workloads' 64/8 GQA; "
                         "32, 16 and 8 run the 4-, 2- and 1-head-group kernel on seeded synthetic queries")
    ap.add_argument("--bq", type=int, default=0,
                    help="query tile of the plan (0: the library's choice for the head counts)")
    ap.add_argument("--fused-versions", action="store_true",
                    help="build no version buffers: the attention rotates version rows as it stages key tiles")
    ap.add_argument("--repos-sets", type=int, default=4, help="repos buffer sets rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only", default="", help="comma list of stages to run (profiling aid): "
                                               "restore,repos,decode")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before timing, run an elementwise multiply reading and writing this many MiB "
                         "(3 times) so hardware byte counters can be scaled against a known transfer")
    return ap.parse_args()


def attn_kernel_name(hq, hkv, bq, fused):
    """The segment-attention kernel the library launches for these heads and plan
    query tile (its launcher's choice)."""
    g = hq // hkv
    if g == 8:
        return ("segment attention (seg_attn_bf16_pp, 8 query heads per kv head"
                + (", version rows rotated at staging)" if fused else ")"))
    if bq != 64:
        return (f"segment attention (seg_attn_bf16_pp, {g} query heads per kv head, query tiles of {bq} "
                f"tokens in {bq // 64} parts" + (", version rows rotated at staging)" if fused else ")"))
    if g == 4 and hkv % 2 == 0:
        return "segment attention (seg_attn_bf16_pp, 4 query heads per kv head, two kv heads per workgroup)"
    return f"segment attention (seg_attn_bf16<{g}>)"


def attn_src_hash():
    """Hash of the attention kernel's code: its source, the two local headers it
    includes, and the plan builder (whose work order decides how much of the K/V
    traffic the L2 absorbs), with comments removed and whitespace collapsed, so an
    edit of the comments alone keeps the counters that were taken on the same code."""
    h = hashlib.sha256()
    for path in ATTN_SRCS:
        with open(path) as f:
            code = re.sub(r"/\*.*?\*/", " ", f.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode() + b"\0")
    return h.hexdigest()[:16]


def read_traffic(cfg):
    """HBM bytes per segment-attention launch measured with rocprofv3 counters, if
    the file was taken on this exact kernel source and workload; else None."""
    path = TRAFFIC_FILES.get(cfg)
    if not path or not os.path.exists(path):
        return None
    txt = open(path).read()
    h = re.search(r"kernel code sha256\[:16\]:\s*([0-9a-f]{16})", txt)
    b = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.e+]+)", txt)
    if not h or not b or h.group(1) != attn_src_hash():
        return None
    return float(b.group(1))


class _Bf16Rows:
    """Decode rows of a bf16-bits array to float64 on indexing (the oracle reads a
    few rows of a multi-hundred-MB input)."""

    def __init__(self, bits):
        self.bits, self.shape = bits, bits.shape

    def __getitem__(self, idx):
        from segmented_attention_seq_amd.workload import bf16_bits_to_f32
        return bf16_bits_to_f32(self.bits[idx]).astype(np.float64)


def cpu_baseline(tr, q, k, v, target_s):
    """Time the CPU oracle (as it stands) on a seeded sample of query rows of the
    same restore workload; report its rate in the metric's unit.  The oracle spreads
    its (query chunk, head) products and key rotations over a thread pool of the
    host's cores (at most 16, the box's share); `cores` is that pool, and the
    parallelism it reached (process CPU time over wall time) is reported with it."""
    import oracle
    from threadpoolctl import threadpool_limits
    threads = max(1, min(16, os.cpu_count() or 1))
    ops = oracle.canonical_ops(tr.msg_len, tr.drop, tr.reposition)
    ev = oracle.replay_events(ops)
    ep = ev.epoch_of_token()
    T, hq, d = q.shape
    order = np.random.default_rng(12345).permutation(T)
    n, done, secs, cpu, flop = 64, 0, 0.0, 0.0, 0.0
    while secs < target_s and done < T:
        rows = np.sort(order[done:done + n])
        t0, c0 = time.perf_counter(), time.process_time()
        with threadpool_limits(1):
            oracle.segment_attention(_Bf16Rows(q), _Bf16Rows(k), _Bf16Rows(v), ev=ev, rows=rows,
                                     base=150000.0, compact=True, threads=threads)
        secs += time.perf_counter() - t0
        cpu += time.process_time() - c0
        for i in rows:   # keys row i attends to: version rows and own tokens j <= i not yet dropped
            tb, te, src = ev.epochs[ep[i]]
            nvis = int((ev.tok_drop[src] > i).sum() + (ev.tok_drop[tb:i + 1] > i).sum())
            flop += 4.0 * d * hq * nvis
        done += rows.size
        n = int(min(4 * n, max(64, n * (target_s - secs) / max(secs, 1e-3))))
    return {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "parallelism": round(cpu / secs, 2),
            "sample": f"{done} random query rows (all {hq} heads) of the restore workload, float64 "
                      f"NumPy oracle on a pool of {threads} threads (BLAS single-threaded inside it), "
                      f"{secs:.1f} s wall, {cpu:.1f} s CPU"}


def _back_to_back(ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"b2b_us": ms * 1e3, "b2b_achieved": gbs, "b2b_frac": gbs / PEAK_HBM_GBS}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: each GPU would run these kernels on its own kv heads or requests",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from segmented_attention_seq_amd import akv, workload
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    only = set(args.only.split(",")) if args.only else {"restore", "repos", "decode"}

    def t_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- inputs (resident in HBM before timing)
    tr, q, k, v = workload.config_prefill(args.config)
    if args.hq != q.shape[1]:
        q = workload.prefill_tensors(tr.n_tokens, args.hq, k.shape[1], k.shape[2], seed=7000 + args.hq)[0]
    T, hq, d = q.shape
    hkv = k.shape[1]
    qd, kd, vd = t_bf16(q), t_bf16(k), t_bf16(v)
    req_ops = (tr.msg_len, tr.drop, tr.reposition)
    bq = args.bq or akv.attention_bq(args.hq, k.shape[1])
    plan0 = akv.build_visibility(akv.ops_from_messages(*req_ops), bq=bq)
    nv = int(plan0.info["n_versions"])
    pairs = int(plan0.info["visible_pairs"])
    attn_flop = 4.0 * d * hq * pairs
    fused = args.fused_versions
    nvb = 0 if fused else nv    # version buffers are not built with fused versions
    bufs = {"k_rot": torch.empty_like(kd),
            "k_ver": torch.empty((nvb, hkv, d), dtype=torch.bfloat16, device=dev),
            "v_ver": torch.empty((nvb, hkv, d), dtype=torch.bfloat16, device=dev),
            "rot_ws": torch.empty(max(akv.rot_table_bytes(plan0, d), 4), dtype=torch.uint8, device=dev),
            "out": torch.empty_like(qd)}

    rb = workload.repos_batch() if "repos" in only else workload.repos_batch(n_keys=64)
    nrep = rb.slots.size
    repos_sets = []
    for s in range(args.repos_sets if "repos" in only else 1):
        pool = torch.zeros((rb.pool_slots, rb.hkv, rb.d), dtype=torch.bfloat16, device=dev)
        pool[torch.from_numpy(rb.slots.astype(np.int64)).to(dev)] = t_bf16(rb.k_rows)
        repos_sets.append((pool, torch.empty((nrep, rb.hkv, rb.d), dtype=torch.bfloat16, device=dev)))
    r_from = torch.from_numpy(rb.pos_from).to(dev)
    r_to = torch.from_numpy(rb.pos_to).to(dev)
    r_idx = torch.from_numpy(rb.slots).to(dev)
    repos_bytes = nrep * rb.hkv * rb.d * 2 * 2 + 12 * nrep

    db = workload.decode_batch() if "decode" in only else workload.decode_batch(batch=1, lo=64, hi=65)
    pool_k = torch.zeros((db.pool_slots, db.hkv, db.d), dtype=torch.bfloat16, device=dev)
    pool_v = torch.zeros_like(pool_k)
    didx = torch.from_numpy(db.indices.astype(np.int64)).to(dev)
    pool_k[didx] = t_bf16(db.k_rows)
    pool_v[didx] = t_bf16(db.v_rows)
    dq = t_bf16(db.q)
    d_indptr = torch.from_numpy(db.indptr).to(dev)
    d_indices = torch.from_numpy(db.indices).to(dev)
    max_n = int(np.diff(db.indptr).max())
    n_keys = int(db.indptr[-1])
    dout = torch.empty((db.q.shape[0], db.hq, db.d), dtype=torch.bfloat16, device=dev)
    dws = torch.empty(akv.decode_workspace_bytes(db.q.shape[0], db.hq, db.hkv, db.d, max_n),
                      dtype=torch.uint8, device=dev)
    decode_bytes = n_keys * db.hkv * db.d * 2 * 2 + 4 * n_keys + 2 * dq.numel() * 2
    torch.cuda.synchronize()
    if args.copy_mb:
        # a plain elementwise kernel that reads and writes exactly copy_mb MiB each
        src = torch.ones((args.copy_mb << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ev_names = ["rope", "versions", "attn", "repos", "decode"]
    stage_ms = {n: [] for n in ev_names}
    build_ms, upload_ev = [], []
    keep_plans = []
    dev_plans = [torch.empty(int(plan0.info["device_bytes"]), dtype=torch.uint8, device=dev) for _ in range(2)]
    copy_stream = torch.cuda.Stream(device=dev)     # default priority
    plan_free = [None, None]    # per device buffer: the attention that last read it has finished

    def mark():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(i, timed):
        ev = {}
        last = None
        if "restore" in only:
            # A1 on the host while the GPU still runs the previous step; the image goes up
            # on the copy stream into the buffer the step before the previous one used
            t0 = time.perf_counter()
            plan = akv.build_visibility(akv.ops_from_messages(*req_ops), bq=bq)
            t1 = time.perf_counter()
            buf = dev_plans[i % 2]
            if plan_free[i % 2] is not None:
                copy_stream.wait_event(plan_free[i % 2])
            up0 = torch.cuda.Event(enable_timing=True)
            up0.record(copy_stream)
            akv._check(akv._lib.akv_plan_upload(plan.handle, buf.data_ptr(), buf.numel(), copy_stream.cuda_stream),
                       "akv_plan_upload")
            uploaded = torch.cuda.Event(enable_timing=True)
            uploaded.record(copy_stream)
            torch.cuda.current_stream().wait_event(uploaded)
            plan._dev[str(dev)] = buf
            keep_plans.append(plan)
            del keep_plans[:-3]      # host images stay alive until their copies ran
            build_ms.append((t1 - t0) * 1e3)
            upload_ev.append((up0, uploaded))   # the copy itself, on the copy stream
            # One event between consecutive stages (each record is a marker packet
            # of a few microseconds on the GPU timeline): stage k runs from mark k to
            # mark k+1.
            m0 = mark()
            akv.rope_apply(plan, bufs["k_rot"], kd)   # queries are rotated inside the attention
            m1 = mark()
            m2 = m1
            if nv and not fused:
                akv.build_kv_versions(plan, bufs["k_rot"], vd, bufs["k_ver"], bufs["v_ver"])
                m2 = mark()
            if fused:   # the run table fill and the attention
                akv.segment_attention_fused(plan, qd, bufs["k_rot"], vd, bufs["out"], rope_base=workload.ROPE_BASE,
                                            ws=bufs["rot_ws"])
            else:
                akv.segment_attention(plan, qd, bufs["k_rot"], vd, bufs["k_ver"], bufs["v_ver"], bufs["out"],
                                      rope_base=workload.ROPE_BASE)
            last = mark()
            plan_free[i % 2] = last
            ev.update(rope=(m0, m1), versions=(m1, m2), attn=(m2, last))
        if "repos" in only:
            pool, out = repos_sets[i % len(repos_sets)]
            start = last if last is not None else mark()
            akv.rope_repos(out, pool, r_to, r_from, r_idx)
            last = mark()
            ev["repos"] = (start, last)
        if "decode" in only:
            start = last if last is not None else mark()
            akv.decode_attention(dq, pool_k, pool_v, d_indptr, d_indices, max_n, dout, ws=dws)
            last = mark()
            ev["decode"] = (start, last)
        return ev

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    pending = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        pending.append(step(args.warmup + i, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for evs in pending:
        for n, (a, b) in evs.items():
            stage_ms[n].append(a.elapsed_time(b))
    ms_per_step = wall * 1e3 / args.steps
    avg = {n: (float(np.mean(v)) if v else None) for n, v in stage_ms.items()}

    # The short kernels once more, back to back between one pair of events per round,
    # so the marker packets of the per-stage events (a few microseconds each) do not
    # count against them: repos over the rotating buffer sets (together larger than
    # the last-level cache), decode over its 1.9 GB of gathered rows.
    # Each is the median over several rounds, since one round of a 35 us kernel moves
    # by several percent from round to round.
    b2b, b2b_rounds = {}, {}

    def rounds(launch, n, k):
        per = []
        for _ in range(k):
            e0 = mark()
            for j in range(n):
                launch(j)
            e1 = mark()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
        return float(np.median(per)), per

    if "repos" in only:
        def repos_launch(j):
            pool, out = repos_sets[j % len(repos_sets)]
            akv.rope_repos(out, pool, r_to, r_from, r_idx)
        b2b["repos"], b2b_rounds["repos"] = rounds(repos_launch, 4 * len(repos_sets), 5)
    if "decode" in only:
        b2b["decode"], b2b_rounds["decode"] = rounds(
            lambda j: akv.decode_attention(dq, pool_k, pool_v, d_indptr, d_indices, max_n, dout, ws=dws), 8, 3)

    value = attn_flop / (ms_per_step * 1e-3) / 1e12 if "restore" in only else 0.0
    attn_tflops = attn_flop / (avg["attn"] * 1e-3) / 1e12 if avg["attn"] else None
    # counters were taken on 64/8 with version buffers
    traffic = read_traffic(args.config) if hq // hkv == 8 and not fused else None
    comps = {"host_plan_build_ms": float(np.mean(build_ms)) if build_ms else None,
             "host_plan_upload_ms": (float(np.mean([a.elapsed_time(b) for a, b in upload_ev]))
                                     if upload_ev else None),
             "plan_device_bytes": int(plan0.info["device_bytes"])}
    for n in ev_names:
        comps[f"{n}_ms"] = avg[n]
    if avg["repos"]:
        gbs = repos_bytes / (avg["repos"] * 1e-3) / 1e9
        comps["repos"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": gbs / PEAK_HBM_GBS, "bytes_per_launch": repos_bytes, "keys": nrep}
        comps["repos"].update(_back_to_back(b2b["repos"], repos_bytes))
        comps["repos"]["b2b_rounds_us"] = [round(x * 1e3, 2) for x in b2b_rounds["repos"]]
    if avg["decode"]:
        gbs = decode_bytes / (avg["decode"] * 1e-3) / 1e9
        comps["decode"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gbs / PEAK_HBM_GBS, "bytes_per_launch": decode_bytes,
                           "gathered_keys": n_keys, "requests": int(db.q.shape[0])}
        comps["decode"].update(_back_to_back(b2b["decode"], decode_bytes))
        comps["decode"]["b2b_rounds_us"] = [round(x * 1e3, 2) for x in b2b_rounds["decode"]]
    if avg["rope"]:
        rope_bytes = 2 * kd.numel() * 2 + 4 * T
        comps["rope_apply_gbs"] = rope_bytes / (avg["rope"] * 1e-3) / 1e9
    if avg["versions"] and nv and not fused:
        comps["versions_gbs"] = (nv * hkv * d * 2 * 4 + 12 * nv) / (avg["versions"] * 1e-3) / 1e9

    workload_name = {2: "48k-token 20-round agent trajectory, rolling drop keep 12 (8 drops)",
                     3: "300,200-token 100-round trajectory, keep 12 + repos at the 96k position window",
                     4: "192k-token 200-round trajectory, keep 12 + repos every round"}[args.config]
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"restore of a {workload_name} ({hq}/{hkv} GQA heads, d=64, RoPE base 150000) "
                               f"+ batched repos of {nrep} keys + decode of {db.q.shape[0]} requests over "
                               f"{n_keys} gathered keys", "restore_tokens": T, "visible_pairs": pairs,
                   "attn_flop_per_step": attn_flop, "version_rows": nv,
                   "versions": "rotated while key tiles are staged" if fused else "built into buffers",
                   "stages": sorted(only)},
        "roofline": {"bound": "mfma", "kernel": attn_kernel_name(hq, hkv, bq, fused),
                     "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": (attn_tflops / PEAK_BF16_TFLOPS) if attn_tflops else None,
                     "traffic": traffic},
        "components": comps,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and "restore" in only:
        line["cpu_baseline"] = cpu_baseline(tr, q, k, v, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
