"""Benchmark of the packed FlashMask forward on one MI355X.

One step = one pass of the whole hot path over the workload, inputs already
resident in HBM:  block extrema (N2) -> tile classes + work list (N3) ->
attention (N4, plus the split merge when rows are split).  Small problems
take the fused path (one attention launch in which every workgroup plans its
own items, then the merge); the others the planning launches and the
plan-reading attention launch.  The metric is effective TFLOP/s: attending
(query, key, head) triples times 4 D flops, divided by the time of one step.

Timing (K = --steps, W = --warmup):
  1. W untimed steps, then K steps back to back between two HIP events on
     the library's stream (a spin kernel queued first lets the host enqueue
     all K ahead): value and ms_per_step.
  2. K steps, each between its own pair of events: the median and p10/p90
     of one step (an event between launches keeps the next launch from
     starting while the previous one drains, so these run a little longer).
  3. Up to 20 steps, each after a 512 MiB write that evicts the caches: the
     cold-cache step.
  4. The dominant launches alone, K back to back between two events: the
     attention kernel (+ merge) of the step on the fused path, the
     plan-reading attention launches with a plan built once on the planned
     path: roofline.achieved.  roofline.profiled and roofline.traffic come
     from the rocprofv3 runs summarised in profiles/ while the forward
     sources are the ones they were taken from.
The oracle (fp64 NumPy, the parity reference) is timed on the host cores on
a bounded sample of the same workload as the CPU baseline.  For bf16
workloads the line also reports, for information, the backward (dq, dk, dv)
and the fused q/k rotary embedding on the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, packed masked attn fwd"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 1000 on the small varlen workload, 200 on the others)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload config id (1..5); 2 is the headline")
    ap.add_argument("--split", type=int, default=-1, help="max key blocks per item (-1 auto, 0 none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="leave out the backward and rotary-embedding legs")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only the warm-up and the timed back-to-back steps (for profiler runs whose "
                         "per-kernel averages should be those of the timed steps)")
    ap.add_argument("--seeds", type=int, default=1, help="measure this many seeds (seed, seed + 1, ...), one line each")
    ap.add_argument("--planned", action="store_true",
                    help="time the planning launches + plan-reading attention even where the fused path applies")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on oracle CPU time")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--seed", type=int, default=None, help="workload seed (default 1000 + config)")
    ap.add_argument("--sparsity-sweep", action="store_true",
                    help="instead of the step: step latency against the unmasked fraction on the varlen shape")
    ap.add_argument("--packing-sweep", action="store_true",
                    help="instead of the step: the workload's documents in four packings (varlen, mask-only "
                         "with cu = [0, N], zero-padded, zero-padded with the padding masked), step time each")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward step: time the backward (dq, dk, dv) on the workload")
    ap.add_argument("--dropout", type=float, default=None, metavar="P",
                    help="time the forward and the backward with attention dropout P beside the plain ones "
                         "on workload --config")
    ap.add_argument("--rope", action="store_true",
                    help="instead of the forward step: time the fused q/k rotary embedding on the workload")
    ap.add_argument("--packings", default=",".join(("varlen", "mask_only", "padded", "padded_masked")),
                    help="comma-separated packings the packing sweep runs")
    ap.add_argument("--preprocess-sweep", action="store_true",
                    help="instead of the step: time the block-extrema pass alone for N = 2^16 .. 2^26 "
                         "(n_vec = 4, non-causal) and report its achieved HBM GB/s")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 1000 if args.config == 2 else 200
    return args


FWD_SOURCES = ("fm_api.cpp", "fm_attn_bf16.hip", "fm_common.hpp", "fm_internal.h", "fm_own_plan.h", "fm_plan.hip")


def source_hash():
    """sha256 over the sources of the forward bf16 path (the planning and
    attention kernels and the host code that launches them) and the build
    script (its compiler flags): stored counter figures apply only to the
    kernels they were taken from."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "packed_varlen_masked_amd")
    for name in FWD_SOURCES:
        h.update(name.encode())
        with open(os.path.join(pkg, "csrc", name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def stored_profile(key):
    """Per-launch figures of the dominant kernels from the rocprofv3 runs
    summarised in profiles/ (profiles/roofline.json): HBM bytes from the
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain-copy calibration) and the
    kernel-trace average durations, or None when absent or taken from other
    sources than the current ones."""
    try:
        with open(os.path.join(ROOT, "profiles", "roofline.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get("entries", {}).get(key)
    if not e or e.get("src_sha256") != source_hash():
        return None
    return e


def count_pairs(w, device=None):
    """Attending (query, key) pairs per head of workload w: pairs of one
    sequence whose key column does not hide the query row.  Column j hides
    rows [LTS_j, LTE_j) and, without the causal flag, [UTS_j, UTE_j); the
    causal flag hides keys after the query; absent stored vectors take the
    defaults LTS = UTS = 0, LTE = UTE = N (FlashMask article, section 2).
    Evaluated densely per sequence in row chunks with torch (on the GPU when
    there is one); the effective FLOPs of the metric are 4 D H times this."""
    import torch
    dev = device or (torch.device("cuda:0") if torch.cuda.is_available() else torch.device("cpu"))
    N = w.N
    sv = torch.from_numpy(np.asarray(w.startend, np.int64)).to(dev)
    full = torch.full((N,), N, dtype=torch.int64, device=dev)
    zero = torch.zeros(N, dtype=torch.int64, device=dev)
    if w.causal:
        lts, lte, uts, ute = sv[0], (sv[1] if w.n_vec == 2 else full), zero, zero
    elif w.n_vec == 2:
        lts, lte, uts, ute = sv[0], full, zero, sv[1]
    else:
        lts, lte, uts, ute = sv[0], sv[1], sv[2], sv[3]
    cu = [int(x) for x in w.cu_seqlens]
    total = 0
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e <= s:
            continue
        j = torch.arange(s, e, device=dev)[None, :]
        for r0 in range(s, e, 2048):
            i = torch.arange(r0, min(r0 + 2048, e), device=dev)[:, None]
            hid = (lts[j] <= i) & (i < lte[j])
            if w.causal:
                hid |= j > i
            else:
                hid |= (uts[j] <= i) & (i < ute[j])
            total += int((~hid).sum().item())
    return total


def host_info():
    """CPU model, usable cores and the NumPy BLAS behind the oracle."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = "%s %s" % (libs[0].get("internal_api"), libs[0].get("version"))
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)), "blas": blas}


_POOL_W = None


def _oracle_task(task):
    """One (sequence, head) of the oracle, rebased to the sequence (pairs of
    different sequences never attend): seconds and effective FLOPs."""
    import oracle as O
    w = _POOL_W
    s, e, h = task
    sv = w.startend[:, s:e].astype(np.int64) - s
    sl = (slice(s, e), slice(h, h + 1))
    t0 = time.perf_counter()
    O.attention(w.q[sl], w.k[sl], w.v[sl], np.array([0, e - s]), sv, w.n_vec, w.causal, w.scale)
    dt = time.perf_counter() - t0
    pairs = O.unmasked_pairs(np.array([0, e - s]), sv, w.n_vec, w.causal)
    return dt, O.effective_flops(pairs, 1, w.D)


def cpu_baseline(w, budget_s):
    """The oracle (fp64 NumPy) on the host cores: a process pool of C
    workers (C = the usable cores, at most 16), one BLAS thread each, over
    (sequence, head) pieces of the workload, longest sequences first, until
    about budget_s seconds of wall time are spent (the whole workload when it
    fits).  Throughput = effective FLOPs of the pieces done / wall time."""
    import multiprocessing as mp
    global _POOL_W
    info = host_info()
    C = max(1, min(16, info["host_cpus"]))
    cu = [int(x) for x in w.cu_seqlens]
    tasks = sorted(((cu[b], cu[b + 1], h) for b in range(len(cu) - 1) if cu[b + 1] > cu[b] for h in range(w.H)),
                   key=lambda t: -(t[1] - t[0]))
    _POOL_W = w
    old = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in old:
        os.environ[k] = "1"
    done_flops, pieces = 0, 0
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            ctx = mp.get_context("fork")
            with ctx.Pool(C) as pool:
                t0 = time.perf_counter()
                for dt, fl in pool.imap_unordered(_oracle_task, tasks, chunksize=1):
                    done_flops += fl
                    pieces += 1
                    if time.perf_counter() - t0 > budget_s:
                        pool.terminate()
                        break
                wall = time.perf_counter() - t0
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    res = {"value": done_flops / wall / 1e12, "unit": "TFLOP/s", "cores": C, "kind": "oracle",
           "sample": "%d of %d (sequence, head) pieces, %.3g effective GFLOP, %.2f s wall, fp64 NumPy, "
                     "process pool of %d workers x 1 BLAS thread" % (pieces, len(tasks), done_flops / 1e9, wall, C)}
    res.update(info)
    return res


def preprocess_sweep(args):
    """Block-extrema pass (fm_preprocess_mask) alone: synthetic int32 mask
    vectors [4, N] (uniform in [0, N)), documents of 2^20 tokens (one when N
    is smaller), Bc = 64.  Algorithmic bytes: the vectors read once
    (16 B per token), cu_seqlens read, kb_off and the extrema (32 B per key
    block) written.  Time: K calls between HIP events after W warm-up calls."""
    import torch
    import packed_varlen_masked_amd as pv
    dev = torch.device("cuda:0")
    n_vec, Bc, K = 4, 64, max(args.steps, 10)
    rows = []
    for lg in range(16, 27, 2):
        N = 1 << lg
        B = max(1, N >> 20)
        cu = (torch.arange(B + 1, dtype=torch.int64, device=dev) * (N // B)).to(torch.int32)
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + lg)
        sv = torch.randint(0, N, (n_vec, N), dtype=torch.int32, device=dev, generator=g)
        cap = -(-N // Bc) + B
        kb_off = torch.empty(B + 1, dtype=torch.int32, device=dev)
        ext = torch.empty(cap, 8, dtype=torch.int32, device=dev)
        scal = torch.zeros(2, dtype=torch.int32, device=dev)

        def call():
            pv._check(pv._lib.fm_preprocess_mask(pv._ptr(sv), n_vec, 0, pv._ptr(cu), B, N, Bc, pv._ptr(kb_off),
                                                 pv._ptr(ext), cap, pv._ptr(scal[0:1]),
                                                 __import__("ctypes").c_void_p(scal.data_ptr() + 4), pv._stream()))
        for _ in range(max(args.warmup, 3)):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            call()
        e1.record()
        torch.cuda.synchronize()
        nkb, status = (int(x) for x in scal.cpu())
        assert status == 0 and nkb == -(-N // Bc), (status, nkb)
        us = e0.elapsed_time(e1) / K * 1e3
        nbytes = 4 * n_vec * N + 4 * (B + 1) + 4 * (B + 1) + 32 * nkb
        rows.append({"N": N, "B": B, "key_blocks": nkb, "us": round(us, 3), "algorithmic_bytes": nbytes,
                     "GB_per_s": round(nbytes / us / 1e3, 1), "frac_of_8TB_s": round(nbytes / us / 1e3 / 8000.0, 4)})
        del sv, ext
    print(json.dumps({"metric": "block-extrema pass (fm_preprocess_mask) achieved HBM GB/s", "unit": "GB/s",
                      "higher_is_better": True, "n_vec": n_vec, "causal": False, "block_k": Bc, "calls_timed": K,
                      "peak_GB_per_s": 8000.0, "data": "synthetic (uniform random int32 mask vectors)",
                      "sweep": rows}), flush=True)


def make_setup(w, args):
    """Device inputs, the plan and the step function for workload w."""
    import torch
    import workloads as W
    import packed_varlen_masked_amd as pv
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float32
    q = torch.from_numpy(w.q).to(dt).to(dev)
    k = torch.from_numpy(w.k).to(dt).to(dev)
    v = torch.from_numpy(w.v).to(dt).to(dev)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(dev)
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).to(dev)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, dt, max_kb_per_item=args.split)
    out = torch.empty_like(q)
    lse = torch.empty(w.H, w.N, dtype=torch.float32, device=dev)
    S = plan.max_kb_per_item
    # small problems: one fused launch plans in LDS and attends; otherwise the
    # planning launches fill the workspace and the attention launch reads it
    fused = pv.fused_path(w.N, w.B, w.H, w.D, dt, w.n_vec, w.causal, S) and not args.planned
    ws = torch.zeros_like(plan.workspace)

    def attn_with_plan():   # the attention launch(es) reading a built plan
        pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan, out=out, lse=lse)

    if fused:
        def step(ev_a=None, ev_b=None):
            if ev_a is not None:
                ev_a.record()
            pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S,
                        out=out, lse=lse, workspace=ws)
            if ev_b is not None:
                ev_b.record()
    else:
        def step(ev_a=None, ev_b=None):
            pv.build_plan_into(plan, cu, sv)
            if ev_a is not None:
                ev_a.record()
            attn_with_plan()
            if ev_b is not None:
                ev_b.record()
    hdr = plan.header   # the plan built above (the fused path writes none)
    return dict(dt=dt, dev=dev, step=step, attn_with_plan=attn_with_plan, plan=plan, S=S, fused=fused, hdr=hdr,
                tensors=(q, k, v, cu, sv))


def spin():
    """Queue a spin kernel so the host enqueues the timed launches ahead of the GPU."""
    import torch
    try:
        torch.cuda._sleep(int(2e8))
        return True
    except Exception:
        return False


def time_calls(fn, K):
    """Mean ms per call of K back-to-back calls between two HIP events."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ahead = spin()
    th0 = time.perf_counter()
    t0.record()
    for _ in range(K):
        fn()
    t1.record()
    host_ms = (time.perf_counter() - th0) * 1e3 / K
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / K, host_ms, ahead


def sparsity_sweep(args):
    """Step time against unmasked work at the shape of workload --config
    (the varlen workload: N = 4352, H = 2; the SFT packing: N = 16384,
    H = 32; D = 128, causal documents): the documents are resized (k equal
    documents, plus the workload's own length mix), which moves the unmasked
    fraction 1 - rho of the N x N score matrix; the FlashMask article (§4.3)
    expects latency linear in it."""
    import workloads as W
    base = W.make_config(args.config, seed=args.seed, with_qkv=False)
    N, H = base.N, base.H
    ks = (1, 2, 4, 8, 17, 34) if N <= 8192 else (1, 2, 4, 8, 16, 32, 64, 128)
    cases = [[N // k] * (k - 1) + [N - (N // k) * (k - 1)] for k in ks] + [[int(x) for x in base.lengths]]
    rows = []
    for lens in cases:
        w = W.document_workload(lens, H=H, D=128, seed=base.meta["seed"])
        st = make_setup(w, args)
        for _ in range(args.warmup):
            st["step"]()
        ms, _, _ = time_calls(st["step"], args.steps)
        pairs = count_pairs(w)
        rows.append({"documents": len(lens), "lengths": lens[:4] + (["..."] if len(lens) > 4 else []),
                     "unmasked_fraction": round(pairs / float(N * N), 5), "unmasked_pairs_per_head": int(pairs),
                     "path": "fused" if st["fused"] else "planned", "max_kb_per_item": st["S"],
                     "us_per_step": round(ms * 1e3, 2),
                     "effective_TFLOP_s": round(4 * w.D * w.H * pairs / (ms * 1e-3) / 1e12, 2)})
    x = np.array([r["unmasked_fraction"] for r in rows])
    y = np.array([r["us_per_step"] for r in rows])
    slope, icpt = np.polyfit(x, y, 1)
    r2 = 1.0 - float(np.sum((y - (slope * x + icpt)) ** 2)) / float(np.sum((y - y.mean()) ** 2))
    print(json.dumps({"metric": "step latency against unmasked fraction (shape of %s)" % base.name, "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
                      "fit": {"us_per_unit_fraction": round(float(slope), 2), "intercept_us": round(float(icpt), 2),
                              "r2": round(r2, 4)},
                      "data": "synthetic (seeded N(0,1) q/k/v)", "sweep": rows}), flush=True)


def packing_sweep(args):
    """The documents of a causal document workload (default: the varlen
    workload [128, 128, 4096]) packed four ways through the same library:
    back to back with one sequence each (varlen), back to back with
    cu = [0, N] and only the mask separating them (mask_only, the FlashMask
    article's ZeroPadding packing), zero-padded to the longest document
    with a plain causal mask (padded, the Varlen-Packing document's padded
    baseline), and zero-padded with the padding masked by the interval
    (padded_masked).  Useful work is the documents' own unmasked pairs in
    every case; `computed_pairs_per_head` is what the layout leaves
    unmasked."""
    import workloads as W
    base = W.make_config(args.config, seed=args.seed)
    useful = count_pairs(base)
    flops = 4 * base.D * base.H * useful
    rows = []
    for kind in [x for x in args.packings.split(",") if x]:
        w = W.packed_as(base, kind)
        st = make_setup(w, args)
        for _ in range(args.warmup):
            st["step"]()
        ms, _, _ = time_calls(st["step"], args.steps)
        st["attn_with_plan"]()
        ms_r, _, _ = time_calls(st["attn_with_plan"], args.steps)
        hdr = st["hdr"]()
        pairs = count_pairs(w)
        rows.append({"packing": kind, "tokens_stored": w.N, "sequences": w.B, "n_vec": w.n_vec,
                     "path": "fused" if st["fused"] else "planned", "max_kb_per_item": st["S"],
                     "n_items": hdr["n_items"], "class_counts": hdr["class_counts"],
                     "computed_pairs_per_head": int(pairs),
                     "us_per_step": round(ms * 1e3, 2), "us_attention_reused_plan": round(ms_r * 1e3, 2),
                     "effective_TFLOP_s": round(flops / (ms * 1e-3) / 1e12, 2)})
    print(json.dumps({"metric": "step time of the same documents in four packings", "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
                      "workload": base.name, "lengths": [int(x) for x in base.lengths][:16],
                      "H": base.H, "D": base.D, "useful_pairs_per_head": int(useful),
                      "effective_gflop": round(flops / 1e9, 4),
                      "data": "synthetic (seeded N(0,1) q/k/v, zero pad tokens)", "sweep": rows}), flush=True)


def backward_bench(args):
    """The backward on workload --config: dq, dk, dv from q, k, v, the
    forward's out and lse, and a seeded N(0, 1) output gradient.  One step =
    one fm_attn_bwd call (block extrema, Delta, dK/dV, dQ).  Useful work =
    five products per attending pair (S recomputed, dP, dV, dK, dQ), i.e.
    2.5 x the forward's effective FLOPs; the dQ launch recomputes S and dP,
    which is not counted."""
    import torch
    import workloads as W
    import packed_varlen_masked_amd as pv
    w = W.make_config(args.config, seed=args.seed)
    if w.dtype != W.BF16:
        raise SystemExit("the backward is built for the bf16 workloads (configs 2-5)")
    st = make_setup(w, args)
    dev = st["dev"]
    q, k, v, cu, sv = st["tensors"]
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale))
    g = torch.from_numpy(np.random.default_rng(w.meta["seed"] + 2).standard_normal(
        (w.N, w.H, w.D), dtype=np.float32)).to(torch.bfloat16).to(dev)
    ws = torch.zeros(pv.bwd_workspace_size(w.N, w.B, w.H, w.D, torch.bfloat16), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    side = torch.cuda.Stream()   # the dQ launches overlap dK/dV on it (fm_attn_bwd_streams)

    def step():
        pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale), workspace=ws,
                    dq=dq, dk=dk, dv=dv, dq_stream=side)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, host_ms, ahead = time_calls(step, args.steps)
    pairs = count_pairs(w)
    flops = 2.5 * 4 * w.D * w.H * pairs
    value = flops / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "backward effective TFLOP/s (5 products per unmasked pair) + % bf16 MFMA peak",
                      "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
                      "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/k/v/dout)",
                      "config": {"workload": w.name, "N": w.N, "B": w.B, "H": w.H, "D": w.D,
                                 "causal": bool(w.causal), "n_vec": w.n_vec,
                                 "unmasked_pairs_per_head": int(pairs), "useful_gflop": round(flops / 1e9, 4)},
                      "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
                      "timing": {"host_enqueue_ms_per_step": round(host_ms, 4), "host_ran_ahead": ahead}}),
          flush=True)


def dropout_bench(args):
    """Forward and backward with attention dropout p (Philox4x32-10 keep
    mask regenerated per element in both) beside the plain ones, on the same
    inputs; the useful work is counted as without dropout."""
    import torch
    import workloads as W
    import packed_varlen_masked_amd as pv
    w = W.make_config(args.config, seed=args.seed)
    if w.dtype != W.BF16:
        raise SystemExit("dropout is built for the bf16 workloads (configs 2-5)")
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(dev)
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).to(dev)
    g = torch.from_numpy(np.random.default_rng(w.meta["seed"] + 2).standard_normal(
        (w.N, w.H, w.D), dtype=np.float32)).to(torch.bfloat16).to(dev)
    wsb = torch.zeros(pv.bwd_workspace_size(w.N, w.B, w.H, w.D, torch.bfloat16), dtype=torch.uint8, device=dev)
    pairs = count_pairs(w)
    flops = 4 * w.D * w.H * pairs
    res = {}
    for p in (0.0, args.dropout):
        kw = dict(dropout_p=p, seed=0x5EED, offset=1) if p > 0 else {}
        plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16, max_kb_per_item=args.split)
        out = torch.empty_like(q)
        lse = torch.empty(w.H, w.N, dtype=torch.float32, device=dev)
        wsf = torch.zeros_like(plan.workspace)
        fused = pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal, plan.max_kb_per_item) and p == 0

        def fwd():
            if fused:
                pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=plan.max_kb_per_item,
                            out=out, lse=lse, workspace=wsf)
            else:
                pv.build_plan_into(plan, cu, sv)
                pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan, out=out, lse=lse, **kw)
        grads = [torch.empty_like(q) for _ in range(3)]

        side = torch.cuda.Stream()   # the dQ launches overlap dK/dV on it, with and without dropout

        def bwd():
            pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale), workspace=wsb,
                        dq=grads[0], dk=grads[1], dv=grads[2], dq_stream=side, **kw)
        for _ in range(args.warmup):
            fwd()
            bwd()
        torch.cuda.synchronize()
        ms_f, _, _ = time_calls(fwd, args.steps)
        ms_b, _, _ = time_calls(bwd, args.steps)
        res["p=%g" % p] = {"forward_ms": round(ms_f, 6), "forward_TFLOP_s": round(flops / (ms_f * 1e-3) / 1e12, 3),
                           "backward_ms": round(ms_b, 6),
                           "backward_TFLOP_s": round(2.5 * flops / (ms_b * 1e-3) / 1e12, 3),
                           "path": "fused" if fused else "planned"}
    print(json.dumps({"metric": "forward and backward with attention dropout, effective TFLOP/s (work counted "
                                "as without dropout)", "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/k/v/dout)",
                      "config": {"workload": w.name, "N": w.N, "B": w.B, "H": w.H, "D": w.D,
                                 "causal": bool(w.causal), "n_vec": w.n_vec, "dropout_p": args.dropout},
                      "results": res}), flush=True)


def rope_bench(args):
    """The fused rotary embedding of the workload's q and k in place (one
    launch for both, positions restarting per document).  HBM-bound:
    algorithmic bytes = q and k read and written once, plus one cos and one
    sin row (D/2 fp32 each) per token."""
    import torch
    import workloads as W
    import packed_varlen_masked_amd as pv
    w = W.make_config(args.config, seed=args.seed)
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float32
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w.q).to(dt).to(dev)
    k = torch.from_numpy(w.k).to(dt).to(dev)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(dev)
    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rope_tables(int(w.lengths.max()), w.D))

    def step():   # forward then inverse, so the data stays bounded over many steps
        pv.rope_qk_(q, k, cu, cos, sin)
        pv.rope_qk_(q, k, cu, cos, sin, inverse=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms2, host_ms, ahead = time_calls(step, args.steps)
    ms = ms2 / 2
    esz = 2 if dt == torch.bfloat16 else 4
    nbytes = 2 * 2 * w.N * w.H * w.D * esz + w.N * w.D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "fused q/k rotary embedding, achieved HBM GB/s (algorithmic bytes)",
                      "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_call": round(ms, 6), "higher_is_better": True,
                      "dtype": "bf16" if dt == torch.bfloat16 else "f32", "data": "synthetic (seeded N(0,1) q/k)",
                      "config": {"workload": w.name, "N": w.N, "B": w.B, "Hq": w.H, "Hk": w.H, "D": w.D},
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                                   "frac": round(gbs / 8000.0, 4), "algorithmic_bytes": int(nbytes)},
                      "timing": {"host_enqueue_ms_per_step": round(host_ms / 2, 4), "host_ran_ahead": ahead,
                                 "what": "mean of a forward and an inverse call"}}), flush=True)


def extra_legs(w, st, K, flops):
    """Beside the headline (the forward step): the backward and the fused
    q/k rotary embedding on the same workload and inputs, each timed over K
    back-to-back calls (informational; the metric is the forward's)."""
    import torch
    import packed_varlen_masked_amd as pv
    import workloads as W
    q, k, v, cu, sv = st["tensors"]
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale))
    g = torch.from_numpy(np.random.default_rng(w.meta["seed"] + 2).standard_normal(
        (w.N, w.H, w.D), dtype=np.float32)).to(torch.bfloat16).to(q.device)
    ws = torch.zeros(pv.bwd_workspace_size(w.N, w.B, w.H, w.D, torch.bfloat16), dtype=torch.uint8, device=q.device)
    grads = [torch.empty_like(q) for _ in range(3)]
    side = torch.cuda.Stream()   # the dQ launches overlap dK/dV on it (fm_attn_bwd_streams)

    def bwd():
        pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale), workspace=ws,
                    dq=grads[0], dk=grads[1], dv=grads[2], dq_stream=side)
    for _ in range(5):
        bwd()
    ms_b, _, _ = time_calls(bwd, K)
    qr, kr = q.clone(), k.clone()
    cos, sin = (torch.from_numpy(t).to(q.device) for t in W.rope_tables(int(w.lengths.max()), w.D))

    def rope():   # forward then inverse: the data stays bounded
        pv.rope_qk_(qr, kr, cu, cos, sin)
        pv.rope_qk_(qr, kr, cu, cos, sin, inverse=True)
    for _ in range(5):
        rope()
    ms_r, _, _ = time_calls(rope, K)
    rope_bytes = 2 * 2 * w.N * w.H * w.D * 2 + w.N * w.D * 4
    return {"backward": {"what": "fm_attn_bwd_streams (dq, dk, dv; dQ on a second stream) on the same inputs; "
                                 "useful work = 5 products per unmasked pair = 2.5 x the forward's effective FLOPs",
                         "ms_per_call": round(ms_b, 6),
                         "effective_TFLOP_s": round(2.5 * flops / (ms_b * 1e-3) / 1e12, 3)},
            "rope": {"what": "fm_rope_qk on the workload's q and k in place (mean of a forward and an inverse call)",
                     "ms_per_call": round(ms_r / 2, 6),
                     "achieved_GB_s": round(rope_bytes / (ms_r / 2 * 1e-3) / 1e9, 1)}}


def main():
    args = parse()
    if args.preprocess_sweep:
        preprocess_sweep(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.sparsity_sweep:
        sparsity_sweep(args)
        return
    if args.packing_sweep:
        packing_sweep(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.dropout is not None:
        dropout_bench(args)
        return
    if args.rope:
        rope_bench(args)
        return
    import torch
    import workloads as W
    seeds = [args.seed if args.seed is not None else 1000 + args.config]
    seeds += [seeds[0] + i for i in range(1, max(1, args.seeds))]
    for sd in seeds:
        res = measure(W.make_config(args.config, seed=sd), args)
        print(json.dumps(res), flush=True)


def measure(w, args):
    """The bench line of workload w (see the module docstring)."""
    import torch
    import workloads as W
    import packed_varlen_masked_amd as pv
    st = make_setup(w, args)
    dt, dev, step, plan, S, fused = st["dt"], st["dev"], st["step"], st["plan"], st["S"], st["fused"]

    # algorithmic work: attending pairs per head (the bench's own count from
    # the interval vectors), 4 D flops per pair and head
    pairs = count_pairs(w)
    flops = 4 * w.D * w.H * pairs
    hdr = st["hdr"]()
    Br, Bc = plan.layout.block_q, plan.layout.block_k
    # tiles the kernels visit: PARTIAL + UNMASKED of the library's own plan,
    # each a full Br x Bc MFMA tile for every head
    visited = int(hdr["class_counts"][1] + hdr["class_counts"][2])
    mfma_flops = 4 * w.D * w.H * visited * Br * Bc

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps

    # pass 1: the timed steps, back to back between two events
    ms_step, host_ms, host_ahead = time_calls(step, K)
    if args.only_timed:
        return {"metric": METRIC, "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
                "higher_is_better": True, "config": {"workload": w.name, "seed": w.meta["seed"]},
                "path": "fused" if fused else "planned", "only_timed": True}
    # pass 2: every step between its own two events (the median and spread of
    # one step; an event between launches keeps the next launch from starting
    # while the previous one drains, so these run a little longer than pass 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    spin()
    for a_, b_ in ev:
        a_.record()
        step()
        b_.record()
    torch.cuda.synchronize()
    one = np.array([a_.elapsed_time(b_) for a_, b_ in ev])
    # pass 3: cold caches: a 512 MiB write (twice the 256 MiB last-level
    # cache) before each of up to 20 steps
    n_cold = min(K, 20)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    for a_, b_ in evc:
        flush.fill_(1)
        a_.record()
        step()
        b_.record()
    torch.cuda.synchronize()
    cold = np.array([a_.elapsed_time(b_) for a_, b_ in evc])
    del flush
    # pass 4: the dominant launches (the attention kernel and, when rows are
    # split, the merge) back to back: on the fused path they are the whole
    # step; on the planned path the attention launches reading a plan built
    # once (the per-layer cost when layers share a mask)
    st["attn_with_plan"]()
    ms_reuse, _, _ = time_calls(st["attn_with_plan"], K)
    ms_kernel = ms_step if fused else ms_reuse
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12

    path = "fused" if fused else "planned"
    kernels = (["fm_fused_bf16_kernel"] if fused else ["fm_attn_bf16_kernel<false>"]) + (
        ["fm_merge_bf16_kernel"] if S > 0 else [])
    prof = stored_profile("%s:%s:S%d" % (w.name, path, S))
    esz = 2 if dt == torch.bfloat16 else 4
    algo_bytes = 4 * w.N * w.H * w.D * esz + 4 * w.N * w.H   # q, k, v read once, out and lse written
    roof = {"bound": "mfma", "kernel": " + ".join(kernels),
            "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": prof.get("bytes_per_launch") if prof else None,
            "algorithmic_bytes": int(algo_bytes),
            "avg_launch_ms": round(ms_kernel, 6),
            "duration_from": "HIP events around K back-to-back calls of the launch(es) on the library's stream"}
    if prof and prof.get("kernel_avg_us"):
        us = float(sum(prof["kernel_avg_us"].values()))
        roof["profiled"] = {"avg_us": round(us, 3), "per_kernel_avg_us": prof["kernel_avg_us"],
                            "frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                            "summary": prof.get("summary")}
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, page-derived lengths and masks)",
        "config": {"workload": w.name, "seed": w.meta["seed"], "N": w.N, "B": w.B, "H": w.H, "D": w.D,
                   "lengths": [int(x) for x in w.lengths][:16], "causal": bool(w.causal),
                   "n_vec": w.n_vec, "block_q": Br, "block_k": Bc,
                   "max_kb_per_item": S, "n_items": hdr["n_items"],
                   "class_counts": hdr["class_counts"], "unmasked_pairs_per_head": int(pairs),
                   "effective_gflop": round(flops / 1e9, 4)},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "visited_tile_overhead": round((mfma_flops - flops) / flops, 4) if flops else None,
        "step_ms": {"back_to_back_mean": round(ms_step, 6),
                    "one_step_p10_p50_p90": [round(float(x), 6) for x in np.percentile(one, [10, 50, 90])],
                    "cold_cache_p10_p50_p90": [round(float(x), 6) for x in np.percentile(cold, [10, 50, 90])],
                    "cold_cache": "512 MiB written before each of %d steps" % n_cold},
        "timing": {"host_enqueue_ms_per_step": round(host_ms, 4), "host_ran_ahead": host_ahead},
        "path": path,
        "roofline": roof,
        "reused_plan": {"what": "attention launches alone, plan built once (fm_attn_bf16_kernel%s)" % (
                            " + fm_merge_bf16_kernel" if S > 0 else ""),
                        "ms_per_call": round(ms_reuse, 6),
                        "effective_TFLOP_s": round(flops / (ms_reuse * 1e-3) / 1e12, 3)},
    }
    if dt == torch.bfloat16 and not args.no_extra:
        res.update(extra_legs(w, st, K, flops))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    return res


if __name__ == "__main__":
    main()
