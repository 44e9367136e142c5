#!/usr/bin/env python3
"""Benchmark of ragged paged attention with KV append on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --workload chunked_gqa --one-shot   # the 8192-token prompt in one step
    python bench.py --copy-calibration      # 1 GiB device copy, for HBM counter scaling

A step is one pass of the hot path over one batch: KV append of the batch's
new tokens, then batched attention (all kernels, split-piece merge included),
with the step's plan built and uploaded beforehand (the plan is host work done
once per step and reused by every layer; its host time is reported as
plan_ms).  Inputs are synthetic and seeded (workloads.py) and resident in HBM
before timing starts.

Default workload: the mixed chunked-prefill step (32 decodes with kv_len
U{512..4096} plus one 512-token chunk at kv_len 1536; 32/32 heads, d 128,
bf16, page 16).  `value` is its KV-read bandwidth: algorithmic KV bytes (every
valid K and V row of every KV head read once) per second of step time.
`parts` times the decode requests and the prefill chunk as batches of their
own: decode KV-read GB/s and chunk TFLOP/s, each against the MI355X roofline.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV-read HBM GB/s + prefill-chunk attention TFLOP/s (1 GPU, % roofline)"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
KERNELS = ("append", "generic", "decode", "prefill", "mla", "merge", "merge_state", "page_copy")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic work (valid tokens only; page padding, split partials and the
# merge are overhead, not work)
# ----------------------------------------------------------------------------


def work(spec, qo_lens, kv_lens):
    elem = spec.elem_bytes
    row_stored = spec.head_dim_qk + (0 if spec.shared_latent else spec.head_dim_v)
    pairs = 0
    kv_bytes = 0
    total_q = 0
    for n, L in zip(qo_lens, kv_lens):
        n, L = int(n), int(L)
        c = L - n
        pairs += (n * c + n * (n + 1) // 2) if spec.causal else n * L
        kv_bytes += L * spec.num_kv_heads * row_stored * elem
        total_q += n
    qo_bytes = total_q * spec.num_qo_heads * (spec.head_dim_qk + spec.head_dim_v) * elem \
        + total_q * spec.num_qo_heads * 4
    return {
        "pairs": pairs,
        "flops": spec.num_qo_heads * pairs * 2 * (spec.head_dim_qk + spec.head_dim_v),
        "kv_bytes": kv_bytes,
        "qo_bytes": qo_bytes,
        "append_bytes": 2 * total_q * spec.num_kv_heads * row_stored * elem,
    }


# ----------------------------------------------------------------------------
# Setup
# ----------------------------------------------------------------------------


def sub_batch(meta, requests, tensors):
    """A batch of some requests of `meta` over the same pools (rows re-packed)."""
    import numpy as np
    import torch
    import workloads
    qo = [int(meta.qo_indptr[r + 1] - meta.qo_indptr[r]) for r in requests]
    pages = [meta.kv_page_indices[meta.kv_page_indptr[r]:meta.kv_page_indptr[r + 1]]
             for r in requests]
    sub = workloads.Meta(
        qo_indptr=np.concatenate([[0], np.cumsum(qo)]).astype(np.int32),
        kv_len=np.array([meta.kv_len[r] for r in requests], dtype=np.int32),
        kv_page_indptr=np.concatenate([[0], np.cumsum([len(p) for p in pages])]).astype(np.int32),
        kv_page_indices=np.concatenate(pages).astype(np.int32),
        num_pages=meta.num_pages, page_size=meta.page_size)
    rows = np.concatenate([np.arange(meta.qo_indptr[r], meta.qo_indptr[r + 1]) for r in requests])
    idx = torch.from_numpy(rows).to(tensors["q"].device)
    t = dict(tensors)
    for k in ("q", "k_new", "v_new"):
        if t[k] is not None:
            t[k] = t[k].index_select(0, idx).contiguous()
    return sub, t


def make_plan(spec, meta, tree_masks=None):
    import ragged_paged_kv_append_amd as rpa
    cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                          spec.page_size, spec.dtype, spec.causal, spec.sm_scale)
    return rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages, tree_masks=tree_masks)


def tree_of(parents):
    """Ancestor-or-self mask of a draft tree given each node's parent (-1: root)."""
    import numpy as np
    n = len(parents)
    m = np.zeros((n, n), dtype=bool)
    for t in range(n):
        u = t
        while u >= 0:
            m[t, u] = True
            u = parents[u]
    return m


def plan_host_ms(spec, meta, reps=20):
    import ragged_paged_kv_append_amd as rpa
    cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                          spec.page_size, spec.dtype, spec.causal, spec.sm_scale)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        h = rpa.rpa_plan_create(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                                meta.kv_page_indices, meta.num_pages)
        ts.append(time.perf_counter() - t0)
        rpa.rpa_plan_destroy(h)
    ts.sort()
    return 1e3 * ts[len(ts) // 2]


def request_classes(plan):
    items = plan.debug("items").reshape(-1, 8)
    return {int(r): int(k) for r, k in zip(items[:, 0], items[:, 7])}


# ----------------------------------------------------------------------------
# Timing
# ----------------------------------------------------------------------------


ATTN_KERNELS = ("generic", "decode", "prefill", "mla")
SCRUB_BYTES = 1 << 30   # > 2x the 256 MB MALL: evicts it (and every L2) between timed steps

_hip = None
_scrub = None


def hip_events(n):
    """n timing events without the system-scope fence (creating them through
    torch would add a cache flush of several microseconds to each record)."""
    import ctypes
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if _hip.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    return evs


def scrub():
    """Writes SCRUB_BYTES of device memory (outside the timed events), so that
    no step finds the previous step's data in the MALL or an L2."""
    import torch
    global _scrub
    if _scrub is None:
        _scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")
    _scrub.fill_(int(time.perf_counter_ns() & 0xffff))


def timed_steps(step, steps, warmup):
    """Runs `warmup` steps, then times exactly `steps` steps.  Each timed step
    is bracketed by its own pair of HIP events on the launch stream, with a
    SCRUB_BYTES write before it (outside the events).  Returns a dict with the
    median, minimum and mean step time (ms), the wall-clock time of the whole
    timed loop per step (scrubs included), and per-kernel timings
    {kernel: (avg ms, launches per step)}.

    A short profiling pass first (every kernel bracketed by events, scrubbed
    steps, outside the timed loop) finds the attention kernel that takes the
    most time per step; the timed steps carry library events around that
    kernel only, which give its average launch time over the timed region.
    The other kernels' figures come from the profiling pass."""
    import ctypes
    import statistics
    import torch
    import ragged_paged_kv_append_amd as rpa
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    def read_all(n_steps):
        out = {}
        for name in KERNELS:
            tot, n = rpa.rpa_profile_read(name)
            if n:
                out[name] = (tot / n, n / n_steps)
        return out

    prof_steps = max(3, min(steps, 10))
    rpa.rpa_profile_reset()
    rpa.rpa_profile_select(None)
    rpa.rpa_profile_enable(True)
    for _ in range(prof_steps):
        scrub()
        step()
    torch.cuda.synchronize()
    rpa.rpa_profile_enable(False)
    kernels = read_all(prof_steps)
    attn = [k for k in kernels if k in ATTN_KERNELS]
    only = [max(attn, key=lambda k: kernels[k][0] * kernels[k][1])] if attn else ["append"]

    evs = hip_events(2 * steps)
    stream = torch.cuda.current_stream().cuda_stream
    rpa.rpa_profile_reset()
    rpa.rpa_profile_select(only)
    rpa.rpa_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        scrub()
        _hip.hipEventRecord(evs[2 * i], stream)
        step()
        _hip.hipEventRecord(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rpa.rpa_profile_enable(False)
    rpa.rpa_profile_select(None)
    kernels.update(read_all(steps))
    per_step = []
    for i in range(steps):
        ms = ctypes.c_float()
        _hip.hipEventSynchronize(evs[2 * i + 1])
        if _hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        per_step.append(float(ms.value))
    for e in evs:
        _hip.hipEventDestroy(e)
    return {"median_ms": statistics.median(per_step), "min_ms": min(per_step),
            "mean_ms": statistics.fmean(per_step), "wall_ms": 1e3 * (t1 - t0) / steps,
            "kernels": kernels}


def run_batch(spec, meta, tensors, steps, warmup, tree_masks=None):
    plan = make_plan(spec, meta, tree_masks)

    def step():
        plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
        plan.attention(tensors["q"], tensors["k_pool"], tensors["v_pool"], o=out["o"],
                       lse=out["lse"])

    import torch
    out = {"o": torch.empty((meta.total_q, spec.num_qo_heads, spec.head_dim_v),
                            dtype=tensors["q"].dtype, device=tensors["q"].device),
           "lse": torch.empty((meta.total_q, spec.num_qo_heads), dtype=torch.float32,
                              device=tensors["q"].device)}
    tm = timed_steps(step, steps, warmup)
    if not torch.isfinite(out["o"].float()).all():
        raise RuntimeError("non-finite attention output")
    return plan, tm


KERNEL_SOURCES = {"generic": "basic.hip", "decode": "decode.hip", "prefill": "prefill.hip",
                  "mla": "mla.hip"}
SHARED_SOURCES = ("kernels/common.h", "launch.h", "rpa_internal.h", "plan.cpp")


def kernel_source_hash(kernel):
    """Hash of the sources a kernel's launches depend on (its file, the shared
    device header, the launch declarations, the plan layout and the planner)."""
    import hashlib
    csrc = os.path.join(ROOT, "ragged_paged_kv_append_amd", "csrc")
    h = hashlib.sha256()
    for rel in ("kernels/" + KERNEL_SOURCES[kernel],) + SHARED_SOURCES:
        with open(os.path.join(csrc, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when no run exists for
    this kernel and workload or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f).get(workload, {}).get(kernel)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("src_hash") != kernel_source_hash(kernel):
        return None
    return entry["traffic_bytes"]


def append_entry(w, kernels):
    """KV append as bandwidth: every appended byte is read once and written once."""
    if "append" not in kernels:
        return None
    us = kernels["append"][0] * 1e3
    nbytes = w["append_bytes"]
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"us": us, "bytes": nbytes, "gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}


def roofline_for(spec, meta, plan, kernels):
    """Roofline entry of the attention kernel that takes the most time per step."""
    attn = {k: v for k, v in kernels.items() if k in ("generic", "decode", "prefill", "mla")}
    if not attn:
        return None
    name = max(attn, key=lambda k: attn[k][0] * attn[k][1])
    avg_ms, per_step = attn[name]
    cls_id = {"generic": 0, "decode": 1, "prefill": 2, "mla": 3}[name]
    rc = request_classes(plan)
    reqs = [r for r in range(meta.batch_size) if rc.get(r) == cls_id]
    qo = [int(meta.qo_indptr[r + 1] - meta.qo_indptr[r]) for r in reqs]
    kv = [int(meta.kv_len[r]) for r in reqs]
    w = work(spec, qo, kv)
    launch_s = avg_ms * 1e-3
    if name in ("prefill", "mla"):
        achieved = w["flops"] / per_step / launch_s / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic(spec.name, name),
                "avg_launch_us": avg_ms * 1e3,
                "algorithmic_per_launch": {"flops": w["flops"] / per_step}}
    nbytes = (w["kv_bytes"] + w["qo_bytes"]) / per_step
    achieved = nbytes / launch_s / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(spec.name, name),
            "avg_launch_us": avg_ms * 1e3, "algorithmic_per_launch": {"bytes": nbytes}}


def run_chunked(spec, steps, warmup, parts=True):
    """The 8192-token GQA prompt run as 16 chunks of 512 (append, then
    attention over the pages, per chunk) and one-shot.  Every chunk step is
    timed on its own after the whole prompt has been appended once (the append
    is idempotent, and a chunk's attention reads only keys below its end)."""
    import numpy as np
    import torch
    import workloads
    import ragged_paged_kv_append_amd as rpa
    L, C = spec.extra["prompt_len"], spec.extra["chunk"]
    q, k, v = workloads.make_prompt(spec, spec.seed, device="cuda")
    meta = workloads.make_meta([L], [L], spec.page_size, spec.seed)
    pages = meta.kv_page_indices
    shape = (meta.num_pages, spec.num_kv_heads, spec.page_size, spec.head_dim_qk)
    k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    v_pool = k_pool.clone()
    o = torch.empty((L, spec.num_qo_heads, spec.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, spec.num_qo_heads), dtype=torch.float32, device="cuda")
    cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                          spec.page_size, spec.dtype, spec.causal, spec.sm_scale)

    def step_of(a, n):
        plan = rpa.Plan(cfg, [0, n], [a + n], [0, len(pages)], pages, meta.num_pages)

        def step():
            plan.append(k[a:a + n], v[a:a + n], k_pool, v_pool)
            plan.attention(q[a:a + n], k_pool, v_pool, o=o[a:a + n], lse=lse[a:a + n])
        return step

    chunks = [step_of(a, min(C, L - a)) for a in range(0, L, C)]
    for st in chunks:
        st()
    torch.cuda.synchronize()
    per_chunk = []
    for i, st in enumerate(chunks):
        a = i * C
        n = min(C, L - a)
        tm = timed_steps(st, steps, warmup)
        kernels = tm["kernels"]
        w = work(spec, [n], [a + n])
        attn_ms = sum(t * c for name, (t, c) in kernels.items() if name != "append")
        per_chunk.append({"chunk": i, "kv_len": a + n, "ms_per_step": tm["median_ms"],
                          "ms_per_step_min": tm["min_ms"], "attention_ms": attn_ms,
                          "flops": w["flops"], "tflops": w["flops"] / (attn_ms * 1e-3) / 1e12,
                          "kernels_us": {kk: t * 1e3 for kk, (t, c) in kernels.items()},
                          "launches": {kk: c for kk, (t, c) in kernels.items()}})
    # the same chunks in split form: cache part (cross attention over the
    # pages) and own part (causal, over the chunk's own K/V rows) in one
    # launch, then their merge, all in one library call; timed like the fused
    # form (the sum of its attention kernels' times), the call's span on the
    # stream (launch gaps included) reported beside it
    o_s = torch.empty_like(o)
    lse_s = torch.empty_like(lse)
    split_chunks = []
    for i in range(len(chunks) if parts else 0):
        a = i * C
        n = min(C, L - a)
        sp = rpa.SplitChunkAttention(cfg, [0, n], [a + n], [0, len(pages)], pages, meta.num_pages)

        def st(sp=sp, a=a, n=n):
            sp.run(q[a:a + n], k[a:a + n], v[a:a + n], k_pool, v_pool, o=o_s[a:a + n],
                   lse=lse_s[a:a + n])
        tm = timed_steps(st, steps, warmup)
        kernels = tm["kernels"]
        w = work(spec, [n], [a + n])
        attn_ms = sum(t * c for name, (t, c) in kernels.items() if name != "append")
        split_chunks.append({"chunk": i, "kv_len": a + n, "attention_ms": attn_ms,
                             "span_ms": tm["median_ms"],
                             "flops": w["flops"], "tflops": w["flops"] / (attn_ms * 1e-3) / 1e12,
                             "kernels_us": {kk: t * 1e3 for kk, (t, c) in kernels.items()},
                             "launches": {kk: c for kk, (t, c) in kernels.items()}})
    if not parts:
        return per_chunk, None, split_chunks
    one = step_of(0, L)
    tm1 = timed_steps(one, max(3, steps // 4), 1)
    k1 = tm1["kernels"]
    w1 = work(spec, [L], [L])
    attn1 = sum(t * c for name, (t, c) in k1.items() if name != "append")
    one_shot = {"ms_per_step": tm1["median_ms"], "attention_ms": attn1, "flops": w1["flops"],
                "tflops": w1["flops"] / (attn1 * 1e-3) / 1e12,
                "kernels_us": {kk: t * 1e3 for kk, (t, c) in k1.items()}}
    return per_chunk, one_shot, split_chunks


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample, on this host's cores
# ----------------------------------------------------------------------------


def cpu_baseline(spec, meta, tensors, requests, unit):
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None

    def raw(t):
        import torch
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def f64(a):
        return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    sub, t = sub_batch(meta, requests, tensors)
    # the sample's pages, renumbered (input preparation, not timed)
    pages = sub.kv_page_indices
    import torch
    pidx = torch.from_numpy(pages.astype(np.int64)).to(tensors["k_pool"].device)
    kp = f64(raw(tensors["k_pool"].index_select(0, pidx)))
    vp = None if tensors["v_pool"] is None else f64(raw(tensors["v_pool"].index_select(0, pidx)))
    q = f64(raw(t["q"]))
    b = oracle.Batch(sub.qo_indptr, sub.kv_len, sub.kv_page_indptr,
                     np.arange(len(pages)), sub.page_size)
    t0 = time.perf_counter()
    oracle.attend(q, kp, vp, b, spec.num_qo_heads, spec.num_kv_heads, spec.sm_scale,
                  head_dim_v=spec.head_dim_v, causal=spec.causal)
    secs = time.perf_counter() - t0
    qo = [int(sub.qo_indptr[r + 1] - sub.qo_indptr[r]) for r in range(sub.batch_size)]
    w = work(spec, qo, sub.kv_len)
    value = (w["kv_bytes"] / secs / 1e9) if unit == "GB/s" else (w["flops"] / secs / 1e12)
    return {"value": value, "unit": unit, "cores": cores, "blas_threads": blas_threads,
            "kind": "oracle", "seconds": secs,
            "sample": f"fp64 numpy oracle attention over {len(requests)} of {meta.batch_size} "
                      f"requests of the same workload ({w['kv_bytes'] / 1e9:.3f} GB of KV, "
                      f"{w['flops'] / 1e9:.2f} GFLOP)"}


# ----------------------------------------------------------------------------
# Main
# ----------------------------------------------------------------------------


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain copy of known size: each launch reads and writes `nbytes`."""
    import torch
    torch.cuda.set_device(0)
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "ms_per_copy": dt * 1e3,
                      "gbps_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # Compute-bound kernels speed up by 7-10% over the first few hundred
    # milliseconds of load (clock ramp): the default warm-up covers that.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="mixed_7b",
                    choices=["mixed_7b", "decode_verify_gqa", "mla_absorbed", "chunked_gqa"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true",
                    help="time the workload's step only (no sub-batch or variant parts), "
                         "so that a profiler's per-kernel averages cover that step alone")
    ap.add_argument("--one-shot", action="store_true",
                    help="chunked_gqa only: time the whole 8192-token prompt as one step "
                         "(append, then attention) and nothing else, for profiler runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the known-size "
                         "kernel that FETCH_SIZE / WRITE_SIZE counter readings are scaled by)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import ragged_paged_kv_append_amd as rpa

    rpa.lib()
    torch.cuda.set_device(0)
    name = args.workload
    if name == "chunked_gqa":
        if args.one_shot:
            main_one_shot(args)
        else:
            main_chunked(args)
        return
    log(f"workload {name}: generating inputs")
    spec, meta, tensors = workloads.workload(name, device="cuda")
    torch.cuda.synchronize()
    qo = [int(meta.qo_indptr[r + 1] - meta.qo_indptr[r]) for r in range(meta.batch_size)]
    w = work(spec, qo, meta.kv_len)

    log(f"workload {name}: timing {args.steps} steps after {args.warmup} warmup")
    plan, tm = run_batch(spec, meta, tensors, args.steps, args.warmup)
    ms, kernels = tm["median_ms"], tm["kernels"]
    roof = roofline_for(spec, meta, plan, kernels)
    plan_ms = plan_host_ms(spec, meta)

    unit = "TFLOP/s" if name == "mla_absorbed" else "GB/s"
    if unit == "GB/s":
        value = w["kv_bytes"] / (ms * 1e-3) / 1e9
    else:
        value = w["flops"] / (ms * 1e-3) / 1e12

    parts = {}
    if name == "mixed_7b" and not args.no_parts:
        dec = [r for r in range(meta.batch_size) if qo[r] == 1]
        pre = [r for r in range(meta.batch_size) if qo[r] > 1]
        for label, reqs in (("decode", dec), ("prefill_chunk", pre)):
            sm, st = sub_batch(meta, reqs, tensors)
            log(f"part {label}: {len(reqs)} requests")
            sqo = [int(sm.qo_indptr[r + 1] - sm.qo_indptr[r]) for r in range(sm.batch_size)]
            sw = work(spec, sqo, sm.kv_len)
            _, ptm = run_batch(spec, sm, st, args.steps, args.warmup)
            pms, pk = ptm["median_ms"], ptm["kernels"]
            attn_ms = sum(v[0] * v[1] for k, v in pk.items() if k != "append")
            entry = {"requests": len(reqs), "ms_per_step": pms, "attention_ms": attn_ms,
                     "kernels_us": {k: v[0] * 1e3 for k, v in pk.items()}}
            if label == "decode":
                gbps = (sw["kv_bytes"] + sw["qo_bytes"]) / (attn_ms * 1e-3) / 1e9
                entry.update({"kv_read_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS})
            else:
                tf = sw["flops"] / (attn_ms * 1e-3) / 1e12
                entry.update({"tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS})
            parts[label] = entry

    if name == "decode_verify_gqa" and not args.no_parts:
        # the same step with every verify request's 4 new tokens as a draft
        # tree (root, two children of the root, one grandchild) instead of a
        # chain: the mask applies to the tiles holding new tokens only
        masks = [tree_of([-1, 0, 0, 1]) if qo[r] == 4 else None for r in range(meta.batch_size)]
        log("part tree_verify: verify requests as draft trees")
        _, ttm = run_batch(spec, meta, tensors, args.steps, args.warmup, tree_masks=masks)
        tms, tk = ttm["median_ms"], ttm["kernels"]
        attn_ms = sum(v[0] * v[1] for k, v in tk.items() if k != "append")
        gbps = (w["kv_bytes"] + w["qo_bytes"]) / (attn_ms * 1e-3) / 1e9
        base_ms = sum(v[0] * v[1] for k, v in kernels.items() if k != "append")
        parts["tree_verify"] = {"ms_per_step": tms, "attention_ms": attn_ms,
                                "kernels_us": {k: v[0] * 1e3 for k, v in tk.items()},
                                "kv_read_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
                                "slowdown_vs_chain": attn_ms / base_ms,
                                "tree_parents": [-1, 0, 0, 1]}

    if name == "decode_verify_gqa" and not args.no_parts:
        # page export for a sharded transfer: the K and V pages of the first 64
        # requests, each as two half-head shards, gathered from the HND pools
        # into packed shard buffers (one contiguous run per page and shard)
        reqs = list(range(64))
        pages = np.concatenate([meta.kv_page_indices[meta.kv_page_indptr[r]:
                                                     meta.kv_page_indptr[r + 1]] for r in reqs])
        pid = torch.as_tensor(pages.astype(np.int32), device="cuda")
        H = spec.num_kv_heads
        bufs = [torch.empty((len(pages), H // 2, spec.page_size, spec.head_dim_qk),
                            dtype=tensors["k_pool"].dtype, device="cuda") for _ in range(4)]

        def export_step():
            for j, pool in enumerate((tensors["k_pool"], tensors["v_pool"])):
                for s_ in range(2):
                    rpa.copy_pages(pool, bufs[2 * j + s_], src_pages=pid,
                                   src_head0=s_ * (H // 2), num_heads=H // 2)
        log(f"part page_export: {len(pages)} pages x 2 pools x 2 shards")
        etm = timed_steps(export_step, args.steps, args.warmup)
        ems, ek = etm["median_ms"], etm["kernels"]
        copied = 2 * len(pages) * H * spec.page_size * spec.head_dim_qk * spec.elem_bytes
        cms = ek["page_copy"][0] * ek["page_copy"][1]
        parts["page_export"] = {"pages": int(len(pages)), "bytes_copied": copied,
                                "ms_per_step": ems, "kernel_ms": cms,
                                "hbm_gbps": 2 * copied / (cms * 1e-3) / 1e9,
                                "hbm_frac": 2 * copied / (cms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                "launches": ek["page_copy"][1]}

    if name == "decode_verify_gqa" and not args.no_parts:
        # prefix-cache page sharing: the first 64 requests read one common
        # 960-token prefix (60 read-only pages of request 0, page aligned, so
        # no shared page is appended to) and their own pages after it; timed
        # against the same batch with every request on its own pages.  The
        # logical KV bytes are the same; the shared pages are read from HBM
        # once and from the caches after.
        import dataclasses
        reqs = list(range(64))
        sm, st = sub_batch(meta, reqs, tensors)
        share = 960 // spec.page_size
        idx = sm.kv_page_indices.copy()
        shared = idx[sm.kv_page_indptr[0]:sm.kv_page_indptr[0] + share].copy()
        for i in range(len(reqs)):
            idx[sm.kv_page_indptr[i]:sm.kv_page_indptr[i] + share] = shared
        shm = dataclasses.replace(sm, kv_page_indices=idx)
        sqo = [int(sm.qo_indptr[r + 1] - sm.qo_indptr[r]) for r in range(sm.batch_size)]
        sw = work(spec, sqo, sm.kv_len)
        per_tok = spec.num_kv_heads * (spec.head_dim_qk + spec.head_dim_v) * spec.elem_bytes
        unique = sw["kv_bytes"] - (len(reqs) - 1) * share * spec.page_size * per_tok
        entry = {"requests": len(reqs), "shared_prefix_tokens": share * spec.page_size,
                 "logical_kv_bytes": sw["kv_bytes"], "unique_kv_bytes": int(unique)}
        for label, m_ in (("own_pages", sm), ("shared_prefix", shm)):
            log(f"part prefix_share: {label}")
            _, ptm = run_batch(spec, m_, st, args.steps, args.warmup)
            pms, pk = ptm["median_ms"], ptm["kernels"]
            attn_ms = sum(v[0] * v[1] for k, v in pk.items() if k != "append")
            entry[label] = {"ms_per_step": pms, "attention_ms": attn_ms,
                            "kernels_us": {k: v[0] * 1e3 for k, v in pk.items()},
                            "logical_kv_gbps": (sw["kv_bytes"] + sw["qo_bytes"]) /
                                               (attn_ms * 1e-3) / 1e9}
        entry["shared_prefix"]["unique_kv_gbps"] = (unique + sw["qo_bytes"]) / (
            entry["shared_prefix"]["attention_ms"] * 1e-3) / 1e9
        parts["prefix_share"] = entry

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        if name == "mixed_7b":
            sample = list(range(meta.batch_size))
        elif name == "decode_verify_gqa":
            sample = list(range(0, meta.batch_size, 16))
        else:
            sample = list(range(0, meta.batch_size, 8))
        cpu = cpu_baseline(spec, meta, tensors, sample, unit)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_min": tm["min_ms"],
        "ms_per_step_mean": tm["mean_ms"],
        "timing": f"median of {args.steps} steps, each between its own pair of HIP events, "
                  f"after a {SCRUB_BYTES >> 20} MiB device write outside the events "
                  f"(wall clock of the timed loop, writes included: {tm['wall_ms']:.4f} ms/step)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": name, "requests": meta.batch_size, "total_q": meta.total_q,
                   "num_qo_heads": spec.num_qo_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim_qk": spec.head_dim_qk, "head_dim_v": spec.head_dim_v,
                   "page_size": spec.page_size, "kv_tokens": int(np.sum(meta.kv_len)),
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "work": {"kv_bytes": w["kv_bytes"], "flops": w["flops"], "qo_bytes": w["qo_bytes"]},
        "kernels_us": {k: v[0] * 1e3 for k, v in kernels.items()},
        "launches_per_step": {k: v[1] for k, v in kernels.items()},
        "plan_ms": plan_ms,
        "append": append_entry(w, kernels),
        "parts": parts,
    }
    print(json.dumps(line), flush=True)


def main_one_shot(args):
    """The 8192-token GQA prompt of chunked_gqa attended in one step (one plan
    over the whole prompt): the prefill kernel at its largest single-request
    size.  One JSON line with the step's attention TFLOP/s."""
    import torch
    import workloads
    import ragged_paged_kv_append_amd as rpa
    spec = workloads.SPECS["chunked_gqa"]
    L = spec.extra["prompt_len"]
    q, k, v = workloads.make_prompt(spec, spec.seed, device="cuda")
    meta = workloads.make_meta([L], [L], spec.page_size, spec.seed)
    shape = (meta.num_pages, spec.num_kv_heads, spec.page_size, spec.head_dim_qk)
    k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    v_pool = k_pool.clone()
    o = torch.empty((L, spec.num_qo_heads, spec.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, spec.num_qo_heads), dtype=torch.float32, device="cuda")
    cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                          spec.page_size, spec.dtype, spec.causal, spec.sm_scale)
    plan = rpa.Plan(cfg, [0, L], [L], meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)

    def step():
        plan.append(k, v, k_pool, v_pool)
        plan.attention(q, k_pool, v_pool, o=o, lse=lse)
    log(f"workload chunked_gqa one-shot: timing {args.steps} steps after {args.warmup} warmup")
    tm = timed_steps(step, args.steps, args.warmup)
    w = work(spec, [L], [L])
    kernels = tm["kernels"]
    attn = sum(t * c for name, (t, c) in kernels.items() if name != "append")
    pre = kernels.get("prefill", (None, 0))[0]
    print(json.dumps({"workload": "chunked_gqa one-shot", "prompt_len": L, "flops": w["flops"],
                      "ms_per_step": tm["median_ms"], "attention_ms": attn,
                      "tflops": w["flops"] / (attn * 1e-3) / 1e12,
                      "prefill_kernel_tflops": None if not pre else w["flops"] / (pre * 1e-3) / 1e12,
                      "kernels_us": {kk: t * 1e3 for kk, (t, c) in kernels.items()}}), flush=True)


def main_chunked(args):
    """Chunked prefill of one 8192-token GQA prompt (16 chunks of 512): value
    is the aggregate attention TFLOP/s over the 16 chunk steps."""
    import workloads
    spec = workloads.SPECS["chunked_gqa"]
    log(f"workload chunked_gqa: timing each of 16 chunk steps, {args.steps} steps after "
        f"{args.warmup} warmup")
    per_chunk, one_shot, split_chunks = run_chunked(spec, args.steps, args.warmup,
                                                    parts=not args.no_parts)
    flops = sum(c["flops"] for c in per_chunk)
    attn_ms = sum(c["attention_ms"] for c in per_chunk)
    step_ms = sum(c["ms_per_step"] for c in per_chunk)
    pre_us = [c["kernels_us"].get("prefill", 0.0) * c["launches"].get("prefill", 0.0)
              for c in per_chunk]
    launches = sum(c["launches"].get("prefill", 0.0) for c in per_chunk)
    achieved = flops / (sum(pre_us) * 1e-6) / 1e12 if sum(pre_us) > 0 else None
    roof = None
    if achieved is not None:
        roof = {"kernel": "prefill", "bound": "mfma", "achieved": achieved,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic("chunked_gqa", "prefill"),
                "avg_launch_us": sum(pre_us) / launches,
                "algorithmic_per_launch": {"flops": flops / launches}}
    line = {
        "metric": METRIC, "value": flops / (attn_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": "chunked_gqa", "prompt_len": spec.extra["prompt_len"],
                   "chunk": spec.extra["chunk"], "num_qo_heads": spec.num_qo_heads,
                   "num_kv_heads": spec.num_kv_heads, "head_dim_qk": spec.head_dim_qk,
                   "head_dim_v": spec.head_dim_v, "page_size": spec.page_size,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof, "cpu_baseline": None,
        "work": {"flops": flops},
        "parts": {"chunks": [{k: c[k] for k in ("chunk", "kv_len", "tflops", "attention_ms",
                                                "kernels_us")} for c in per_chunk],
                  "one_shot": one_shot,
                  "split": None if not split_chunks else {
                      "tflops": sum(c["flops"] for c in split_chunks)
                      / (sum(c["attention_ms"] for c in split_chunks) * 1e-3) / 1e12,
                      # the same chunks fused (after the append), attention kernels only
                      "fused_tflops": sum(c["flops"] for c in per_chunk)
                      / (sum(c["attention_ms"] for c in per_chunk) * 1e-3) / 1e12,
                      # each call's span on the stream, launch gaps included
                      "span_tflops": sum(c["flops"] for c in split_chunks)
                      / (sum(c["span_ms"] for c in split_chunks) * 1e-3) / 1e12,
                      "timing": "split and fused: the sum of their attention kernels' times "
                                "(span_tflops: each split call's span on the stream)",
                      "chunks": [{k: c[k] for k in ("chunk", "tflops", "attention_ms", "span_ms",
                                                    "kernels_us")} for c in split_chunks]}},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
