"""Benchmark of paged GQA attention at head_dim 512 on one MI355X.

Prints ONE JSON line.  The headline is paged decode HBM throughput on the GQA decode
workload (batch 32, 24 query / 4 KV heads, head_dim 512, page size 16, KV lengths
uniform in [1024, 8192], bf16), split by the balanced planner: ``value`` is algorithmic
bytes per step divided by the measured step time, with the inputs resident in HBM.  A
step is one pass of the decode hot path: the split-K partial kernel and the log-sum-exp
merge kernel (the plan is host work, made and uploaded once before timing).  The other
workloads (the same GQA inputs with a fixed split-K of 8, FP8 decode, sliding-window
decode, causal prefill) are reported under ``secondary``.

Algorithmic work:
  decode bytes  = sum_b Hkv * |visible keys_b| * (Dqk + Dvo) * bytes_per_kv_element
                  + Q bytes + output bytes + 4 * (pages touched) + 4 * (2B + 1)
  prefill flops = sum_b sum_i Hq * |visible keys of row i| * 2 * (Dqk + Dvo)
Both are counted from the realised seeded lengths.

Timing: `ms_per_step` (and `value`) come from one pair of HIP events on the launch stream
around K back-to-back steps; `protocol` gives the median, minimum and mean of 50 further
iterations timed one by one (an event between consecutive iterations); the dominant
kernel's average duration (`roofline.kernel_avg_ms`): for prefill the step itself (one
launch, or the split kernel and its merge); for decode the step less the merge kernel, whose
duration comes from K back-to-back merge launches between one pair of events (consecutive
launches abut, so no event sits between kernels).  The sliding-window workloads at head_dim 256 (about 0.4 GB of visible KV,
close to the 256 MB last-level cache) alternate between two copies of the pool in every
timed loop.  Every line carries the oracle's CPU throughput on a bounded sample of the same
workload (`cpu_baseline`).

`--profile` runs only W + K launches of the named workload's hot path (no other timing,
no baseline, no secondary workloads), for rocprofv3: its kernel averages then cover exactly
those calls.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-secondary] [--no-cpu-baseline] [--profile]
"""

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "paged decode attn HBM GB/s (% peak) at hd512 GQA; prefill TFLOP/s"
# Kernel sources per kernel family, for tying counter summaries to the code they were
# taken on; the host planner decides the kernels' work split, so it counts too.
_SHARED_SOURCES = ["paged_attention_hd512_amd/csrc/pa_device.hpp",
                   "paged_attention_hd512_amd/csrc/pa_internal.hpp",
                   "paged_attention_hd512_amd/csrc/pa_host.cpp"]
KERNEL_SOURCES = {
    "decode": ["paged_attention_hd512_amd/csrc/pa_decode.hip"] + _SHARED_SOURCES,
    "prefill": ["paged_attention_hd512_amd/csrc/pa_prefill.hip"] + _SHARED_SOURCES,
}


def kernel_source_hash(family):
    """Hash of one kernel family's sources' code: comments and whitespace are dropped, so
    editing a comment does not mark counters taken on the same code as stale."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, p)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def kernel_family(workload):
    return "prefill" if "prefill" in workload else "decode"


# ----------------------------------------------------------------------------- work counts

def decode_algorithmic_bytes(case, requests=None):
    import numpy as np
    reqs = range(case.batch) if requests is None else requests
    # Bytes per KV element: bf16 2, FP8 1, NVFP4 half a byte plus one E4M3 block scale
    # per 16 elements.
    esz = {"bf16": 2.0, "fp8": 1.0, "nvfp4": 0.5 + 1.0 / 16}[case.kv_dtype]
    out_sz = 4 if case.out_dtype == "fp32" else 2
    total = 0
    for b in reqs:
        L = int(case.kv_lens[b])
        start = max(0, L - case.window) if case.window > 0 else 0
        vis = L - start
        pages = 0 if vis == 0 else (L - 1) // case.page_size - start // case.page_size + 1
        total += int(case.num_kv_heads * vis * (case.head_dim_qk + case.head_dim_vo) * esz)
        total += case.num_qo_heads * (case.head_dim_qk * 2 + case.head_dim_vo * out_sz)
        total += 4 * pages
    total += 4 * (2 * len(list(reqs)) + 1)
    return int(total)


def prefill_algorithmic_flops(case, requests=None):
    reqs = range(case.batch) if requests is None else requests
    total = 0
    for b in reqs:
        q_len, L = int(case.qo_lens[b]), int(case.kv_lens[b])
        for i in range(q_len):
            pos = L - q_len + i
            hi = pos + 1 if case.causal else L
            lo = max(0, pos - case.window + 1) if case.window > 0 else 0
            total += case.num_qo_heads * max(0, hi - lo) * 2 * (case.head_dim_qk + case.head_dim_vo)
    return int(total)


def extend_algorithmic_bytes(case):
    """HBM bytes a short-query prefill must move: for each (request, KV head) the K and V
    rows of every key some row of the request sees, plus Q and the output."""
    total = 0
    for b in range(case.batch):
        q_len, L = int(case.qo_lens[b]), int(case.kv_lens[b])
        if q_len == 0:
            continue
        lo = max(0, L - q_len - case.window + 1) if case.window > 0 else 0
        hi = L if case.causal else L
        total += case.num_kv_heads * max(0, hi - lo) * (case.head_dim_qk + case.head_dim_vo) * 2
        total += q_len * case.num_qo_heads * (case.head_dim_qk * 2 + case.head_dim_vo * 2)
    return int(total)


# ----------------------------------------------------------------------------- timing

def time_steps(launch, stream, steps):
    """ms per step of `steps` back-to-back steps, from one pair of HIP events on the launch
    stream around them (events recorded between the kernels would themselves add several
    microseconds to every step), and the host wall-clock per step."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def time_protocol(launch, stream, iters=50):
    """Median, minimum and mean (ms) of `iters` iterations timed one by one: one HIP event
    between consecutive iterations on the launch stream."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(iters):
        launch()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    med = (t[(iters - 1) // 2] + t[iters // 2]) / 2
    return {"iters": iters, "median_ms": round(med, 5), "min_ms": round(t[0], 5),
            "mean_ms": round(sum(t) / iters, 5)}


def settle(launch, ms):
    """Untimed steps for at least `ms` of host wall time; returns how many ran.  After an
    idle gap (host work such as the oracle baseline) the GPU's clock takes tens of
    milliseconds under load to return to its loaded level: causal prefill steps measured one
    by one go from about 2.0 ms to 1.57 ms over their first 20 steps, so a line measured right
    after host work without this would time part of that ramp."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            launch()
        n += 4
        torch.cuda.synchronize()
    return n


class Rotation:
    """Calls the launches of several copies of a workload in turn (one per call)."""

    def __init__(self, fns):
        self.fns, self.i = fns, 0

    def __call__(self):
        f = self.fns[self.i]
        self.i = (self.i + 1) % len(self.fns)
        f()


def decode_runner(case):
    from paged_attention_hd512_amd import PagedDecode
    return PagedDecode(case.k_pool, case.v_pool, case.kv_indptr, case.kv_indices,
                       case.kv_last_page_len, case.num_qo_heads, kv_dtype=case.kv_dtype,
                       k_scale=case.k_scale, v_scale=case.v_scale, sm_scale=case.sm_scale,
                       window=case.window, num_splits=case.num_splits, out_dtype=case.out_dtype,
                       k_sf=case.k_sf, v_sf=case.v_sf)


def pool_copy(case):
    """The same case over a second copy of its KV pool (and block scales)."""
    import copy
    c2 = copy.copy(case)
    if case.cache is not None:
        c2.cache = case.cache.clone()
        c2.k_pool, c2.v_pool = c2.cache[:, 0], c2.cache[:, 1]
    else:
        c2.k_pool, c2.v_pool = case.k_pool.clone(), case.v_pool.clone()
    if case.sf_cache is not None:
        c2.sf_cache = case.sf_cache.clone()
        c2.k_sf, c2.v_sf = c2.sf_cache[:, 0], c2.sf_cache[:, 1]
    elif case.k_sf is not None:
        c2.k_sf, c2.v_sf = case.k_sf.clone(), case.v_sf.clone()
    return c2


def time_decode(case, steps, warmup, copies=1, profile=False, settle_ms=0.0):
    """Returns (ms_per_step, partial_kernel_ms, merge_ms, wall_ms, plan, protocol): the step
    time of back-to-back decode steps, then the two kernels' durations from events around
    each, then the 50-iteration protocol.  With copies = 2 every loop alternates between
    two copies of the pool.  With settle_ms, untimed steps run for that long after the warmup
    ones.  With profile, only the warmup steps, the settle steps and `steps` more run."""
    import torch
    import paged_attention_hd512_amd.pa as pa

    cases = [case] + [pool_copy(case) for _ in range(copies - 1)]
    sh = pa.current_stream_handle()
    argsets = []
    runners = []
    for c in cases:
        run = decode_runner(c)
        out, lse = run.run(c.q)
        runners.append((run, out, lse))
        argsets.append((run.plan, c.q.data_ptr(), run.cache, run.table, run.params,
                        out.data_ptr(), lse.data_ptr(), run.workspace.data_ptr(),
                        run.workspace.numel(), sh))
    stream = torch.cuda.current_stream()
    step_fn = Rotation([lambda a=a: pa.pa_paged_decode(*a) for a in argsets])
    for _ in range(warmup):
        step_fn()
    if profile:
        settled = settle(step_fn, settle_ms)
        for _ in range(steps):
            step_fn()
        torch.cuda.synchronize()
        return None, None, None, None, runners[0][0].plan, {"settle_calls": settled}
    settled = settle(step_fn, settle_ms)
    step, wall = time_steps(step_fn, stream, steps)
    # The merge alone, back to back (it is idempotent: it re-reads the partials); consecutive
    # launches abut, so this average carries none of the few microseconds that an event
    # recorded between two kernels adds.  The partial kernel's duration inside the step is
    # then the step time less the merge's.  (Timing the partial kernel alone back to back
    # would give a shorter time than it takes inside a step, so it is not used.)
    merge, _ = time_steps(Rotation([lambda a=a: pa.pa_paged_decode_merge(*a) for a in argsets]),
                          stream, steps) if runners[0][0].plan.num_merges > 0 else (0.0, 0.0)
    part = step - merge
    proto = time_protocol(step_fn, stream)
    if settle_ms > 0:
        proto.update(settle_ms=settle_ms, settle_steps=settled)
    return max(step, 1e-9), part, merge, wall, runners[0][0].plan, proto


def time_decode_graph(case, steps, warmup):
    """The same decode step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: ms per replayed step, from HIP events around `steps` back-to-back replays."""
    import torch
    from paged_attention_hd512_amd import PagedDecode

    run = PagedDecode(case.k_pool, case.v_pool, case.kv_indptr, case.kv_indices,
                      case.kv_last_page_len, case.num_qo_heads, kv_dtype=case.kv_dtype,
                      k_scale=case.k_scale, v_scale=case.v_scale, sm_scale=case.sm_scale,
                      window=case.window, num_splits=case.num_splits, out_dtype=case.out_dtype,
                      k_sf=case.k_sf, v_sf=case.v_sf)
    out, lse = run.run(case.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.run(case.q, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.run(case.q, out=out, lse=lse)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_prefill(case, steps, warmup, profile=False, settle_ms=0.0):
    """Returns (ms_per_step, kernel_ms, wall_ms, plan, protocol): back-to-back prefill steps,
    then the duration of one step's launch(es) from events around it, then the 50-iteration
    protocol.  With settle_ms, untimed steps run for that long after the warmup ones.  With
    profile, only the warmup steps, the settle steps and `steps` more run."""
    import torch
    from paged_attention_hd512_amd import PagedPrefill
    import paged_attention_hd512_amd.pa as pa

    run = PagedPrefill(case.k_pool, case.v_pool, case.qo_indptr, case.kv_indptr,
                       case.kv_indices, case.kv_last_page_len, case.num_qo_heads,
                       kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                       sm_scale=case.sm_scale, window=case.window, causal=case.causal,
                       out_dtype=case.out_dtype, k_sf=case.k_sf, v_sf=case.v_sf)
    out, lse = run.run(case.q)
    stream = torch.cuda.current_stream()
    sh = pa.current_stream_handle()
    args = (run.plan, case.q.data_ptr(), run.qo_indptr_d.data_ptr(), run.cache, run.table,
            run.params, out.data_ptr(), lse.data_ptr(), run.workspace.data_ptr(),
            run.workspace.numel(), sh)
    for _ in range(warmup):
        pa.pa_paged_prefill(*args)
    if profile:
        settled = settle(lambda: pa.pa_paged_prefill(*args), settle_ms)
        for _ in range(steps):
            pa.pa_paged_prefill(*args)
        torch.cuda.synchronize()
        return None, None, None, run.plan, {"settle_calls": settled}
    settled = settle(lambda: pa.pa_paged_prefill(*args), settle_ms)
    step, wall = time_steps(lambda: pa.pa_paged_prefill(*args), stream, steps)
    # A prefill step is its kernel launch(es): back-to-back steps abut, so the step average
    # is the launch duration (events between launches would add a few microseconds each).
    kern = step
    proto = time_protocol(lambda: pa.pa_paged_prefill(*args), stream)
    if settle_ms > 0:
        proto.update(settle_ms=settle_ms, settle_steps=settled)
    return step, kern, wall, run.plan, proto


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_decode_baseline(case, budget_s=12.0):
    """The oracle, as it stands, timed on the requests of the same batch, pass after pass,
    until the budget is spent; throughput in algorithmic GB/s of the requests it finished.
    Each request's inputs are extracted once, outside the timed calls."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    from synth import extract_requests

    threads = cpu_threads()
    inputs = {}

    def request_inputs(b):
        if b not in inputs:
            sub = extract_requests(case, [b])
            dt = torch.int16 if case.kv_dtype == "bf16" else torch.uint8
            kp = sub["k_pool"].contiguous().view(dt).numpy()
            vp = sub["v_pool"].contiguous().view(dt).numpy()
            if case.kv_dtype == "bf16":
                kp, vp = kp.view(np.uint16), vp.view(np.uint16)
            sf = {}
            if case.kv_dtype == "nvfp4":
                sf = {n: sub[n].contiguous().numpy() for n in ("k_sf", "v_sf")}
            q = oracle.bf16_bits_to_f64(sub["q"].contiguous().view(torch.int16).numpy().view(np.uint16))
            inputs[b] = (q, kp, vp, sub["kv_indptr"], sub["kv_indices"], sub["kv_last_page_len"], sf)
        return inputs[b]

    done, spent = [], 0.0
    with threadpool_limits(limits=threads):
        while spent < budget_s:
            for b in range(case.batch):
                q, kp, vp, ip, ix, la, sf = request_inputs(b)
                t0 = time.perf_counter()
                oracle.decode_ref(q, kp, vp, ip, ix, la, case.page_size, case.sm_scale,
                                  window=case.window, kv_dtype=case.kv_dtype,
                                  k_scale=case.k_scale, v_scale=case.v_scale, **sf)
                spent += time.perf_counter() - t0
                done.append(b)
                if spent >= budget_s:
                    break
    nbytes = decode_algorithmic_bytes(case, done)
    passes = len(done) / case.batch
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(done)} request decodes ({passes:.1f} passes over the {case.batch} "
                      f"requests of the same batch), fp64 numpy on {cpu_model()}, {spent:.1f} s"}


def oracle_prefill_baseline(case, budget_s=12.0):
    """The oracle, as it stands, on rows of request 0 (64 query tokens at a time, all
    heads, the longest rows first) until the budget is spent; algorithmic TFLOP/s of the
    rows it finished."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    import oracle

    threads = cpu_threads()
    dt = torch.int16
    extra = {}
    if case.kv_dtype == "nvfp4":
        kp = case.k_pool.contiguous().cpu().numpy()
        vp = case.v_pool.contiguous().cpu().numpy()
        extra = dict(kv_dtype="nvfp4", k_scale=case.k_scale, v_scale=case.v_scale,
                     k_sf=case.k_sf.contiguous().cpu().numpy(),
                     v_sf=case.v_sf.contiguous().cpu().numpy())
    elif case.kv_dtype == "fp8":
        kp = case.k_pool.contiguous().cpu().view(torch.uint8).numpy()
        vp = case.v_pool.contiguous().cpu().view(torch.uint8).numpy()
        extra = dict(kv_dtype="fp8", k_scale=case.k_scale, v_scale=case.v_scale)
    else:
        kp = case.k_pool.contiguous().cpu().view(dt).numpy().view(np.uint16)
        vp = case.v_pool.contiguous().cpu().view(dt).numpy().view(np.uint16)
    q = oracle.bf16_bits_to_f64(case.q.contiguous().cpu().view(dt).numpy().view(np.uint16))
    flops, spent, rows = 0, 0.0, 0
    with threadpool_limits(limits=threads):
        # Rows of request 0 in chunks of 64 tokens, last (longest) rows first.
        q_len = int(case.qo_lens[0])
        for end in range(q_len, 0, -64):
            toks = np.arange(max(0, end - 64), end)
            t0 = time.perf_counter()
            oracle.prefill_ref(q, case.qo_indptr, kp, vp, case.kv_indptr, case.kv_indices,
                               case.kv_last_page_len, case.page_size, case.sm_scale,
                               causal=case.causal, window=case.window, tokens=toks, **extra)
            spent += time.perf_counter() - t0
            L = int(case.kv_lens[0])
            for i in toks:
                pos = L - q_len + int(i)
                flops += case.num_qo_heads * (pos + 1) * 2 * (case.head_dim_qk + case.head_dim_vo)
            rows += len(toks)
            if spent >= budget_s:
                break
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of {int(case.qo_lens.sum())} query tokens (all heads) of "
                      f"request 0, fp64 numpy on {cpu_model()}, {spent:.1f} s"}


def oracle_extend_baseline(case, budget_s=12.0):
    """The oracle, as it stands, on whole requests of the short-query workload (all their new
    tokens and heads), request after request until the budget is spent; algorithmic GB/s of
    the requests it finished."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    from synth import extract_requests

    threads = cpu_threads()
    done, spent, nbytes = [], 0.0, 0
    with threadpool_limits(limits=threads):
        while spent < budget_s:
            for b in range(case.batch):
                sub = extract_requests(case, [b])
                kp = sub["k_pool"].contiguous().view(torch.int16).numpy().view(np.uint16)
                vp = sub["v_pool"].contiguous().view(torch.int16).numpy().view(np.uint16)
                q = oracle.bf16_bits_to_f64(
                    sub["q"].contiguous().view(torch.int16).numpy().view(np.uint16))
                t0 = time.perf_counter()
                oracle.prefill_ref(q, sub["qo_indptr"], kp, vp, sub["kv_indptr"],
                                   sub["kv_indices"], sub["kv_last_page_len"], case.page_size,
                                   case.sm_scale, causal=case.causal, window=case.window)
                spent += time.perf_counter() - t0
                done.append(b)
                if spent >= budget_s:
                    break
    one = extend_algorithmic_bytes(case) / case.batch  # every request has the same shape
    return {"value": round(one * len(done) / spent / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(done)} whole requests ({case.qo_lens[0]} new tokens each, all heads), "
                      f"fp64 numpy on {cpu_model()}, {spent:.1f} s"}


def cpu_baseline_for(res, budget_s):
    case = res["case"]
    if res.get("kind") == "extend":
        return oracle_extend_baseline(case, budget_s)
    if "flops" in res:
        return oracle_prefill_baseline(case, budget_s)
    return oracle_decode_baseline(case, budget_s)


# ----------------------------------------------------------------------------- counters

def traffic_for(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash(kernel_family(workload)):
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- workloads

def decode_config(case):
    return {"workload": case.name, "batch": case.batch, "num_qo_heads": case.num_qo_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim_qk": case.head_dim_qk,
            "head_dim_vo": case.head_dim_vo, "page_size": case.page_size,
            "kv_dtype": case.kv_dtype, "window": case.window,
            "split_k": case.num_splits if case.num_splits > 0 else "balanced",
            "kv_len_min": int(case.kv_lens.min()), "kv_len_max": int(case.kv_lens.max()),
            "kv_len_mean": float(case.kv_lens.mean()), "out_dtype": case.out_dtype}


def measure_decode(name, steps, warmup, variant=None, profile=False, settle_ms=0.0):
    import torch
    from synth import decode_workload
    case = decode_workload(name, device="cuda", variant=variant)
    if isinstance(variant, str):
        case.name = f"{name}_{variant}"
    elif variant is not None:
        case.name = f"{name}_d{variant[0]}_p{variant[1]}"
    # Sliding window at head_dim 256: the visible KV (~0.4 GB) is close to the 256 MB
    # last-level cache, so the timed loops alternate between two copies of the pool.
    copies = 2 if name == "window_decode" and case.head_dim_qk == 256 else 1
    step_ms, part_ms, merge_ms, wall_ms, plan, proto = time_decode(case, steps, warmup, copies,
                                                                   profile, settle_ms)
    if profile:
        return {"case": case, "profiled_calls": warmup + proto["settle_calls"] + steps,
                "settle_calls": proto["settle_calls"], "pool_copies": copies}
    nbytes = decode_algorithmic_bytes(case)
    achieved = nbytes / (part_ms * 1e-3) / 1e9
    res = {
        "case": case, "bytes": nbytes, "step_ms": step_ms, "wall_ms": wall_ms,
        "kernel_ms": part_ms, "merge_ms": merge_ms,
        "value": nbytes / (step_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(case.name), "kernel": "decode_partial_kernel",
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel_avg_ms": round(part_ms, 5)},
        "plan": {"segments": plan.num_items, "waves": plan.num_workers,
                 "merged_pairs": plan.num_merges, "partial_slots": plan.num_slots,
                 "max_wave_blocks": plan.chunk_blocks},
        "protocol": dict(proto, pool_copies=copies),
    }
    return res


def measure_prefill(name, steps, warmup, head_dim_vo, profile=False, settle_ms=0.0):
    from synth import prefill_workload
    case = prefill_workload(name, device="cuda", head_dim_vo=head_dim_vo)
    case.name = f"{name}_qk512_vo{head_dim_vo}"
    step_ms, kern_ms, wall_ms, plan, proto = time_prefill(case, steps, warmup, profile,
                                                          settle_ms)
    if profile:
        return {"case": case, "profiled_calls": warmup + proto["settle_calls"] + steps,
                "settle_calls": proto["settle_calls"]}
    flops = prefill_algorithmic_flops(case)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    return {
        "case": case, "flops": flops, "step_ms": step_ms, "wall_ms": wall_ms,
        "kernel_ms": kern_ms, "value": flops / (step_ms * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(case.name),
                     "kernel": ("nvfp4_stage_kernel + prefill_kernel" if plan.staged_pages > 0
                                else "prefill_kernel"),
                     "algorithmic_flops_per_launch": flops, "kernel_avg_ms": round(kern_ms, 5)},
        "protocol": proto,
    }


def measure_extend(name, steps, warmup, profile=False, settle_ms=0.0):
    """Short-query extend: the whole call (prefill kernel over key chunks + merge) against
    the algorithmic HBM bytes."""
    from synth import prefill_workload
    case = prefill_workload(name, device="cuda", head_dim_vo=512)
    step_ms, kern_ms, wall_ms, plan, proto = time_prefill(case, steps, warmup, profile,
                                                          settle_ms)
    if profile:
        return {"case": case, "profiled_calls": warmup + proto["settle_calls"] + steps,
                "settle_calls": proto["settle_calls"], "kind": "extend"}
    nbytes = extend_algorithmic_bytes(case)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    return {
        "case": case, "bytes": nbytes, "step_ms": step_ms, "wall_ms": wall_ms, "kind": "extend",
        "kernel_ms": kern_ms, "value": nbytes / (step_ms * 1e-3) / 1e9, "protocol": proto,
        "plan": {"items": plan.num_items, "split_tiles": plan.num_merges,
                 "partial_slots": plan.num_slots, "chunk_stages": plan.chunk_blocks},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(case.name),
                     "kernel": "prefill_kernel + prefill_merge_kernel",
                     "algorithmic_bytes_per_launch": nbytes, "kernel_avg_ms": round(kern_ms, 5)},
    }


def copy_calibration(nbytes=1 << 30, steps=5):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "steps": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_decode",
                    help="gqa_decode | gqa_decode_splitk8 | fp8_decode | nvfp4_decode | "
                         "window_decode_d512_p1 | ... | "
                         "causal_prefill_vo512 | causal_prefill_vo256 | fp8_prefill_vo512 | "
                         "fp8_prefill_vo256 | nvfp4_prefill | extend_prefill")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="run only the warmup launches, the --settle-ms launches and then "
                         "`steps` launches of the workload (for rocprofv3)")
    ap.add_argument("--baseline-seconds", type=float, default=10.0,
                    help="oracle time for the headline's cpu_baseline (secondaries: a quarter)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="secondary lines: untimed steps for this long after the warmup steps")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    def run_named(wl, profile=False, settle_ms=0.0):
        st, wu, sm = args.steps, args.warmup, settle_ms
        if wl.startswith("window_decode_d"):
            d, p = wl[len("window_decode_d"):].split("_p")
            return measure_decode("window_decode", st, wu, (int(d), int(p)), profile, sm)
        if wl.startswith("causal_prefill_vo"):
            return measure_prefill("causal_prefill", st, wu, int(wl[len("causal_prefill_vo"):]),
                                   profile, sm)
        if wl.startswith("fp8_prefill_vo"):
            return measure_prefill("fp8_prefill", st, wu, int(wl[len("fp8_prefill_vo"):]),
                                   profile, sm)
        if wl == "extend_prefill":
            return measure_extend(wl, st, wu, profile, sm)
        if wl == "nvfp4_prefill":
            return measure_prefill(wl, st, wu, 256, profile, sm)
        if wl.startswith("gqa_decode_splitk"):
            return measure_decode("gqa_decode", st, wu, wl[len("gqa_decode_"):], profile, sm)
        return measure_decode(wl, st, wu, None, profile, sm)

    if args.profile:
        # Untimed calls for --settle-ms come before the last `steps` calls, so those run at
        # the settled clock, as a secondary line's timed steps do.
        r = run_named(args.workload, profile=True, settle_ms=args.settle_ms)
        print(json.dumps({"profile": args.workload, "workload": r["case"].name,
                          "calls": r["profiled_calls"], "warmup": args.warmup,
                          "settle_ms": args.settle_ms, "settle_calls": r["settle_calls"],
                          "steps": args.steps,
                          "kernel_source_hash": {f: kernel_source_hash(f)
                                                 for f in KERNEL_SOURCES}}), flush=True)
        return

    main_res = run_named(args.workload)
    case = main_res["case"]
    is_prefill = "flops" in main_res or main_res.get("kind") == "extend"
    line = {
        "metric": METRIC,
        "value": round(main_res["value"], 3),
        "unit": "TFLOP/s" if "flops" in main_res else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_res["step_ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if case.kv_dtype == "bf16" else f"{case.kv_dtype}-kv/bf16",
        "data": "synthetic",
        "config": decode_config(case) if not is_prefill else {
            "workload": case.name, "batch": case.batch, "qo_len": int(case.qo_lens[0]),
            "kv_len": int(case.kv_lens[0]), "num_qo_heads": case.num_qo_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim_qk": case.head_dim_qk,
            "head_dim_vo": case.head_dim_vo, "page_size": case.page_size, "causal": True},
        "roofline": main_res["roofline"],
        "protocol": main_res["protocol"],
        "wall_ms_per_step": round(main_res["wall_ms"], 5),
        "kernel_source_hash": {f: kernel_source_hash(f) for f in KERNEL_SOURCES},
    }
    if "merge_ms" in main_res:
        line["merge_ms"] = round(main_res["merge_ms"], 5)
        # The same step replayed from a captured HIP graph (no per-call host work).
        line["graph_ms_per_step"] = round(time_decode_graph(case, args.steps, args.warmup), 5)
    if "plan" in main_res:
        line["plan"] = main_res["plan"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_for(main_res, args.baseline_seconds)
    del main_res, case
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        names = ["gqa_decode", "gqa_decode_splitk8", "fp8_decode", "nvfp4_decode",
                 "window_decode_d512_p1", "window_decode_d512_p32",
                 "window_decode_d256_p1", "window_decode_d256_p32",
                 "causal_prefill_vo512", "causal_prefill_vo256",
                 "fp8_prefill_vo512", "fp8_prefill_vo256", "nvfp4_prefill", "extend_prefill"]
        for wl in names:
            if wl == args.workload:
                continue
            try:
                # Each secondary follows the previous line's oracle baseline (host work, GPU
                # idle), so its timed steps start once the clock has settled under load.
                r = run_named(wl, settle_ms=args.settle_ms)
                unit = "TFLOP/s" if "flops" in r else "GB/s"
                sec[wl] = {"value": round(r["value"], 3), "unit": unit,
                           "ms_per_step": round(r["step_ms"], 5), "roofline": r["roofline"],
                           "protocol": r["protocol"]}
                if "plan" in r and wl == "extend_prefill":
                    sec[wl]["plan"] = r["plan"]
                if not args.no_cpu_baseline:
                    sec[wl]["cpu_baseline"] = cpu_baseline_for(r, args.baseline_seconds / 4)
            except Exception as e:  # report, keep measuring the rest
                sec[wl] = {"error": f"{type(e).__name__}: {e}"}
            r = None
            torch.cuda.empty_cache()
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
