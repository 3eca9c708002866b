#!/usr/bin/env python3
"""Decode-step benchmark of the prefix-tree two-phase attention on one MI355X.

One step = one ca_attend (chunk-first, sequence-first and merge kernels) over
the whole batch, with the chunk table already uploaded and Q resident in HBM.
Before each timed step a 1 GiB scratch buffer is read (outside the timing
events), so neither the 256 MB Infinity Cache nor the L2s hold KV: the
figures are cold-cache HBM figures.  The flush only reads, so the caches hold
clean lines that cost nothing to evict (a writing flush would leave dirty
lines whose write-back competes with the step).  Warm (back-to-back) figures
are reported alongside, labelled.

Prints one JSON line.  Its top level is the headline workload (by default
the multi-branch tree: 128 sequences x 32 heads, a 1,024-token root, four
1,024-token branches, private suffixes of 64..1,024 tokens):
  value        attended KV tokens/s (sum of sequence lengths / step time)
  roofline     the dominant kernel's unique-KV bytes / its own average
               duration (HIP events on the launching stream), against the
               8 TB/s HBM peak; traffic as recorded by the counter passes
               under profiles/ for the same kernel source
  comparator   the same step on the unshared paged layout (every sequence
               keeps its own copy of every chunk; no chunk-first phase)
  comparator_shared_pages  the prefix stored once but no chunk-first phase
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
per_config holds the same figures for the other workloads (and the 1,766-token
prefix, and chunk sizes 32 and 128); ns_sweep_batch32 the shared-prompt sweep
(0..4096 shared tokens, batch 32); decode_progression the decode sweeps over
completion length and batch (2,048 shared prompt tokens); decode_host_overlap
the host time of structural and fill-only decode steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--headline-only]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
METRIC = "attended KV tokens/s per decode step; unique-KV HBM GB/s vs 8 TB/s peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="headline workload 1..5 (default 5: the multi-branch tree, 128 seq x 32 heads)")
    ap.add_argument("--no-comparator", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (headline)")
    ap.add_argument("--cpu-seconds-per-config", type=float, default=4.0,
                    help="target CPU time of the oracle sample of each other workload")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline workload (no per_config entries, no decode point)")
    ap.add_argument("--no-decode", action="store_true", help="leave out the decode-progression point")
    ap.add_argument("--prefix-len", type=int, default=None,
                    help="instead of a numbered workload: --n-seq sequences x 32 heads with this shared prefix "
                         "length (any length, e.g. 1766) and --suffix-len private tokens each")
    ap.add_argument("--suffix-len", type=int, default=512)
    ap.add_argument("--chunk", type=int, default=64, choices=(32, 64, 128),
                    help="chunk size of the cache (the workloads are defined at 64)")
    ap.add_argument("--n-seq", type=int, default=32, help="sequences of the --prefix-len workload")
    ap.add_argument("--decode", action="store_true",
                    help="decode progression instead: n_s = 2048 shared prompt tokens, one token appended per "
                         "sequence per step (completion length n_c sweep at batch 32, batch sweep at n_c = 512), "
                         "as ca_decode_step and as append + attend, with the shared-pages comparator")
    ap.add_argument("--decode-only", default=None, metavar="MODE:BATCH:NC",
                    help="with --decode: one run only, e.g. decode_step:32:512 (modes decode_step, two_phase, "
                         "shared_pages_no_chunk_first), for profiling one configuration")
    ap.add_argument("--row-appends", type=int, default=1, choices=(0, 1),
                    help="with --decode: chunks made by appends stored row-major (1, the library default) or "
                         "as tiles (0)")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the step timing loop (for rocprofv3 runs): warmup steps, then cold steps as "
                         "ca_attend runs them; prints the event mean")
    ap.add_argument("--phases", action="store_true",
                    help="with --profile-only: launch the chunk-first and sequence-first parts of the partials "
                         "kernel separately (then the merge), so counters can be read per phase")
    return ap.parse_args()


class Flusher:
    """Reads a 1 GiB buffer: evicts KV from the Infinity Cache and L2s and
    leaves only clean lines behind."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.acc = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        # same dtype in and out: one reduction kernel, no conversion copy
        self.torch.sum(self.buf, dim=0, out=self.acc)


def time_steps(torch, fn, steps, flush=None):
    """Per-step event times (ms) of fn() on the current stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush()
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def time_launches(torch, ca, q, out, steps, flush, phases):
    """Event times (ms) of each launch in `phases` (ca_attend_phase ids),
    launched one after another on the current stream, cold."""
    ca.prepare()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        ev[i][0].record()
        for j, ph in enumerate(phases):
            ca.attend_phase(ph, q, out)
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    return np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(phases))] for i in range(steps)])


def step_kernel_digest():
    """sha256 over the device sources of the decode-step kernels."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_attention_prefix_tree_amd", "csrc")
    h = hashlib.sha256()
    for name in ("kernels.hip", "kernels.h", "tile_layout.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def recorded_traffic(config):
    """HBM bytes per partials launch from the committed counter summary, if it
    was taken on this workload with the kernel source as it is now; else None."""
    root = os.path.dirname(os.path.abspath(__file__))
    prof = os.path.join(root, "profiles", f"partials_kernel_workload{config}_traffic.md")
    if not os.path.exists(prof):
        return None
    fields = {}
    for line in open(prof):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    digest = step_kernel_digest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, seconds_target):
    """The fp64 oracle on the host cores: one thread per worker over the
    sequences (BLAS limited to one thread each), repeated passes over a
    sample of the workload's sequences until about seconds_target of wall
    time; tokens/s from the median pass.  Also a one-thread rate."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    workers = len(os.sched_getaffinity(0))

    def one(i):
        k, v = wl.seq_kv(i)
        return A.attend_sequence(wl.q[i], k, v)

    ctx = threadpool_limits(1) if threadpool_limits else None
    try:
        # size the sample from one row: a pass should take at most a third of the budget
        t0 = time.perf_counter()
        one(0)
        t_row = time.perf_counter() - t0
        n = wl.n_seq
        if t_row * n / min(workers, n) > seconds_target / 3:
            n = max(min(workers, wl.n_seq), int(seconds_target / 3 * workers / max(t_row, 1e-6)))
        sample = list(range(min(n, wl.n_seq)))
        passes = []
        with ThreadPoolExecutor(max_workers=workers) as ex:
            start = time.perf_counter()
            while len(passes) < 3 or (time.perf_counter() - start < seconds_target and len(passes) < 500):
                t0 = time.perf_counter()
                list(ex.map(one, sample))
                passes.append(time.perf_counter() - t0)
            total = time.perf_counter() - start
        # one thread, on as many rows as take about a second
        k1 = max(1, min(len(sample), int(1.0 / max(t_row, 1e-6))))
        t0 = time.perf_counter()
        for i in range(k1):
            one(i)
        t1 = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    toks = int(sum(wl.seq_len(i) for i in sample))
    used = min(workers, len(sample))
    med = float(np.median(passes))
    return {"value": toks / med, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "single_thread_tokens_per_s": int(sum(wl.seq_len(i) for i in range(k1))) / t1,
            "cpu_model": cpu_model(),
            "sample": f"{len(sample)} of {wl.n_seq} sequences ({toks} attended tokens, all {wl.heads} heads) per pass, "
                      f"{len(passes)} passes in {total:.1f} s, median pass {med * 1e3:.1f} ms; fp64 numpy oracle, "
                      f"{used} threads over sequences, BLAS 1 thread each"}


def decode_progression(torch, n_seq, n_shared, checkpoints, two_phase, flush, window=16, heads=32, seed=7,
                       one_call=False, row_appends=1):
    """Decode steps from a fully shared prompt: each step appends one token per
    sequence and attends, either as ca_append_batch + ca_attend or, with
    one_call, as ca_decode_step.  Returns, per checkpoint n_c (the completion
    length reached), the mean cold GPU time of the append and the attend (or
    of the whole step) over the `window` steps ending there, and the host time
    per step (each timed call is made with only the flush ahead of it on the
    stream)."""
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    gen = torch.Generator(device="cuda").manual_seed(seed)
    max_c = max(checkpoints)
    cap = (n_shared + 63) // 64 + n_seq * ((max_c + 63) // 64 + 1) + 8
    ca = ChunkAttention(heads, cap, device="cuda:0", two_phase=two_phase)
    ca.set_option(_capi.CA_OPT_ROW_APPENDS, row_appends)
    ks = torch.randn((n_shared, heads, 128), generator=gen, device="cuda").half()
    vs = torch.randn((n_shared, heads, 128), generator=gen, device="cuda").half()
    prompt = np.arange(n_shared, dtype=np.int32)
    for i in range(n_seq):
        ca.insert(i, prompt, ks, vs)
    ids = list(range(n_seq))
    out = torch.empty((n_seq, heads, 128), dtype=torch.float16, device="cuda")
    res, pending = {}, []
    for c in range(1, max_c + 1):
        k = torch.randn((n_seq, heads, 128), generator=gen, device="cuda").half()
        v = torch.randn((n_seq, heads, 128), generator=gen, device="cuda").half()
        q = torch.randn((n_seq, heads, 128), generator=gen, device="cuda").half()
        timed = any(cp - window < c <= cp for cp in checkpoints)
        toks = np.full(n_seq, c, np.int32)
        if timed:
            # untimed steps let the host run far ahead of the GPU; drain the
            # queue first so that the call's host time is its own work and not
            # a wait for queue space or a staging buffer the GPU still reads
            torch.cuda.synchronize()
            flush()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            h0 = time.perf_counter()
            e[0].record()
            if one_call:
                e[1] = e[0]  # one call: the whole step is reported as the attend column
                ca.decode_step(toks, k, v, q, out)
            else:
                ca.append_batch(ids, toks, k, v)
                e[1].record()
                ca.attend(q, out)
            e[2].record()
            pending.append((c, e, time.perf_counter() - h0))
        elif one_call:
            ca.decode_step(toks, k, v, q, out)
        else:
            ca.append_batch(ids, toks, k, v)
            ca.attend(q, out)
        if c in checkpoints:
            torch.cuda.synchronize()
            rows = [(e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), h) for cc, e, h in pending]
            app = float(np.mean([r[0] for r in rows])) * 1e3
            att = float(np.mean([r[1] for r in rows])) * 1e3
            host = float(np.mean([r[2] for r in rows])) * 1e6
            host_p50 = float(np.median([r[2] for r in rows])) * 1e6
            host_max = float(np.max([r[2] for r in rows])) * 1e6
            st = ca.stats()
            # with one_call the append column is 0 and attend is the whole step
            res[c] = {"append_us": app, "attend_us": att, "host_us_per_step": host,
                      "host_us_p50": host_p50, "host_us_max": host_max,
                      "generated_tokens_per_s": n_seq / ((app + att) * 1e-6),
                      "attended_tokens_per_s": st["attended_tokens"] / (att * 1e-6),
                      "unique_kv_gbps": st["unique_kv_bytes"] / (att * 1e-6) / 1e9,
                      "table_rebuilds": st["table_rebuilds"], "table_uploads": st["table_uploads"],
                      "patched_appends": st["patched_appends"]}
            pending = []
    del ca
    torch.cuda.synchronize()
    return res


def decode_host_overlap(torch, n_seq, n_shared, n_steps, prebuild, heads=32, seed=11):
    """Decode steps as a sampling loop runs them: after each ca_decode_step the
    host waits for the GPU (the next token would come from that step's
    output).  Per step: the host time of the call and the wall time from call
    to finished step, split into structural steps (a chunk filled up: the
    table changes shape and is uploaded), the steps just before them (which,
    with the prebuild on, also build the next table after their launch,
    while the GPU runs) and the other fill-only steps."""
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    gen = torch.Generator(device="cuda").manual_seed(seed)
    cap = (n_shared + 63) // 64 + n_seq * ((n_steps + 63) // 64 + 1) + 8
    ca = ChunkAttention(heads, cap, device="cuda:0")
    ca.set_option(_capi.CA_OPT_PREBUILD_PLAN, 1 if prebuild else 0)
    ks = torch.randn((n_shared, heads, 128), generator=gen, device="cuda").half()
    prompt = np.arange(n_shared, dtype=np.int32)
    for i in range(n_seq):
        ca.insert(i, prompt, ks, ks)
    out = torch.empty((n_seq, heads, 128), dtype=torch.float16, device="cuda")
    ca.ensure_workspace()
    k = torch.randn((n_seq, heads, 128), generator=gen, device="cuda").half()
    q = torch.randn((n_seq, heads, 128), generator=gen, device="cuda").half()
    ca.attend(q, out)
    torch.cuda.synchronize()
    rows = []
    toks = np.zeros(n_seq, np.int32)
    for c in range(1, n_steps + 1):
        toks[:] = c
        t0 = time.perf_counter()
        ca.decode_step(toks, k, k, q, out)
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        # the prompt fills whole chunks, so every 64th append opens new chunks
        kind = "structural" if (c - 1) % 64 == 0 else "before_structural" if c % 64 == 0 else "fill_only"
        rows.append((kind, (t1 - t0) * 1e6, (t2 - t0) * 1e6))
    st = ca.stats()
    del ca
    torch.cuda.synchronize()
    res = {"prebuild": bool(prebuild), "steps": n_steps, "prebuilt_plans": st["prebuilt_plans"],
           "table_uploads": st["table_uploads"]}
    for name in ("structural", "before_structural", "fill_only"):
        sel = [r for r in rows[1:] if r[0] == name]  # the first step warms up
        res[name] = {"steps": len(sel), "call_us": float(np.mean([r[1] for r in sel])) if sel else None,
                     "wall_us": float(np.mean([r[2] for r in sel])) if sel else None,
                     "call_us_p50": float(np.median([r[1] for r in sel])) if sel else None,
                     "wall_us_p50": float(np.median([r[2] for r in sel])) if sel else None}
    return res


def decode_main(args, torch):
    flush = Flusher(torch)
    line = {"metric": "decode progression: generated tokens/s (ca_decode_step: one token per sequence "
                      "appended and attended per call)",
            "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "n_s = 2048 shared prompt tokens, heads 32, head_dim 128, chunk 64",
                       "cache": "cold (1 GiB read before each timed step)"}}
    modes = (("decode_step", True, True), ("two_phase", True, False), ("shared_pages_no_chunk_first", False, False))
    if args.decode_only:
        mode, batch, nc = args.decode_only.split(":")
        two_phase, one_call = {m[0]: m[1:] for m in modes}[mode]
        line["config"].update({"mode": mode, "batch": int(batch), "n_c": int(nc), "row_appends": args.row_appends})
        r = decode_progression(torch, int(batch), 2048, [int(nc)], two_phase, flush, one_call=one_call,
                               row_appends=args.row_appends)[int(nc)]
        line.update(r)
        line["value"] = r["generated_tokens_per_s"]
        print(json.dumps(line), flush=True)
        return
    for name, two_phase, one_call in modes:
        log(f"decode n_c sweep, {name}")
        line.setdefault("nc_sweep_batch32", {})[name] = decode_progression(
            torch, 32, 2048, [512, 1024, 2048], two_phase, flush, one_call=one_call)
        log(f"decode batch sweep, {name}")
        line.setdefault("batch_sweep_nc512", {})[name] = {
            b: decode_progression(torch, b, 2048, [512], two_phase, flush, one_call=one_call)[512]
            for b in (16, 32, 64, 96)}
    sw = line["nc_sweep_batch32"]

    def step_us(r):
        return r["append_us"] + r["attend_us"]

    line["speedup_vs_shared_pages"] = {
        nc: step_us(sw["shared_pages_no_chunk_first"][nc]) / step_us(sw["decode_step"][nc]) for nc in sw["decode_step"]}
    line["value"] = sw["decode_step"][512]["generated_tokens_per_s"]
    print(json.dumps(line), flush=True)


def step_stats(ms):
    """mean / p10 / p50 / p90 in microseconds of per-step event times (ms)."""
    return {"mean": float(ms.mean()) * 1e3, "p10": float(np.percentile(ms, 10)) * 1e3,
            "p50": float(np.median(ms)) * 1e3, "p90": float(np.percentile(ms, 90)) * 1e3}


def comparator(torch, wl, q, steps, warmup, flush, t_ours, seg_cache, kind, **kw):
    """The same step on another layout of the same workload, timed the same way."""
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed
    cmp_ca = ChunkAttention(wl.heads, slots_needed(wl, share=kw.get("share", True)) + 8, device="cuda:0", **kw)
    load_workload(cmp_ca, wl, segments=seg_cache)
    cmp_ca.ensure_workspace()
    out2 = torch.empty_like(q)

    def cstep():
        cmp_ca.attend(q, out2)

    for _ in range(warmup):
        cstep()
    cc = time_steps(torch, cstep, steps, flush)
    tc = float(cc.mean()) * 1e-3
    cst = cmp_ca.stats()
    res = {"kind": kind, "ms_per_step": tc * 1e3, "attended_tokens_per_s": cst["attended_tokens"] / tc,
           "stored_kv_gbps": cst["unique_kv_bytes"] / tc / 1e9,
           # bytes the kernels ask for, counting every re-read of a shared chunk;
           # caches (L2, Infinity Cache) serve many of them, so this is not HBM traffic
           "logical_kv_read_gbps": (cst["sf_chunk_reads"] + cst["cf_chunk_reads"]) * 4 * 64 * wl.heads * 128
           / tc / 1e9,
           "speedup": tc / t_ours}
    del cmp_ca
    torch.cuda.synchronize()
    return res


def measure(torch, args, wl, flush, full, seg_cache, chunk=64, comparators=True, cpu_seconds=None):
    """One workload: the step timed cold over args.steps steps (after
    args.warmup untimed ones), its launches timed apart, the comparators and
    the oracle on the host.  full: also warm steps and the phases alone."""
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi, load_workload, slots_needed
    ca = ChunkAttention(wl.heads, slots_needed(wl, chunk=chunk) + 8, device="cuda:0", chunk_size=chunk)
    load_workload(ca, wl, segments=seg_cache)
    q = torch.from_numpy(wl.q).cuda()
    out = torch.empty_like(q)
    ca.ensure_workspace()
    st = ca.stats()
    torch.cuda.synchronize()

    def step():
        ca.attend(q, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    cold = time_steps(torch, step, args.steps, flush)
    wall = time.perf_counter() - wall0
    one_launch = bool(st["one_launch_step"])
    lt = time_launches(torch, ca, q, out, args.steps, flush, (_capi.CA_PHASE_PARTIALS, _capi.CA_PHASE_MERGE))
    unique_b = st["unique_kv_bytes"]
    t_mean = float(cold.mean()) * 1e-3
    # The dominant kernel: the partials launch (chunk-first and sequence-first
    # blocks in one grid), or, in the one-launch step, that launch with the
    # merge blocks, which is the whole step.  Algorithmic bytes per launch: the
    # unique KV bytes (each shared chunk once, each private chunk once).
    dom_t = t_mean if one_launch else float(lt[:, 0].mean()) * 1e-3
    res = {
        "workload": wl.description, "n_seq": wl.n_seq, "heads": wl.heads, "chunk": chunk,
        "launches_per_step": 1 if one_launch else 2,
        "cf_chunks_per_task": st["cf_chunks_per_task"], "sf_chunks_per_task": st["sf_chunks_per_task"],
        "step_us": step_stats(cold),
        "attended_tokens_per_s": st["attended_tokens"] / t_mean,
        "unique_kv_gbps": unique_b / t_mean / 1e9,
        "frac": unique_b / t_mean / 1e9 / HBM_PEAK_GBPS,
        "queries_per_s": wl.n_seq / t_mean,
        "dominant_kernel": {"kernel": "partials_kernel" + (" (one-launch step, merge blocks included)"
                                                           if one_launch else ""),
                            "avg_launch_us": dom_t * 1e6, "gbps": unique_b / dom_t / 1e9,
                            "frac": unique_b / dom_t / 1e9 / HBM_PEAK_GBPS},
        "launch_us_two_launch_form": {"partials_kernel": float(lt[:, 0].mean()) * 1e3,
                                      "merge_kernel": float(lt[:, 1].mean()) * 1e3},
        "tokens": {"attended": st["attended_tokens"], "unique": st["unique_tokens"],
                   "shared": st["shared_tokens"], "private": st["private_tokens"]},
        "unique_kv_bytes": unique_b,
        "timed_wall_s": wall,
    }
    if full:
        per_tok = 4 * wl.heads * wl.head_dim
        warm = time_steps(torch, step, args.steps)
        ph = time_launches(torch, ca, q, out, args.steps, flush,
                           (_capi.CA_PHASE_CHUNK_FIRST, _capi.CA_PHASE_SEQUENCE_FIRST))
        res["warm_step_us"] = {"mean": float(warm.mean()) * 1e3, "p50": float(np.median(warm)) * 1e3,
                               "unique_kv_gbps": unique_b / (float(warm.mean()) * 1e-3) / 1e9}
        res["phase_alone_us"] = {"chunk_first": float(ph[:, 0].mean()) * 1e3,
                                 "sequence_first": float(ph[:, 1].mean()) * 1e3,
                                 "sequence_first_gbps": st["private_tokens"] * per_tok
                                 / (float(ph[:, 1].mean()) * 1e-3) / 1e9}
    del ca
    torch.cuda.synchronize()
    if comparators and not args.no_comparator:
        log("  comparator: unshared paged layout")
        res["comparator"] = comparator(
            torch, wl, q, args.steps, args.warmup, flush, t_mean, seg_cache,
            "unshared paged decode (own HIP kernel, every sequence keeps its own 64-token blocks)", share=False)
        log("  comparator: shared pages, no chunk-first phase")
        res["comparator_shared_pages"] = comparator(
            torch, wl, q, args.steps, args.warmup, flush, t_mean, seg_cache,
            "shared pages without two-phase partition (prefix stored once, every sequence streams its "
            "whole path)", two_phase=False)
    if cpu_seconds and not args.no_cpu_baseline:
        log("  cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange; only the one-GPU share is run here)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed
    from workloads import CONFIG_NAMES, make_config, make_prefix_suffix

    torch.cuda.set_device(0)
    if args.decode:
        decode_main(args, torch)
        return
    if args.prefix_len is not None:
        wl = make_prefix_suffix(args.prefix_len, [args.suffix_len] * args.n_seq, heads=32,
                                seed=2000 + args.prefix_len)
        workload_name = "prefix-suffix: " + wl.description
        args.config = None
    else:
        wl = make_config(args.config)
        workload_name = CONFIG_NAMES[args.config]
    log(f"building workload {workload_name}")
    flush = Flusher(torch)

    if args.profile_only:
        from decode_attention_prefix_tree_amd import _capi
        ca = ChunkAttention(wl.heads, slots_needed(wl, chunk=args.chunk) + 8, device="cuda:0",
                            chunk_size=args.chunk)
        load_workload(ca, wl)
        q = torch.from_numpy(wl.q).cuda()
        out = torch.empty_like(q)
        ca.ensure_workspace()
        st = ca.stats()
        torch.cuda.synchronize()

        def step():
            ca.attend(q, out)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        one_launch = bool(st["one_launch_step"])
        if not args.phases:
            # the real step (ca_attend): one launch whose grid ends with the
            # merge blocks, or the partials launch and the merge launch
            names = ("step (partials_kernel, merge blocks included)" if one_launch
                     else "step (partials_kernel + merge_kernel)",)
            lt = time_steps(torch, step, args.steps, flush)[:, None]
        elif args.phases:
            names = ("chunk_first", "sequence_first", "merge_kernel")
            lt = time_launches(torch, ca, q, out, args.steps, flush,
                               (_capi.CA_PHASE_CHUNK_FIRST, _capi.CA_PHASE_SEQUENCE_FIRST, _capi.CA_PHASE_MERGE))
        # Calibration for hardware byte counters: a plain device copy of a known
        # size (256 MiB read + 256 MiB written), cold like the steps.
        src = torch.ones(1 << 27, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            flush()
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"launch_us_mean": {n: float(lt[:, j].mean()) * 1e3 for j, n in enumerate(names)},
                          "cf_units": st["cf_units"], "heads": wl.heads, "shared_chunks": st["shared_chunks"],
                          "unique_kv_bytes": st["unique_kv_bytes"], "copy_calibration_bytes": src.numel() * 2,
                          "steps": args.steps, "config": args.config}), flush=True)
        return

    log(f"headline: {workload_name}")
    seg_cache = {}
    head = measure(torch, args, wl, flush, True, seg_cache, chunk=args.chunk, cpu_seconds=args.cpu_seconds)
    del seg_cache
    dom = head["dominant_kernel"]
    traffic = recorded_traffic(args.config) if args.config and args.chunk == 64 else None
    roof = {"kernel": dom["kernel"], "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "achieved": dom["gbps"], "frac": dom["gbps"] / HBM_PEAK_GBPS,
            "traffic": traffic,
            "traffic_source": (f"recorded: profiles/partials_kernel_workload{args.config}_traffic.md "
                               "(FETCH_SIZE and WRITE_SIZE passes, per launch; its kernel source sha256 "
                               "matches the sources built here)") if traffic else
                              "none recorded for this workload and kernel source",
            "bytes_per_launch": head["unique_kv_bytes"], "avg_launch_us": dom["avg_launch_us"]}
    t_mean = head["step_us"]["mean"] * 1e-6
    result = {
        "metric": METRIC,
        "value": head["attended_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_mean * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": workload_name, "n_seq": wl.n_seq, "heads": wl.heads,
                   "head_dim": wl.head_dim, "chunk": args.chunk, "cache": "cold (1 GiB read before each step)",
                   "cf_chunks_per_task": head["cf_chunks_per_task"],
                   "sf_chunks_per_task": head["sf_chunks_per_task"],
                   "launches_per_step": head["launches_per_step"]},
        "unique_kv_gbps": head["unique_kv_gbps"],
        "hbm_frac_unique": head["frac"],
        "queries_per_s": head["queries_per_s"],
        "step_us": head["step_us"],
        "roofline": roof,
    }
    for key in ("warm_step_us", "launch_us_two_launch_form", "phase_alone_us", "tokens", "timed_wall_s",
                "comparator", "comparator_shared_pages", "cpu_baseline"):
        if key in head:
            result[key] = head[key]
    del wl

    if not args.headline_only and args.prefix_len is None:
        per = {}
        cases = [(str(k), k, 64) for k in (1, 2, 3, 4, 5) if k != args.config]
        cases += [("prefix1766", None, 64), ("2_chunk32", 2, 32), ("2_chunk128", 2, 128)]
        for name, k, chunk in cases:
            if k is None:
                # the plugin system prompt of the pages (1,766 tokens) with 512-token suffixes
                w = make_prefix_suffix(1766, [512] * 32, heads=32, seed=2000 + 1766)
            else:
                w = make_config(k)
            log(f"per config: {name}: {w.description}, chunk {chunk}")
            cache = {}
            main_case = chunk == 64
            per[str(name)] = measure(torch, args, w, flush, False, cache, chunk=chunk, comparators=main_case,
                                     cpu_seconds=args.cpu_seconds_per_config if main_case else None)
            del cache, w
        result["per_config"] = per
    if not args.headline_only and args.prefix_len is None:
        # The pages' shared-prompt sweep (summary section 4.1, Table 3: chunk 64,
        # batch 32, shared tokens 0..4096), here with 512 private tokens each,
        # against shared pages without the chunk-first phase and the unshared
        # paged layout.
        log("shared-prompt sweep: 32 seq x 32 heads, n_s 0 / 1024 / 2048 / 4096 + 512 private")
        sweep = {}
        for ns in (0, 1024, 2048, 4096):
            w = make_prefix_suffix(ns, [512] * 32, heads=32, seed=3000 + ns)
            cache = {}
            r = measure(torch, args, w, flush, False, cache, cpu_seconds=None)
            sweep[str(ns)] = {"step_us": r["step_us"]["mean"], "unique_kv_gbps": r["unique_kv_gbps"], "frac": r["frac"],
                              "attended_tokens_per_s": r["attended_tokens_per_s"],
                              "shared_pages_step_us": r["comparator_shared_pages"]["ms_per_step"] * 1e3,
                              "unshared_step_us": r["comparator"]["ms_per_step"] * 1e3,
                              "speedup_vs_shared_pages": r["comparator_shared_pages"]["speedup"],
                              "speedup_vs_unshared": r["comparator"]["speedup"]}
            del cache, w
        result["ns_sweep_batch32"] = sweep
    if not args.headline_only and not args.no_decode:
        # The decode progression (Figures 3 and 4): 2,048 shared prompt tokens,
        # one token per sequence per step; completion lengths 512..2048 at batch
        # 32 and batches 16..96 at 512 completion tokens.
        log("decode progression: n_c 512 / 1024 / 2048 at batch 32, batch 16 / 32 / 64 / 96 at n_c 512")
        modes = (("decode_step", True, True), ("append_then_attend", True, False),
                 ("shared_pages_no_chunk_first", False, False))
        nc_sweep = {m: decode_progression(torch, 32, 2048, [512, 1024, 2048], tp, flush, one_call=oc)
                    for m, tp, oc in modes}
        batch_sweep = {m: {b: (nc_sweep[m][512] if b == 32 else
                               decode_progression(torch, b, 2048, [512], tp, flush, one_call=oc)[512])
                           for b in (16, 32, 64, 96)} for m, tp, oc in modes}

        def step_us(r):
            return r["append_us"] + r["attend_us"]

        result["decode_progression"] = {
            "workload": "32 heads, a 2,048-token prompt shared by every sequence, one token appended per sequence "
                        "per step; each point the mean of the 16 cold steps ending at that completion length",
            "nc_sweep_batch32": nc_sweep,
            "batch_sweep_nc512": batch_sweep,
            "generated_tokens_per_s_decode_step": {
                "nc": {nc: nc_sweep["decode_step"][nc]["generated_tokens_per_s"] for nc in (512, 1024, 2048)},
                "batch": {b: batch_sweep["decode_step"][b]["generated_tokens_per_s"] for b in (16, 32, 64, 96)}},
            "speedup_decode_step_vs_shared_pages": {
                "nc": {nc: step_us(nc_sweep["shared_pages_no_chunk_first"][nc]) / step_us(nc_sweep["decode_step"][nc])
                       for nc in (512, 1024, 2048)},
                "batch": {b: step_us(batch_sweep["shared_pages_no_chunk_first"][b]) /
                          step_us(batch_sweep["decode_step"][b]) for b in (16, 32, 64, 96)}}}
        log("decode host overlap: batch 32 and 96, 1024 steps, waiting for each step")
        result["decode_host_overlap"] = {
            f"batch{b}": {("prebuild_on" if pb else "prebuild_off"): decode_host_overlap(torch, b, 2048, 1024, pb)
                          for pb in (True, False)} for b in (32, 96)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
