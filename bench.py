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

Prints one JSON line:
  value        attended KV tokens/s (sum of sequence lengths / step time)
  roofline     the dominant kernel's unique-KV bytes / its own average
               duration, against the 8 TB/s HBM peak
  comparator   the same step on the unshared paged layout (every sequence
               keeps its own copy of every chunk; no chunk-first phase)
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
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
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: 32 seq, 1024+512)")
    ap.add_argument("--no-comparator", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
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
    ap.add_argument("--profile-only", action="store_true",
                    help="only the per-kernel timing loop (for rocprofv3 runs); prints its event means")
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
                       one_call=False):
    """Decode steps from a fully shared prompt: each step appends one token per
    sequence and attends, either as ca_append_batch + ca_attend or, with
    one_call, as ca_decode_step.  Returns, per checkpoint n_c (the completion
    length reached), the mean cold GPU time of the append and the attend (or
    of the whole step) over the `window` steps ending there, and the host time
    per step."""
    from decode_attention_prefix_tree_amd import ChunkAttention
    gen = torch.Generator(device="cuda").manual_seed(seed)
    max_c = max(checkpoints)
    cap = (n_shared + 63) // 64 + n_seq * ((max_c + 63) // 64 + 1) + 8
    ca = ChunkAttention(heads, cap, device="cuda:0", two_phase=two_phase)
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
            st = ca.stats()
            # with one_call the append column is 0 and attend is the whole step
            res[c] = {"append_us": app, "attend_us": att, "host_us_per_step": host,
                      "generated_tokens_per_s": n_seq / ((app + att) * 1e-6),
                      "attended_tokens_per_s": st["attended_tokens"] / (att * 1e-6),
                      "unique_kv_gbps": st["unique_kv_bytes"] / (att * 1e-6) / 1e9,
                      "table_rebuilds": st["table_rebuilds"], "table_uploads": st["table_uploads"],
                      "patched_appends": st["patched_appends"]}
            pending = []
    del ca
    torch.cuda.synchronize()
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
        line["config"].update({"mode": mode, "batch": int(batch), "n_c": int(nc)})
        r = decode_progression(torch, int(batch), 2048, [int(nc)], two_phase, flush, one_call=one_call)[int(nc)]
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
    ca = ChunkAttention(wl.heads, slots_needed(wl, chunk=args.chunk) + 8, device="cuda:0", chunk_size=args.chunk)
    load_workload(ca, wl)
    q = torch.from_numpy(wl.q).cuda()
    out = torch.empty_like(q)
    ca.ensure_workspace()
    st = ca.stats()
    torch.cuda.synchronize()
    flush = Flusher(torch)

    def step():
        ca.attend(q, out)

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    from decode_attention_prefix_tree_amd import _capi
    step_launches = (_capi.CA_PHASE_PARTIALS, _capi.CA_PHASE_MERGE)
    one_launch = bool(st["one_launch_step"])
    if args.profile_only:
        if one_launch and not args.phases:
            # the step is one launch (merge blocks close the partials grid)
            names = ("partials_kernel (one-launch step)",)
            lt = time_steps(torch, step, args.steps, flush)[:, None]
        elif args.phases:
            names = ("chunk_first", "sequence_first", "merge_kernel")
            lt = time_launches(torch, ca, q, out, args.steps, flush,
                               (_capi.CA_PHASE_CHUNK_FIRST, _capi.CA_PHASE_SEQUENCE_FIRST, _capi.CA_PHASE_MERGE))
        else:
            names = ("partials_kernel", "merge_kernel")
            lt = time_launches(torch, ca, q, out, args.steps, flush, step_launches)
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

    log(f"timing {args.steps} cold steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    cold = time_steps(torch, step, args.steps, flush)
    wall = time.perf_counter() - wall0

    log("timing warm steps")
    warm = time_steps(torch, step, args.steps)
    log("timing launches")
    lt = time_launches(torch, ca, q, out, args.steps, flush, step_launches)
    ph = time_launches(torch, ca, q, out, args.steps, flush,
                       (_capi.CA_PHASE_CHUNK_FIRST, _capi.CA_PHASE_SEQUENCE_FIRST))

    unique_b = st["unique_kv_bytes"]
    per_tok = 4 * wl.heads * wl.head_dim
    shared_b = st["shared_tokens"] * per_tok
    private_b = st["private_tokens"] * per_tok
    t_mean = float(cold.mean()) * 1e-3
    value = st["attended_tokens"] / t_mean

    # The dominant kernel: the partials launch of a step (chunk-first and
    # sequence-first blocks in one grid; in the one-launch step it also holds
    # the merge blocks, and the step is that launch).  Its algorithmic bytes
    # are the unique KV bytes (each shared chunk once, each private chunk once).
    dom_t = t_mean if one_launch else float(lt[:, 0].mean()) * 1e-3
    roof = {"kernel": "partials_kernel" + (" (one-launch step, merge blocks included)" if one_launch else ""),
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "achieved": unique_b / dom_t / 1e9,
            "traffic": recorded_traffic(args.config) if args.config and not one_launch else None,
            "bytes_per_launch": unique_b, "avg_launch_us": dom_t * 1e6}
    roof["frac"] = roof["achieved"] / HBM_PEAK_GBPS

    result = {
        "metric": METRIC,
        "value": value,
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
                   "cf_chunks_per_task": st["cf_chunks_per_task"], "sf_chunks_per_task": st["sf_chunks_per_task"],
                   "launches_per_step": 1 if one_launch else 2},
        "unique_kv_gbps": unique_b / t_mean / 1e9,
        "hbm_frac_unique": unique_b / t_mean / 1e9 / HBM_PEAK_GBPS,
        "queries_per_s": wl.n_seq / t_mean,
        "step_us": {"mean": t_mean * 1e6, "p10": float(np.percentile(cold, 10)) * 1e3,
                    "p50": float(np.median(cold)) * 1e3, "p90": float(np.percentile(cold, 90)) * 1e3},
        "warm_step_us": {"mean": float(warm.mean()) * 1e3, "p50": float(np.median(warm)) * 1e3,
                         "unique_kv_gbps": unique_b / (float(warm.mean()) * 1e-3) / 1e9},
        "launch_us": {"partials_kernel": float(lt[:, 0].mean()) * 1e3, "merge_kernel": float(lt[:, 1].mean()) * 1e3},
        "phase_alone_us": {"chunk_first": float(ph[:, 0].mean()) * 1e3, "sequence_first": float(ph[:, 1].mean()) * 1e3,
                           "sequence_first_gbps": private_b / (float(ph[:, 1].mean()) * 1e-3) / 1e9},
        "tokens": {"attended": st["attended_tokens"], "unique": st["unique_tokens"],
                   "shared": st["shared_tokens"], "private": st["private_tokens"]},
        "timed_wall_s": wall,
        "roofline": roof,
    }

    if not args.no_comparator:
        def comparator(kind, **kw):
            cmp_ca = ChunkAttention(wl.heads, slots_needed(wl, share=kw.get("share", True)) + 8,
                                    device="cuda:0", **kw)
            load_workload(cmp_ca, wl)
            cmp_ca.ensure_workspace()
            out2 = torch.empty_like(q)

            def cstep():
                cmp_ca.attend(q, out2)

            for _ in range(args.warmup):
                cstep()
            cc = time_steps(torch, cstep, args.steps, flush)
            tc = float(cc.mean()) * 1e-3
            cst = cmp_ca.stats()
            res = {"kind": kind, "ms_per_step": tc * 1e3, "attended_tokens_per_s": cst["attended_tokens"] / tc,
                   "stored_kv_gbps": cst["unique_kv_bytes"] / tc / 1e9,
                   "read_kv_gbps": (cst["sf_chunk_reads"] + cst["cf_chunk_reads"]) * 4 * 64 * wl.heads * 128
                   / tc / 1e9,
                   "speedup": tc / t_mean}
            del cmp_ca
            torch.cuda.synchronize()
            return res

        log("comparator: unshared paged layout")
        result["comparator"] = comparator(
            "unshared paged decode (own HIP kernel, every sequence keeps its own 64-token blocks)", share=False)
        log("comparator: shared pages, no chunk-first phase")
        result["comparator_shared_pages"] = comparator(
            "shared pages without two-phase partition (prefix stored once, every sequence streams its "
            "whole path)", two_phase=False)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
