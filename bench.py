#!/usr/bin/env python3
"""Decode throughput of one DSA layer step at 128K context on one MI355X.

Workload (the headline): batch 16, context 131072 per sequence, RoPE layer, fp8 E4M3FN index keys
(one fp32 scale per token) and fp8 latent cache (one fp32 scale per 64 elements), bf16 queries.
One step = lightning-indexer scores over every cached key -> exact top-2048 -> sparse MLA decode
(64 heads, 512 + 64 dims).  The NoPE-layer and shared-indexer variants of the same shape, the
4096-token chunked prefill on a 61440-token prefix, the 512K block-sparse decode and the batch-64
16K-32K decode are timed the same way and reported beside it.  All inputs are seeded synthetic
tensors generated on the GPU and resident in HBM before timing starts; every timed loop cycles
through three copies of its workload's caches, so each call reads HBM as in a multi-layer decode.

Inside the timed steps the library's timing hook records every kernel's own duration (the start
and stop events of its dispatch); the roofline figure is the score kernel's average there.  --only NAME times one
configuration alone (for profiles of that configuration's kernels).

Prints one JSON line.  --gpus N > 1 is refused: this build runs on one GPU.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at 128K ctx (indexer+top-2048+sparse MLA); % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F16_PEAK_TFLOPS = 2500.0
INDEX_BYTES_PER_KEY = 128 + 4 + 4      # fp8 key row + fp32 scale read, fp32 score written
LATENT_BYTES_PER_KEY = 576 + 9 * 4     # fp8 latent row + 9 fp32 scales
MLA_FLOP_PER_KEY_HEAD = 2 * (576 + 512)   # QK^T over 576 dims and PV over 512, per selected key and head
INDEX_COUNTERS = os.path.join(ROOT, "profiles", "index_scores_fp8_b16_ctx128k_counters.txt")
INDEX_SOURCES = ["dsa_sparse_attention_indexer_amd/csrc/indexer.hip", "dsa_sparse_attention_indexer_amd/csrc/topk_common.h",
                 "dsa_sparse_attention_indexer_amd/csrc/dsa_internal.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


N_COPIES = 3   # copies of each workload's caches cycled through by the timed loops


def cache_copies(wl, n=N_COPIES):
    """The workload plus n - 1 copies whose caches (index keys, latents and their scales) are clones.

    A decode step of one layer reads that layer's caches once; between two steps of the same layer
    every other layer streams its own.  Timing back-to-back steps on one copy would instead serve part
    of the 285 MB index-key stream from the 256 MB last-level cache.  Cycling through copies (4+ GB)
    makes every timed step read HBM, as in a multi-layer decode."""
    out = [wl]
    for _ in range(n - 1):
        out.append(dataclasses.replace(
            wl, index_k=wl.index_k.clone(),
            index_k_scale=None if wl.index_k_scale is None else wl.index_k_scale.clone(),
            kv=wl.kv.clone(), kv_scale=None if wl.kv_scale is None else wl.kv_scale.clone()))
    return out


def cycling(fn, wls):
    """fn(workload) over the copies in turn."""
    i = [0]

    def call():
        fn(wls[i[0] % len(wls)])
        i[0] += 1
    return call


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per index-score launch from the committed rocprofv3 counter summary, or None if
    it is missing or was taken on a different version of the kernel's source."""
    try:
        with open(INDEX_COUNTERS) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("source_digest") != source_digest(INDEX_SOURCES):
            return None
        return float(kv["traffic_bytes_per_dispatch"])
    except (OSError, KeyError, ValueError):
        return None


def cache_writer_rates(dsa, timed, dev):
    """Per-call device time and algorithmic bandwidth of the cache writers (and the wall-clock
    time per call through the binding) for one decode step's 16 new tokens and one 4096-token
    prefill chunk.  Keys read: x (2 B x hidden per token) and the
    key projection's weight (2 B x 128 x hidden, once per call); written: 132 B per token.  Latent
    rows: 1152 B read, 612 B written per token.  The destination rows are numbered densely (the
    writers' cost does not depend on where the rows lie)."""
    import torch
    import workloads
    out = {}
    for name, b in (("decode_b16", workloads.insert_decode(device=dev)),
                    ("prefill_4096", workloads.insert_prefill(device=dev))):
        T, D = b.x.shape
        slot = torch.arange(T, dtype=torch.int64, device=dev)
        kc = torch.empty((T, 128), dtype=torch.uint8, device=dev)
        ks = torch.empty((T,), dtype=torch.float32, device=dev)
        lc = torch.empty((T, 576), dtype=torch.uint8, device=dev)
        ls = torch.empty((T, 9), dtype=torch.float32, device=dev)
        d = dsa.index_k_desc(b.x, D, 64, b.eps, T)
        ws = torch.empty(dsa.dsa_index_k_insert_workspace_size(d), dtype=torch.uint8, device=dev)
        fk = lambda: dsa.dsa_index_k_insert(b.x, b.wk, b.ln_w, b.ln_b, b.pos, slot, kc, ks,
                                            inv_freq=b.inv_freq, eps=b.eps, ws=ws)
        fl = lambda: dsa.dsa_latent_insert(b.kv, b.pos, slot, lc, ls, inv_freq=b.inv_freq)
        tk, tl = timed(fk), timed(fl)
        dk, dl = device_time(fk, dev), device_time(fl, dev)
        kbytes = T * 2 * D + 2 * 128 * D + T * 132
        lbytes = T * (2 * 576 + 576 + 36)
        out[f"index_k_insert_{name}"] = {"us_per_call": dk * 1e6, "gb_per_s": kbytes / dk / 1e9,
                                          "bytes_per_call": kbytes, "us_per_call_wall": tk * 1e6}
        out[f"latent_insert_{name}"] = {"us_per_call": dl * 1e6, "gb_per_s": lbytes / dl / 1e9,
                                         "bytes_per_call": lbytes, "us_per_call_wall": tl * 1e6}
    return out


def device_time(fn, dev, n=20):
    """Device time per call of a short call: a ~1 ms device copy is queued first, so all n calls
    are enqueued before the GPU reaches them and the events between them see device time only
    (launch gaps included), not the Python binding's per-call cost."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    del src, dst
    return e0.elapsed_time(e1) * 1e-3 / n


def oracle_rate(wl, seconds, block_sparse=False, max_queries=None):
    """Queries per second of the float64 oracle on whole queries of wl (scores over the full
    context, selection, sparse MLA), timed one query at a time until `seconds` have been spent."""
    import workloads
    from oracle import dsa_oracle as O
    n = wl.num_q if max_queries is None else min(wl.num_q, max_queries)
    done, elapsed = 0, 0.0
    while done == 0 or (elapsed < seconds and done < n):
        sub = workloads.slice_query(wl, done)
        t0 = time.perf_counter()
        O.decode_layer(sub, [0], block_sparse=block_sparse)
        elapsed += time.perf_counter() - t0
        done += 1
    return done / elapsed, done, elapsed


def oracle_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max((i.get("num_threads") or 1) for i in info) if info else None
    except Exception:
        return None


def cpu_baseline(wl, seconds):
    """The float64 oracle on whole queries of the headline workload, on this host's cores."""
    rate, done, elapsed = oracle_rate(wl, seconds)
    return {"value": rate, "unit": "tok/s", "cores": oracle_threads() or os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {wl.num_q} decode queries at context {wl.max_ctx} (full indexer scan, "
                      f"top-{wl.topk}, sparse MLA), float64 numpy, {elapsed:.1f} s"}


def mla_rates(wl, lengths, us):
    """Algorithmic MFMA rate and latent-gather bandwidth of a sparse-MLA stage that took `us`."""
    sel = int(lengths.long().sum())
    flops = sel * wl.mla_heads * MLA_FLOP_PER_KEY_HEAD
    tflops = flops / (us * 1e-6) / 1e12
    gbs = sel * LATENT_BYTES_PER_KEY / (us * 1e-6) / 1e9
    return {"us": us, "selected_keys": sel, "heads": wl.mla_heads, "tflops": tflops,
            "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS, "gather_gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def index_rates(wl, us):
    """MFMA rate of a many-query score kernel (prefill, verify blocks) that took `us`: every visible
    (query, key) pair is a 32-head x 128-dim product per fp16 term of q', and the kernel issues two
    terms (the hi and lo parts); the algorithmic rate counts the real heads and one term."""
    keys = int((wl.q_pos.long().clamp(min=-1, max=wl.max_ctx - 1) + 1).sum())
    issued = keys * 2 * 2 * 32 * 128
    alg = keys * 2 * wl.num_heads * 128
    return {"us": us, "visible_keys": keys, "issued_tflops": issued / (us * 1e-6) / 1e12,
            "frac_f16_peak": issued / (us * 1e-6) / 1e12 / F16_PEAK_TFLOPS,
            "algorithmic_tflops": alg / (us * 1e-6) / 1e12}


def mean(xs):
    return sum(xs) / len(xs)


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def _demangle_kernel(m):
    """The kernel identifier and its integer / bool template arguments from an Itanium-mangled
    name ('_ZN3dsa12_GLOBAL__N_112k_mla_fp8_wsILi64EEEvNS_9MlaLaunchE' -> 'k_mla_fp8_ws<64>')."""
    import re
    for hit in re.finditer(r"k_", m):
        p = hit.start()
        q = p
        while q > 0 and m[q - 1].isdigit():
            q -= 1
        for L in range(1, p - q + 1):
            n = int(m[p - L:p])
            ident = m[p:p + n]
            rest = m[p + n:]
            if len(ident) == n and re.fullmatch(r"k_\w+", ident) and rest[:1] in ("E", "I"):
                if not rest.startswith("I"):
                    return ident
                args = re.findall(r"L([ib])(\d+)E", rest[:rest.find("EE") + 2])
                vals = [("true" if v == "1" else "false") if t == "b" else v for t, v in args]
                return f"{ident}<{', '.join(vals)}>"
    return m


def short_name(name):
    """'void dsa::(anonymous namespace)::k_mla_fp8_ws<64>(dsa::MlaLaunch)' (or its mangled form)
    -> 'k_mla_fp8_ws<64>'."""
    if name.startswith("_Z"):
        return _demangle_kernel(name)
    head = name.split("(dsa::")[0] if "(dsa::" in name else name
    if "<" not in head:
        return head.rsplit("::", 1)[-1]
    cut = head.rfind("::", 0, head.index("<"))
    return head if cut < 0 else head[cut + 2:]


def stage_of(kernel):
    if kernel.startswith("k_index"):
        return "scores"
    if kernel.startswith(("k_topk", "k_block")):
        return "select"
    if kernel.startswith("k_mla"):
        return "sparse_mla"
    return "other"


def staged_steps(dsa, pipeline, wls, n, buf, *, prefill=False, block_sparse=False, shared_from=None):
    """n layer steps over the cache copies, timed on the wall clock, with each library kernel's own
    device duration taken by the library's timing hook (start and stop events of the kernels' own
    dispatches, so nothing is added to the stream).
    Returns (wall seconds per step, {kernel: [us per launch]}, {stage: us per step})."""
    import torch
    timer = dsa.KernelTimer(8 * n)
    with timer:
        t0 = time.perf_counter()
        for i in range(n):
            pipeline.layer_step(wls[i % len(wls)], buf, prefill=prefill, block_sparse=block_sparse,
                                shared_from=shared_from)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / n
    per = {}
    stages = {"scores": 0.0, "select": 0.0, "sparse_mla": 0.0}
    for name, us in timer.results():
        k = short_name(name)
        per.setdefault(k, []).append(us)
        st = stage_of(k)
        stages[st] = stages.get(st, 0.0) + us / n
    return wall, per, stages


# name -> (workload maker, step kind); the headline is the first
CONFIGS = {
    "decode_b16_ctx128k": (lambda w, dev: w.config2("a", device=dev), {}),
    "decode_b16_ctx128k_nope": (lambda w, dev: w.config2("b", device=dev), {}),
    "decode_b64_ctx16k_32k": (lambda w, dev: w.config1(device=dev), {}),
    "prefill_4096_on_61440": (lambda w, dev: w.config3(device=dev), {"prefill": True}),
    "blocksparse_b4_ctx512k": (lambda w, dev: w.config4(device=dev), {"block_sparse": True}),
    "decode_b1_ctx8192_f32": (lambda w, dev: w.config0(device=dev), {}),
    "verify_b16x4_ctx128k": (lambda w, dev: w.verify_blocks(device=dev, batch=16, tokens=4, ctx=131072), {}),
}


def run_config(dsa, pipeline, wls, kind, steps, warmup, shared_from=None, buf=None):
    """Warmup, then `steps` timed layer steps: wall time per step, each kernel's mean and median
    device time, and the per-step device time of each stage."""
    import torch
    if buf is None:
        buf = pipeline.alloc_buffers(wls[0], prefill=kind.get("prefill", False),
                                     block_sparse=kind.get("block_sparse", False))
    for i in range(warmup):
        pipeline.layer_step(wls[i % len(wls)], buf, shared_from=shared_from, **kind)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        pipeline.layer_step(wls[i % len(wls)], buf, shared_from=shared_from, **kind)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    _, per, stages = staged_steps(dsa, pipeline, wls, steps, buf, shared_from=shared_from, **kind)
    out = {"us_per_step": wall * 1e6, "tok_per_s": wls[0].num_q / wall,
           "kernels_us_mean": {k: mean(v) for k, v in per.items()},
           "kernels_us_median": {k: median(v) for k, v in per.items()},
           "stages_us_per_step": stages}
    if shared_from is None and not kind.get("block_sparse", False):
        # the same step with the selection as two calls (scores written, then the top-k over them)
        for i in range(warmup):
            pipeline.layer_step(wls[i % len(wls)], buf, fused=False, **kind)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            pipeline.layer_step(wls[i % len(wls)], buf, fused=False, **kind)
        torch.cuda.synchronize()
        out["us_per_step_separate_selection"] = (time.perf_counter() - t0) / steps * 1e6
    src = buf if shared_from is None else shared_from
    idx_main = [v for k, v in per.items() if k.startswith(("k_index_scores_fp8_grouped", "k_index_scores_fp8_qtile"))]
    if idx_main and shared_from is None:
        out["index_scores_kernel"] = index_rates(wls[0], mean(idx_main[0]))
    mla_main = [v for k, v in per.items() if k.startswith("k_mla") and "combine" not in k]
    if mla_main:
        out["sparse_mla_kernel"] = mla_rates(wls[0], src.length, mean(mla_main[0]))
    out["sparse_mla_stage"] = mla_rates(wls[0], src.length, stages["sparse_mla"])
    return out, buf, per


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time on the headline workload (the other configs get a third of it each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the back-to-back score-kernel loop (profiles of the in-step kernel only)")
    ap.add_argument("--only", choices=sorted(CONFIGS), default=None,
                    help="time one configuration's staged layer steps only and print its figures")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the DSA path here is built and measured on one MI355X; "
              "multi-GPU sharding is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import dsa_sparse_attention_indexer_amd as dsa
    from dsa_sparse_attention_indexer_amd import pipeline

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "dispatches": 5}))
        return

    if args.only is not None:
        make, kind = CONFIGS[args.only]
        log(f"generating {args.only} on the GPU ...")
        wls = cache_copies(make(workloads, dev))
        res, _, _ = run_config(dsa, pipeline, wls, kind, args.steps, args.warmup)
        res["config"] = args.only
        print(json.dumps(res), flush=True)
        return

    log("generating the 128K decode workload (RoPE layer) on the GPU ...")
    wa = workloads.config2("a", device=dev)
    T = wa.num_q
    buf_a = pipeline.alloc_buffers(wa)
    torch.cuda.synchronize()
    was = cache_copies(wa)

    # ---- headline: K timed layer steps ------------------------------------------------------------
    # Every step reads a different copy of the caches, so each reads HBM as inside a multi-layer
    # decode.  The library's timing hook gives every kernel's own duration inside these steps; the
    # score kernel's average there is the roofline's time.
    for i in range(args.warmup):
        pipeline.layer_step(was[i % len(was)], buf_a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pipeline.layer_step(was[i % len(was)], buf_a)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ms_per_step = 1e3 * wall
    # the same steps again with the timing hook on (it lengthens the step on the wall clock, not
    # the kernels): every kernel's own duration
    hooked_wall, per, stages = staged_steps(dsa, pipeline, was, args.steps, buf_a)
    score_name = next((k for k in per if k.startswith("k_index_scores")), None)
    if score_name is None:
        raise RuntimeError(f"no score kernel among the timed kernels: {sorted(per)}")
    t_idx = mean(per[score_name])
    t_mla = stages["sparse_mla"]
    log(f"layer step: {ms_per_step * 1e3:.1f} us wall; in-step kernels " +
        ", ".join(f"{k} {mean(v):.1f}" for k, v in per.items()) + " us")

    keys = int((wa.q_pos.long() + 1).sum())
    idx_bytes = keys * INDEX_BYTES_PER_KEY
    achieved = idx_bytes / (t_idx * 1e-6) / 1e9
    isolated = None
    if not args.no_isolated:
        # The score kernel alone, back to back over the copies, with the histogram but without the
        # candidate emission (dsa_indexer_scores_hist); its histograms pile up in a scratch
        # workspace and are discarded.
        tmp = pipeline.alloc_buffers(wa)
        f = cycling(lambda w: pipeline.index_scores_hist(w, tmp), was)
        for _ in range(2):
            f()
        timer = dsa.KernelTimer(args.steps)
        with timer:
            for _ in range(args.steps):
                f()
        t_iso = mean([us for _, us in timer.results()])
        isolated = {"us": t_iso, "achieved": idx_bytes / (t_iso * 1e-6) / 1e9,
                    "frac": idx_bytes / (t_iso * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "note": "score kernel alone, back to back, histogram but no candidate emission"}
        del tmp
        log(f"score kernel back to back: {t_iso:.1f} us")
    mla_name = next(k for k in per if k.startswith("k_mla") and "combine" not in k)
    headline_mla = {"kernel": mla_rates(wa, buf_a.length, mean(per[mla_name])),
                    "stage": mla_rates(wa, buf_a.length, t_mla)}

    variants = {}
    oracle_rates = {}
    cpu_s = args.cpu_seconds / 3
    if not args.no_variants:
        buf_c = pipeline.alloc_buffers(wa)   # shared-indexer layer: its own outputs, a's selection
        variants["shared_indexer_layer_b16_ctx128k"], _, _ = run_config(
            dsa, pipeline, was, {}, args.steps, args.warmup, shared_from=buf_a, buf=buf_c)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            s0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - s0) / args.steps

        tf = timed(cycling(lambda w: pipeline.layer_step(w, buf_c, fused=False), was))   # two separate calls
        variants["separate_index_topk_layer_b16_ctx128k"] = {"us_per_step": tf * 1e6, "tok_per_s": T / tf}
        del buf_c, was
        for name, (make, kind) in list(CONFIGS.items())[1:]:
            log(f"generating {name} ...")
            wls = cache_copies(make(workloads, dev))
            variants[name], _, _ = run_config(dsa, pipeline, wls, kind, args.steps, args.warmup)
            if not args.no_cpu_baseline:
                r, done, el = oracle_rate(wls[0], cpu_s, block_sparse=kind.get("block_sparse", False))
                oracle_rates[name] = {"tok_per_s": r, "sample": f"{done} of {wls[0].num_q} queries, {el:.1f} s"}
            del wls
            torch.cuda.synchronize()
        log("variants: " + ", ".join(f"{k} {v['us_per_step']:.1f} us" for k, v in variants.items()))
        variants["cache_writers"] = cache_writer_rates(dsa, timed, dev)
        log("cache writers: " + ", ".join(f"{k} {v['us_per_call']:.1f} us" for k, v in variants["cache_writers"].items()))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on host cores ...")
        cpu = cpu_baseline(wa, args.cpu_seconds)
        if oracle_rates:
            cpu["other_configs"] = oracle_rates

    res = {
        "metric": METRIC,
        "value": T / wall,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 caches; f16 (indexer) / bf16 (MLA) MFMA; fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "decode layer step (RoPE layer): indexer + top-2048 + sparse MLA",
                   "batch": T, "context": wa.max_ctx, "index_heads": wa.num_heads, "mla_heads": wa.mla_heads,
                   "topk": wa.topk, "kv_cache": "fp8 e4m3fn + fp32 scales"},
        "roofline": {"bound": "hbm", "kernel": score_name + " (scores + first-digit histogram + candidate emission)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(), "bytes_per_launch": idx_bytes,
                     "launch_us_in_step_mean": t_idx, "launch_us_in_step_median": median(per[score_name]),
                     "launches": len(per[score_name]), "isolated_back_to_back": isolated},
        "kernels_us_mean": {k: mean(v) for k, v in per.items()},
        "kernels_us_median": {k: median(v) for k, v in per.items()},
        "stages_us_per_step": stages,
        "us_per_step_with_timing_hook": hooked_wall * 1e6,
        "keys_scored_per_s": keys / (t_idx * 1e-6),
        "sparse_mla": headline_mla,
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
