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
    import torch
    import workloads
    """Per-call device time and algorithmic bandwidth of the cache writers (and the wall-clock
    time per call through the binding) for one decode step's 16 new tokens and one 4096-token
    prefill chunk.  Keys read: x (2 B x hidden per token) and the
    key projection's weight (2 B x 128 x hidden, once per call); written: 132 B per token.  Latent
    rows: 1152 B read, 612 B written per token.  The destination rows are numbered densely (the
    writers' cost does not depend on where the rows lie)."""
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


def cpu_baseline(wl, seconds):
    """The float64 oracle on whole queries of the same workload, on this host's cores."""
    import workloads
    from oracle import dsa_oracle as O
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads") or 1) for i in info) if info else None
    except Exception:
        pass
    done, elapsed, t = 0, 0.0, 0
    while done == 0 or (elapsed < seconds and done < wl.num_q):
        sub = workloads.slice_query(wl, t)
        t0 = time.perf_counter()
        O.decode_layer(sub, [0])
        elapsed += time.perf_counter() - t0
        done += 1
        t += 1
    return {"value": done / elapsed, "unit": "tok/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {wl.num_q} decode queries at context {wl.max_ctx} (full indexer scan, "
                      f"top-{wl.topk}, sparse MLA), float64 numpy, {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
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

    log("generating the 128K decode workload (RoPE layer) on the GPU ...")
    wa = workloads.config2("a", device=dev)
    T = wa.num_q
    buf_a = pipeline.alloc_buffers(wa)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    was = cache_copies(wa)
    step_a = cycling(lambda w: pipeline.layer_step(w, buf_a), was)

    # ---- headline: K timed layer steps --------------------------------------------------------
    for _ in range(args.warmup):
        step_a()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_a()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    log(f"layer step: {ms_per_step * 1e3:.1f} us")

    # ---- per-stage durations: K back-to-back calls between two events on the launch stream -------
    def per_call_us(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    # Every stage is timed over calls that cycle through the cache copies, so each call reads HBM
    # (as inside a real decode step), not lines left in the last-level cache by the previous call.
    # The score kernel (with the histogram, as in the step) back to back on scratch buffers (their
    # histogram piles up over the calls and is discarded), then score kernel + top-k pairs: the
    # top-k's share is the difference.
    tmp = pipeline.alloc_buffers(wa)
    t_idx = per_call_us(cycling(lambda w: pipeline.index_scores_hist(w, tmp), was))
    del tmp

    def pair(w):
        pipeline.index_scores_hist(w, buf_a)
        pipeline.select_hist(w, buf_a)

    t_topk = per_call_us(cycling(pair, was)) - t_idx
    t_mla = per_call_us(cycling(lambda w: pipeline.attend(w, buf_a), was))
    keys = int((wa.q_pos.long() + 1).sum())
    idx_bytes = keys * INDEX_BYTES_PER_KEY
    achieved = idx_bytes / (t_idx * 1e-6) / 1e9
    sel = int(buf_a.length.long().sum())
    mla_flops = sel * wa.mla_heads * MLA_FLOP_PER_KEY_HEAD
    mla_tflops = mla_flops / (t_mla * 1e-6) / 1e12
    mla_gbs = sel * LATENT_BYTES_PER_KEY / (t_mla * 1e-6) / 1e9
    log(f"index {t_idx:.1f} us, top-k {t_topk:.1f} us, MLA {t_mla:.1f} us")

    variants = {}
    if not args.no_variants:
        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            s0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - s0) / args.steps

        buf_c = pipeline.alloc_buffers(wa)   # shared-indexer layer: its own outputs, a's selection
        tc = timed(cycling(lambda w: pipeline.layer_step(w, buf_c, shared_from=buf_a), was))
        variants["shared_indexer_layer_b16_ctx128k"] = {"us_per_step": tc * 1e6, "tok_per_s": T / tc}
        tf = timed(cycling(lambda w: pipeline.layer_step(w, buf_c, fused=False), was))   # two separate calls
        variants["separate_index_topk_layer_b16_ctx128k"] = {"us_per_step": tf * 1e6, "tok_per_s": T / tf}
        del buf_c
        del was
        log("generating the NoPE-layer workload ...")
        wb = cache_copies(workloads.config2("b", device=dev))
        bb = pipeline.alloc_buffers(wb[0])
        tb = timed(cycling(lambda w: pipeline.layer_step(w, bb), wb))
        variants["nope_layer_b16_ctx128k"] = {"us_per_step": tb * 1e6, "tok_per_s": wb[0].num_q / tb}
        del wb, bb
        log("generating the 4096-on-61440 chunked prefill ...")
        w3 = cache_copies(workloads.config3(device=dev))
        b3 = pipeline.alloc_buffers(w3[0], prefill=True)
        t3 = timed(cycling(lambda w: pipeline.layer_step(w, b3, prefill=True), w3))
        variants["chunked_prefill_4096_on_61440"] = {"us_per_step": t3 * 1e6, "tok_per_s": w3[0].num_q / t3}
        del w3, b3
        log("generating the 512K block-sparse decode ...")
        w4 = cache_copies(workloads.config4(device=dev))
        b4 = pipeline.alloc_buffers(w4[0], block_sparse=True)
        t4 = timed(cycling(lambda w: pipeline.layer_step(w, b4, block_sparse=True), w4))
        variants["block_sparse_b4_ctx512k"] = {"us_per_step": t4 * 1e6, "tok_per_s": w4[0].num_q / t4}
        del w4, b4
        log("generating the batch-64 16K-32K decode ...")
        w1 = cache_copies(workloads.config1(device=dev))
        b1 = pipeline.alloc_buffers(w1[0])
        t1 = timed(cycling(lambda w: pipeline.layer_step(w, b1), w1))
        variants["decode_b64_ctx16k_32k"] = {"us_per_step": t1 * 1e6, "tok_per_s": w1[0].num_q / t1}
        del w1, b1
        log("variants: " + ", ".join(f"{k} {v['us_per_step']:.1f} us" for k, v in variants.items()))
        variants["cache_writers"] = cache_writer_rates(dsa, timed, dev)
        log("cache writers: " + ", ".join(f"{k} {v['us_per_call']:.1f} us" for k, v in variants["cache_writers"].items()))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on host cores ...")
        cpu = cpu_baseline(wa, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": T / (elapsed / args.steps),
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
        "roofline": {"bound": "hbm", "kernel": "index scores + first-digit histogram (fp8 keys)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(), "bytes_per_launch": idx_bytes},
        "stages_us": {"index_scores_hist": t_idx, "topk_from_hist": t_topk, "sparse_mla": t_mla},
        "keys_scored_per_s": keys / (t_idx * 1e-6),
        "sparse_mla": {"tflops": mla_tflops, "frac_bf16_peak": mla_tflops / BF16_PEAK_TFLOPS,
                       "gather_gbs": mla_gbs, "frac_hbm_peak": mla_gbs / HBM_PEAK_GBS},
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
