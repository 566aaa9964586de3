"""Benchmark: decode attention over the rotated FP4 KV cache on one MI355X.

Workload (synthetic, seeded): batch 32, 8 KV / 64 query heads, head_dim 128,
context 32768 tokens per sequence, page size 16 with randomly permuted block
tables; keys/values/queries bf16 N(0,1) with 2 outlier channels x20 per KV
head.  One step = append one new token per sequence to the FP4 cache
(rotate + quantise + store) and one FP4 decode-attention pass over the whole
cache, in one call (kvq_append_decode_attn_fp4).  The cache is replicated
(as the layers of a model would be) and the steps rotate over the replicas,
so no step finds its cache in the 256 MB last-level cache.  The FP8 (E4M3 +
per-32 scale) comparator cache is built from the same bf16 inputs and timed
in ABBA order against FP4.

Prints ONE JSON line.  `value` is KV-cache bytes streamed per second by the
whole step (GB/s, inputs resident in HBM); `roofline` is that step call
(query prologue with the append, page-scan and split-merge kernels):
algorithmic bytes per call over its mean HIP-event duration, against the
8 TB/s HBM peak, with the HBM traffic the committed counter summary records
for these kernel sources; `cpu_baseline` times the CPU oracle on a bounded
sample.  Further sections time the bulk append of the whole cache, the
agentic MTP mix and a forked batch (plain and shared-prefix decode), an
extend chunk and the latent workload (plain and selected positions); each
can be left out with its --no-* flag.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "b32_l32k"
# HBM traffic of one append + decode call, measured with rocprofv3 counters and
# scaled by a plain copy kernel; valid only for the kernel source it names.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_fp4_b32_l32k_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_quantized_kv_rotate_amd", "csrc", f)
                  for f in ("kvq_decode.hip", "kvq_decode_common.h", "kvq_device.h", "kvq_append_dev.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the page scan's time settles over the first ~150 back-to-back steps of a
    # run (the device's clocks under sustained HBM load: 175-260 us per call at
    # first, 176-181 us once settled), so the untimed warmup runs past that
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--replicas", type=int, default=3,
                    help="cache copies the steps rotate over (defeats last-level-cache reuse)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle baseline sample")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the parallel oracle sample (0: host cores, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-mla", action="store_true", help="skip the head_dim 512 latent decode")
    ap.add_argument("--no-mix", action="store_true", help="skip the shared-prefix MTP mix")
    ap.add_argument("--no-extend", action="store_true", help="skip the extend-chunk attention")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain fp32 elementwise kernel over 2 x 512 MiB "
                         "(reference for the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 of the decode kernel sources without comments and blank lines
    (a comment edit keeps the measured traffic valid; a code edit does not)."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            for line in fh:
                line = re.sub(r"//.*", "", line).strip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    when there is none or it was taken on another version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def build_cache(kvq, syn, wl, plan, fmt, dev):
    """One cache of format `fmt` holding every sequence's tokens; returns the
    cache and, per sequence, the last tokens (re-appended by every step)."""
    P, H, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    c = kvq.KVCache(fmt, H, D, P, plan.num_pages, kv_shared=wl.kv_shared)
    n_app = max(wl.append_tokens, 1)
    for p in range(wl.n_prefixes):
        pages = plan.prefix_pages[p]
        kv = {t: syn.full_prefix(wl, plan, t, p, dev) for t in syn.tensor_names(wl)}
        slots = torch_from(syn.slots_for(pages, len(pages) * P, P), dev)
        kvq.rotate_quantize_append(c, kv["k"], kv.get("v"), slots)
    last = {}
    for b in range(wl.batch):
        L = int(plan.context_lens[b])
        n_sh = plan.n_shared_pages[b] * P
        kv = {t: syn.private_tokens(wl, t, b, L - n_sh, dev) for t in syn.tensor_names(wl)}
        slots = torch_from(syn.slots_for(plan.private_pages[b], L - n_sh, P), dev)
        kvq.rotate_quantize_append(c, kv["k"], kv.get("v"), slots)
        last[b] = ({t: x[-n_app:].contiguous() for t, x in kv.items()}, slots[-n_app:])
    return c, last


def torch_from(a, dev):
    import torch
    return torch.from_numpy(a).to(dev)


def replicate(kvq, c, n):
    """n caches with identical contents (the first is `c` itself)."""
    reps = [c]
    for _ in range(n - 1):
        r = kvq.KVCache(c.fmt, c.num_kv_heads, c.head_dim, c.page_size, c.num_pages,
                        rotate=c.rotate, kv_shared=c.kv_shared)
        r.k_codes.copy_(c.k_codes)
        r.k_scales.copy_(c.k_scales)
        if not c.kv_shared:
            r.v_codes.copy_(c.v_codes)
            r.v_scales.copy_(c.v_scales)
        reps.append(r)
    return reps


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_kv_rotate_amd as kvq
    import kvq_synth as syn

    torch.cuda.set_device(0)
    wl = syn.WORKLOADS[args.workload]
    plan = syn.page_plan(wl)
    P, H, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    B, HQ, NQ = wl.batch, wl.num_q_heads, wl.n_q
    R = max(1, args.replicas)
    dev = torch.device("cuda", 0)

    # ---------------- caches (FP4 and FP8 from identical bf16 inputs)
    t0 = time.time()
    c4, last = build_cache(kvq, syn, wl, plan, kvq.FMT_FP4_E2M1, dev)
    c8 = None
    if not args.no_fp8:
        c8, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP8_E4M3, dev)
    torch.cuda.synchronize()
    c4s = replicate(kvq, c4, R)
    c8s = None if c8 is None else replicate(kvq, c8, R)
    torch.cuda.synchronize()
    log("caches built in %.1fs: fp4 %.3f GB x %d%s" % (
        time.time() - t0, c4.nbytes / 1e9, R,
        "" if c8 is None else ", fp8 %.3f GB x %d" % (c8.nbytes / 1e9, R)))

    step_k = torch.cat([last[b][0]["k"] for b in range(B)], 0)
    step_v = None if wl.kv_shared else torch.cat([last[b][0]["v"] for b in range(B)], 0)
    step_slots = torch.cat([last[b][1] for b in range(B)], 0)
    q = syn.queries(wl, dev)
    bt = torch_from(plan.block_tables, dev)
    cl = torch_from(plan.context_lens, dev)
    maxL = int(plan.context_lens.max())
    out4 = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    out8 = torch.empty_like(out4)
    ws_bytes = max(kvq.decode_workspace_bytes(c4, B, HQ, NQ, maxL),
                   0 if c8 is None else kvq.decode_workspace_bytes(c8, B, HQ, NQ, maxL))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        # one decode step in one call: append the new token of every sequence,
        # then attend over the whole cache
        kvq.append_decode_attn_fp4(c4s[i % R], step_k, step_v, step_slots, q, bt, cl, maxL, out=out4,
                                   workspace=ws, stream=stream)

    def dec4(i):
        kvq.decode_attn_fp4(c4s[i % R], q, bt, cl, maxL, out=out4, workspace=ws, stream=stream)

    def dec8(i):
        kvq.decode_attn_fp8(c8s[i % R], q, bt, cl, maxL, out=out8, workspace=ws, stream=stream)

    # ---------------- W untimed steps, then exactly K timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        step(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = [e[0].elapsed_time(e[1]) for e in ev]
    ms_per_step = wall * 1e3 / args.steps

    # ---------------- bytes
    Ls = plan.context_lens.astype(np.int64)
    n_t = 1 if wl.kv_shared else 2
    per_tok_fp4 = (D // 2 + D // 32) * n_t     # 136 at d128 (K and V)
    per_tok_fp8 = (D + D // 32) * n_t          # 264 at d128
    kv_fp4 = int(Ls.sum()) * H * per_tok_fp4
    kv_fp8 = int(Ls.sum()) * H * per_tok_fp8
    q_bytes = B * NQ * HQ * D * 2
    bt_bytes = int(sum((l + P - 1) // P for l in Ls)) * H * 4   # each (seq, KV head) reads its table
    out_bytes = B * NQ * HQ * D * 4
    # the step's append: bf16 K and V rows in, FP4 codes + scales out, slots
    n_new = int(step_slots.numel())
    step_app = n_new * H * n_t * (2 * D + D // 2 + D // 32) + n_new * 4
    dec_alg = kv_fp4 + q_bytes + bt_bytes + out_bytes + step_app
    value = kv_fp4 / (ms_per_step * 1e-3) / 1e9
    mean_step = statistics.fmean(step_ms)
    achieved = dec_alg / (mean_step * 1e-3) / 1e9

    # ---------------- FP4 vs FP8, ABBA (median of three paired-mean ratios)
    fp8 = None
    if c8 is not None:
        def timed(fn, n):
            es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n)]
            for i, (a, b) in enumerate(es):
                a.record(stream)
                fn(i)
                b.record(stream)
            torch.cuda.synchronize()
            return statistics.median([a.elapsed_time(b) for a, b in es])
        for i in range(5):
            dec8(i)
        torch.cuda.synchronize()
        ratios, t4s, t8s = [], [], []
        n = max(args.steps // 2, 24)
        for _ in range(3):
            a1 = timed(dec4, n)
            b1 = timed(dec8, n)
            b2 = timed(dec8, n)
            a2 = timed(dec4, n)
            t4, t8 = (a1 + a2) / 2, (b1 + b2) / 2
            t4s.append(t4)
            t8s.append(t8)
            ratios.append(t8 / t4)
        t8m, t4m = statistics.median(t8s), statistics.median(t4s)
        fp8 = {
            "decode_ms": round(t8m, 4),
            "kv_gbs": round(kv_fp8 / (t8m * 1e-3) / 1e9, 1),
            "hbm_frac": round(kv_fp8 / (t8m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fp4_decode_ms": round(t4m, 4),
            "fp4_kv_gbs": round(kv_fp4 / (t4m * 1e-3) / 1e9, 1),
            "speedup_fp4_vs_fp8": round(statistics.median(ratios), 3),
            "kv_bytes": kv_fp8,
            "byte_ratio": round(kv_fp8 / kv_fp4, 4),
        }

    # ---------------- bulk append: the whole cache build in one call (every
    # sequence's tokens, 4.29 GB of bf16 K and V in, 1.14 GB of FP4 codes and
    # scales out), re-appended over a replica (rewrites identical codes)
    parts = {t: [] for t in syn.tensor_names(wl)}
    sl_parts = []
    for b in range(B):
        n_sh = plan.n_shared_pages[b] * P
        Lb = int(plan.context_lens[b]) - n_sh
        for t in parts:
            parts[t].append(syn.private_tokens(wl, t, b, Lb, dev))
        sl_parts.append(torch_from(syn.slots_for(plan.private_pages[b], Lb, P), dev))
    kv0 = {t: torch.cat(x) for t, x in parts.items()}
    sl0 = torch.cat(sl_parts)
    del parts, sl_parts
    L0 = int(sl0.numel())
    torch.cuda.synchronize()
    app_ms = []
    for r in range(12):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        kvq.rotate_quantize_append(c4s[r % R], kv0["k"], kv0.get("v"), sl0, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        app_ms.append(a.elapsed_time(b))
    app_t = statistics.median(app_ms[2:])
    app_bytes = L0 * H * n_t * (2 * D + D // 2 + D // 32) + L0 * 4
    append_bulk = {
        "tokens": L0, "ms": round(app_t, 4),
        "bytes": app_bytes, "gbs": round(app_bytes / (app_t * 1e-3) / 1e9, 1),
        "hbm_frac": round(app_bytes / (app_t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "note": "the whole cache build in one call: bf16 K and V read, FP4 codes + scales written, slot ids read",
    }
    del kv0, sl0

    if args.copy_calibration:
        # torch's elementwise kernel: reads 512 MiB, writes 512 MiB
        src = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- agentic mix: shared prefixes, MTP verify positions
    mix = fork = None
    if not args.no_mix:
        mix = bench_mix(kvq, syn, dev, stream, max(args.steps // 2, 20), R)
        fork = bench_mix(kvq, syn, dev, stream, max(args.steps // 2, 20), R, name="fork_b32_l32k")

    # ---------------- extend chunk (many query rows per KV head, MFMA-bound)
    ext = None
    if not args.no_extend:
        ext = bench_extend(kvq, syn, dev, stream, max(args.steps // 10, 10), R)

    # ---------------- latent-width decode (head_dim 512, MFMA-bound)
    mla = None
    if not args.no_mla:
        mla = bench_latent(kvq, syn, dev, stream, max(args.steps // 2, 20), R)

    # ---------------- CPU oracle baseline on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, plan, args.cpu_seconds, args.cpu_threads)

    res = {
        "metric": "FP4-KV decode attention: KV bytes/s as % of HBM peak; speedup vs FP8-KV kernel",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 e2m1 cache; scaled fp4 x fp6 MFMA scores, bf16 hi/lo MFMA PV, fp32 accumulate",
        "data": "synthetic (seeded bf16 N(0,1) + outlier channels; no trace or dataset)",
        "config": {
            "workload": "%s: %s" % (wl.name, wl.description),
            "batch": B, "kv_heads": H, "q_heads": HQ, "head_dim": D, "context": maxL,
            "page_size": P, "query_positions": NQ, "parallelism": "single GPU",
            "cache_replicas": R,
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv_fp4,
        "step_ms_events_median": round(statistics.median(step_ms), 4),
        "step_ms_events_mean": round(mean_step, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "kernel": "one FP4 append + decode call (the step): qprep_append_kernel + decode_kernel + merge_kernel",
            "bytes_per_launch": dec_alg,
        },
        "fp8_comparator": fp8,
        "append_bulk": append_bulk,
        "agentic_mix": mix,
        "fork_prefix": fork,
        "extend_chunk": ext,
        "latent_512": mla,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


# dense MFMA peaks of MI355X (TFLOP/s)
PEAK_FP4_FP6 = 10100.0
PEAK_BF16 = 2500.0


def bench_mix(kvq, syn, dev, stream, steps, R, name="mtp_mixed_b32"):
    """Decode over a batch with shared prefixes and 3 MTP verify positions:
    the agentic mix (mtp_mixed_b32: contexts 4K-128K, 92% of each sequence's
    pages shared from 4 prefixes, so members share prefixes of different
    lengths) or a fork (fork_b32_l32k: 32 sequences of 32K tokens whose first
    30K tokens are one prefix).  Mean HIP-event time of one FP4 decode call
    over cache replicas, plain and through the shared-prefix entry point.
    Reports logical KV bytes (every sequence's pages, shared ones counted
    per sequence) and unique bytes (each physical page once)."""
    import numpy as np
    import torch
    wl = syn.WORKLOADS[name]
    plan = syn.page_plan(wl)
    c, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP4_E2M1, dev)
    cs = replicate(kvq, c, R)
    q = syn.queries(wl, dev)
    bt = torch_from(plan.block_tables, dev)
    cl = torch_from(plan.context_lens, dev)
    maxL = int(plan.context_lens.max())
    B, HQ, NQ, D = wl.batch, wl.num_q_heads, wl.n_q, wl.head_dim
    out = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL), dtype=torch.uint8, device=dev)
    for i in range(5):
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(es):
        a.record(stream)
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    t = statistics.fmean([a.elapsed_time(b) for a, b in es])

    # the same call through the shared-prefix entry point: each prefix's pages
    # read once for all the sequences that share it
    P = wl.page_size
    shared = [plan.n_shared_pages[b] * P for b in range(B)]
    groups = kvq.PrefixGroups.from_lists(
        [[b for b in range(B) if plan.prefix_of[b] == g and shared[b] > 0] for g in range(wl.n_prefixes)],
        plan.prefix_pages, shared, [int(x) for x in plan.context_lens], device=dev)
    ws2 = torch.empty(kvq.decode_shared_workspace_bytes(c, B, HQ, NQ, groups), dtype=torch.uint8, device=dev)
    out2 = torch.empty_like(out)
    for i in range(5):
        kvq.decode_attn_fp4_shared(cs[i % R], q, bt, cl, groups, out=out2, workspace=ws2, stream=stream)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(es):
        a.record(stream)
        kvq.decode_attn_fp4_shared(cs[i % R], q, bt, cl, groups, out=out2, workspace=ws2, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    t2 = statistics.fmean([a.elapsed_time(b) for a, b in es])
    max_diff = float((out2 - out).abs().max())

    per_tok = (D // 2 + D // 32) * 2 * wl.num_kv_heads
    logical = int(plan.context_lens.astype(np.int64).sum()) * per_tok
    used = set()
    for b in range(B):
        n = (int(plan.context_lens[b]) + P - 1) // P
        used.update(int(x) for x in plan.block_tables[b][:n])
    unique = len(used) * P * per_tok
    del cs, c
    return {
        "workload": "%s: %s" % (wl.name, wl.description),
        "decode_ms_events_mean": round(t, 4),
        "logical_kv_bytes": logical,
        "unique_kv_bytes": unique,
        "logical_gbs": round(logical / (t * 1e-3) / 1e9, 1),
        "unique_gbs": round(unique / (t * 1e-3) / 1e9, 1),
        "shared_prefix": {
            "decode_ms_events_mean": round(t2, 4),
            "speedup_vs_plain": round(t / t2, 3),
            "logical_gbs": round(logical / (t2 * 1e-3) / 1e9, 1),
            "unique_gbs": round(unique / (t2 * 1e-3) / 1e9, 1),
            "max_abs_diff_vs_plain": max_diff,
            "note": "kvq_decode_attn_fp4_shared, one group per prefix (%d)" % wl.n_prefixes,
        },
    }


def bench_extend(kvq, syn, dev, stream, steps, R, chunk=1024):
    """Attention of an extend (prefill) chunk over the FP4 cache: batch 4,
    8 KV / 64 query heads, head_dim 128, context 32768 whose last `chunk`
    tokens are the new chunk (position j sees tokens 0 .. L - chunk + j).
    Mean HIP-event time of one call over cache replicas, against the MFMA
    time of the instructions the kernel issues (four FP4 x FP6 query terms
    for QK^T, bf16 hi + lo for PV)."""
    import torch
    wl = syn.Workload("extend_b4_l32k", batch=4, num_kv_heads=8, num_q_heads=64, head_dim=128,
                      page_size=16, context=32768, n_q=chunk,
                      description="batch 4, 8 KV / 64 Q heads, d128, context 32768 of which the "
                                  "last %d tokens are the chunk" % chunk)
    plan = syn.page_plan(wl)
    c, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP4_E2M1, dev)
    cs = replicate(kvq, c, R)
    q = syn.queries(wl, dev)
    bt = torch_from(plan.block_tables, dev)
    cl = torch_from(plan.context_lens, dev)
    maxL = int(plan.context_lens.max())
    B, HQ, NQ, D = wl.batch, wl.num_q_heads, wl.n_q, wl.head_dim
    out = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL), dtype=torch.uint8, device=dev)
    for i in range(3):
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(es):
        a.record(stream)
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    t = statistics.fmean([a.elapsed_time(b) for a, b in es])
    L = wl.context
    visible = NQ * (L - NQ) + NQ * (NQ + 1) // 2          # (position, token) pairs per query head
    row_tokens = float(visible) * HQ * B
    alg_flops = 4.0 * D * row_tokens
    qk_flops = 2.0 * D * row_tokens * 4
    pv_flops = 2.0 * D * row_tokens * 2
    t_peak = qk_flops / (PEAK_FP4_FP6 * 1e12) + pv_flops / (PEAK_BF16 * 1e12)
    issued = qk_flops + pv_flops
    del cs, c
    return {
        "workload": "extend_b4_l32k: %s" % wl.description,
        "chunk_tokens": NQ,
        "rows_per_kv_head": wl.group * NQ,
        "decode_ms_events_mean": round(t, 4),
        "algorithmic_tflops": round(alg_flops / (t * 1e-3) / 1e12, 1),
        "tokens_per_s": round(B * NQ / (t * 1e-3), 1),
        "roofline": {
            "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(issued / (t * 1e-3) / 1e12, 1),
            "peak": round(issued / t_peak / 1e12, 1),
            "frac": round(t_peak / (t * 1e-3), 4),
            "traffic": None,
            "note": "issued MFMA flops (QK^T 4 FP4xFP6 terms at 10.1 PF/s, PV bf16 hi+lo at 2.5 PF/s); "
                    "peak = their time-weighted dense peak",
        },
    }


def bench_latent(kvq, syn, dev, stream, steps, R, name="mla_b16_l128k"):
    """Decode over the latent cache (batch 16, one K = V head of width 512,
    64 absorbed query heads, context 131072, page 64): mean HIP-event time
    of one decode call over cache replicas, against the MFMA time the
    kernel's instructions need at the dense peaks (QK^T: four FP4 x FP6
    terms; PV: bf16 hi + lo)."""
    import numpy as np
    import torch
    wl = syn.WORKLOADS[name]
    plan = syn.page_plan(wl)
    c, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP4_E2M1, dev)
    cs = replicate(kvq, c, R)
    q = syn.queries(wl, dev)
    bt = torch_from(plan.block_tables, dev)
    cl = torch_from(plan.context_lens, dev)
    maxL = int(plan.context_lens.max())
    B, HQ, NQ, D = wl.batch, wl.num_q_heads, wl.n_q, wl.head_dim
    out = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL), dtype=torch.uint8, device=dev)
    for i in range(10):
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(es):
        a.record(stream)
        kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    t = statistics.fmean([a.elapsed_time(b) for a, b in es])
    tokens = int(plan.context_lens.astype(np.int64).sum()) * wl.num_kv_heads
    rows = wl.group * NQ
    alg_flops = 4.0 * D * rows * tokens                 # QK^T + PV, single term
    qk_flops = 2.0 * D * rows * tokens * 4              # four FP6 query terms
    pv_flops = 2.0 * D * rows * tokens * 2              # P hi + lo
    t_peak = qk_flops / (PEAK_FP4_FP6 * 1e12) + pv_flops / (PEAK_BF16 * 1e12)
    issued = qk_flops + pv_flops
    kv_bytes = tokens * (D // 2 + D // 32)

    # selected-position decode over the same cache: per sequence 512 pooled
    # four-token groups plus the 3 most recent tokens (2,051 positions)
    sels = [syn.selected_positions(wl, plan, b) for b in range(B)]
    max_sel = max(len(x) for x in sels)
    sel = np.zeros((B, max_sel), dtype=np.int32)
    for b, x in enumerate(sels):
        sel[b, : len(x)] = x
    sel_d = torch_from(sel, dev)
    sel_lens = torch_from(np.array([len(x) for x in sels], dtype=np.int32), dev)
    ws_s = torch.empty(kvq.decode_selected_workspace_bytes(c, B, HQ, max_sel), dtype=torch.uint8, device=dev)
    out_s = torch.empty((B, 1, HQ, D), dtype=torch.float32, device=dev)
    for i in range(10):
        kvq.decode_attn_fp4_selected(cs[i % R], q, bt, sel_d, sel_lens, out=out_s, workspace=ws_s, stream=stream)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(es):
        a.record(stream)
        kvq.decode_attn_fp4_selected(cs[i % R], q, bt, sel_d, sel_lens, out=out_s, workspace=ws_s, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    t_sel = statistics.fmean([a.elapsed_time(b) for a, b in es])
    n_sel = int(sum(len(x) for x in sels)) * wl.num_kv_heads
    del cs, c
    return {
        "workload": "%s: %s" % (wl.name, wl.description),
        "selected": {
            "positions_per_sequence": max_sel,
            "decode_ms_events_mean": round(t_sel, 4),
            "speedup_vs_full_scan": round(t / t_sel, 2),
            "selected_kv_gbs": round(n_sel * (D // 2 + D // 32) / (t_sel * 1e-3) / 1e9, 1),
            "note": "kvq_decode_attn_fp4_selected: 512 pooled four-token groups + 3 recent tokens per sequence",
        },
        "decode_ms_events_mean": round(t, 4),
        "kv_gbs": round(kv_bytes / (t * 1e-3) / 1e9, 1),
        "hbm_frac": round(kv_bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_tflops": round(alg_flops / (t * 1e-3) / 1e12, 1),
        "roofline": {
            "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(issued / (t * 1e-3) / 1e12, 1),
            "peak": round(issued / t_peak / 1e12, 1),
            "frac": round(t_peak / (t * 1e-3), 4),
            "traffic": None,
            "note": "issued MFMA flops (QK^T 4 FP4xFP6 terms at 10.1 PF/s, PV bf16 hi+lo at 2.5 PF/s); "
                    "peak = their time-weighted dense peak",
        },
    }


def cpu_baseline(wl, plan, target_s, threads):
    """Time the oracle - dequantise the FP4 cache of one (sequence, KV head)
    and run fp64 decode attention for its query heads - over (sequence, KV
    head) items: first single-threaded until about target_s seconds, then on
    `threads` host threads (the oracle's C code runs without the GIL) for
    about target_s seconds of CPU time.  Reports KV GB/s."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    import kvq_synth as syn
    import oracle

    dev = torch.device("cuda", 0)
    q = syn.bf16_bits(syn.queries(wl, dev))
    g = wl.group
    sm = 1.0 / math.sqrt(wl.head_dim)
    if threads <= 0:
        threads = min(16, os.cpu_count() or 1)
    # sequence-major, so each sequence's K/V is drawn once per pass
    order = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    seq_cache = {}

    def item(b, h):
        """Quantised FP4 K/V of one (sequence, KV head) - not timed."""
        if b not in seq_cache:
            seq_cache.clear()
            k = syn.bf16_bits(syn.sequence_kv(wl, plan, "k", b, dev))
            v = None if wl.kv_shared else syn.bf16_bits(syn.sequence_kv(wl, plan, "v", b, dev))
            seq_cache[b] = (k, v)
        k, v = seq_cache[b]
        kc, ks = oracle.quantize_fp4(np.ascontiguousarray(k[:, h:h + 1]), True)
        vc, vs = (None, None) if v is None else oracle.quantize_fp4(np.ascontiguousarray(v[:, h:h + 1]), True)
        return kc, ks, vc, vs

    def work(b, h, kc, ks, vc, vs):
        khat = oracle.dequant_fp4(kc, ks)
        vhat = None if vc is None else oracle.dequant_fp4(vc, vs)
        oracle.decode(q[b][:, h * g:(h + 1) * g], khat, vhat, True, sm)
        return kc.shape[0] * (kc.shape[-1] + ks.shape[-1]) * (1 if vc is None else 2)

    # single thread
    t1, b1, n1 = 0.0, 0, 0
    for b, h in order:
        args = item(b, h)
        t0 = time.perf_counter()
        b1 += work(b, h, *args)
        t1 += time.perf_counter() - t0
        n1 += 1
        if t1 >= target_s:
            break
    per_item = t1 / n1
    # parallel: enough items for about target_s of CPU time, inputs prepared first
    n_par = max(threads, int(math.ceil(target_s / per_item / threads)) * threads)
    items = [(b, h) + item(b, h) for b, h in (order * (n_par // len(order) + 1))[:n_par]]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        bpar = sum(ex.map(lambda a: work(*a), items))
    tpar = time.perf_counter() - t0
    return {
        "value": round(bpar / tpar / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d (sequence, KV head) items of %s (%d tokens each): dequantise the "
                  "FP4 K/V and run fp64 decode attention for %d query heads, on %d threads "
                  "in %.2f s wall" % (n_par, wl.name, int(plan.context_lens[0]), g, threads, tpar),
        "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "items": n1,
                          "seconds": round(t1, 2)},
        "cpu": cpu_model(),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
