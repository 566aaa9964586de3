"""Benchmark: decode attention over the rotated FP4 KV cache on one MI355X.

Workload (synthetic, seeded): batch 32, 8 KV / 64 query heads, head_dim 128,
context 32768 tokens per sequence, page size 16 with randomly permuted block
tables; keys/values/queries bf16 N(0,1) with 2 outlier channels x20 per KV
head.  One step = append one new token per sequence to the FP4 cache
(rotate + quantise + store) and one FP4 decode-attention pass over the whole
cache.  The FP8 (E4M3 + per-32 scale) comparator cache is built from the
same bf16 inputs and timed in ABBA order against FP4.

Prints ONE JSON line.  `value` is KV-cache bytes streamed per second by the
whole step (GB/s, inputs resident in HBM); `roofline` is the FP4 decode
kernel's algorithmic bytes per launch over its HIP-event duration against
the 8 TB/s HBM peak; `cpu_baseline` times the CPU oracle on a bounded sample.
"""
import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
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
    dev = torch.device("cuda", 0)

    # ---------------- build both caches from identical bf16 inputs
    t0 = time.time()
    c4 = kvq.KVCache(kvq.FMT_FP4_E2M1, H, D, P, plan.num_pages, kv_shared=wl.kv_shared)
    c8 = None if args.no_fp8 else kvq.KVCache(kvq.FMT_FP8_E4M3, H, D, P, plan.num_pages,
                                              kv_shared=wl.kv_shared)
    n_app = max(wl.append_tokens, 1)
    last_tok = {}
    for p in range(wl.n_prefixes):
        pages = plan.prefix_pages[p]
        kv = {t: syn.full_prefix(wl, plan, t, p, dev) for t in syn.tensor_names(wl)}
        slots = torch.from_numpy(syn.slots_for(pages, len(pages) * P, P)).to(dev)
        for c in (c4, c8):
            if c is not None:
                kvq.rotate_quantize_append(c, kv["k"], kv.get("v"), slots)
    for b in range(B):
        L = int(plan.context_lens[b])
        n_sh = plan.n_shared_pages[b] * P
        kv = {t: syn.private_tokens(wl, t, b, L - n_sh, dev) for t in syn.tensor_names(wl)}
        slots = torch.from_numpy(syn.slots_for(plan.private_pages[b], L - n_sh, P)).to(dev)
        for c in (c4, c8):
            if c is not None:
                kvq.rotate_quantize_append(c, kv["k"], kv.get("v"), slots)
        # the last n_app tokens are re-appended by every step
        last_tok[b] = ({t: x[-n_app:].contiguous() for t, x in kv.items()}, slots[-n_app:])
        del kv
    torch.cuda.synchronize()
    build_s = time.time() - t0
    log("cache build %.1fs: fp4 %.3f GB" % (build_s, c4.nbytes / 1e9))

    step_k = torch.cat([last_tok[b][0]["k"] for b in range(B)], 0)
    step_v = None if wl.kv_shared else torch.cat([last_tok[b][0]["v"] for b in range(B)], 0)
    step_slots = torch.cat([last_tok[b][1] for b in range(B)], 0)
    q = syn.queries(wl, dev)
    bt = torch.from_numpy(plan.block_tables).to(dev)
    cl = torch.from_numpy(plan.context_lens).to(dev)
    maxL = int(plan.context_lens.max())
    out4 = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    out8 = torch.empty_like(out4)
    ws_bytes = kvq.decode_workspace_bytes(c4, B, HQ, NQ, maxL)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()

    def step():
        kvq.rotate_quantize_append(c4, step_k, step_v, step_slots, stream=stream)
        kvq.decode_attn_fp4(c4, q, bt, cl, maxL, out=out4, workspace=ws, stream=stream)

    def dec4():
        kvq.decode_attn_fp4(c4, q, bt, cl, maxL, out=out4, workspace=ws, stream=stream)

    def dec8():
        kvq.decode_attn_fp8(c8, q, bt, cl, maxL, out=out8, workspace=ws, stream=stream)

    # ---------------- timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        kvq.rotate_quantize_append(c4, step_k, step_v, step_slots, stream=stream)
        evd[i][0].record(stream)
        kvq.decode_attn_fp4(c4, q, bt, cl, maxL, out=out4, workspace=ws, stream=stream)
        evd[i][1].record(stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = [a.elapsed_time(b) for a, b in ev]
    dec_ms = [a.elapsed_time(b) for a, b in evd]
    ms_per_step = wall * 1e3 / args.steps

    # ---------------- bytes
    Ls = plan.context_lens.astype(np.int64)
    per_tok_fp4 = (D // 2 + D // 32) * (1 if wl.kv_shared else 2)     # 136 at d128
    per_tok_fp8 = (D + D // 32) * (1 if wl.kv_shared else 2)          # 264 at d128
    kv_fp4 = int(Ls.sum()) * H * per_tok_fp4
    kv_fp8 = int(Ls.sum()) * H * per_tok_fp8
    q_bytes = B * NQ * HQ * D * 2
    bt_bytes = int(sum((l + P - 1) // P for l in Ls)) * H * 4   # each (seq, KV head) reads its table
    out_bytes = B * NQ * HQ * D * 4
    dec_alg = kv_fp4 + q_bytes + bt_bytes + out_bytes
    value = kv_fp4 / (ms_per_step * 1e-3) / 1e9

    med_dec = statistics.median(dec_ms)
    achieved = dec_alg / (med_dec * 1e-3) / 1e9

    # ---------------- FP4 vs FP8, ABBA (median of three paired-mean ratios)
    fp8 = None
    if c8 is not None:
        def timed(fn, n):
            es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n)]
            for a, b in es:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return statistics.median([a.elapsed_time(b) for a, b in es])
        for _ in range(3):
            dec8()
        torch.cuda.synchronize()
        ratios, t4s, t8s = [], [], []
        n = max(args.steps, 10)
        for _ in range(3):
            a1 = timed(dec4, n)
            b1 = timed(dec8, n)
            b2 = timed(dec8, n)
            a2 = timed(dec4, n)
            t4, t8 = (a1 + a2) / 2, (b1 + b2) / 2
            t4s.append(t4)
            t8s.append(t8)
            ratios.append(t8 / t4)
        t8m = statistics.median(t8s)
        fp8 = {
            "decode_ms": round(t8m, 4),
            "kv_gbs": round(kv_fp8 / (t8m * 1e-3) / 1e9, 1),
            "hbm_frac": round(kv_fp8 / (t8m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fp4_decode_ms_abba": round(statistics.median(t4s), 4),
            "speedup_fp4_vs_fp8": round(statistics.median(ratios), 3),
            "kv_bytes": kv_fp8,
        }

    # ---------------- evicted check: a 1 GiB write between decodes
    evict = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ev_ms = []
    for _ in range(5):
        evict.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dec4()
        b.record(stream)
        torch.cuda.synchronize()
        ev_ms.append(a.elapsed_time(b))
    del evict

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- CPU oracle baseline on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, plan, args.cpu_seconds)

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
        "dtype": "fp4 e2m1 cache -> bf16 hi/lo MFMA, f32 accumulate",
        "data": "synthetic (seeded bf16 N(0,1) + outlier channels; no trace or dataset)",
        "config": {
            "workload": "%s: %s" % (wl.name, wl.description),
            "batch": B, "kv_heads": H, "q_heads": HQ, "head_dim": D, "context": maxL,
            "page_size": P, "query_positions": NQ, "parallelism": "single GPU",
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv_fp4,
        "step_ms_events_median": round(statistics.median(step_ms), 4),
        "decode_ms_events_median": round(med_dec, 4),
        "decode_ms_evicted_median": round(statistics.median(ev_ms), 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "decode_kernel<fp4> + split merge (one decode call)",
            "bytes_per_launch": dec_alg,
        },
        "fp8_comparator": fp8,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(wl, plan, target_s):
    """Time the oracle (dequantise the FP4 cache of one (sequence, KV head)
    and run fp64 decode attention for its query heads) on (sequence, KV head)
    pairs until about target_s seconds of CPU work; report KV GB/s."""
    import numpy as np
    import torch
    import kvq_synth as syn
    import oracle

    dev = torch.device("cuda", 0)
    q = syn.bf16_bits(syn.queries(wl, dev))
    g = wl.group
    sm = 1.0 / math.sqrt(wl.head_dim)
    total_s, total_bytes, pairs = 0.0, 0, []
    rng = np.random.default_rng(0)
    order = rng.permutation(wl.batch * wl.num_kv_heads)
    for idx in order:
        b, h = int(idx // wl.num_kv_heads), int(idx % wl.num_kv_heads)
        k = syn.bf16_bits(syn.sequence_kv(wl, plan, "k", b, dev)[:, h:h + 1])
        v = None if wl.kv_shared else syn.bf16_bits(syn.sequence_kv(wl, plan, "v", b, dev)[:, h:h + 1])
        kc, ks = oracle.quantize_fp4(k, True)
        vc, vs = (None, None) if v is None else oracle.quantize_fp4(v, True)
        t0 = time.perf_counter()
        khat = oracle.dequant_fp4(kc, ks)
        vhat = None if v is None else oracle.dequant_fp4(vc, vs)
        oracle.decode(q[b][:, h * g:(h + 1) * g], khat, vhat, True, sm)
        dt = time.perf_counter() - t0
        total_s += dt
        L = k.shape[0]
        total_bytes += L * (kc.shape[-1] + ks.shape[-1]) * (1 if v is None else 2)
        pairs.append((b, h))
        if total_s >= target_s:
            break
    return {
        "value": round(total_bytes / total_s / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d (sequence, KV head) pairs of %s: dequantise their FP4 K/V "
                  "(%d tokens each) and run fp64 decode attention for %d query heads; "
                  "%.1f s single-threaded" % (len(pairs), wl.name, int(plan.context_lens[0]), g, total_s),
        "seconds": round(total_s, 2),
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
