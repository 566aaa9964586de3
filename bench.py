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
algorithmic bytes per call over its mean duration by one HIP event pair
around the timed steps on the step's stream, against the
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
QK_FLAGS = 0          # decode flags of the FP4 calls (KVQ_QK_CONVERT with --qk-convert)
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
                    help="target time of the single-threaded oracle sample")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the parallel oracle leg (0: every CPU this process may run on)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-mla", action="store_true", help="skip the head_dim 512 latent decode")
    ap.add_argument("--no-mix", action="store_true", help="skip the shared-prefix MTP mix")
    ap.add_argument("--no-extend", action="store_true", help="skip the extend-chunk attention")
    ap.add_argument("--sections", default="all",
                    help="comma list of the sections run after the timed step: fp8 (also the 8K "
                         "comparison), append, mix, fork, extend, latent, cpu; default all")
    ap.add_argument("--qk-convert", action="store_true",
                    help="FP4 decode calls compute scores by converting the K codes to bf16 "
                         "(KVQ_QK_CONVERT), the route the native scaled-MFMA scores are compared with")
    ap.add_argument("--clock-trace", action="store_true",
                    help="sample the shader clock (one side-stream wave) during the warmup and "
                         "timed steps, and record clocks and socket power over 2.5 s of "
                         "sustained FP4 steps and FP8 calls (needs bench_clock.so)")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="wall time of back-to-back calls before each section's timed calls "
                         "(the record's step keeps --warmup)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain fp32 elementwise kernel over 2 x 512 MiB "
                         "(reference for the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 of the decode kernel sources without comments and blank lines,
    and of the compiler flags they are built with (a comment edit keeps the
    measured traffic valid; a code or flag edit does not)."""
    import re
    sys.path.insert(0, ROOT)
    from bit_quantized_kv_rotate_amd import _build
    h = hashlib.sha256()
    flags = [x for x in _build.COMMON if not x.startswith("-I")] + _build.SOURCES["kvq_decode.hip"]
    h.update(repr(flags).encode() + b"\n")
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


def step_bytes(wl, plan, n_new):
    """Algorithmic bytes of one step call over a workload's cache: the FP4
    and FP8 KV bytes every decode call streams (codes plus one scale byte per
    32 channels, K and V, every cached token of every KV head), and the
    step's whole traffic: FP4 KV + the bf16 queries + each (sequence, KV
    head)'s block-table entries + the fp32 outputs + the append of n_new
    tokens (bf16 K and V rows in, FP4 codes and scales out, slot ids)."""
    import numpy as np
    D, H, P = wl.head_dim, wl.num_kv_heads, wl.page_size
    B, HQ, NQ = wl.batch, wl.num_q_heads, wl.n_q
    Ls = plan.context_lens.astype(np.int64)
    n_t = 1 if wl.kv_shared else 2
    kv_fp4 = int(Ls.sum()) * H * (D // 2 + D // 32) * n_t      # 136 B per token and head at d128
    kv_fp8 = int(Ls.sum()) * H * (D + D // 32) * n_t           # 264
    q_bytes = B * NQ * HQ * D * 2
    bt_bytes = int(sum((l + P - 1) // P for l in Ls)) * H * 4
    out_bytes = B * NQ * HQ * D * 4
    app = n_new * H * n_t * (2 * D + D // 2 + D // 32) + n_new * 4
    return kv_fp4, kv_fp8, kv_fp4 + q_bytes + bt_bytes + out_bytes + app


def timed_calls(fn, n, stream):
    """ms per call of n back-to-back calls fn(0) .. fn(n - 1): one HIP event
    pair on `stream` around all of them (an event record between calls costs
    the stream several microseconds of its own)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def abba(stream, fa, fb, n):
    """Paired timing in ABBA order (a, b, b, a), three repeats: returns the
    median of the paired means of a and b (ms per call, each the mean of n
    back-to-back calls under one HIP event pair) and the median of the
    paired ratios b / a."""

    def timed(fn):
        return timed_calls(fn, n, stream)

    ta, tb, ratios = [], [], []
    for _ in range(3):
        a1 = timed(fa)
        b1 = timed(fb)
        b2 = timed(fb)
        a2 = timed(fa)
        ta.append((a1 + a2) / 2)
        tb.append((b1 + b2) / 2)
        ratios.append(tb[-1] / ta[-1])
    return statistics.median(ta), statistics.median(tb), statistics.median(ratios)


SETTLE_S = 0.15


def settle(fn, seconds=None):
    """Back-to-back calls of fn(i) for `seconds` of wall time, before a
    section's timed calls.  The device's power controller cuts the shader
    clock for some tens of milliseconds after the device leaves idle (the
    section set-up idles it), and the compute-bound section kernels then take
    up to a fifth longer per call; the section figures are of the settled
    device.  The record's step keeps the driver's own warmup count."""
    import torch
    seconds = SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


class ClockSampler:
    """Shader clock over time: one wave of bench_clock.so on a side stream (at
    the default priority) records (wall clock, shader clock) pairs every 5 us
    while the work under test runs on the main stream."""

    def __init__(self, dev, stream):
        import ctypes
        import torch
        path = os.path.join(ROOT, "bench_clock.so")
        if not os.path.exists(path):
            raise RuntimeError("--clock-trace needs bench_clock.so (run __graft_entry__.build())")
        self.lib = ctypes.CDLL(path)
        self.lib.bench_clock_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_ulonglong, ctypes.c_void_p]
        khz = ctypes.c_int(0)
        if self.lib.bench_clock_wall_khz(ctypes.byref(khz)) != 0 or khz.value <= 0:
            raise RuntimeError("wall-clock rate unavailable")
        self.wall_khz = khz.value
        self.dev, self.stream = dev, stream
        self.side = torch.cuda.Stream(device=dev)
        # first launch (module load, side queue) before anything is timed
        buf = torch.zeros(2, dtype=torch.int64, device=dev)
        if self.lib.bench_clock_launch(ctypes.c_void_p(buf.data_ptr()), 1, 1,
                                       ctypes.c_void_p(self.side.cuda_stream)) != 0:
            raise RuntimeError("bench_clock_launch failed")
        torch.cuda.synchronize()

    def start(self, ms):
        import ctypes
        import torch
        self.interval = max(1, self.wall_khz // 200)          # 5 us
        self.n = int(ms * 200)
        self.buf = torch.zeros(2 * self.n, dtype=torch.int64, device=self.dev)
        self.base = torch.cuda.Event(enable_timing=True)
        self.base.record(self.stream)
        self.side.wait_stream(self.stream)
        rc = self.lib.bench_clock_launch(ctypes.c_void_p(self.buf.data_ptr()), self.n, self.interval,
                                         ctypes.c_void_p(self.side.cuda_stream))
        if rc != 0:
            raise RuntimeError("bench_clock_launch failed (%d)" % rc)
        time.sleep(0.001)   # let the sampling wave start before the work under test

    def finish(self, window_ms=1.0):
        import torch
        torch.cuda.synchronize()
        s = self.buf.view(self.n, 2).cpu().numpy().astype("float64")
        k = max(1, int(window_ms * 200))
        out = []
        for i in range(0, self.n - k, k):
            dw = s[i + k, 0] - s[i, 0]
            out.append(round((s[i + k, 1] - s[i, 1]) / dw * self.wall_khz / 1000.0) if dw > 0 else None)
        return out


def cold_start_trace(fn, stream, sampler, idle_s, n):
    """After idle_s seconds of idle device, n calls of fn back to back with
    the shader clock sampled beside them: the clock per 1 ms window and each
    call's HIP-event time, on one time base (ms from the sampler's start)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    time.sleep(idle_s)
    sampler.start(max(40.0, 0.5 * n))
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
    stream.synchronize()
    return {
        "idle_s_before": idle_s,
        "sclk_mhz_per_ms": sampler.finish(),
        "call_ms": [round(a.elapsed_time(b), 4) for a, b in ev],
        "call_start_ms": [round(sampler.base.elapsed_time(a), 3) for a, _ in ev],
        "note": "shader clock from one sampling wave on a side stream, per 1 ms window; "
                "call_start_ms on the same time base",
    }


def sustained(fn, stream, seconds, sampler=None):
    """Call fn back to back for about `seconds`; report the mean time per
    call, the mean shader clock (sampling wave) and the socket power and
    clocks the SMU reports (amdsmi, updated about once a second) after the
    first second."""
    import torch
    smi = None
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        smi = (amdsmi, amdsmi.amdsmi_get_processor_handles()[0])
    except Exception:
        smi = None
    if sampler:
        sampler.start(seconds * 1000.0 + 50.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    n, power, gfx = 0, [], []
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn(n)
            n += 1
        stream.synchronize()   # not the device: the sampling wave runs on another stream
        if smi and time.perf_counter() - t0 > 1.0:
            try:
                m = smi[0].amdsmi_get_gpu_metrics_info(smi[1])
                ts = m.get("firmware_timestamp")
                if not power or ts != power[-1][0]:
                    power.append((ts, m.get("current_socket_power")))
                    gfx.append(sum(m["current_gfxclks"]) / len(m["current_gfxclks"]))
            except Exception:
                pass
    e1.record(stream)
    stream.synchronize()
    res = {"calls": n, "ms_per_call": round(e0.elapsed_time(e1) / n, 4)}
    if sampler:
        clk = [x for x in sampler.finish(window_ms=100.0) if x]
        res["sclk_mhz_mean"] = round(statistics.fmean(clk[10:])) if len(clk) > 10 else None
    if power:
        res["socket_power_w"] = [p for _, p in power]
        res["smi_gfxclk_mhz"] = [round(g) for g in gfx]
    if smi:
        try:
            smi[0].amdsmi_shut_down()
        except Exception:
            pass
    return res


def main():
    args = parse()
    global SETTLE_S
    SETTLE_S = args.settle_ms / 1e3
    want = set(s.strip() for s in args.sections.split(",")) if args.sections != "all" else None
    on = lambda s: want is None or s in want
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_kv_rotate_amd as kvq
    import kvq_synth as syn

    torch.cuda.set_device(0)
    global QK_FLAGS
    QK_FLAGS = kvq.QK_CONVERT if args.qk_convert else 0
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
    if not args.no_fp8 and on("fp8"):
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
    ws_bytes = max(kvq.decode_workspace_bytes(c4, B, HQ, NQ, maxL, QK_FLAGS),
                   0 if c8 is None else kvq.decode_workspace_bytes(c8, B, HQ, NQ, maxL))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        # one decode step in one call: append the new token of every sequence,
        # then attend over the whole cache
        kvq.append_decode_attn_fp4(c4s[i % R], step_k, step_v, step_slots, q, bt, cl, maxL, out=out4,
                                   workspace=ws, stream=stream, flags=QK_FLAGS)

    def dec4(i):
        kvq.decode_attn_fp4(c4s[i % R], q, bt, cl, maxL, out=out4, workspace=ws, stream=stream, flags=QK_FLAGS)

    def dec8(i):
        kvq.decode_attn_fp8(c8s[i % R], q, bt, cl, maxL, out=out8, workspace=ws, stream=stream)

    # ---------------- W untimed steps, then exactly K timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # One HIP event pair on the step's stream brackets the K steps: an event
    # record between consecutive steps costs the stream ~7 us per step on
    # MI355X (back-to-back b32_l32k steps: 188-190 us of wall time per step
    # with a pair around each step, 180-182 us without), so per-step events
    # would time themselves as well as the step.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    mean_step = ev[0].elapsed_time(ev[1]) / args.steps

    # ---------------- bytes
    n_new = int(step_slots.numel())
    kv_fp4, kv_fp8, dec_alg = step_bytes(wl, plan, n_new)
    value = kv_fp4 / (ms_per_step * 1e-3) / 1e9
    achieved = dec_alg / (mean_step * 1e-3) / 1e9

    # ---------------- FP4 vs FP8, ABBA (median of three paired-mean ratios)
    fp8 = None
    if c8 is not None:
        for i in range(5):
            dec8(i)
        torch.cuda.synchronize()
        t4m, t8m, ratio = abba(stream, dec4, dec8, max(args.steps // 2, 24))
        fp8 = {
            "decode_ms": round(t8m, 4),
            "kv_gbs": round(kv_fp8 / (t8m * 1e-3) / 1e9, 1),
            "hbm_frac": round(kv_fp8 / (t8m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fp4_decode_ms": round(t4m, 4),
            "fp4_kv_gbs": round(kv_fp4 / (t4m * 1e-3) / 1e9, 1),
            "speedup_fp4_vs_fp8": round(ratio, 3),
            "kv_bytes": kv_fp8,
            "byte_ratio": round(kv_fp8 / kv_fp4, 4),
        }

    # ---------------- bulk append: the whole cache build in one call (every
    # sequence's tokens, 4.29 GB of bf16 K and V in, 1.14 GB of FP4 codes and
    # scales out), re-appended over a replica (rewrites identical codes)
    append_bulk = None
    if on("append"):
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
        n_t = 1 if wl.kv_shared else 2
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

    # ---------------- 8K context: FP4 vs FP8 (ABBA), replicas past the last-level cache
    small = None
    if not args.no_fp8 and on("fp8"):
        small = bench_small(kvq, syn, dev, stream, max(args.steps // 2, 24))

    # ---------------- agentic mix: shared prefixes, MTP verify positions
    mix = fork = None
    if not args.no_mix and on("mix"):
        mix = bench_mix(kvq, syn, dev, stream, max(args.steps // 2, 20), R, fp8=not args.no_fp8 and on("fp8"))
    if not args.no_mix and on("fork"):
        fork = bench_mix(kvq, syn, dev, stream, max(args.steps // 2, 20), R, name="fork_b32_l32k")

    # ---------------- extend chunk (many query rows per KV head, MFMA-bound)
    ext = None
    if not args.no_extend and on("extend"):
        ext = bench_extend(kvq, syn, dev, stream, max(args.steps // 10, 10), R)

    # ---------------- latent-width decode (head_dim 512, MFMA-bound)
    mla = None
    if not args.no_mla and on("latent"):
        mla = bench_latent(kvq, syn, dev, stream, max(args.steps // 2, 20), R)

    # ---------------- shader clock of a cold start, clocks and socket power
    # under sustained calls (diagnostic: after the timed region)
    clock_trace = None
    if args.clock_trace:
        sampler = ClockSampler(dev, stream)
        clock_trace = {"cold_start": cold_start_trace(step, stream, sampler, 1.5, 5 + 100)}
        time.sleep(1.0)
        clock_trace["sustained_fp4_step"] = sustained(step, stream, 2.5, sampler)
        time.sleep(1.0)
        if c8 is not None:
            # without the sampling wave: at 252 registers two FP8 decode waves
            # fill a SIMD's register file, so the sampler would take a slot
            clock_trace["sustained_fp8_decode"] = sustained(dec8, stream, 2.5)

    # ---------------- CPU oracle baseline on a bounded sample
    cpu = None
    if not args.no_cpu_baseline and on("cpu"):
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
        "dtype": ("fp4 e2m1 cache; scaled fp4 x fp6 MFMA scores, bf16 hi/lo MFMA PV, fp32 accumulate"
                  if not args.qk_convert else
                  "fp4 e2m1 cache; codes converted to bf16 for bf16 hi/lo MFMA scores, bf16 hi/lo MFMA PV, "
                  "fp32 accumulate"),
        "data": "synthetic (seeded bf16 N(0,1) + outlier channels; no trace or dataset)",
        "config": {
            "workload": "%s: %s" % (wl.name, wl.description),
            "batch": B, "kv_heads": H, "q_heads": HQ, "head_dim": D, "context": maxL,
            "page_size": P, "query_positions": NQ, "parallelism": "single GPU",
            "cache_replicas": R,
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv_fp4,
        "step_ms_events_mean": round(mean_step, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "kernel": "one FP4 append + decode call (the step): qprep_append_kernel + decode_kernel + merge_kernel",
            "bytes_per_launch": dec_alg,
        },
        "fp8_comparator": fp8,
        "context_8k": small,
        "append_bulk": append_bulk,
        "section_settle_ms": args.settle_ms,
        "agentic_mix": mix,
        "fork_prefix": fork,
        "extend_chunk": ext,
        "latent_512": mla,
        "cpu_baseline": cpu,
    }
    if clock_trace:
        res["clock_trace"] = clock_trace
    print(json.dumps(res), flush=True)


# dense MFMA peaks of MI355X (TFLOP/s)
PEAK_FP4_FP6 = 10100.0
PEAK_BF16 = 2500.0


def mfma_roofline(D, row_tokens, t_ms):
    """MFMA roofline of an attention call over row_tokens (query row, token)
    pairs at head_dim D.  Algorithmic work: 2 D flops for the score and 2 D
    for the value product per pair, each priced at the dense MFMA peak of the
    type it runs in (scores: FP4 cache x FP6 query, 10.1 PF/s; values: bf16,
    2.5 PF/s).  frac = the time that work needs at those peaks over the
    measured time.  The flops the kernels issue are larger (four FP6 query
    terms, P as bf16 hi + lo): their fraction is issued_frac."""
    t = t_ms * 1e-3
    qk, pv = 2.0 * D * row_tokens, 2.0 * D * row_tokens
    t_alg = qk / (PEAK_FP4_FP6 * 1e12) + pv / (PEAK_BF16 * 1e12)
    qk_i, pv_i = qk * 4, pv * 2
    t_iss = qk_i / (PEAK_FP4_FP6 * 1e12) + pv_i / (PEAK_BF16 * 1e12)
    return {
        "bound": "mfma", "unit": "TFLOP/s",
        "achieved": round((qk + pv) / t / 1e12, 1),
        "peak": round((qk + pv) / t_alg / 1e12, 1),
        "frac": round(t_alg / t, 4),
        "traffic": None,
        "issued_tflops": round((qk_i + pv_i) / t / 1e12, 1),
        "issued_frac": round(t_iss / t, 4),
        "note": "algorithmic flops (4 D per row-token: QK^T at the FP4 x FP6 peak 10.1 PF/s, PV at the "
                "bf16 peak 2.5 PF/s); issued: four FP6 query terms and bf16 hi + lo P",
    }


def bench_small(kvq, syn, dev, stream, steps, name="b8_l8k", min_bytes=512e6):
    """FP4 against FP8 decode at 8K context (batch 8, 8 KV / 64 query heads,
    head_dim 128, permuted pages): ABBA timings of one decode call, each
    format rotating over enough cache replicas that they total more than
    512 MB, so that no call finds its cache (71 MB FP4, 138 MB FP8) in the
    256 MB last-level cache left by the calls before it."""
    import numpy as np
    import torch
    wl = syn.WORKLOADS[name]
    plan = syn.page_plan(wl)
    c4, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP4_E2M1, dev)
    c8, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP8_E4M3, dev)
    r4 = int(math.ceil(min_bytes / c4.nbytes)) + 1
    r8 = int(math.ceil(min_bytes / c8.nbytes)) + 1
    c4s, c8s = replicate(kvq, c4, r4), replicate(kvq, c8, r8)
    q = syn.queries(wl, dev)
    bt = torch_from(plan.block_tables, dev)
    cl = torch_from(plan.context_lens, dev)
    maxL = int(plan.context_lens.max())
    B, HQ, NQ, D, H = wl.batch, wl.num_q_heads, wl.n_q, wl.head_dim, wl.num_kv_heads
    out = torch.empty((B, NQ, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kvq.decode_workspace_bytes(c4, B, HQ, NQ, maxL),
                         kvq.decode_workspace_bytes(c8, B, HQ, NQ, maxL)), dtype=torch.uint8, device=dev)

    def d4(i):
        kvq.decode_attn_fp4(c4s[i % r4], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)

    def d8(i):
        kvq.decode_attn_fp8(c8s[i % r8], q, bt, cl, maxL, out=out, workspace=ws, stream=stream)

    for i in range(2 * max(r4, r8)):
        d4(i)
        d8(i)
    settle(lambda i: (d4(i), d8(i)))
    t4, t8, ratio = abba(stream, d4, d8, steps)
    tok = int(plan.context_lens.astype(np.int64).sum()) * H
    kv4, kv8 = tok * (D // 2 + D // 32) * 2, tok * (D + D // 32) * 2
    del c4s, c8s, c4, c8
    return {
        "workload": "%s: %s" % (wl.name, wl.description),
        "replicas": {"fp4": r4, "fp8": r8},
        "fp4_decode_ms": round(t4, 4),
        "fp4_kv_gbs": round(kv4 / (t4 * 1e-3) / 1e9, 1),
        "fp4_hbm_frac": round(kv4 / (t4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "fp8_decode_ms": round(t8, 4),
        "fp8_kv_gbs": round(kv8 / (t8 * 1e-3) / 1e9, 1),
        "fp8_hbm_frac": round(kv8 / (t8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "speedup_fp4_vs_fp8": round(ratio, 3),
        "kv_bytes": {"fp4": kv4, "fp8": kv8},
    }


def bench_mix(kvq, syn, dev, stream, steps, R, name="mtp_mixed_b32", fp8=False):
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
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL, QK_FLAGS), dtype=torch.uint8, device=dev)
    settle(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                         flags=QK_FLAGS))
    t = timed_calls(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                                  flags=QK_FLAGS), steps, stream)

    # the same call through the shared-prefix entry point: each prefix's pages
    # read once for all the sequences that share it
    P = wl.page_size
    shared = [plan.n_shared_pages[b] * P for b in range(B)]
    groups = kvq.PrefixGroups.from_lists(
        [[b for b in range(B) if plan.prefix_of[b] == g and shared[b] > 0] for g in range(wl.n_prefixes)],
        plan.prefix_pages, shared, [int(x) for x in plan.context_lens], device=dev)
    ws2 = torch.empty(kvq.decode_shared_workspace_bytes(c, B, HQ, NQ, groups), dtype=torch.uint8, device=dev)
    out2 = torch.empty_like(out)
    settle(lambda i: kvq.decode_attn_fp4_shared(cs[i % R], q, bt, cl, groups, out=out2, workspace=ws2,
                                                stream=stream, max_context_len=maxL))
    t2 = timed_calls(lambda i: kvq.decode_attn_fp4_shared(cs[i % R], q, bt, cl, groups, out=out2, workspace=ws2,
                                                          stream=stream, max_context_len=maxL), steps, stream)
    max_diff = float((out2 - out).abs().max())

    # the same plain decode over an FP8 cache of the same inputs, ABBA
    fp8_res = None
    if fp8:
        c8, _ = build_cache(kvq, syn, wl, plan, kvq.FMT_FP8_E4M3, dev)
        c8s = replicate(kvq, c8, R)
        ws8 = torch.empty(kvq.decode_workspace_bytes(c8, B, HQ, NQ, maxL), dtype=torch.uint8, device=dev)
        out8 = torch.empty_like(out)

        def d4(i):
            kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream, flags=QK_FLAGS)

        def d8(i):
            kvq.decode_attn_fp8(c8s[i % R], q, bt, cl, maxL, out=out8, workspace=ws8, stream=stream)

        settle(lambda i: (d4(i), d8(i)))
        t4a, t8a, ratio = abba(stream, d4, d8, steps)
        logical8 = int(plan.context_lens.astype(np.int64).sum()) * (D + D // 32) * 2 * wl.num_kv_heads
        fp8_res = {
            "fp4_decode_ms": round(t4a, 4),
            "fp8_decode_ms": round(t8a, 4),
            "speedup_fp4_vs_fp8": round(ratio, 3),
            "fp8_logical_gbs": round(logical8 / (t8a * 1e-3) / 1e9, 1),
            "note": "plain decode, ABBA; the FP8 kernel runs the 24 rows per KV head as three 8-row tiles "
                    "of one wave, the FP4 call the many-row kernel",
        }
        del c8s, c8

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
        "fp8_comparator": fp8_res,
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
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL, QK_FLAGS), dtype=torch.uint8, device=dev)
    settle(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                         flags=QK_FLAGS))
    t = timed_calls(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                                  flags=QK_FLAGS), steps, stream)
    L = wl.context
    visible = NQ * (L - NQ) + NQ * (NQ + 1) // 2          # (position, token) pairs per query head
    row_tokens = float(visible) * HQ * B
    alg_flops = 4.0 * D * row_tokens
    roof = mfma_roofline(D, row_tokens, t)
    del cs, c
    return {
        "workload": "extend_b4_l32k: %s" % wl.description,
        "chunk_tokens": NQ,
        "rows_per_kv_head": wl.group * NQ,
        "decode_ms_events_mean": round(t, 4),
        "algorithmic_tflops": round(alg_flops / (t * 1e-3) / 1e12, 1),
        "tokens_per_s": round(B * NQ / (t * 1e-3), 1),
        "roofline": roof,
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
    ws = torch.empty(kvq.decode_workspace_bytes(c, B, HQ, NQ, maxL, QK_FLAGS), dtype=torch.uint8, device=dev)
    settle(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                         flags=QK_FLAGS))
    t = timed_calls(lambda i: kvq.decode_attn_fp4(cs[i % R], q, bt, cl, maxL, out=out, workspace=ws, stream=stream,
                                                  flags=QK_FLAGS), steps, stream)
    tokens = int(plan.context_lens.astype(np.int64).sum()) * wl.num_kv_heads
    rows = wl.group * NQ
    alg_flops = 4.0 * D * rows * tokens                 # QK^T + PV, single term
    roof = mfma_roofline(D, float(rows) * tokens, t)
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
    settle(lambda i: kvq.decode_attn_fp4_selected(cs[i % R], q, bt, sel_d, sel_lens, out=out_s, workspace=ws_s,
                                                  stream=stream))
    t_sel = timed_calls(lambda i: kvq.decode_attn_fp4_selected(cs[i % R], q, bt, sel_d, sel_lens, out=out_s,
                                                               workspace=ws_s, stream=stream), steps, stream)
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
        "roofline": roof,
    }


def cpu_baseline(wl, plan, target_s, threads):
    """Time the oracle on the host over the decode step of the workload: for
    every (sequence, KV head), dequantise its FP4 K/V cache and run fp64
    decode attention for its query heads.  The parallel leg runs every item
    of the step (256 at b32_l32k: the whole 1.14 GB cache) on `threads` host
    threads (the oracle's C code runs without the GIL); the single-threaded
    leg runs items until about target_s seconds.  The oracle quantises the
    FP4 inputs beforehand on the same threads, untimed.  Reports KV GB/s."""
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
        threads = len(os.sched_getaffinity(0))
    order = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]

    def quant(k, v, h):
        kc, ks = oracle.quantize_fp4(np.ascontiguousarray(k[:, h:h + 1]), True)
        vc, vs = (None, None) if v is None else oracle.quantize_fp4(np.ascontiguousarray(v[:, h:h + 1]), True)
        return kc, ks, vc, vs

    def work(b, h, kc, ks, vc, vs):
        khat = oracle.dequant_fp4(kc, ks)
        vhat = None if vc is None else oracle.dequant_fp4(vc, vs)
        oracle.decode(q[b][:, h * g:(h + 1) * g], khat, vhat, True, sm)
        return kc.shape[0] * (kc.shape[-1] + ks.shape[-1]) * (1 if vc is None else 2)

    # inputs of every item, quantised by the oracle on the host threads (untimed)
    t_prep = time.perf_counter()
    items = {}
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for b in range(wl.batch):
            k = syn.bf16_bits(syn.sequence_kv(wl, plan, "k", b, dev))
            v = None if wl.kv_shared else syn.bf16_bits(syn.sequence_kv(wl, plan, "v", b, dev))
            futs = {h: ex.submit(quant, k, v, h) for h in range(wl.num_kv_heads)}
            for h, fu in futs.items():
                items[(b, h)] = fu.result()
    t_prep = time.perf_counter() - t_prep

    # single thread, a sample
    t1, b1, n1 = 0.0, 0, 0
    for b, h in order:
        t0 = time.perf_counter()
        b1 += work(b, h, *items[(b, h)])
        t1 += time.perf_counter() - t0
        n1 += 1
        if t1 >= target_s:
            break
    # all items of the step on the host threads
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        bpar = sum(ex.map(lambda bh: work(bh[0], bh[1], *items[bh]), order))
    tpar = time.perf_counter() - t0
    return {
        "value": round(bpar / tpar / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "the whole decode step of %s: all %d (sequence, KV head) items (%d tokens each, "
                  "%d B of FP4 KV): dequantise and run fp64 decode attention for %d query heads, on %d "
                  "threads in %.2f s wall (inputs quantised by the oracle beforehand in %.1f s, untimed)"
                  % (wl.name, len(order), int(plan.context_lens[0]), bpar, g, threads, tpar, t_prep),
        "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "items": n1,
                          "seconds": round(t1, 2)},
        "host_cpus": os.cpu_count(),
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
