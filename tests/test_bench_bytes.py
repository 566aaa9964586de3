"""The benchmark's algorithmic byte counts against the per-unit figures they
are built from: one 16-token tile of one (sequence, KV head) is 1,024 B of
FP4 codes and 64 B of scale bytes per tensor (2,176 B for K and V; FP8 4,224
B), and a b32_l32k step call adds the bf16 queries, the block-table entries,
the fp32 outputs and the append of one token per sequence."""
import importlib.util
import os

import kvq_synth as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_step_bytes_b32_l32k():
    b = _bench()
    wl = syn.WORKLOADS["b32_l32k"]
    plan = syn.page_plan(wl)
    kv4, kv8, step = b.step_bytes(wl, plan, n_new=32)
    tiles = 32 * 8 * 32768 // 16                  # (sequence, KV head) tiles of 16 tokens
    assert kv4 == tiles * 2176 == 1140850688
    assert kv8 == tiles * 4224
    q = 32 * 64 * 128 * 2
    bt = 32 * 8 * (32768 // 16) * 4                # one int32 page id per page and KV head
    out = 32 * 64 * 128 * 4
    append = 32 * 8 * 2 * (256 + 64 + 4) + 32 * 4  # bf16 row in, codes + scales out, slot id
    assert step == kv4 + q + bt + out + append == 1144686720


def test_step_bytes_latent_reads_the_shared_cache_once():
    b = _bench()
    wl = syn.WORKLOADS["mla_b16_l128k"]
    plan = syn.page_plan(wl)
    kv4, kv8, _ = b.step_bytes(wl, plan, n_new=0)
    tokens = int(plan.context_lens.sum())
    assert kv4 == tokens * (256 + 16)              # K = V: 512 channels, one tensor
    assert kv8 == tokens * (512 + 16)
