"""Decode attention at the full benchmark sizes, in the launch configuration
the benchmark times (automatic split count, one call), against the oracle on
sampled (sequence, KV head) pairs: every query row of a sampled pair is
compared element by element (max |err| <= 2e-3, relative L2 <= 1e-3).

  b32_l32k       batch 32, 8 KV / 64 Q heads, d128, context 32768, page 16
                 (FP4 cache and the FP8 comparator)
  mtp_mixed_b32  batch 32, contexts 4K-128K log-uniform, 92% of pages shared
                 from 4 prefixes, 3 MTP verify positions (24 rows per KV head);
                 plain and shared-prefix decode
  fork_b32_l32k  batch 32, context 32768 whose first 30720 tokens are one
                 prefix of every sequence, 3 MTP verify positions
                 (shared-prefix decode)
  mla_b16_l128k  batch 16, one latent head of width 512 (K = V), 64 absorbed
                 query heads, context 131072, page 64
  extend         batch 4, 8 KV / 64 Q heads, context 32768 whose last 64
                 tokens are a new chunk (512 rows per KV head)
"""
import numpy as np
import pytest
import torch

import kvq_synth as syn
from kvq_gpu_util import Filled, assert_close, oracle_decode_pairs

pytestmark = pytest.mark.gpu


def _pairs(wl, n, seed):
    """n distinct (sequence, KV head) pairs, covering the first and last
    sequence and every KV head at least once when n allows."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (wl.batch - 1, wl.num_kv_heads - 1)}
    for h in range(min(wl.num_kv_heads, n - 2)):
        pairs.add((int(rng.integers(wl.batch)), h))
    while len(pairs) < n:
        pairs.add((int(rng.integers(wl.batch)), int(rng.integers(wl.num_kv_heads))))
    return sorted(pairs)


def _check(name, fmt, n_pairs, seed, shared=False):
    wl = syn.WORKLOADS[name]
    f = Filled(wl, fmt, gen_device="cuda")
    q = syn.queries(wl, "cuda")
    out = (f.decode_shared(q) if shared else f.decode(q)).cpu().numpy()
    torch.cuda.synchronize()
    qh = syn.bf16_bits(q)
    g = wl.group
    pairs = _pairs(wl, n_pairs, seed)
    want = oracle_decode_pairs(f, qh, pairs)
    worst = (0.0, 0.0)
    for (b, h), ref in want.items():
        got = out[b][:, h * g:(h + 1) * g]
        r = assert_close(got, ref, "%s %s seq %d kv head %d (L=%d)" % (name, fmt, b, h, int(f.plan.context_lens[b])))
        worst = (max(worst[0], r[0]), max(worst[1], r[1]))
    # every output is finite, including the rows not sampled
    assert np.isfinite(out).all()
    print("%s %s%s: %d pairs, worst max_abs %.3g rel_l2 %.3g" % (name, fmt, " shared-prefix" if shared else "",
                                                                len(pairs), worst[0], worst[1]))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_fullsize_b32_l32k_sampled(gpu, fmt):
    _check("b32_l32k", fmt, 24, 1)


def test_fullsize_mtp_mixed_b32_sampled(gpu):
    _check("mtp_mixed_b32", "fp4", 16, 2)


def test_fullsize_mtp_mixed_b32_shared_prefix_sampled(gpu):
    """The same agentic mix through the shared-prefix entry point (each
    prefix group's pages read once for all its members)."""
    _check("mtp_mixed_b32", "fp4", 16, 5, shared=True)


def test_fullsize_fork_b32_l32k_shared_prefix_sampled(gpu):
    """32 sequences forked from one 30K-token prefix, through the
    shared-prefix entry point (768 gathered rows per KV head)."""
    _check("fork_b32_l32k", "fp4", 16, 6, shared=True)


def test_fullsize_mla_b16_l128k_sampled(gpu):
    """Four whole sequences (all 64 rows) of the latent workload."""
    _check("mla_b16_l128k", "fp4", 4, 3)


def test_fullsize_extend_chunk_sampled(gpu):
    """An extend chunk over a 32K cache: the many-row kernel at full length."""
    wl = syn.Workload("extend_b4_l32k_c64", batch=4, num_kv_heads=8, num_q_heads=64, head_dim=128,
                      page_size=16, context=32768, n_q=64)
    syn.WORKLOADS.setdefault(wl.name, wl)
    _check(wl.name, "fp4", 4, 4)
