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
                 tokens are a new chunk (512 rows per KV head); and the
                 benchmark's 1024-token chunk on sampled positions

and, for b32_l32k, the bulk append of the whole cache in one call (bit-exact
on sampled tokens) and the one-call step (append + decode) the benchmark
times.
"""
import numpy as np
import pytest
import torch

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
import oracle
from kvq_gpu_util import Filled, assert_close, gather_codes, oracle_decode_pairs

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


def test_fullsize_extend_1024_chunk_sampled_rows(gpu):
    """The benchmark's extend chunk exactly (batch 4, 8 KV / 64 query heads,
    context 32768 whose last 1024 tokens are the chunk: 8192 rows per KV
    head, one call): sampled chunk positions of two sequences, all 64 heads
    each, against the oracle's attention over the tokens the position sees
    (its own and every earlier one)."""
    import math

    wl = syn.Workload("extend_b4_l32k", batch=4, num_kv_heads=8, num_q_heads=64, head_dim=128,
                      page_size=16, context=32768, n_q=1024)
    f = Filled(wl, "fp4", gen_device="cuda")
    q = syn.queries(wl, "cuda")
    out = f.decode(q).cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(out).all()
    qh = syn.bf16_bits(q)
    worst = 0.0
    for b in (0, wl.batch - 1):
        L = int(f.plan.context_lens[b])
        kc, ks = oracle.quantize_fp4(f.host["k"][b], True)
        vc, vs = oracle.quantize_fp4(f.host["v"][b], True)
        khat, vhat = oracle.dequant_fp4(kc, ks), oracle.dequant_fp4(vc, vs)
        for j in (0, 1, 511, 766, 1022, 1023):
            seen = L - wl.n_q + j + 1
            want = oracle.decode(qh[b][j:j + 1], khat[:seen], vhat[:seen], True, 1.0 / math.sqrt(wl.head_dim))
            worst = max(worst, assert_close(out[b][j], want[0], "extend chunk seq %d position %d" % (b, j))[0])
    print("extend_b4_l32k (1024-token chunk): 12 sampled positions x 64 heads, worst max_abs %.3g" % worst)


def test_fullsize_b32_l32k_bulk_append_sampled(gpu):
    """The whole b32_l32k cache (32 sequences x 32768 tokens x 8 KV heads)
    built by one append call, the launch the benchmark times as its bulk
    append: codes and scale bytes bit-exact against the oracle on the first
    and last token of every sequence and 2,000 random tokens, every head and
    both tensors."""
    wl = syn.WORKLOADS["b32_l32k"]
    plan = syn.page_plan(wl)
    P = wl.page_size
    cache = kvq.KVCache(kvq.FMT_FP4_E2M1, wl.num_kv_heads, wl.head_dim, P, plan.num_pages)
    ks, vs, sls, starts = [], [], [], []
    n = 0
    for b in range(wl.batch):
        L = int(plan.context_lens[b])
        ks.append(syn.private_tokens(wl, "k", b, L, "cuda"))
        vs.append(syn.private_tokens(wl, "v", b, L, "cuda"))
        sls.append(syn.slots_for(plan.private_pages[b], L, P))
        starts.append(n)
        n += L
    k, v = torch.cat(ks), torch.cat(vs)
    slots = np.concatenate(sls)
    del ks, vs
    kvq.rotate_quantize_append(cache, k, v, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    idx = set(rng.integers(n, size=2000).tolist())
    for b in range(wl.batch):
        idx.update((starts[b], starts[b] + int(plan.context_lens[b]) - 1))
    idx = np.array(sorted(idx), dtype=np.int64)
    sel = torch.from_numpy(idx).cuda()
    for t, x in (("k", k), ("v", v)):
        want_c, want_s = oracle.quantize_fp4(syn.bf16_bits(x[sel]), True)
        got_c, got_s = gather_codes(cache, t, slots[idx])
        bad_s = np.argwhere(got_s != want_s)
        assert bad_s.size == 0, "%s: scale mismatch at %s" % (t, bad_s[:5].tolist())
        bad_c = np.argwhere(got_c != want_c)
        assert bad_c.size == 0, "%s: code mismatch at %s" % (t, bad_c[:5].tolist())
    print("b32_l32k bulk append: %d tokens in one call, %d sampled tokens bit-exact" % (n, len(idx)))


def test_fullsize_b32_l32k_step_call(gpu):
    """The benchmark's step at full size: one kvq_append_decode_attn_fp4 call
    that re-appends the last token of every sequence, then attends.  The
    tokens re-appended are the stored ones, so the cache keeps every byte,
    and the output is bitwise that of the decode-only call (which the
    sampled test above checks against the oracle)."""
    wl = syn.WORKLOADS["b32_l32k"]
    f = Filled(wl, "fp4", gen_device="cuda", keep_host=False)
    q = syn.queries(wl, "cuda")
    plain = f.decode(q)
    k1, v1, s1 = [], [], []
    for b in range(wl.batch):
        L = int(f.plan.context_lens[b])
        k1.append(syn.private_tokens(wl, "k", b, L, "cuda")[-1:])
        v1.append(syn.private_tokens(wl, "v", b, L, "cuda")[-1:])
        s1.append(syn.slots_for(f.plan.private_pages[b], L, wl.page_size)[-1:])
    before = [x.clone() for x in (f.cache.k_codes, f.cache.k_scales, f.cache.v_codes, f.cache.v_scales)]
    out = kvq.append_decode_attn_fp4(f.cache, torch.cat(k1), torch.cat(v1), torch.from_numpy(np.concatenate(s1)).cuda(),
                                     q, f.block_tables, f.context_lens, f.max_context)
    torch.cuda.synchronize()
    after = (f.cache.k_codes, f.cache.k_scales, f.cache.v_codes, f.cache.v_scales)
    assert all(torch.equal(x, y) for x, y in zip(before, after)), "the re-append changed the cache"
    assert torch.equal(out, plain), "step call differs from the decode-only call"
