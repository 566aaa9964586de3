"""kvq_append_decode_attn_fp4 (append the step's new tokens, then decode, in
one call) through the C ABI: it leaves exactly the cache bytes the separate
append leaves (bit-exact), and its output is plain decode's, bit for bit, on
the one-wave path (append inside the query prologue launch), the many-row
path and the latent path (append as a launch of its own)."""
import math

import numpy as np
import pytest
import torch

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
from kvq_gpu_util import Filled, assert_close, oracle_decode_batch, to_dev_i32

pytestmark = pytest.mark.gpu


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _cache_bytes(c):
    parts = [c.k_codes, c.k_scales] + ([] if c.kv_shared else [c.v_codes, c.v_scales])
    return [t.clone() for t in parts]


@pytest.mark.parametrize("group,n_q,D", [(8, 1, 128), (4, 3, 128), (8, 3, 128), (16, 1, 512)])
def test_append_decode_equals_separate_calls(gpu, group, n_q, D):
    latent = D == 512
    wl = syn.Workload("appdec_g%d_nq%d_d%d" % (group, n_q, D), batch=4, num_kv_heads=1 if latent else 2,
                      num_q_heads=group if latent else 2 * group, head_dim=D, page_size=64 if latent else 16,
                      context=0, n_q=n_q, ctx_range=(200, 900), kv_shared=latent,
                      std=math.sqrt(0.5) if latent else 1.0)
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    want = f.decode(q).cpu().numpy()
    before = _cache_bytes(f.cache)
    # each sequence's last token, and its slot
    slots = to_dev_i32([int(f.seq_slots(b)[-1]) for b in range(wl.batch)])
    k_last = _bf16(np.stack([f.host["k"][b][-1] for b in range(wl.batch)]))
    v_last = None if latent else _bf16(np.stack([f.host["v"][b][-1] for b in range(wl.batch)]))
    # overwrite those slots with other values, then restore them in the fused call
    junk = torch.ones_like(k_last)
    kvq.rotate_quantize_append(f.cache, junk, None if latent else junk, slots)
    assert any(not torch.equal(a, b) for a, b in zip(_cache_bytes(f.cache), before))
    out = kvq.append_decode_attn_fp4(f.cache, k_last, v_last, slots, q, f.block_tables, f.context_lens,
                                     f.max_context).cpu().numpy()
    for a, b in zip(_cache_bytes(f.cache), before):
        assert torch.equal(a, b), "cache bytes differ from the separate append"
    assert np.array_equal(out, want)
    # and the oracle agrees (the cache is the one it was built from)
    ref = oracle_decode_batch(f, syn.bf16_bits(q.cpu()))
    for b in range(wl.batch):
        assert_close(out[b], ref[b], "append+decode g%d n_q%d D%d seq %d" % (group, n_q, D, b))


def test_append_decode_without_tokens_is_decode(gpu):
    wl = syn.WORKLOADS["tiny_b1_l256"]
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    want = f.decode(q).cpu().numpy()
    empty = torch.zeros((0, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out = kvq.append_decode_attn_fp4(f.cache, empty, empty, to_dev_i32(np.zeros(0, np.int32)), q, f.block_tables,
                                     f.context_lens, f.max_context).cpu().numpy()
    assert np.array_equal(out, want)
