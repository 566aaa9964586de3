"""kvq_decode_attn_fp4_scratch (the decode that takes no workspace and uses
the library's static device scratch) through the C ABI: two calls in a row,
the second with a smaller input, each bitwise equal to kvq_decode_attn_fp4 on
a caller workspace and within the acceptance bound of the oracle; a shape
that needs more scratch than the array holds is refused."""
import numpy as np
import pytest
import torch

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
from kvq_gpu_util import Filled, assert_close, oracle_decode_batch

pytestmark = pytest.mark.gpu


def _case(wl):
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    return f, q


def _scratch_call(f, q):
    B, n_q, hq, d = q.shape
    out = torch.full((B, n_q, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    kvq.decode_attn_fp4_scratch(f.cache, q, f.block_tables, f.context_lens, f.max_context, out=out)
    return out


def test_scratch_decode_two_calls_second_smaller(gpu):
    big = syn.Workload("scratch_big", batch=6, num_kv_heads=4, num_q_heads=32, head_dim=128,
                       page_size=16, context=0, n_q=1, ctx_range=(300, 5000))
    small = syn.Workload("scratch_small", batch=2, num_kv_heads=1, num_q_heads=4, head_dim=128,
                         page_size=16, context=0, n_q=3, ctx_range=(20, 400))
    for wl in (big, small):
        f, q = _case(wl)
        assert 0 < kvq.decode_workspace_bytes(f.cache, wl.batch, wl.num_q_heads, wl.n_q,
                                              f.max_context) <= kvq.SCRATCH_BYTES
        got = _scratch_call(f, q)
        ref = f.decode(q)                           # same kernels on a caller workspace
        torch.cuda.synchronize()
        assert torch.equal(got, ref), wl.name
        want = oracle_decode_batch(f, syn.bf16_bits(q.cpu()))
        for b in range(wl.batch):
            assert_close(got[b].cpu().numpy(), want[b], "%s seq %d" % (wl.name, b))


def test_scratch_decode_latent_and_many_rows(gpu):
    """The other kernel families (latent width, many rows per KV head) on the
    same static array, each equal to the workspace call."""
    for wl in (syn.Workload("scratch_latent", batch=2, num_kv_heads=1, num_q_heads=16, head_dim=512,
                            page_size=64, context=0, n_q=1, ctx_range=(100, 3000), kv_shared=True,
                            std=0.7, n_outliers=4, outlier_mult=16.0),
               syn.Workload("scratch_many", batch=2, num_kv_heads=2, num_q_heads=32, head_dim=128,
                            page_size=16, context=0, n_q=3, ctx_range=(100, 3000))):
        f, q = _case(wl)
        got = _scratch_call(f, q)
        ref = f.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), wl.name


def test_scratch_decode_refuses_oversize(gpu):
    f, q = _case(syn.WORKLOADS["tiny_b1_l256"])
    big_ctx = 1 << 20
    need = kvq.decode_workspace_bytes(f.cache, 64, 64, 1, big_ctx)
    assert need > kvq.SCRATCH_BYTES
    qb = torch.zeros((64, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, big_ctx // 16), dtype=torch.int32, device="cuda")
    cl = torch.ones(64, dtype=torch.int32, device="cuda")
    out = torch.empty((64, 1, 64, 128), dtype=torch.float32, device="cuda")
    cache = kvq.KVCache(kvq.FMT_FP4_E2M1, 64, 128, 16, 1)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_fp4_scratch(cache, qb, bt, cl, big_ctx, out=out)
    assert e.value.status == -7
