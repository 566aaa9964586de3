"""Selected-position decode over the latent-width FP4 cache (head_dim 512),
through the C ABI, against the oracle's attention over the same selected
positions (max |err| <= 2e-3, relative L2 <= 1e-3 over every output), plus
invariances: selecting every position is plain decode, the split count
changes only rounding."""
import math

import numpy as np
import pytest
import torch

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
import oracle
from kvq_gpu_util import SPLIT_ATOL, SPLIT_RTOL, Filled, assert_close, to_dev_i32

pytestmark = pytest.mark.gpu


def _latent(name, batch, hq, ctx, P=64, shared=True):
    return syn.Workload(name, batch=batch, num_kv_heads=1, num_q_heads=hq, head_dim=512, page_size=P, context=0,
                        kv_shared=shared, ctx_range=ctx, std=math.sqrt(0.5), n_outliers=4, outlier_mult=16.0)


def _sel_tensors(sels):
    width = max(1, max(len(x) for x in sels))
    a = np.zeros((len(sels), width), dtype=np.int32)
    for b, x in enumerate(sels):
        a[b, : len(x)] = x
    return to_dev_i32(a), to_dev_i32(np.array([len(x) for x in sels], dtype=np.int32))


def _oracle(f, qh, b, sel):
    v = None if f.wl.kv_shared else f.host["v"][b]
    return oracle.reference_decode_selected(qh[b], f.host["k"][b], v, sel, "fp4", f.cache.rotate,
                                            1.0 / math.sqrt(f.wl.head_dim))


@pytest.mark.parametrize("hq,P,shared", [(64, 64, True), (16, 64, True), (48, 16, False), (8, 32, True)])
def test_selected_matches_oracle(gpu, hq, P, shared):
    wl = _latent("sel_h%d_p%d_%s" % (hq, P, shared), batch=5, hq=hq, ctx=(300, 5000), P=P, shared=shared)
    f = Filled(wl, "fp4")
    q = syn.queries(wl)
    qh = syn.bf16_bits(q)
    sels = [syn.selected_positions(wl, f.plan, b, n_groups=40) for b in range(wl.batch)]
    sels[1] = sels[1][:17]                       # a list that ends inside a tile
    sels[2] = np.array([int(f.plan.context_lens[2]) - 1], dtype=np.int32)   # one position
    sels[3] = np.concatenate([sels[3][:30], sels[3][:30]])                   # every position twice
    sels[4] = np.zeros(0, dtype=np.int32)       # nothing selected: zeros
    sel, lens = _sel_tensors(sels)
    out = kvq.decode_attn_fp4_selected(f.cache, q.cuda(), f.block_tables, sel, lens).cpu().numpy()
    for b in range(wl.batch):
        if len(sels[b]) == 0:
            assert np.array_equal(out[b], np.zeros_like(out[b])), "empty selection"
            continue
        assert_close(out[b], _oracle(f, qh, b, sels[b]), "selected hq%d P%d seq %d (%d positions)"
                     % (hq, P, b, len(sels[b])))


def test_selected_every_position_is_plain_decode(gpu):
    wl = _latent("sel_all", batch=3, hq=64, ctx=(200, 3000))
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    sels = [np.arange(int(L), dtype=np.int32) for L in f.plan.context_lens]
    sel, lens = _sel_tensors(sels)
    got = kvq.decode_attn_fp4_selected(f.cache, q, f.block_tables, sel, lens).cpu().numpy()
    plain = f.decode(q).cpu().numpy()
    np.testing.assert_allclose(got, plain, rtol=SPLIT_RTOL, atol=SPLIT_ATOL)


def test_selected_split_invariance(gpu):
    wl = _latent("sel_split", batch=2, hq=64, ctx=(3000, 6000))
    f = Filled(wl, "fp4")
    q = syn.queries(wl)
    sels = [syn.selected_positions(wl, f.plan, b, n_groups=300) for b in range(wl.batch)]
    sel, lens = _sel_tensors(sels)
    ref = kvq.decode_attn_fp4_selected(f.cache, q.cuda(), f.block_tables, sel, lens,
                                       flags=kvq.splits_flag(1)).cpu().numpy()
    qh = syn.bf16_bits(q)
    for b in range(wl.batch):
        assert_close(ref[b], _oracle(f, qh, b, sels[b]), "selected one split seq %d" % b)
    for s in (2, 5, 16):
        got = kvq.decode_attn_fp4_selected(f.cache, q.cuda(), f.block_tables, sel, lens,
                                           flags=kvq.splits_flag(s)).cpu().numpy()
        np.testing.assert_allclose(got, ref, rtol=SPLIT_RTOL, atol=SPLIT_ATOL)


def test_fullsize_mla_b16_l128k_selected_sampled(gpu):
    """The latent workload at full size with the index's bound (512 pooled
    groups + 3 recent tokens = 2,051 positions per sequence), in the launch
    configuration the benchmark times; four sequences against the oracle."""
    wl = syn.WORKLOADS["mla_b16_l128k"]
    f = Filled(wl, "fp4", gen_device="cuda")
    q = syn.queries(wl, "cuda")
    sels = [syn.selected_positions(wl, f.plan, b) for b in range(wl.batch)]
    sel, lens = _sel_tensors(sels)
    out = kvq.decode_attn_fp4_selected(f.cache, q, f.block_tables, sel, lens).cpu().numpy()
    torch.cuda.synchronize()
    qh = syn.bf16_bits(q)
    assert np.isfinite(out).all()
    worst = 0.0
    for b in (0, 5, 10, wl.batch - 1):
        # quantisation is per token: quantising only the selected rows gives
        # the same codes as quantising the whole cache
        rows = f.host["k"][b][sels[b]]
        want = oracle.reference_decode_selected(qh[b], rows, None, np.arange(len(sels[b])), "fp4", True,
                                                1.0 / math.sqrt(wl.head_dim))
        worst = max(worst, assert_close(out[b], want, "mla selected seq %d" % b)[0])
    print("mla_b16_l128k selected: worst max_abs %.3g" % worst)
