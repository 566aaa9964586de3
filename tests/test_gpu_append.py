"""Write path on the GPU against the oracle, bit for bit: codes and UE8M0
scale bytes of every appended (token, head, group), read back through the
documented layout; and the GPU dequantiser against the oracle's."""
import dataclasses

import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from kvq_gpu_util import Filled, gather_codes, to_dev_i32

pytestmark = pytest.mark.gpu


def _check_bitexact(f: Filled, rotate: bool):
    quant = oracle.quantize_fp4 if f.fmt == "fp4" else oracle.quantize_fp8
    for b in range(f.wl.batch):
        slots = f.seq_slots(b)
        for t in syn.tensor_names(f.wl):
            want_c, want_s = quant(f.host[t][b], rotate)
            got_c, got_s = gather_codes(f.cache, t, slots)
            bad_s = np.argwhere(got_s != want_s)
            assert bad_s.size == 0, "seq %d %s: scale mismatch at %s" % (b, t, bad_s[:5].tolist())
            bad_c = np.argwhere(got_c != want_c)
            assert bad_c.size == 0, "seq %d %s: code mismatch at %s" % (b, t, bad_c[:5].tolist())


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_append_bitexact_tiny(gpu, fmt):
    f = Filled(syn.WORKLOADS["tiny_b1_l256"], fmt)
    _check_bitexact(f, f.cache.rotate)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_append_bitexact_b8_l8k(gpu, fmt):
    f = Filled(syn.WORKLOADS["b8_l8k"], fmt)
    _check_bitexact(f, f.cache.rotate)


@pytest.mark.parametrize("fmt,rotate", [("fp4", False), ("fp8", True)])
def test_append_bitexact_other_rotation(gpu, fmt, rotate):
    wl = dataclasses.replace(syn.WORKLOADS["tiny_b1_l256"], name="tiny_rot_%s" % rotate)
    f = Filled(wl, fmt, rotate=rotate)
    _check_bitexact(f, rotate)


@pytest.mark.parametrize("d", [32, 64, 256, 512, 1024])
@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_append_bitexact_head_dims(gpu, d, fmt):
    wl = syn.Workload("dims_%d" % d, batch=2, num_kv_heads=2, num_q_heads=2, head_dim=d,
                      page_size=32, context=70, n_outliers=3)
    f = Filled(wl, fmt)
    _check_bitexact(f, f.cache.rotate)


def _bf16_from_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_append_every_bf16_value_unrotated(gpu, fmt):
    """Every finite bf16 bit pattern goes through the encoder at least once,
    in groups whose maxima span the scale range (zero, subnormal and huge
    groups included), without rotation so the values reach it unchanged."""
    import bit_quantized_kv_rotate_amd as kvq
    b = np.arange(1 << 16, dtype=np.uint32)
    f32 = (b << 16).astype(np.uint32).view(np.float32)
    vals = b[np.isfinite(f32)].astype(np.uint16)
    rng = np.random.default_rng(0)
    rng.shuffle(vals)
    d = 128
    n_vec = (len(vals) + d - 1) // d
    x = np.zeros(n_vec * d, np.uint16)
    x[: len(vals)] = vals
    x = x.reshape(n_vec, 1, d)
    extra = np.zeros((5, 1, d), np.uint16)
    extra[1, 0, 5] = 0x8000                     # -0.0 alone
    extra[2, 0, :32] = 0x0001                   # smallest subnormal
    sub = (0x0040 + np.arange(64)).astype(np.uint16)
    extra[3, 0, :64] = sub                      # subnormal groups that need codes > 0
    extra[3, 0, 64:] = sub | 0x8000
    extra[4, 0, :] = 0x7F7F                     # largest finite bf16 everywhere
    x = np.concatenate([x, extra], 0)
    n = x.shape[0]
    P = 16
    pages = (n + P - 1) // P
    cache = kvq.KVCache(kvq.FMT_FP4_E2M1 if fmt == "fp4" else kvq.FMT_FP8_E4M3, 1, d, P, pages,
                        rotate=False)
    slots = np.random.default_rng(1).permutation(pages * P)[:n].astype(np.int32)
    kx = _bf16_from_bits(x).cuda()
    kvq.rotate_quantize_append(cache, kx, kx, to_dev_i32(slots))
    quant = oracle.quantize_fp4 if fmt == "fp4" else oracle.quantize_fp8
    want_c, want_s = quant(x, False)
    for t in ("k", "v"):
        got_c, got_s = gather_codes(cache, t, slots)
        assert np.array_equal(got_s, want_s)
        bad = np.argwhere(got_c != want_c)
        assert bad.size == 0, bad[:5].tolist()


def test_dequant_matches_oracle(gpu):
    import bit_quantized_kv_rotate_amd as kvq
    for fmt in ("fp4", "fp8"):
        f = Filled(syn.WORKLOADS["tiny_b1_l256"], fmt)
        slots = f.seq_slots(0)
        k, v = kvq.dequant(f.cache, to_dev_i32(slots))
        deq = oracle.dequant_fp4 if fmt == "fp4" else oracle.dequant_fp8
        for t, got in (("k", k), ("v", v)):
            c, s = gather_codes(f.cache, t, slots)
            want = deq(c, s)
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_append_in_one_call_equals_token_by_token(gpu):
    import bit_quantized_kv_rotate_amd as kvq
    wl = syn.WORKLOADS["tiny_b1_l256"]
    f = Filled(wl, "fp4")
    one = kvq.KVCache(kvq.FMT_FP4_E2M1, 1, 128, 16, f.plan.num_pages)
    k = _bf16_from_bits(f.host["k"][0]).cuda()
    v = _bf16_from_bits(f.host["v"][0]).cuda()
    slots = f.seq_slots(0).astype(np.int32)
    for i in range(0, len(slots), 37):
        j = min(i + 37, len(slots))
        kvq.rotate_quantize_append(one, k[i:j], v[i:j], to_dev_i32(slots[i:j]))
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(one, name), getattr(f.cache, name)), name


def test_negative_slots_are_skipped(gpu):
    import bit_quantized_kv_rotate_amd as kvq
    cache = kvq.KVCache(kvq.FMT_FP4_E2M1, 2, 128, 16, 2)
    x = torch.randn(4, 2, 128).to(torch.bfloat16).cuda()
    kvq.rotate_quantize_append(cache, x, x, to_dev_i32([3, -1, 17, -5]))
    torch.cuda.synchronize()
    written = set()
    c, s = gather_codes(cache, "k", np.arange(32))
    for slot in range(32):
        if np.any(s[slot] != 0) or np.any(c[slot] != 0):
            written.add(slot)
    assert written == {3, 17}
