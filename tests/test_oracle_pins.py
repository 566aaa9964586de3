"""Pins of the CPU oracle against facts that do not come from the oracle:
closed forms, library routines (scipy's Sylvester Hadamard matrix, torch's
fp8 casts), hand-written tables from the format definitions, the byte
arithmetic stated by the ROCm blog "UltraQuant on AMD Instinct", and brute
force on tiny inputs.  CPU only."""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
from conftest import read_golden

DIMS = [32, 64, 128, 256, 512, 1024]


def f32(x):
    return np.float32(x)


def bits(x):
    return int(np.float32(x).view(np.uint32))


# ------------------------------------------------------------ rotation

@pytest.mark.parametrize("d", DIMS)
def test_fwht_unit_vectors_exact_sylvester_signs(d):
    """H e_k has entries exactly +-fp32(1/sqrt d), with scipy's Sylvester
    sign pattern (which is (-1)^popcount(i & k))."""
    H = scipy.linalg.hadamard(d)
    consts = {int(r[0]): int(r[1], 16) for r in read_golden("fwht_constants.txt")}
    c = np.array([consts[d]], dtype=np.uint32).view(np.float32)[0]
    for k in [0, 1, d // 2 - 1, d // 2, d - 1, 5 % d]:
        e = np.zeros(d, np.float32)
        e[k] = 1.0
        y = oracle.fwht_f32(e)
        expect = (H[:, k] * c).astype(np.float32)
        assert np.array_equal(y.view(np.uint32), expect.view(np.uint32)), k
        pop = np.array([bin(i & k).count("1") % 2 for i in range(d)])
        assert np.array_equal(np.sign(y), np.where(pop == 1, -1.0, 1.0))


@pytest.mark.parametrize("d", DIMS)
def test_fwht_f64_equals_sylvester_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((4, d))
    H = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    np.testing.assert_allclose(oracle.fwht_f64(x), x @ H.T, rtol=0, atol=1e-12 * math.sqrt(d))


@pytest.mark.parametrize("d", DIMS)
def test_fwht_f32_close_to_exact_and_involution(d):
    rng = np.random.default_rng(100 + d)
    x = rng.standard_normal((8, d)).astype(np.float32)
    H = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    y = oracle.fwht_f32(x)
    exact = x.astype(np.float64) @ H.T
    ulp = np.abs(exact).max() * 2.0 ** -23
    assert np.abs(y - exact).max() <= (math.log2(d) + 2) * ulp
    # H is symmetric and orthogonal: applying it twice gives x back
    z = oracle.fwht_f32(y)
    assert np.abs(z - x).max() <= 2 * (math.log2(d) + 2) * np.abs(x).max() * 2.0 ** -23
    # Parseval
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)


def test_fwht_symmetric():
    d = 64
    cols = np.stack([oracle.fwht_f64(np.eye(d)[k]) for k in range(d)], 1)
    assert np.array_equal(cols, cols.T)


# ------------------------------------------------------------ scale byte

@pytest.mark.parametrize("emax,off", [(2, 125), (8, 119)])
def test_scale_byte_closed_form(emax, off):
    """amax in [2^e, 2^(e+1)) gives byte max(e + 127 - emax, 0) for every
    exponent from the smallest subnormal up to the largest finite fp32."""
    assert oracle.scale_byte(0.0, emax) == 0
    for e in range(-149, 128):
        lo = np.float32(2.0 ** e)
        hi = np.nextafter(np.float32(2.0 ** (e + 1)) if e < 127 else np.float32(np.inf),
                          np.float32(0), dtype=np.float32)
        want = max(e + off, 0)
        assert oracle.scale_byte(float(lo), emax) == want, e
        assert oracle.scale_byte(float(hi), emax) == want, e


def test_scale_value_matches_torch_e8m0():
    b = torch.arange(0, 255, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([oracle.scale_value(int(i)) for i in range(255)])
    assert np.array_equal(ref, ours)


# ------------------------------------------------------------ E2M1 codes

def test_e2m1_decode_table():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert abs(v) == grid[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_e2m1_rounding_table():
    for r, want in read_golden("e2m1_rounding.txt"):
        r, want = float(r), float(want)
        for sgn in (1.0, -1.0):
            code = oracle.e2m1_encode(sgn * r, 0)
            assert abs(oracle.e2m1_value(code)) == want, (r, code)
            assert (code >> 3) == (1 if sgn < 0 else 0)


def _generic_rne_e2m1(r):
    """Round-to-nearest-even onto a float format with 2 exponent bits (bias 1)
    and 1 mantissa bit, saturating at 6 -- written as a generic float
    rounding (quantum 2^(e-1) above 1, 0.5 below) with numpy's
    half-to-even rounding, independent of the oracle's grid search."""
    a = np.abs(r).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 1.0)))
    q = np.where(a < 1.0, 0.5, 2.0 ** (e - 1))
    v = np.round(a / q) * q
    return np.minimum(v, 6.0)


def test_e2m1_matches_generic_rne_on_all_bf16():
    """Every finite bf16 value with |x| < 8 at unit scale."""
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (b << 16).astype(np.uint32).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 8)]
    got = np.array([abs(oracle.e2m1_value(oracle.e2m1_encode(float(v), 0))) for v in x])
    assert np.array_equal(got, _generic_rne_e2m1(x))


def test_e2m1_matches_generic_rne_random_fp32_and_scales():
    rng = np.random.default_rng(7)
    x = rng.uniform(-8, 8, 20000).astype(np.float32)
    for e_s in (-127, -40, -3, 0, 5, 60, 125):
        y = (x.astype(np.float64) * 2.0 ** e_s).astype(np.float32)
        keep = np.isfinite(y)
        r = y[keep].astype(np.float64) * 2.0 ** -e_s
        got = np.array([abs(oracle.e2m1_value(oracle.e2m1_encode(float(v), e_s))) for v in y[keep]])
        assert np.array_equal(got, _generic_rne_e2m1(r)), e_s


def test_e2m1_grid_round_trips_at_every_scale():
    for e_s in range(-127, 126):
        for c in range(16):
            y = np.float32(oracle.e2m1_value(c) * 2.0 ** e_s)
            assert oracle.e2m1_encode(float(y), e_s) == c, (e_s, c)


def test_e2m1_sign_of_zero_and_saturation():
    assert oracle.e2m1_encode(0.0, 0) == 0
    assert oracle.e2m1_encode(-0.0, 0) == 8
    assert oracle.e2m1_encode(-0.01, 0) == 8
    assert oracle.e2m1_encode(7.99, 0) == 7
    assert oracle.e2m1_encode(-7.99, 0) == 15


# ------------------------------------------------------------ E4M3 codes

def test_e4m3_decode_matches_torch():
    c = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    ref = c.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_value(i) for i in range(256)])
    finite = np.isfinite(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[finite], ours[finite])


def test_e4m3_encode_matches_torch_cast():
    """torch's cast is round-to-nearest-even without saturation, so compare
    where it is finite (|x| <= 464), on every finite bf16 value plus random
    fp32 and all midpoints between neighbouring codes."""
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    xs = [(b << 16).astype(np.uint32).view(np.float32)]
    xs.append(np.random.default_rng(3).uniform(-464, 464, 20000).astype(np.float32))
    vals = np.array([oracle.e4m3_value(i) for i in range(127)])
    xs.append(((vals[1:] + vals[:-1]) / 2).astype(np.float32))
    x = np.concatenate(xs)
    x = x[np.isfinite(x) & (np.abs(x) <= 464)]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(v), 0) for v in x], dtype=np.uint8)
    # torch keeps -0.0 as 0x80 like the oracle
    assert np.array_equal(ref, ours)


def test_e4m3_saturates_and_round_trips():
    assert oracle.e4m3_encode(500.0, 0) == 0x7E
    assert oracle.e4m3_encode(-511.0, 0) == 0xFE
    for e_s in (-127, -20, 0, 20, 119):
        for c in list(range(0, 127)) + list(range(128, 255)):
            y = np.float32(oracle.e4m3_value(c) * 2.0 ** e_s)
            assert oracle.e4m3_encode(float(y), e_s) == c, (e_s, c)


# ------------------------------------------------------------ whole vectors

def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_byte_budget_matches_page():
    g = {r[0]: float(r[1]) for r in read_golden("byte_budget.txt")}
    d = 128
    codes, scales = oracle.quantize_fp4(_bf16(np.zeros(d)), rotate=True)
    per_group = (codes.nbytes + scales.nbytes) / (d // 32)
    assert per_group == g["fp4_group_bytes"] == 17
    assert g["values_per_group"] == 32
    assert round(100 * (1 - per_group / g["fp8_group_bytes"])) == g["capacity_reduction_percent"]
    assert round(g["fp8_group_bytes"] / per_group, 2) == g["values_per_byte_ratio"]


def test_nibble_order_and_scale_of_a_known_vector():
    x = np.zeros(64, np.float32)
    x[0], x[1], x[2], x[3] = 0.5, 6.0, -1.0, 3.0       # group 0: amax 6 -> e_s 0
    x[32], x[33] = 40.0, -0.1                          # group 1: amax 40 -> e_s 3
    codes, scales = oracle.quantize_fp4(_bf16(x), rotate=False)
    assert list(scales) == [127, 130]
    assert codes[0] == 0x71 and codes[1] == 0x5A
    # 40 / 8 = 5 -> tie between 4 and 6 -> 4 (code 6); -0.1/8 -> -0 (code 8)
    assert codes[16] == 0x86


@pytest.mark.parametrize("d", [32, 128, 512])
def test_quantize_error_bound_and_scale_rule(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((64, d)).astype(np.float32)
    x[:, 3] *= 20
    xb = _bf16(x)
    codes, scales = oracle.quantize_fp4(xb, rotate=True)
    y = oracle.fwht_f32(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy())
    yhat = oracle.dequant_fp4(codes, scales)
    for g in range(d // 32):
        seg = slice(32 * g, 32 * g + 32)
        amax = np.abs(y[:, seg]).max(axis=1)
        s = 2.0 ** (scales[:, g].astype(np.float64) - 127)
        # largest element lands in [4, 8) of the group scale
        assert np.all((amax / s >= 4) & (amax / s < 8))
        # error: half the grid spacing (<= 1 scale unit) or the saturation gap (< 2)
        err = np.abs(y[:, seg] - yhat[:, seg]).max(axis=1)
        assert np.all(err <= 2 * s)
        small = np.abs(y[:, seg]) <= 6 * s[:, None]
        assert np.all(np.abs(y[:, seg] - yhat[:, seg])[small] <= (s[:, None] * np.ones_like(y[:, seg]))[small])


def test_fp8_vector_error_bound():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 128)).astype(np.float32) * 3
    codes, scales = oracle.quantize_fp8(_bf16(x), rotate=False)
    xf = torch.from_numpy(_bf16(x).view(np.int16)).view(torch.bfloat16).float().numpy()
    xhat = oracle.dequant_fp8(codes, scales)
    s = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    r = np.abs(xf) / s                        # value in units of the group scale
    err = np.abs(xhat - xf)
    # the group maximum lands in [256, 512); E4M3 normals (>= 2^-6) keep 4
    # significant bits (relative error <= 2^-4) up to 448 ...
    normal = (r >= 2.0 ** -6) & (r <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf)[normal])
    # ... and beyond 448 saturate to 448
    sat = r > 448
    assert np.all(xhat[sat] == np.sign(xf[sat]) * 448 * s[sat])
    assert np.all(r < 512)


# ------------------------------------------------------------ attention

def _np_attention(q, k, v, sm_scale, n_q):
    """Independent fp64 restatement using numpy matmul and scipy's softmax."""
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    out = np.zeros((n, hq, d))
    for j in range(n):
        last = L - n_q + j
        for h in range(hq):
            kv = h // g
            s = sm_scale * (k[: last + 1, kv, :].astype(np.float64) @ q[j, h])
            p = scipy.special.softmax(s)
            out[j, h] = p @ v[: last + 1, kv, :].astype(np.float64)
    return out


@pytest.mark.parametrize("L,n_q,hq,hkv,d", [(1, 1, 2, 1, 32), (7, 1, 4, 2, 64), (33, 3, 8, 2, 32), (64, 1, 4, 1, 128)])
def test_attend_matches_numpy_scipy(L, n_q, hq, hkv, d):
    rng = np.random.default_rng(L * 7 + d)
    q = rng.standard_normal((n_q, hq, d))
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    sm = 1 / math.sqrt(d)
    got = oracle.attend(q, k, v, sm)
    np.testing.assert_allclose(got, _np_attention(q, k, v, sm, n_q), rtol=0, atol=1e-12)
    # values equal to keys when vhat is omitted
    np.testing.assert_allclose(oracle.attend(q, k, None, sm), _np_attention(q, k, k, sm, n_q), atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(5)
    d, hkv, hq = 64, 2, 4
    k = rng.standard_normal((10, hkv, d)).astype(np.float32)
    v = rng.standard_normal((10, hkv, d)).astype(np.float32)
    # one token: output is that token's value
    q = rng.standard_normal((1, hq, d))
    o = oracle.attend(q, k[:1], v[:1], 0.1)
    for h in range(hq):
        np.testing.assert_array_equal(o[0, h], v[0, h // 2].astype(np.float64))
    # zero query: uniform weights, output is the mean value
    o = oracle.attend(np.zeros((1, hq, d)), k, v, 0.1)
    np.testing.assert_allclose(o[0, 0], v[:, 0].astype(np.float64).mean(0), atol=1e-14)
    # a key far ahead of the rest: output is its value
    q = np.zeros((1, hq, d))
    q[0, :, 0] = 1.0
    k2 = k.copy()
    k2[:, :, 0] = 0
    k2[6, :, 0] = 1000.0
    o = oracle.attend(q, k2, v, 1.0)
    np.testing.assert_allclose(o[0, 3], v[6, 1], atol=1e-12)
    # a position with no visible token (MTP verify longer than the context) is zero
    o = oracle.attend(rng.standard_normal((3, hq, d)), k[:1], v[:1], 0.1)
    assert np.all(o[0] == 0) and np.all(o[1] == 0)


def test_mtp_positions_equal_shorter_single_queries():
    rng = np.random.default_rng(9)
    L, d, hkv, hq = 40, 32, 2, 4
    q = rng.standard_normal((3, hq, d))
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    o = oracle.attend(q, k, v, 0.2)
    for j in range(3):
        last = L - 3 + j
        oj = oracle.attend(q[j:j + 1], k[: last + 1], v[: last + 1], 0.2)
        np.testing.assert_array_equal(o[j], oj[0])


def test_gqa_head_mapping():
    rng = np.random.default_rng(12)
    L, d, hkv, hq = 16, 32, 4, 8
    q = rng.standard_normal((1, hq, d))
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    o = oracle.attend(q, k, v, 0.3)
    for h in range(hq):
        kv = h // 2
        oh = oracle.attend(q[:, h:h + 1], k[:, kv:kv + 1], v[:, kv:kv + 1], 0.3)
        np.testing.assert_array_equal(o[0, h], oh[0, 0])


def test_rotation_invariance_without_quantisation():
    """With quantisation bypassed, attention over rotated q, K, V taken back
    by H equals attention in the original basis.  d = 64 makes 1/sqrt(d) =
    1/8, so the rotation of small integers is exact in fp32 and the identity
    can be held to 1e-12."""
    rng = np.random.default_rng(21)
    L, d, hkv, hq = 50, 64, 2, 8
    H = scipy.linalg.hadamard(d) / 8.0
    q = rng.integers(-3, 4, (2, hq, d)).astype(np.float64)
    k = rng.integers(-3, 4, (L, hkv, d)).astype(np.float64)
    v = rng.integers(-3, 4, (L, hkv, d)).astype(np.float64)
    plain = oracle.attend(q, k.astype(np.float32), v.astype(np.float32), 0.05)
    kr, vr = (k @ H).astype(np.float32), (v @ H).astype(np.float32)
    assert np.array_equal(kr.astype(np.float64), k @ H)       # exact
    rotated = oracle.attend(q @ H, kr, vr, 0.05)
    np.testing.assert_allclose(oracle.fwht_f64(rotated), plain, rtol=0, atol=1e-12)


def test_fwht_f32_butterfly_order():
    """The fp32 transform runs its radix-2 stages in the order h = 1, 2, ...,
    d/2 with one rounding per add/sub, then one multiply.  Restated here as
    whole-array numpy stages; a different stage order rounds differently and
    fails this bit-for-bit comparison on random inputs."""
    rng = np.random.default_rng(77)
    for d in (32, 128, 512):
        x = rng.standard_normal((16, d)).astype(np.float32)
        y = x.copy()
        h = 1
        while h < d:
            blk = y.reshape(16, d // (2 * h), 2, h)
            a, b = blk[:, :, 0, :].copy(), blk[:, :, 1, :].copy()
            blk[:, :, 0, :] = a + b
            blk[:, :, 1, :] = a - b
            h *= 2
        y = y * np.float32(1.0 / math.sqrt(d))
        assert np.array_equal(oracle.fwht_f32(x).view(np.uint32), y.view(np.uint32))


def test_decode_rotated_cache_matches_plain_attention():
    """Through the real pipeline (fp32 rotation of bf16 inputs, FP4 codes),
    decode with rotation equals plain attention over the dequantised cache
    rotated back, and an unrotated cache needs no rotation of q."""
    rng = np.random.default_rng(33)
    L, d, hkv, hq = 48, 128, 1, 4
    kb = _bf16(rng.standard_normal((L, hkv, d)))
    vb = _bf16(rng.standard_normal((L, hkv, d)))
    qb = _bf16(rng.standard_normal((1, hq, d)))
    kc, ks = oracle.quantize_fp4(kb, rotate=True)
    vc, vs = oracle.quantize_fp4(vb, rotate=True)
    khat, vhat = oracle.dequant_fp4(kc, ks), oracle.dequant_fp4(vc, vs)
    sm = 1 / math.sqrt(d)
    got = oracle.decode(qb, khat, vhat, True, sm)
    qf = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).float().numpy()
    qrot = oracle.fwht_f32(qf).astype(np.float64)
    H = scipy.linalg.hadamard(d) / math.sqrt(d)
    want = _np_attention(qrot, khat, vhat, sm, 1) @ H
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


# ------------------------------------------------------------ selected positions
# [GLM] "How the serving path works", "Sparse attention and K-pool selection":
# a separate index decides which history positions a token attends to; the
# attention itself reads only those cache rows.

def _selected_case(seed, L=40, d=64, hq=4, shared=False):
    rng = np.random.default_rng(seed)
    kb = _bf16(rng.standard_normal((L, 1, d)))
    vb = None if shared else _bf16(rng.standard_normal((L, 1, d)))
    qb = _bf16(rng.standard_normal((1, hq, d)))
    kc, ks = oracle.quantize_fp4(kb, rotate=True)
    khat = oracle.dequant_fp4(kc, ks)
    vhat = None
    if vb is not None:
        vc, vs = oracle.quantize_fp4(vb, rotate=True)
        vhat = oracle.dequant_fp4(vc, vs)
    return qb, khat, vhat


def test_selected_every_position_is_full_decode():
    qb, khat, vhat = _selected_case(41)
    sm = 1 / math.sqrt(64)
    full = oracle.decode(qb, khat, vhat, True, sm)
    got = oracle.decode_selected(qb, khat, vhat, np.arange(40), True, sm)
    assert np.array_equal(got, full)
    perm = np.random.default_rng(3).permutation(40)
    np.testing.assert_allclose(oracle.decode_selected(qb, khat, vhat, perm, True, sm), full, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shared", [False, True])
def test_selected_single_position_returns_its_value_row(shared):
    """One selected position has weight 1: every head's output is that
    position's value row rotated back (H is its own inverse)."""
    qb, khat, vhat = _selected_case(42, shared=shared)
    H = scipy.linalg.hadamard(64) / math.sqrt(64)
    for t in (0, 7, 39):
        got = oracle.decode_selected(qb, khat, vhat, [t], True, 1 / 8)
        row = (khat if vhat is None else vhat)[t, 0].astype(np.float64) @ H
        for h in range(4):
            np.testing.assert_allclose(got[0, h], row, rtol=0, atol=1e-12)


def test_selected_matches_numpy_over_listed_rows():
    """Independent restatement (numpy matmul, scipy softmax) over the listed
    rows in any order; a position listed twice counts twice."""
    qb, khat, vhat = _selected_case(43)
    sel = [5, 3, 3, 20, 39, 0]
    sm = 1 / 8
    got = oracle.decode_selected(qb, khat, vhat, sel, True, sm)
    qf = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).float().numpy()
    qrot = oracle.fwht_f32(qf).astype(np.float64)
    H = scipy.linalg.hadamard(64) / math.sqrt(64)
    want = _np_attention(qrot, khat[sel], vhat[sel], sm, 1) @ H
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)
    # the duplicate matters: without it the result moves
    other = oracle.decode_selected(qb, khat, vhat, [5, 3, 20, 39, 0], True, sm)
    assert np.abs(other - got).max() > 1e-6


def test_batch_encoders_are_the_single_value_encoders():
    """encode_n (the sweep's batch form) is the per-value encoder applied to
    each input, at several scale exponents, both formats."""
    rng = np.random.default_rng(7)
    for e in (-127, -3, 0, 5, 127):
        x = (rng.standard_normal(300) * 4.0 * 2.0 ** e).astype(np.float32)
        x[:3] = [0.0, -0.0, np.float32(2.5 * 2.0 ** e)]
        np.testing.assert_array_equal(oracle.encode_n(x, e, "fp4"),
                                      [oracle.e2m1_encode(float(v), e) for v in x])
        y = (x.astype(np.float64) * 60.0)
        y = y[np.abs(y) < np.finfo(np.float32).max].astype(np.float32)
        np.testing.assert_array_equal(oracle.encode_n(y, e, "fp8"), [oracle.e4m3_encode(float(v), e) for v in y])
