"""The append's codes come from the gfx950 scaled conversions (FP4 directly,
FP8 after a clamp to +-448 * 2^e_s).  This sweep runs the append's own group
encoders (encode_fp4_group / encode_fp8_group, through the harness in
tests/convert_harness.hip) over fp32 inputs and compares every code with the
CPU oracle's encoders (nearest grid value, a tie to the even code,
saturating, sign copied), computed on host threads from the same inputs:

  - E2M1 at scale byte 127: every finite fp32 pattern with |x| < 8 (the whole
    range a group can hold at that scale: |x| < 2^(floor(log2 amax) + 1) and
    e_s = floor(log2 amax) - 2), 2.18e9 inputs;
  - E2M1 and E4M3 at scale bytes 0, 1, 126, 127, 128, 254: every grid value,
    every tie between neighbouring grid values and the saturation edge, each
    with its nearest fp32 neighbours, both signs;
  - E2M1 and E4M3 at the same bytes: random fp32 patterns over each format's
    whole range at that scale.

The grid is "the FP4 grid that MI355X supports" of the ROCm blog "UltraQuant
on AMD Instinct", section "What is UltraQuant?"; the rounding rule is the
reading the oracle states."""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BYTES = (0, 1, 126, 127, 128, 254)
THREADS = 16


@pytest.fixture(scope="module")
def harness(gpu):
    from bit_quantized_kv_rotate_amd import _build
    path = _build.HARNESS_LIB
    assert os.path.exists(path), "tests/libconvert_harness.so is not built (python __graft_entry__.py)"
    with open(path + ".srchash") as f:
        assert f.read().strip() == _build.harness_hash(), "the conversion harness is stale; rebuild it"
    L = ctypes.CDLL(path)
    L.harness_encode.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.harness_encode_bits.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    return L


def _unpack(packed: np.ndarray, fmt: str) -> np.ndarray:
    """One code per value from the harness output (FP4: channel 2i in the
    low nibble of byte i)."""
    if fmt == "fp8":
        return packed
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out


def _gpu_codes(L, fmt, x=None, bits=None, byte=127):
    """Codes of the harness: from an fp32 array x (a multiple of 32 values),
    or from the bit patterns bits = (u0, n, negative)."""
    n = x.size if x is not None else bits[1]
    per = n // 2 if fmt == "fp4" else n
    out = torch.empty(per, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = 1 if fmt == "fp4" else 2
    if x is not None:
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        rc = L.harness_encode(f, ctypes.c_void_p(xd.data_ptr()), n, byte, ctypes.c_void_p(out.data_ptr()), stream)
    else:
        rc = L.harness_encode_bits(f, bits[0], n, int(bits[2]), byte, ctypes.c_void_p(out.data_ptr()), stream)
    assert rc == 0, rc
    return _unpack(out.cpu().numpy(), fmt)


def _oracle_codes(x: np.ndarray, e_s: int, fmt: str, ex: ThreadPoolExecutor) -> np.ndarray:
    parts = np.array_split(x, THREADS)
    return np.concatenate(list(ex.map(lambda p: oracle.encode_n(p, e_s, fmt), parts)))


def _check(got, want, x, what):
    bad = np.nonzero(got != want)[0]
    if bad.size:
        i = bad[:8]
        pytest.fail("%s: %d of %d codes differ; first inputs %s (bits %s): gpu %s oracle %s" % (
            what, bad.size, x.size, x[i], x[i].view(np.uint32), got[i], want[i]))


def _pad32(x: np.ndarray) -> np.ndarray:
    return np.concatenate([x, np.zeros((-x.size) % 32, dtype=np.float32)]).astype(np.float32)


def test_e2m1_every_fp32_below_8_at_unit_scale(harness):
    top = 0x41000000                      # bits of 8.0
    chunk = 1 << 24
    with ThreadPoolExecutor(THREADS) as ex:
        for neg in (0, 1):
            for u0 in range(0, top, chunk):
                n = min(chunk, top - u0)
                x = (np.arange(u0, u0 + n, dtype=np.uint32) | np.uint32(neg << 31)).view(np.float32)
                got = _gpu_codes(harness, "fp4", bits=(u0, n, neg), byte=127)
                _check(got, _oracle_codes(x, 0, "fp4", ex), x, "E2M1 byte 127 from bits 0x%08x" % u0)


def _grid_points(fmt):
    """Grid magnitudes, the ties between neighbours and the saturation edge
    (beyond the largest value the codes saturate; E4M3 values past 448 are
    clamped first)."""
    if fmt == "fp4":
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
        extra = [6.5, 7.0, 7.5, 7.999]
    else:
        grid = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
        extra = [456.0, 464.0, 472.0, 480.0, 500.0, 511.9]
    ties = (grid[1:] + grid[:-1]) / 2
    return np.concatenate([grid, ties, extra])


def _neighbours(x32: np.ndarray) -> np.ndarray:
    out = [x32]
    up, dn = x32.copy(), x32.copy()
    for _ in range(2):
        up = np.nextafter(up, np.float32(np.inf)).astype(np.float32)
        dn = np.nextafter(dn, np.float32(-np.inf)).astype(np.float32)
        out += [up, dn]
    return np.concatenate(out)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_grid_ties_and_neighbours_at_extreme_scales(harness, fmt):
    r = _grid_points(fmt)
    with ThreadPoolExecutor(THREADS) as ex:
        for byte in BYTES:
            e = byte - 127
            with np.errstate(over="ignore"):
                x = np.ldexp(r, e).astype(np.float32)
            x = _neighbours(x[np.isfinite(x)])
            x = x[np.isfinite(x)]
            x = _pad32(np.concatenate([x, -x]))
            _check(_gpu_codes(harness, fmt, x=x, byte=byte), _oracle_codes(x, e, fmt, ex), x,
                   "%s ties, byte %d" % (fmt, byte))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_random_inputs_over_the_range_at_extreme_scales(harness, fmt):
    """Uniform fp32 bit patterns below the range limit of the scale (8 * 2^e
    for E2M1, 512 * 2^e for E4M3: what a group with that scale byte can
    hold), both signs."""
    rng = np.random.default_rng(20261203)
    lim = 8.0 if fmt == "fp4" else 512.0
    n = 1 << 21
    with ThreadPoolExecutor(THREADS) as ex:
        for byte in BYTES:
            e = byte - 127
            top = np.float32(min(np.ldexp(lim, e), np.finfo(np.float32).max)).view(np.uint32)
            bits = rng.integers(0, int(top), size=n, dtype=np.uint32)
            bits |= (rng.integers(0, 2, size=n, dtype=np.uint32) << np.uint32(31))
            x = bits.view(np.float32)
            _check(_gpu_codes(harness, fmt, x=x, byte=byte), _oracle_codes(x, e, fmt, ex), x,
                   "%s random, byte %d" % (fmt, byte))
