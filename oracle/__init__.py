"""CPU oracle for the rotated 4-bit KV cache and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
(``bit_quantized_kv_rotate_amd``) never imports it, and this package never
imports the product library: the two share no code.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp32 rotation and
quantisation in a fixed order, fp64 attention); this module only marshals
numpy arrays into it.  bf16 values travel as ``numpy.uint16`` bit patterns.

Method source: AMD ROCm blog "UltraQuant on AMD Instinct", sections
"What is UltraQuant?" (Walsh-Hadamard rotation, FP4 E2M1 codes with one
power-of-two scale per 32 channels, 17 bytes per group) and "Why UltraQuant
beats 8-bit KV" (UE8M0 scales, 17 vs 32 bytes per 32 values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double
_F = ctypes.c_float

_SIGNATURES = {
    "orc_bf16_to_f32": (_F, [ctypes.c_uint16]),
    "orc_fwht_f32": (None, [_P, _I]),
    "orc_fwht_f64": (None, [_P, _I]),
    "orc_scale_exponent": (_I, [_F, _I]),
    "orc_scale_byte": (_I, [_F, _I]),
    "orc_scale_value": (_D, [_I]),
    "orc_e2m1_value": (_D, [_I]),
    "orc_e2m1_encode": (_I, [_F, _I]),
    "orc_e4m3_value": (_D, [_I]),
    "orc_e4m3_encode": (_I, [_F, _I]),
    "orc_e2m1_encode_n": (None, [_P, _I64, _I, _P]),
    "orc_e4m3_encode_n": (None, [_P, _I64, _I, _P]),
    "orc_quantize_fp4_n": (None, [_P, _I64, _I, _I, _P, _P]),
    "orc_quantize_fp8_n": (None, [_P, _I64, _I, _I, _P, _P]),
    "orc_dequant_fp4_n": (None, [_P, _P, _I64, _I, _P]),
    "orc_dequant_fp8_n": (None, [_P, _P, _I64, _I, _P]),
    "orc_attend": (None, [_P, _I, _I, _I, _I, _I, _P, _P, _D, _P]),
    "orc_decode": (None, [_P, _I, _I, _I, _I, _I, _P, _P, _I, _D, _P]),
    "orc_version": (_I, []),
}


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file with gcc (no fast-math, no FMA
    contraction, so every fp32 operation rounds once, in program order)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    return compile_source(_SRC, LIB_PATH)


def load(path: str):
    """Load a compiled oracle and declare its C signatures."""
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = None
_override = None


def lib():
    if _override is not None:
        return _override
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("KVQ_ORACLE_LIB")   # another build (the sanitizer run's)
    if alt:
        _lib = load(alt)
        return _lib
    if (not os.path.exists(LIB_PATH)
            or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    _lib = load(LIB_PATH)
    return _lib


class use_library:
    """Context manager: route every function of this module to another
    compiled oracle (used to show that the pins catch planted mistakes)."""

    def __init__(self, L):
        self.L = L

    def __enter__(self):
        global _override
        self.prev = _override
        _override = self.L
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- scalars

def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(int(b) & 0xFFFF)


def scale_exponent(amax: float, emax_elem: int) -> int:
    return lib().orc_scale_exponent(float(amax), int(emax_elem))


def scale_byte(amax: float, emax_elem: int = 2) -> int:
    return lib().orc_scale_byte(float(amax), int(emax_elem))


def scale_value(byte: int) -> float:
    return lib().orc_scale_value(int(byte))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(y: float, e_s: int) -> int:
    return lib().orc_e2m1_encode(float(y), int(e_s))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_encode(y: float, e_s: int) -> int:
    return lib().orc_e4m3_encode(float(y), int(e_s))


# ---------------------------------------------------------------- vectors

def encode_n(y: np.ndarray, e_s: int, fmt: str) -> np.ndarray:
    """Codes (uint8, one per value) of fp32 values y at scale exponent e_s:
    the E2M1 (fmt 'fp4') or E4M3 ('fp8') encoder applied to each value."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    fn = lib().orc_e2m1_encode_n if fmt == "fp4" else lib().orc_e4m3_encode_n
    fn(_ptr(y), y.size, int(e_s), _ptr(out))
    return out


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Rotate every length-d row of ``x`` (float32, d a power of two)."""
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    d = y.shape[-1]
    flat = y.reshape(-1, d)
    for r in range(flat.shape[0]):
        row = flat[r]
        lib().orc_fwht_f32(_ptr(row), d)
    return y


def fwht_f64(x: np.ndarray) -> np.ndarray:
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    d = y.shape[-1]
    flat = y.reshape(-1, d)
    for r in range(flat.shape[0]):
        row = flat[r]
        lib().orc_fwht_f64(_ptr(row), d)
    return y


def quantize_fp4(x_bf16: np.ndarray, rotate: bool = True):
    """x_bf16: uint16 [..., d].  Returns (codes uint8 [..., d/2],
    scales uint8 [..., d/32]); channel 2i is the low nibble of byte i."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    d = x.shape[-1]
    n = x.size // d
    codes = np.empty(x.shape[:-1] + (d // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 32,), dtype=np.uint8)
    lib().orc_quantize_fp4_n(_ptr(x), n, d, int(bool(rotate)), _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_fp8(x_bf16: np.ndarray, rotate: bool = False):
    """x_bf16: uint16 [..., d].  Returns (codes uint8 [..., d] E4M3,
    scales uint8 [..., d/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    d = x.shape[-1]
    n = x.size // d
    codes = np.empty(x.shape[:-1] + (d,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 32,), dtype=np.uint8)
    lib().orc_quantize_fp8_n(_ptr(x), n, d, int(bool(rotate)), _ptr(codes), _ptr(scales))
    return codes, scales


def dequant_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    d = c.shape[-1] * 2
    n = c.size // (d // 2)
    out = np.empty(c.shape[:-1] + (d,), dtype=np.float32)
    lib().orc_dequant_fp4_n(_ptr(c), _ptr(s), n, d, _ptr(out))
    return out


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    d = c.shape[-1]
    n = c.size // d
    out = np.empty(c.shape, dtype=np.float32)
    lib().orc_dequant_fp8_n(_ptr(c), _ptr(s), n, d, _ptr(out))
    return out


# ---------------------------------------------------------------- attention

def attend(q: np.ndarray, khat: np.ndarray, vhat, sm_scale: float) -> np.ndarray:
    """Textbook fp64 attention for one sequence, one basis throughout.
    q: [n_q, hq, d] float64; khat/vhat: [L, hkv, d] float32 (vhat None: V=K)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(khat, dtype=np.float32)
    v = None if vhat is None else np.ascontiguousarray(vhat, dtype=np.float32)
    n_q, hq, d = q.shape
    L, hkv, _ = k.shape
    out = np.empty((n_q, hq, d), dtype=np.float64)
    lib().orc_attend(_ptr(q), n_q, hq, hkv, d, L, _ptr(k),
                     None if v is None else _ptr(v), float(sm_scale), _ptr(out))
    return out


def decode(q_bf16: np.ndarray, khat: np.ndarray, vhat, rotate: bool,
           sm_scale: float) -> np.ndarray:
    """Decode attention for one sequence in the caller's basis.
    q_bf16: uint16 [n_q, hq, d]; khat/vhat: [L, hkv, d] float32 dequantised
    cache (rotated basis when ``rotate``); returns float64 [n_q, hq, d]."""
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    k = np.ascontiguousarray(khat, dtype=np.float32)
    v = None if vhat is None else np.ascontiguousarray(vhat, dtype=np.float32)
    n_q, hq, d = q.shape
    L, hkv, _ = k.shape
    out = np.empty((n_q, hq, d), dtype=np.float64)
    lib().orc_decode(_ptr(q), n_q, hq, hkv, d, L, _ptr(k),
                     None if v is None else _ptr(v), int(bool(rotate)),
                     float(sm_scale), _ptr(out))
    return out


def decode_selected(q_bf16: np.ndarray, khat: np.ndarray, vhat, sel, rotate: bool,
                    sm_scale: float) -> np.ndarray:
    """Attention of one query position over selected history positions only.
    [GLM] "How the serving path works", "Sparse attention and K-pool
    selection": a separate index picks the history each token attends to
    (pooled four-token groups plus a few recent tokens); attention then reads
    the cache rows of the picked positions alone.  sel: int positions into
    the sequence's cache (a position listed twice counts twice).
    q_bf16: uint16 [1, hq, d]; khat/vhat: [L, hkv, d] float32."""
    idx = np.asarray(sel, dtype=np.int64)
    k = np.ascontiguousarray(khat[idx])
    v = None if vhat is None else np.ascontiguousarray(vhat[idx])
    return decode(q_bf16, k, v, rotate, sm_scale)


def reference_decode_selected(q_bf16, k_bf16, v_bf16, sel, fmt: str, rotate: bool,
                              sm_scale: float) -> np.ndarray:
    """Whole pipeline for one sequence and one query position: quantise the
    cache, dequantise it, and attend over the selected positions."""
    q = np.asarray(q_bf16)
    assert q.shape[0] == 1, "one query position per selection"
    if fmt != "fp4":
        raise ValueError(fmt)
    kc, ks = quantize_fp4(k_bf16, rotate)
    khat = dequant_fp4(kc, ks)
    vhat = None
    if v_bf16 is not None:
        vc, vs = quantize_fp4(v_bf16, rotate)
        vhat = dequant_fp4(vc, vs)
    return decode_selected(q, khat, vhat, sel, rotate, sm_scale)


def reference_decode_seq(q_bf16, k_bf16, v_bf16, fmt: str, rotate: bool,
                         sm_scale: float) -> np.ndarray:
    """Whole pipeline for one sequence from bf16 inputs: quantise the cache
    (fp4 or fp8), dequantise it, and run decode attention.
    k_bf16/v_bf16: uint16 [L, hkv, d] (v None: K=V)."""
    if fmt == "fp4":
        kc, ks = quantize_fp4(k_bf16, rotate)
        khat = dequant_fp4(kc, ks)
        vhat = None
        if v_bf16 is not None:
            vc, vs = quantize_fp4(v_bf16, rotate)
            vhat = dequant_fp4(vc, vs)
    elif fmt == "fp8":
        kc, ks = quantize_fp8(k_bf16, rotate)
        khat = dequant_fp8(kc, ks)
        vhat = None
        if v_bf16 is not None:
            vc, vs = quantize_fp8(v_bf16, rotate)
            vhat = dequant_fp8(vc, vs)
    else:
        raise ValueError(fmt)
    return decode(q_bf16, khat, vhat, rotate, sm_scale)
