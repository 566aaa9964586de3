"""libkvq's C interface on the host: the library loads, exports every
function include/kvq.h declares, sizes its buffers as documented, and rejects
bad arguments with the documented status before any HIP call.  No GPU."""
import ctypes
import os
import re

import pytest

import bit_quantized_kv_rotate_amd as kvq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kvq.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = kvq.library()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.kvq_version() == 1


def _desc(fmt=1, hkv=8, d=128, p=16, pages=10, rotate=1, shared=0, ptrs=True):
    x = ctypes.c_void_p(0x1000) if ptrs else None
    return kvq.CacheDesc(fmt, rotate, shared, hkv, d, p, pages, x, x, x, x)


def test_cache_sizes_match_documented_layout():
    L = kvq.library()
    d = _desc(fmt=1, hkv=8, d=128, p=16, pages=10)
    # FP4: 16 code bytes + 1 scale byte per (token, group): 17 per 32 values
    assert L.kvq_cache_code_bytes(ctypes.byref(d)) == 10 * 8 * 4 * 16 * 16
    assert L.kvq_cache_scale_bytes(ctypes.byref(d)) == 10 * 8 * 4 * 16
    d8 = _desc(fmt=2, hkv=1, d=512, p=64, pages=3)
    assert L.kvq_cache_code_bytes(ctypes.byref(d8)) == 3 * 1 * 16 * 64 * 32
    assert L.kvq_cache_scale_bytes(ctypes.byref(d8)) == 3 * 16 * 64
    per_group = (L.kvq_cache_code_bytes(ctypes.byref(d)) + L.kvq_cache_scale_bytes(ctypes.byref(d))) \
        / (10 * 8 * 16 * 4)
    assert per_group == 17


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=16), dict(d=2048), dict(hkv=0), dict(pages=0)])
def test_bad_geometry_sizes_zero(kw):
    d = _desc(**kw)
    assert kvq.library().kvq_cache_code_bytes(ctypes.byref(d)) == 0


def test_strerror_texts():
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert kvq.strerror(st)
    assert "HIP" in kvq.strerror(-6)


def _append(desc, k=0x2000, v=0x3000, slots=0x4000, n=4):
    return kvq.library().kvq_rotate_quantize_append(ctypes.byref(desc) if desc is not None else None,
                                                    k, v, slots, n, None)


def test_append_argument_errors():
    assert _append(None) == -1
    assert _append(_desc(ptrs=False)) == -1
    assert _append(_desc(), k=None) == -1
    assert _append(_desc(), v=None) == -1
    assert _append(_desc(), slots=None) == -1
    assert _append(_desc(), n=-1) == -2
    assert _append(_desc(), n=0) == 0            # nothing to do, no HIP call
    assert _append(_desc(d=96)) == -2
    assert _append(_desc(p=24)) == -4
    assert _append(_desc(fmt=7)) == -3
    assert _append(_desc(rotate=2)) == -2


def _decode(fn="kvq_decode_attn_fp4", desc=None, q=0x10, B=2, hq=16, n_q=1, bt=0x20, maxp=8,
            cl=0x30, maxl=128, sm=0.1, flags=0, out=0x40, ws=0x50, wsb=1 << 30):
    if desc is None:
        desc = _desc(fmt=1 if fn.endswith("fp4") else 2)
    return getattr(kvq.library(), fn)(ctypes.byref(desc), q, B, hq, n_q, bt, maxp, cl, maxl,
                                      sm, flags, out, ws, wsb, None)


def test_decode_argument_errors():
    assert _decode(q=None) == -1
    assert _decode(bt=None) == -1
    assert _decode(cl=None) == -1
    assert _decode(out=None) == -1
    assert _decode(desc=_desc(ptrs=False)) == -1
    assert _decode(hq=12) == -2                  # not a multiple of num_kv_heads
    assert _decode(n_q=0) == -2
    assert _decode(maxp=4, maxl=128) == -2       # 4 pages of 16 cannot hold 128 tokens
    assert _decode(sm=float("inf")) == -2
    assert _decode(flags=0x8) == -2
    assert _shared(flags=kvq.QK_CONVERT) == -2          # decode calls only
    assert _decode(desc=_desc(fmt=2)) == -3      # FP4 entry point, FP8 cache
    assert _decode(fn="kvq_decode_attn_fp8", desc=_desc(fmt=1)) == -3
    assert _decode(desc=_desc(d=64)) == -4       # no kernel for head_dim 64 yet
    # more than 24 rows per KV head: FP4 has the many-row kernel, FP8 does not
    assert _decode(fn="kvq_decode_attn_fp8", hq=8 * 32) == -4
    assert kvq.library().kvq_decode_workspace_bytes(ctypes.byref(_desc()), 2, 8 * 32, 1, 128, 0) > 0
    assert kvq.library().kvq_decode_workspace_bytes(ctypes.byref(_desc()), 2, 8 * 8193, 8, 128, 0) == 0
    # the many-row kernel's limit, 65,536 rows per KV head, exactly: accepted; one more: not
    assert kvq.library().kvq_decode_workspace_bytes(ctypes.byref(_desc()), 2, 8 * 8192, 8, 128, 0) > 0
    assert kvq.library().kvq_decode_workspace_bytes(ctypes.byref(_desc()), 2, 8 * 65537, 1, 128, 0) == 0
    # latent width 512: FP4 up to 64 rows per KV head; no FP8 kernel at 512
    d512 = _desc(d=512, hkv=1, p=64, shared=1)
    L = kvq.library()
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d512), 16, 64, 1, 131072, 0) > 0
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d512), 16, 65, 1, 131072, 0) == 0  # 65 rows
    assert L.kvq_decode_workspace_bytes(ctypes.byref(_desc(fmt=2, d=512, hkv=1, p=64, shared=1)),
                                        16, 64, 1, 131072, 0) == 0
    assert _decode(fn="kvq_decode_attn_fp8", desc=_desc(fmt=2, d=512, hkv=1, p=64, shared=1), hq=64) == -4
    assert _decode(desc=d512, hq=65) == -4
    assert _decode(B=0) == 0                     # empty batch: nothing enqueued
    # host bounds: at most 2^30 tokens of context
    assert _decode(maxl=(1 << 30) + 1, maxp=(1 << 26) + 1) == -2
    assert kvq.library().kvq_decode_workspace_bytes(ctypes.byref(_desc()), 2, 16, 1, (1 << 30) + 1, 0) == 0
    # latent width: the row count in 64 bits (an int product of group and
    # n_q that wraps must not pass as a small count)
    assert _decode(desc=d512, hq=64, n_q=(1 << 26) + 1) == -4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d512), 2, 64, (1 << 26) + 1, 1024, 0) == 0
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d512), 2, 1 << 16, 1 << 16, 1024, 0) == 0


def test_misaligned_code_array_is_rejected():
    L = kvq.library()
    d = _desc()
    d.v_codes = ctypes.c_void_p(0x1008)
    assert L.kvq_rotate_quantize_append(ctypes.byref(d), 0x10, 0x20, 0x30, 4, None) == -2
    assert _decode(desc=d) == -2
    d = _desc()
    d.k_codes = ctypes.c_void_p(0x1004)
    assert L.kvq_rotate_quantize_append(ctypes.byref(d), 0x10, 0x20, 0x30, 4, None) == -2


def test_decode_workspace_checks():
    L = kvq.library()
    d = _desc()
    need = L.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 64, 1, 32768, 0)
    assert need > 0
    assert _decode(B=32, hq=64, maxp=2048, maxl=32768, ws=None, wsb=0) == -5
    assert _decode(B=32, hq=64, maxp=2048, maxl=32768, ws=0x50, wsb=need - 1) == -5
    assert _decode(B=32, hq=64, maxp=2048, maxl=32768, ws=0x58, wsb=need) == -5  # not 16-byte aligned
    # one forced split: only the prepared query operands (FP4: 2 MFMA operands
    # of 8 dwords per lane for each 8-row tile of each (sequence, KV head))
    one = L.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 64, 1, 32768, kvq.splits_flag(1))
    assert one == 32 * d.num_kv_heads * 1 * 64 * 4 * 2 * 8
    assert need > one
    # an empty context is planned like a one-token context; a negative one is invalid
    z = L.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 64, 1, 0, 0)
    assert z > 0 and z == L.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 64, 1, 1, 0)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 32, 64, 1, -1, 0) == 0


def test_decode_workspace_fp8_three_query_terms_and_plan():
    """The FP8 comparator's query operands are three bf16 terms in two sets of
    four k-step operands (8 operands of 4 dwords per lane and 8-row tile), and
    without a device its plan takes the fallback of six page-scan waves per
    compute unit (b32_l32k: 6 splits, as forced), where FP4 takes eight."""
    L = kvq.library()
    d8 = _desc(fmt=2, rotate=0)
    one = L.kvq_decode_workspace_bytes(ctypes.byref(d8), 32, 64, 1, 32768, kvq.splits_flag(1))
    assert one == 32 * d8.num_kv_heads * 1 * 64 * 4 * 8 * 4
    need8 = L.kvq_decode_workspace_bytes(ctypes.byref(d8), 32, 64, 1, 32768, 0)
    assert need8 == L.kvq_decode_workspace_bytes(ctypes.byref(d8), 32, 64, 1, 32768, kvq.splits_flag(6))
    d4 = _desc()
    need4 = L.kvq_decode_workspace_bytes(ctypes.byref(d4), 32, 64, 1, 32768, 0)
    assert need4 == L.kvq_decode_workspace_bytes(ctypes.byref(d4), 32, 64, 1, 32768, kvq.splits_flag(8))


def test_dequant_argument_errors():
    L = kvq.library()
    d = _desc()
    assert L.kvq_dequant(ctypes.byref(d), None, 3, 0x10, 0x20, None) == -1
    assert L.kvq_dequant(ctypes.byref(d), 0x10, 3, None, 0x20, None) == -1
    assert L.kvq_dequant(ctypes.byref(d), 0x10, 3, 0x10, None, None) == -1
    assert L.kvq_dequant(ctypes.byref(d), 0x10, -1, 0x10, 0x20, None) == -2
    assert L.kvq_dequant(ctypes.byref(d), 0x10, 0, 0x10, 0x20, None) == 0


def test_binding_has_no_oracle_dependency():
    """The product package must not import or call the test oracle."""
    pkg = os.path.dirname(kvq.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.lower().replace("no cpu fallback", ""), f


def _groups(G=2, gmax=4, ptrs=True, maxpp=64, suffix=256):
    x = ctypes.c_void_p(0x6000) if ptrs else None
    return kvq.PrefixGroupsDesc(G, gmax, x, x, x, maxpp, x, suffix)


def _shared(desc=None, q=0x10, B=8, hq=64, n_q=3, bt=0x20, maxp=128, cl=0x30, maxl=2048, groups=None, sm=0.1,
            flags=0, out=0x40, ws=0x50, wsb=1 << 34):
    desc = _desc() if desc is None else desc
    g = _groups() if groups is None else groups
    return kvq.library().kvq_decode_attn_fp4_shared(ctypes.byref(desc), q, B, hq, n_q, bt, maxp, cl, maxl,
                                                    ctypes.byref(g), sm, flags, out, ws, wsb, None)


def test_shared_workspace_bytes():
    L = kvq.library()
    d = _desc()
    ws = lambda desc=d, B=8, hq=64, n_q=3, g=None, flags=0: L.kvq_decode_shared_workspace_bytes(
        ctypes.byref(desc), B, hq, n_q, ctypes.byref(g if g is not None else _groups()), flags)
    need = ws()
    assert need > 0
    # the prefix level's operands alone need one 16-row operand block per 16 gathered rows
    assert need > 2 * 8 * (4 * 24 + 127) // 128 * 128 // 16 * 4 * 64 * 8 * 4
    assert ws(desc=_desc(fmt=2)) == 0                     # FP4 only
    assert ws(desc=_desc(d=512, hkv=1, p=64, shared=1), hq=64, n_q=1) == 0
    assert ws(g=_groups(G=0)) == 0
    assert ws(g=_groups(gmax=0)) == 0
    assert ws(g=_groups(maxpp=0)) == 0
    assert ws(g=_groups(suffix=-1)) == 0
    assert ws(g=_groups(gmax=2731)) == 0                  # 2731 x 24 rows > 65536
    assert ws(g=_groups(gmax=2730)) > 0
    assert ws(B=0) == 0
    assert ws(g=_groups(suffix=0)) > 0                    # every token shared
    # a forced split count applies to both levels, at most 32 each
    assert ws(flags=kvq.splits_flag(40)) == ws(flags=kvq.splits_flag(32))


def test_shared_argument_errors():
    assert _shared(q=None) == -1
    assert _shared(bt=None) == -1
    assert _shared(cl=None) == -1
    assert _shared(out=None) == -1
    assert _shared(desc=_desc(ptrs=False)) == -1
    assert _shared(groups=_groups(ptrs=False)) == -1
    assert kvq.library().kvq_decode_attn_fp4_shared(ctypes.byref(_desc()), 0x10, 8, 64, 3, 0x20, 128, 0x30, 2048,
                                                    None, 0.1, 0, 0x40, 0x50, 1 << 34, None) == -1
    assert _shared(desc=_desc(fmt=2)) == -3
    assert _shared(desc=_desc(d=64)) == -4
    assert _shared(hq=12) == -2
    assert _shared(n_q=0) == -2
    assert _shared(sm=float("nan")) == -2
    assert _shared(flags=0x8) == -2
    assert _shared(groups=_groups(G=0)) == -2
    assert _shared(groups=_groups(suffix=128 * 16 + 1), maxl=128 * 16 + 1) == -2  # longer than a table row
    assert _shared(groups=_groups(suffix=300), maxl=299) == -2  # a suffix longer than the longest context
    # a table row must cover the whole context (the suffix scan indexes it by
    # token position), not just the suffix
    assert _shared(groups=_groups(suffix=256), maxp=20, maxl=20 * 16 + 1) == -2
    assert _shared(maxl=-1) == -2
    assert _shared(maxl=(1 << 30) + 1, maxp=(1 << 26) + 1) == -2
    assert _shared(groups=_groups(gmax=2731)) == -4
    assert _shared(ws=None, wsb=0) == -5
    L = kvq.library()
    need = L.kvq_decode_shared_workspace_bytes(ctypes.byref(_desc()), 8, 64, 3, ctypes.byref(_groups()), 0)
    assert _shared(wsb=need - 1) == -5
    assert _shared(ws=0x58, wsb=need) == -5
    assert _shared(B=0) == 0                     # empty batch: nothing enqueued


def _selected(desc=None, q=0x10, B=4, hq=64, bt=0x20, maxp=64, sel=0x30, sel_lens=0x38, max_sel=2051, sm=0.1,
              flags=0, out=0x40, ws=0x50, wsb=1 << 34):
    desc = _desc(d=512, hkv=1, p=64, shared=1) if desc is None else desc
    return kvq.library().kvq_decode_attn_fp4_selected(ctypes.byref(desc), q, B, hq, bt, maxp, sel, sel_lens, max_sel,
                                                      sm, flags, out, ws, wsb, None)


def test_selected_workspace_and_argument_errors():
    L = kvq.library()
    d512 = _desc(d=512, hkv=1, p=64, shared=1)
    need = L.kvq_decode_selected_workspace_bytes(ctypes.byref(d512), 4, 64, 2051, 0)
    assert need > 0
    # the same plan as a one-position decode over a context of max_selected tokens
    assert need == L.kvq_decode_workspace_bytes(ctypes.byref(d512), 4, 64, 1, 2051, 0)
    assert L.kvq_decode_selected_workspace_bytes(ctypes.byref(_desc()), 4, 64, 2051, 0) == 0      # head_dim 128
    assert L.kvq_decode_selected_workspace_bytes(ctypes.byref(d512), 4, 65, 2051, 0) == 0         # 65 rows
    assert L.kvq_decode_selected_workspace_bytes(ctypes.byref(d512), 4, 64, -1, 0) == 0
    assert L.kvq_decode_selected_workspace_bytes(ctypes.byref(d512), 4, 64, 0, 0) > 0
    assert _selected(q=None) == -1
    assert _selected(bt=None) == -1
    assert _selected(sel=None) == -1
    assert _selected(sel_lens=None) == -1
    assert _selected(out=None) == -1
    assert _selected(max_sel=-1) == -2
    assert _selected(sm=float("inf")) == -2
    assert _selected(flags=0x10) == -2
    assert _selected(desc=_desc(fmt=2, d=512, hkv=1, p=64, shared=1)) == -3
    assert _selected(desc=_desc(d=128)) == -4
    assert _selected(hq=65) == -4
    assert _selected(ws=None, wsb=0) == -5
    assert _selected(wsb=need - 1) == -5
    assert _selected(ws=0x58, wsb=need) == -5
    assert _selected(B=0) == 0


def test_append_decode_argument_errors():
    L = kvq.library()
    d = _desc()
    call = lambda desc=d, k=0x60, v=0x68, s=0x70, n=4, q=0x10, B=2, out=0x40, ws=0x50, wsb=1 << 30: \
        L.kvq_append_decode_attn_fp4(ctypes.byref(desc), k, v, s, n, q, B, 16, 1, 0x20, 8, 0x30, 128, 0.1, 0,
                                     out, ws, wsb, None)
    assert call(k=None) == -1
    assert call(v=None) == -1
    assert call(s=None) == -1
    assert call(n=-1) == -2
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(desc=_desc(fmt=2)) == -3
    assert call(ws=None, wsb=0) == -5
    assert call(n=0, k=None, v=None, s=None, B=0) == 0      # nothing to append or attend
    assert call(desc=_desc(d=96)) == -2


def _scratch(desc=None, q=0x10, B=2, hq=16, n_q=1, bt=0x20, maxp=8, cl=0x30, maxl=128, sm=0.1, flags=0,
             out=0x40):
    desc = _desc() if desc is None else desc
    return kvq.library().kvq_decode_attn_fp4_scratch(ctypes.byref(desc), q, B, hq, n_q, bt, maxp, cl, maxl,
                                                     sm, flags, out, None)


def test_scratch_decode_argument_errors():
    """The allocation-free decode checks its arguments like the workspace
    call, and refuses (before any HIP call) sizes that need more than the
    static scratch array holds."""
    assert _scratch(q=None) == -1
    assert _scratch(out=None) == -1
    assert _scratch(hq=12) == -2
    assert _scratch(maxp=4, maxl=128) == -2
    assert _scratch(desc=_desc(fmt=2)) == -3
    assert _scratch(desc=_desc(d=64)) == -4
    assert _scratch(B=0) == 0
    L = kvq.library()
    big = dict(B=64, hq=64, maxl=1 << 20, maxp=(1 << 20) // 16)
    d64 = _desc(hkv=64)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d64), 64, 64, 1, 1 << 20, 0) > kvq.SCRATCH_BYTES
    assert _scratch(desc=d64, **big) == -7
    assert "scratch" in kvq.strerror(-7)


def test_library_refuses_a_stale_build(monkeypatch):
    """library() raises, rather than loading old kernels, when libkvq.so was
    not built from the sources in the tree (the build records their hash)."""
    from bit_quantized_kv_rotate_amd import _build
    with open(_build.HASH_PATH) as f:
        assert f.read().strip() == _build.source_hash()   # the tree's build is current
    saved = kvq._lib
    try:
        kvq._lib = None
        monkeypatch.setattr(_build, "source_hash", lambda: "0" * 64)
        with pytest.raises(RuntimeError, match="stale"):
            kvq.library()
    finally:
        kvq._lib = saved
