"""Python binding of libkvq: a paged, Walsh-Hadamard-rotated 4-bit (E2M1 +
UE8M0 per 32 channels) KV cache and decode attention over it, for MI355X.

Argument marshalling only: every step of the path runs in libkvq's HIP
kernels.  PyTorch supplies device memory and the current stream.  The names
follow the C interface in ``include/kvq.h``:

  rotate_quantize_append(cache, k_new, v_new, slot_mapping)
  decode_attn_fp4(cache, q, block_tables, context_lens, max_context_len, ...)
  decode_attn_fp8(...)            the 8-bit comparator, same arguments
  decode_workspace_bytes(cache, batch, num_q_heads, n_q, max_context_len)
  dequant(cache, slots)

There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch  # loads torch's HIP runtime first; libkvq then shares it

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY names another build of the library (the sanitizer run's)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
FMT_FP4_E2M1 = 1
FMT_FP8_E4M3 = 2
Q_PREROTATED = 0x1
OUT_ROTATED = 0x2
QK_CONVERT = 0x4
SPLITS_SHIFT = 16
SPLITS_MASK = 0x0FFF0000

ERRORS = {
    -1: "KVQ_ERR_NULL", -2: "KVQ_ERR_SHAPE", -3: "KVQ_ERR_FORMAT",
    -4: "KVQ_ERR_UNSUPPORTED", -5: "KVQ_ERR_WORKSPACE", -6: "KVQ_ERR_HIP",
    -7: "KVQ_ERR_SCRATCH",
}
SCRATCH_BYTES = 32 << 20      # KVQ_SCRATCH_BYTES


def splits_flag(n: int) -> int:
    """Flag bits that force the number of context splits (0: automatic)."""
    return (int(n) << SPLITS_SHIFT) & SPLITS_MASK


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(status, "?"), status, msg))
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("kv_shared", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
    ]


class PrefixGroupsDesc(ctypes.Structure):
    _fields_ = [
        ("num_groups", ctypes.c_int32),
        ("max_group_size", ctypes.c_int32),
        ("indptr", ctypes.c_void_p),
        ("members", ctypes.c_void_p),
        ("prefix_tables", ctypes.c_void_p),
        ("max_prefix_pages", ctypes.c_int32),
        ("shared_lens", ctypes.c_void_p),
        ("max_suffix_len", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_DESC = ctypes.POINTER(CacheDesc)
_GROUPS = ctypes.POINTER(PrefixGroupsDesc)

# name -> (restype, argtypes); every symbol include/kvq.h declares
SIGNATURES = {
    "kvq_cache_code_bytes": (_SZ, [_DESC]),
    "kvq_cache_scale_bytes": (_SZ, [_DESC]),
    "kvq_rotate_quantize_append": (ctypes.c_int, [_DESC, _P, _P, _P, _I32, _P]),
    "kvq_decode_workspace_bytes": (_SZ, [_DESC, _I32, _I32, _I32, _I32, _U32]),
    "kvq_decode_attn_fp4": (ctypes.c_int, [_DESC, _P, _I32, _I32, _I32, _P, _I32, _P, _I32,
                                           ctypes.c_float, _U32, _P, _P, _SZ, _P]),
    "kvq_decode_attn_fp8": (ctypes.c_int, [_DESC, _P, _I32, _I32, _I32, _P, _I32, _P, _I32,
                                           ctypes.c_float, _U32, _P, _P, _SZ, _P]),
    "kvq_decode_attn_fp4_scratch": (ctypes.c_int, [_DESC, _P, _I32, _I32, _I32, _P, _I32, _P, _I32,
                                                   ctypes.c_float, _U32, _P, _P]),
    "kvq_append_decode_attn_fp4": (ctypes.c_int, [_DESC, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _P, _I32, _P,
                                                  _I32, ctypes.c_float, _U32, _P, _P, _SZ, _P]),
    "kvq_decode_shared_workspace_bytes": (_SZ, [_DESC, _I32, _I32, _I32, _GROUPS, _U32]),
    "kvq_decode_attn_fp4_shared": (ctypes.c_int, [_DESC, _P, _I32, _I32, _I32, _P, _I32, _P, _I32, _GROUPS,
                                                  ctypes.c_float, _U32, _P, _P, _SZ, _P]),
    "kvq_decode_selected_workspace_bytes": (_SZ, [_DESC, _I32, _I32, _I32, _U32]),
    "kvq_decode_attn_fp4_selected": (ctypes.c_int, [_DESC, _P, _I32, _I32, _P, _I32, _P, _P, _I32,
                                                    ctypes.c_float, _U32, _P, _P, _SZ, _P]),
    "kvq_dequant": (ctypes.c_int, [_DESC, _P, _I32, _P, _P, _P]),
    "kvq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_version": (ctypes.c_int, []),
}

_lib = None


def library(path: str = LIB_PATH):
    """Load libkvq.so: build it first if it does not exist; raise if it was
    built from sources other than the ones in the tree now (a stale build
    would run old kernels)."""
    global _lib
    if _lib is not None:
        return _lib
    from . import _build
    if not os.path.exists(path) and os.path.abspath(path) == os.path.abspath(_build.LIB_PATH):
        _build.build()
    # every build records the hash of its sources beside the library
    try:
        with open(path + ".srchash") as f:
            built = f.read().strip()
    except OSError:
        built = None
    if built != _build.source_hash():
        raise RuntimeError("%s is stale: it was not built from the current csrc/ and include/ "
                           "sources; rebuild it (python __graft_entry__.py)" % path)
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    return library().kvq_strerror(int(status)).decode()


def version() -> int:
    return library().kvq_version()


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, strerror(status))


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class KVCache:
    """A paged cache: caller-side owner of the code and scale arrays (torch
    uint8 device tensors) plus the C description pointing at them."""

    def __init__(self, fmt: int, num_kv_heads: int, head_dim: int, page_size: int,
                 num_pages: int, rotate: Optional[bool] = None, kv_shared: bool = False,
                 device="cuda"):
        if rotate is None:
            rotate = fmt == FMT_FP4_E2M1
        self.fmt = int(fmt)
        self.rotate = bool(rotate)
        self.kv_shared = bool(kv_shared)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.page_size = int(page_size)
        self.num_pages = int(num_pages)
        d = CacheDesc(self.fmt, int(self.rotate), int(self.kv_shared), self.num_kv_heads,
                      self.head_dim, self.page_size, self.num_pages, None, None, None, None)
        L = library()
        cb, sb = L.kvq_cache_code_bytes(ctypes.byref(d)), L.kvq_cache_scale_bytes(ctypes.byref(d))
        if cb == 0 or sb == 0:
            raise KvqError(-2, "invalid cache description")
        self.code_bytes, self.scale_bytes = cb, sb
        self.k_codes = torch.zeros(cb, dtype=torch.uint8, device=device)
        self.k_scales = torch.zeros(sb, dtype=torch.uint8, device=device)
        if self.kv_shared:
            self.v_codes, self.v_scales = None, None
        else:
            self.v_codes = torch.zeros(cb, dtype=torch.uint8, device=device)
            self.v_scales = torch.zeros(sb, dtype=torch.uint8, device=device)
        d.k_codes, d.k_scales = self.k_codes.data_ptr(), self.k_scales.data_ptr()
        if not self.kv_shared:
            d.v_codes, d.v_scales = self.v_codes.data_ptr(), self.v_scales.data_ptr()
        self.desc = d

    @property
    def nbytes(self) -> int:
        return (self.code_bytes + self.scale_bytes) * (1 if self.kv_shared else 2)

    def ref(self):
        return ctypes.byref(self.desc)


def rotate_quantize_append(cache: KVCache, k_new: torch.Tensor, v_new: Optional[torch.Tensor],
                           slot_mapping: torch.Tensor, stream=None) -> None:
    n = int(slot_mapping.shape[0])
    shp = (n, cache.num_kv_heads, cache.head_dim)
    _shape(k_new, shp, "k_new")
    kp = _dev(k_new, torch.bfloat16, "k_new")
    vp = None
    if not cache.kv_shared:
        _shape(v_new, shp, "v_new")
        vp = _dev(v_new, torch.bfloat16, "v_new")
    sp = _dev(slot_mapping, torch.int32, "slot_mapping")
    _check(library().kvq_rotate_quantize_append(cache.ref(), kp, vp, sp, n, _stream(stream)))


def decode_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, n_q: int,
                           max_context_len: int, flags: int = 0) -> int:
    return int(library().kvq_decode_workspace_bytes(cache.ref(), batch, num_q_heads, n_q,
                                                    max_context_len, flags))


def _decode(fn_name, cache, q, block_tables, context_lens, max_context_len, sm_scale, flags,
            out, workspace, stream):
    B, n_q, hq, d = (int(x) for x in q.shape)
    if d != cache.head_dim:
        raise ValueError("q head_dim %d does not match the cache (%d)" % (d, cache.head_dim))
    qp = _dev(q, torch.bfloat16, "q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_pages]")
    bp = _dev(block_tables, torch.int32, "block_tables")
    _shape(context_lens, (B,), "context_lens")
    cp = _dev(context_lens, torch.int32, "context_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, n_q, hq, d), dtype=torch.float32, device=q.device)
    _shape(out, (B, n_q, hq, d), "out")
    op = _dev(out, torch.float32, "out")
    need = decode_workspace_bytes(cache, B, hq, n_q, int(max_context_len), flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp, wbytes = None, 0
    if workspace is not None:
        wp = _dev(workspace, workspace.dtype, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    fn = getattr(library(), fn_name)
    _check(fn(cache.ref(), qp, B, hq, n_q, bp, int(block_tables.shape[1]), cp, int(max_context_len),
              float(sm_scale), int(flags), op, wp, wbytes, _stream(stream)))
    return out


def decode_attn_fp4(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int,
                    sm_scale: Optional[float] = None, flags: int = 0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """q: bf16 [batch, n_q, num_q_heads, head_dim]; returns fp32 of that shape."""
    return _decode("kvq_decode_attn_fp4", cache, q, block_tables, context_lens, max_context_len,
                   sm_scale, flags, out, workspace, stream)


def decode_attn_fp4_scratch(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, max_context_len: int, out: torch.Tensor,
                            sm_scale: Optional[float] = None, flags: int = 0, stream=None) -> torch.Tensor:
    """decode_attn_fp4 on the library's static scratch array (no workspace):
    the caller passes `out`; nothing is allocated."""
    B, n_q, hq, d = (int(x) for x in q.shape)
    if d != cache.head_dim:
        raise ValueError("q head_dim %d does not match the cache (%d)" % (d, cache.head_dim))
    qp = _dev(q, torch.bfloat16, "q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_pages]")
    bp = _dev(block_tables, torch.int32, "block_tables")
    _shape(context_lens, (B,), "context_lens")
    cp = _dev(context_lens, torch.int32, "context_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _shape(out, (B, n_q, hq, d), "out")
    op = _dev(out, torch.float32, "out")
    _check(library().kvq_decode_attn_fp4_scratch(cache.ref(), qp, B, hq, n_q, bp, int(block_tables.shape[1]),
                                                  cp, int(max_context_len), float(sm_scale), int(flags), op,
                                                  _stream(stream)))
    return out


def append_decode_attn_fp4(cache: KVCache, k_new: torch.Tensor, v_new: Optional[torch.Tensor],
                           slot_mapping: torch.Tensor, q: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, max_context_len: int,
                           sm_scale: Optional[float] = None, flags: int = 0,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """rotate_quantize_append(cache, k_new, v_new, slot_mapping) followed by
    decode_attn_fp4(cache, q, ...), in one call."""
    n = int(slot_mapping.shape[0])
    kp = vp = sp = None
    if n:
        shp = (n, cache.num_kv_heads, cache.head_dim)
        _shape(k_new, shp, "k_new")
        kp = _dev(k_new, torch.bfloat16, "k_new")
        if not cache.kv_shared:
            _shape(v_new, shp, "v_new")
            vp = _dev(v_new, torch.bfloat16, "v_new")
        sp = _dev(slot_mapping, torch.int32, "slot_mapping")
    B, n_q, hq, d = (int(x) for x in q.shape)
    if d != cache.head_dim:
        raise ValueError("q head_dim %d does not match the cache (%d)" % (d, cache.head_dim))
    qp = _dev(q, torch.bfloat16, "q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_pages]")
    bp = _dev(block_tables, torch.int32, "block_tables")
    _shape(context_lens, (B,), "context_lens")
    cp = _dev(context_lens, torch.int32, "context_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, n_q, hq, d), dtype=torch.float32, device=q.device)
    _shape(out, (B, n_q, hq, d), "out")
    op = _dev(out, torch.float32, "out")
    need = decode_workspace_bytes(cache, B, hq, n_q, int(max_context_len), flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp, wbytes = None, 0
    if workspace is not None:
        wp = _dev(workspace, workspace.dtype, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    _check(library().kvq_append_decode_attn_fp4(cache.ref(), kp, vp, sp, n, qp, B, hq, n_q, bp,
                                                 int(block_tables.shape[1]), cp, int(max_context_len),
                                                 float(sm_scale), int(flags), op, wp, wbytes, _stream(stream)))
    return out


def decode_attn_fp8(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int,
                    sm_scale: Optional[float] = None, flags: int = 0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    return _decode("kvq_decode_attn_fp8", cache, q, block_tables, context_lens, max_context_len,
                   sm_scale, flags, out, workspace, stream)


class PrefixGroups:
    """Prefix groups of a shared-prefix decode: device int32 tensors plus the
    host-side bounds (the fields of kvq_prefix_groups)."""

    def __init__(self, indptr: torch.Tensor, members: torch.Tensor, prefix_tables: torch.Tensor,
                 shared_lens: torch.Tensor, max_group_size: int, max_suffix_len: int,
                 max_context_len: Optional[int] = None):
        if prefix_tables.dim() != 2 or prefix_tables.shape[0] != indptr.numel() - 1:
            raise ValueError("prefix_tables must be [num_groups, max_prefix_pages]")
        if members.numel() == 0:  # no member at all: a valid pointer is still passed
            members = torch.zeros(1, dtype=torch.int32, device=indptr.device)
        self.indptr, self.members = indptr, members
        self.prefix_tables, self.shared_lens = prefix_tables, shared_lens
        self.max_group_size, self.max_suffix_len = int(max_group_size), int(max_suffix_len)
        # the longest context of the batch, if known (a default for the decode call)
        self.max_context_len = None if max_context_len is None else int(max_context_len)
        self._desc = PrefixGroupsDesc(
            int(indptr.numel() - 1), self.max_group_size, _dev(indptr, torch.int32, "indptr"),
            _dev(members, torch.int32, "members"),
            _dev(prefix_tables, torch.int32, "prefix_tables"), int(prefix_tables.shape[1]),
            _dev(shared_lens, torch.int32, "shared_lens"), self.max_suffix_len)

    @classmethod
    def from_lists(cls, groups: Sequence[Sequence[int]], prefix_pages: Sequence[Sequence[int]],
                   shared_lens: Sequence[int], context_lens: Sequence[int], device="cuda") -> "PrefixGroups":
        """Build the tensors from host lists: groups[g] lists the member
        sequences of prefix g, prefix_pages[g] its physical pages.  Members are
        stored by decreasing shared length (the fastest order)."""
        if len(groups) != len(prefix_pages) or not groups:
            raise ValueError("one page list per group, at least one group")
        indptr, members = [0], []
        for g in groups:
            members.extend(sorted(g, key=lambda b: -int(shared_lens[b])))
            indptr.append(len(members))
        width = max(1, max(len(pp) for pp in prefix_pages))
        tables = torch.zeros((len(groups), width), dtype=torch.int32)
        for i, pp in enumerate(prefix_pages):
            tables[i, : len(pp)] = torch.as_tensor(list(pp), dtype=torch.int32)
        suffix = max((int(L) - int(s) for L, s in zip(context_lens, shared_lens)), default=0)
        as_dev = lambda x: torch.as_tensor(x, dtype=torch.int32).to(device)
        return cls(as_dev(indptr), as_dev(members), tables.to(device), as_dev(list(shared_lens)),
                   max(1, max(len(g) for g in groups)), max(suffix, 0),
                   max((int(L) for L in context_lens), default=0))

    def ref(self):
        return ctypes.byref(self._desc)


def decode_shared_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, n_q: int,
                                  groups: PrefixGroups, flags: int = 0) -> int:
    return int(library().kvq_decode_shared_workspace_bytes(cache.ref(), batch, num_q_heads, n_q,
                                                           groups.ref(), flags))


def decode_attn_fp4_shared(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, groups: PrefixGroups,
                           sm_scale: Optional[float] = None, flags: int = 0,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None, max_context_len: Optional[int] = None) -> torch.Tensor:
    """Shared-prefix decode: the result of decode_attn_fp4 with each group's
    prefix pages read once for all its members.  max_context_len defaults to
    the one the groups were built with."""
    if max_context_len is None:
        max_context_len = groups.max_context_len
    if max_context_len is None:
        raise ValueError("max_context_len is needed (the groups do not know it)")
    B, n_q, hq, d = (int(x) for x in q.shape)
    if d != cache.head_dim:
        raise ValueError("q head_dim %d does not match the cache (%d)" % (d, cache.head_dim))
    qp = _dev(q, torch.bfloat16, "q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_pages]")
    bp = _dev(block_tables, torch.int32, "block_tables")
    _shape(context_lens, (B,), "context_lens")
    cp = _dev(context_lens, torch.int32, "context_lens")
    _shape(groups.shared_lens, (B,), "shared_lens")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, n_q, hq, d), dtype=torch.float32, device=q.device)
    _shape(out, (B, n_q, hq, d), "out")
    op = _dev(out, torch.float32, "out")
    need = decode_shared_workspace_bytes(cache, B, hq, n_q, groups, flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp, wbytes = None, 0
    if workspace is not None:
        wp = _dev(workspace, workspace.dtype, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    _check(library().kvq_decode_attn_fp4_shared(cache.ref(), qp, B, hq, n_q, bp, int(block_tables.shape[1]), cp,
                                                 int(max_context_len), groups.ref(), float(sm_scale), int(flags),
                                                 op, wp, wbytes,
                                                 _stream(stream)))
    return out


def decode_selected_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, max_selected: int,
                                    flags: int = 0) -> int:
    return int(library().kvq_decode_selected_workspace_bytes(cache.ref(), batch, num_q_heads, max_selected, flags))


def decode_attn_fp4_selected(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor,
                             sel: torch.Tensor, sel_lens: torch.Tensor,
                             sm_scale: Optional[float] = None, flags: int = 0,
                             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """Attention of one query position per sequence over its selected
    history positions: q bf16 [batch, 1, num_q_heads, head_dim], sel int32
    [batch, max_selected], sel_lens int32 [batch]; returns fp32 like q."""
    B, n_q, hq, d = (int(x) for x in q.shape)
    if n_q != 1:
        raise ValueError("one query position per sequence")
    if d != cache.head_dim:
        raise ValueError("q head_dim %d does not match the cache (%d)" % (d, cache.head_dim))
    qp = _dev(q, torch.bfloat16, "q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_pages]")
    bp = _dev(block_tables, torch.int32, "block_tables")
    if sel.dim() != 2 or sel.shape[0] != B:
        raise ValueError("sel must be [batch, max_selected]")
    sp = _dev(sel, torch.int32, "sel")
    _shape(sel_lens, (B,), "sel_lens")
    lp = _dev(sel_lens, torch.int32, "sel_lens")
    max_sel = int(sel.shape[1])
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, 1, hq, d), dtype=torch.float32, device=q.device)
    _shape(out, (B, 1, hq, d), "out")
    op = _dev(out, torch.float32, "out")
    need = decode_selected_workspace_bytes(cache, B, hq, max_sel, flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp, wbytes = None, 0
    if workspace is not None:
        wp = _dev(workspace, workspace.dtype, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    _check(library().kvq_decode_attn_fp4_selected(cache.ref(), qp, B, hq, bp, int(block_tables.shape[1]), sp, lp,
                                                   max_sel, float(sm_scale), int(flags), op, wp, wbytes,
                                                   _stream(stream)))
    return out


def dequant(cache: KVCache, slots: torch.Tensor, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fp32 [n, num_kv_heads, head_dim] keys (and values) of the given slots,
    in the stored (rotated) basis."""
    n = int(slots.shape[0])
    sp = _dev(slots, torch.int32, "slots")
    k = torch.empty((n, cache.num_kv_heads, cache.head_dim), dtype=torch.float32, device=slots.device)
    v = None if cache.kv_shared else torch.empty_like(k)
    _check(library().kvq_dequant(cache.ref(), sp, n, k.data_ptr(), None if v is None else v.data_ptr(),
                                 _stream(stream)))
    return k, v
