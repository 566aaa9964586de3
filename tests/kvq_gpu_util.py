"""Helpers for the GPU tests: fill a paged cache through libkvq from a
synthetic workload, read cache bytes back through the layout documented in
include/kvq.h, and compare attention outputs with the oracle's."""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
import oracle

FMT = {"fp4": kvq.FMT_FP4_E2M1, "fp8": kvq.FMT_FP8_E4M3}

# Acceptance: max |gpu - oracle| <= 2e-3 and ||gpu - oracle|| / ||oracle|| <= 1e-3
MAX_ABS = 2e-3
REL_L2 = 1e-3

# Two GPU results of one cache that differ only in how the context is cut
# (split count, shared-prefix levels): each cut rounds its softmax weights to
# bf16 hi + lo (2^-17 relative) against its own running maximum.
SPLIT_RTOL = 5e-5
SPLIT_ATOL = 3e-4


def to_dev_i32(a) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class Filled:
    """A cache filled with every token of a workload, plus what the oracle
    needs (host copies of the bf16 inputs when gen_device is 'cpu')."""

    def __init__(self, wl: syn.Workload, fmt: str, gen_device: str = "cpu",
                 keep_host: bool = True, rotate: Optional[bool] = None,
                 plan: Optional[syn.PagePlan] = None):
        self.wl = wl
        self.fmt = fmt
        self.plan = plan if plan is not None else syn.page_plan(wl)
        P = wl.page_size
        self.cache = kvq.KVCache(FMT[fmt], wl.num_kv_heads, wl.head_dim, P, self.plan.num_pages,
                                 rotate=rotate, kv_shared=wl.kv_shared)
        self.host: Dict[str, List[np.ndarray]] = {t: [] for t in syn.tensor_names(wl)}
        prefix_host = {}
        for p in range(wl.n_prefixes):
            pages = self.plan.prefix_pages[p]
            if len(pages) == 0:
                continue
            kv = {t: syn.full_prefix(wl, self.plan, t, p, gen_device) for t in syn.tensor_names(wl)}
            slots = syn.slots_for(pages, len(pages) * P, P)
            self._append(kv, slots)
            if keep_host:
                prefix_host[p] = {t: syn.bf16_bits(x) for t, x in kv.items()}
        for b in range(wl.batch):
            L = int(self.plan.context_lens[b])
            n_sh = self.plan.n_shared_pages[b] * P
            kv = {t: syn.private_tokens(wl, t, b, L - n_sh, gen_device) for t in syn.tensor_names(wl)}
            slots = syn.slots_for(self.plan.private_pages[b], L - n_sh, P)
            self._append(kv, slots)
            if keep_host:
                for t, x in kv.items():
                    own = syn.bf16_bits(x)
                    if n_sh:
                        own = np.concatenate([prefix_host[self.plan.prefix_of[b]][t][:n_sh], own], 0)
                    self.host[t].append(own)
        self.block_tables = to_dev_i32(self.plan.block_tables)
        self.context_lens = to_dev_i32(self.plan.context_lens)
        self.max_context = int(self.plan.context_lens.max())

    def _append(self, kv, slots):
        if len(slots) == 0:
            return
        k = kv["k"].cuda()
        v = None if self.wl.kv_shared else kv["v"].cuda()
        kvq.rotate_quantize_append(self.cache, k, v, to_dev_i32(slots))

    def decode(self, q: torch.Tensor, flags: int = 0, sm_scale: Optional[float] = None):
        fn = kvq.decode_attn_fp4 if self.fmt == "fp4" else kvq.decode_attn_fp8
        return fn(self.cache, q, self.block_tables, self.context_lens, self.max_context,
                  sm_scale=sm_scale, flags=flags)

    def prefix_groups(self, shared_lens=None) -> kvq.PrefixGroups:
        """The plan's shared prefixes as prefix groups: sequence b shares its
        whole shared pages unless shared_lens says otherwise; a sequence that
        shares nothing is in no group."""
        plan, P = self.plan, self.wl.page_size
        if shared_lens is None:
            shared_lens = [plan.n_shared_pages[b] * P for b in range(self.wl.batch)]
        n_groups = max(1, self.wl.n_prefixes)
        groups = [[b for b in range(self.wl.batch) if plan.prefix_of[b] == g and shared_lens[b] > 0]
                  for g in range(n_groups)]
        pages = [plan.prefix_pages[g] if g < len(plan.prefix_pages) else [] for g in range(n_groups)]
        return kvq.PrefixGroups.from_lists(groups, pages, [int(x) for x in shared_lens],
                                           [int(x) for x in plan.context_lens])

    def decode_shared(self, q: torch.Tensor, groups: Optional[kvq.PrefixGroups] = None, flags: int = 0):
        groups = self.prefix_groups() if groups is None else groups
        return kvq.decode_attn_fp4_shared(self.cache, q, self.block_tables, self.context_lens, groups,
                                          flags=flags)

    def seq_slots(self, b: int) -> np.ndarray:
        L = int(self.plan.context_lens[b])
        t = np.arange(L)
        return (self.plan.block_tables[b][t // self.wl.page_size].astype(np.int64)
                * self.wl.page_size + t % self.wl.page_size)


def gather_codes(cache: kvq.KVCache, tensor: str, slots: np.ndarray):
    """Codes [n, hkv, d/2 or d] and scales [n, hkv, d/32] of the given slots,
    read through the documented layout: group g of (page, head, offset) is at
    ((page * hkv + head) * G + g) * P + offset."""
    P, H, D = cache.page_size, cache.num_kv_heads, cache.head_dim
    G = D // 32
    cb = 16 if cache.fmt == kvq.FMT_FP4_E2M1 else 32
    codes = (cache.k_codes if tensor == "k" else cache.v_codes).cpu().numpy()
    scales = (cache.k_scales if tensor == "k" else cache.v_scales).cpu().numpy()
    slots = np.asarray(slots, dtype=np.int64)
    page, off = slots // P, slots % P
    h = np.arange(H, dtype=np.int64)
    g = np.arange(G, dtype=np.int64)
    idx = ((page[:, None, None] * H + h[None, :, None]) * G + g[None, None, :]) * P + off[:, None, None]
    c = codes.reshape(-1, cb)[idx].reshape(len(slots), H, G * cb)
    s = scales[idx]
    return c, s


def oracle_decode_batch(filled: Filled, q_host: np.ndarray, seqs=None, rotate=None,
                        sm_scale=None, kv_heads=None) -> Dict[int, np.ndarray]:
    """Oracle outputs {b: [n_q, hq, d] float64} from the host bf16 inputs.
    kv_heads restricts the oracle to some KV heads (the rest stay NaN)."""
    wl = filled.wl
    rotate = filled.cache.rotate if rotate is None else rotate
    sm = 1.0 / math.sqrt(wl.head_dim) if sm_scale is None else sm_scale
    out = {}
    for b in (range(wl.batch) if seqs is None else seqs):
        k = filled.host["k"][b]
        v = None if wl.kv_shared else filled.host["v"][b]
        if kv_heads is None:
            out[b] = oracle.reference_decode_seq(q_host[b], k, v, filled.fmt, rotate, sm)
        else:
            g = wl.group
            res = np.full((wl.n_q, wl.num_q_heads, wl.head_dim), np.nan)
            for h in kv_heads:
                r = oracle.reference_decode_seq(q_host[b][:, h * g:(h + 1) * g], k[:, h:h + 1],
                                                None if v is None else v[:, h:h + 1],
                                                filled.fmt, rotate, sm)
                res[:, h * g:(h + 1) * g] = r
            out[b] = res
    return out


def assert_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    mask = ~np.isnan(want)
    d = np.abs(got[mask] - want[mask])
    max_abs = float(d.max()) if d.size else 0.0
    rel = float(np.linalg.norm(got[mask] - want[mask]) / max(np.linalg.norm(want[mask]), 1e-30))
    assert np.all(np.isfinite(got[mask])), "%s: non-finite output" % what
    assert max_abs <= MAX_ABS and rel <= REL_L2, \
        "%s: max_abs %.3g (<= %.1g), rel_l2 %.3g (<= %.1g)" % (what, max_abs, MAX_ABS, rel, REL_L2)
    return max_abs, rel


def oracle_decode_pairs(filled: Filled, q_host: np.ndarray, pairs, threads: int = 16,
                        sm_scale=None) -> Dict[tuple, np.ndarray]:
    """Oracle outputs {(b, kv_head): [n_q, group, d] float64} for sampled
    (sequence, KV head) pairs, computed on host threads (the oracle's C code
    runs without the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    wl = filled.wl
    g = wl.group
    rotate = filled.cache.rotate
    sm = 1.0 / math.sqrt(wl.head_dim) if sm_scale is None else sm_scale

    def one(bh):
        b, h = bh
        k = np.ascontiguousarray(filled.host["k"][b][:, h:h + 1])
        v = None if wl.kv_shared else np.ascontiguousarray(filled.host["v"][b][:, h:h + 1])
        return bh, oracle.reference_decode_seq(q_host[b][:, h * g:(h + 1) * g], k, v, filled.fmt,
                                               rotate, sm)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(one, list(pairs)))
