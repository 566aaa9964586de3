"""Seeded synthetic workloads for decode attention over a paged KV cache.

This module only draws inputs: bf16 queries, keys and values with outlier
channels, per-sequence context lengths, shared-prefix page plans, block tables
and slot mappings.  It contains none of the method's arithmetic (no rotation,
no quantisation, no attention), so both the HIP library's tests and the CPU
oracle can take their inputs from it without sharing code with each other.

Every tensor is drawn from its own ``torch.Generator`` whose seed is derived
from (base seed, workload name, tensor name, index), so one sequence or one
prefix can be regenerated alone.  Values are fp32 N(0, std^2), a few channels
per KV head multiplied by a large factor, rounded to bf16 (round to nearest
even).  The same outlier channels are used in K, V and the query heads that
read that KV head.

The shapes stand in for the serving workload of the ROCm blog "UltraQuant on
AMD Instinct" (long agent prompts with shared prefixes and 91-95% prefix-cache
hits, MTP verify with three query positions): no trace or dataset is used.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    page_size: int
    context: int                      # fixed context length (ignored if ctx_range)
    n_q: int = 1                      # query positions per sequence
    kv_shared: bool = False           # K == V (latent cache)
    std: float = 1.0
    n_outliers: int = 2               # outlier channels per KV head
    outlier_mult: float = 20.0
    permute_pages: bool = True
    ctx_range: Optional[Tuple[int, int]] = None   # log-uniform contexts
    n_prefixes: int = 0               # shared prefixes (0: none)
    shared_frac: float = 0.0          # fraction of a sequence's pages shared
    append_tokens: int = 0            # tokens appended by the decode step
    seed: int = 0
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_b1_l256", batch=1, num_kv_heads=1, num_q_heads=4,
                 head_dim=128, page_size=16, context=256, permute_pages=False,
                 description="batch 1, 1 KV / 4 Q heads, d128, context 256, "
                             "page 16, 2 outlier channels x20"),
        Workload("b8_l8k", batch=8, num_kv_heads=8, num_q_heads=64,
                 head_dim=128, page_size=16, context=8192,
                 description="batch 8, 8 KV / 64 Q heads, d128, context 8192, "
                             "page 16, permuted block tables"),
        Workload("b32_l32k", batch=32, num_kv_heads=8, num_q_heads=64,
                 head_dim=128, page_size=16, context=32768, append_tokens=1,
                 description="batch 32, 8 KV / 64 Q heads, d128, context "
                             "32768, page 16, append 1 token then decode"),
        Workload("mtp_mixed_b32", batch=32, num_kv_heads=8, num_q_heads=64,
                 head_dim=128, page_size=16, context=0, n_q=3,
                 ctx_range=(4096, 131072), n_prefixes=4, shared_frac=0.92,
                 description="batch 32 agentic mix, contexts log-uniform "
                             "4K-128K, 92% of pages from 4 shared prefixes, "
                             "3 MTP verify positions with causal mask"),
        Workload("fork_b32_l32k", batch=32, num_kv_heads=8, num_q_heads=64,
                 head_dim=128, page_size=16, context=32768, n_q=3,
                 n_prefixes=1, shared_frac=0.9375,
                 description="batch 32 forked from one prefix: context 32768, "
                             "the first 30720 tokens shared by every sequence, "
                             "3 MTP verify positions with causal mask"),
        Workload("mla_b16_l128k", batch=16, num_kv_heads=1, num_q_heads=64,
                 head_dim=512, page_size=64, context=131072, kv_shared=True,
                 std=math.sqrt(0.5), n_outliers=4, outlier_mult=16.0,
                 description="latent cache width 512 (K=V), 64 absorbed "
                             "query heads, batch 16, context 131072, page 64"),
    ]
}


def derive_seed(wl: Workload, tensor: str, index: int = 0) -> int:
    key = "%d/%s/%s/%d" % (wl.seed, wl.name, tensor, index)
    return zlib.crc32(key.encode()) & 0x7FFFFFFF


def _gen(wl: Workload, tensor: str, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(wl, tensor, index))
    return g


# ------------------------------------------------------------ structure

def context_lens(wl: Workload) -> np.ndarray:
    """Tokens in the cache per sequence at decode time (appended tokens and
    MTP verify tokens included)."""
    if wl.ctx_range is None:
        return np.full(wl.batch, wl.context, dtype=np.int32)
    g = _gen(wl, "ctx", 0, "cpu")
    lo, hi = wl.ctx_range
    u = torch.rand(wl.batch, generator=g, dtype=torch.float64).numpy()
    L = np.rint(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return np.clip(L, lo, hi).astype(np.int32)


def outlier_channels(wl: Workload) -> np.ndarray:
    """[num_kv_heads, n_outliers] channel indices (distinct within a head)."""
    g = _gen(wl, "outliers", 0, "cpu")
    rows = [torch.randperm(wl.head_dim, generator=g)[: wl.n_outliers].numpy()
            for _ in range(wl.num_kv_heads)]
    return np.stack(rows).astype(np.int64)


@dataclass
class PagePlan:
    """Where every token of every sequence lives in the paged cache."""
    num_pages: int
    block_tables: np.ndarray            # int32 [batch, max_pages]
    context_lens: np.ndarray            # int32 [batch]
    # Pages each sequence owns (physical ids, logical order) and, for shared
    # prefixes, which prefix and how many of its pages a sequence starts with.
    private_pages: List[np.ndarray]
    prefix_of: List[int]                # -1: no shared prefix
    n_shared_pages: List[int]
    prefix_pages: List[np.ndarray]      # physical ids of each prefix's pages

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])


def page_plan(wl: Workload, lens: Optional[List[int]] = None,
              shared_pages: Optional[List[int]] = None) -> PagePlan:
    """The workload's page plan; ``lens`` and ``shared_pages`` (whole pages
    sequence b takes from prefix b mod n_prefixes) override the drawn context
    lengths and the shared fraction, for edge cases."""
    P = wl.page_size
    L = context_lens(wl) if lens is None else np.asarray(lens, dtype=np.int32)
    n_pages = [(int(l) + P - 1) // P for l in L]
    prefix_of = [-1] * wl.batch
    n_shared = [0] * wl.batch
    prefix_need = [0] * wl.n_prefixes
    if wl.n_prefixes:
        for b in range(wl.batch):
            p = b % wl.n_prefixes
            prefix_of[b] = p
            if shared_pages is None:
                n_shared[b] = int(math.floor(wl.shared_frac * n_pages[b]))
            else:
                n_shared[b] = min(int(shared_pages[b]), int(L[b]) // P)
            prefix_need[p] = max(prefix_need[p], n_shared[b])
    total = sum(prefix_need) + sum(n_pages[b] - n_shared[b] for b in range(wl.batch))
    if wl.permute_pages:
        g = _gen(wl, "pages", 0, "cpu")
        phys = torch.randperm(total, generator=g).numpy().astype(np.int32)
    else:
        phys = np.arange(total, dtype=np.int32)
    cur = 0
    prefix_pages = []
    for p in range(wl.n_prefixes):
        prefix_pages.append(phys[cur: cur + prefix_need[p]])
        cur += prefix_need[p]
    private = []
    maxp = max(n_pages) if n_pages else 0
    bt = np.zeros((wl.batch, max(maxp, 1)), dtype=np.int32)
    for b in range(wl.batch):
        own = phys[cur: cur + n_pages[b] - n_shared[b]]
        cur += n_pages[b] - n_shared[b]
        private.append(own)
        row = []
        if prefix_of[b] >= 0:
            row.extend(prefix_pages[prefix_of[b]][: n_shared[b]].tolist())
        row.extend(own.tolist())
        bt[b, : len(row)] = row
    return PagePlan(num_pages=total, block_tables=bt, context_lens=L,
                    private_pages=private, prefix_of=prefix_of,
                    n_shared_pages=n_shared, prefix_pages=prefix_pages)


def slots_for(pages: np.ndarray, n_tokens: int, page_size: int,
              first_token: int = 0) -> np.ndarray:
    """Slot ids (page * page_size + offset) of tokens first_token ..
    first_token + n_tokens - 1 of a run of pages."""
    t = np.arange(first_token, first_token + n_tokens, dtype=np.int64)
    return (pages[t // page_size].astype(np.int64) * page_size
            + t % page_size).astype(np.int32)


# ------------------------------------------------------------ values

def _draw(wl: Workload, shape, tensor: str, index: int, heads_axis: int,
          head_of, device) -> torch.Tensor:
    """fp32 N(0, std^2) of ``shape`` with the outlier channels of each KV head
    multiplied, rounded to bf16.  ``head_of[i]`` maps index i along
    ``heads_axis`` to its KV head."""
    g = _gen(wl, tensor, index, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if wl.std != 1.0:
        x = x * wl.std
    if wl.n_outliers:
        oc = outlier_channels(wl)
        mult = torch.ones(shape[heads_axis], wl.head_dim, device=device)
        for i in range(shape[heads_axis]):
            mult[i, torch.as_tensor(oc[head_of[i]], device=device)] = wl.outlier_mult
        view = [1] * len(shape)
        view[heads_axis] = shape[heads_axis]
        view[-1] = wl.head_dim
        x = x * mult.view(view)
    return x.to(torch.bfloat16)


def prefix_tokens(wl: Workload, tensor: str, prefix: int, n_tokens: int,
                  device="cpu") -> torch.Tensor:
    """bf16 [n_tokens, num_kv_heads, head_dim] of shared prefix ``prefix``."""
    return _draw(wl, (n_tokens, wl.num_kv_heads, wl.head_dim),
                 tensor + "/prefix", prefix, 1, list(range(wl.num_kv_heads)), device)


def private_tokens(wl: Workload, tensor: str, seq: int, n_tokens: int,
                   device="cpu") -> torch.Tensor:
    """bf16 [n_tokens, num_kv_heads, head_dim]: a sequence's own tokens."""
    return _draw(wl, (n_tokens, wl.num_kv_heads, wl.head_dim),
                 tensor + "/seq", seq, 1, list(range(wl.num_kv_heads)), device)


def sequence_kv(wl: Workload, plan: PagePlan, tensor: str, seq: int,
                device="cpu") -> torch.Tensor:
    """The whole logical sequence [L_b, num_kv_heads, head_dim] in bf16:
    shared-prefix tokens first (if any), then the sequence's own tokens."""
    L = int(plan.context_lens[seq])
    n_sh = plan.n_shared_pages[seq] * wl.page_size
    parts = []
    if n_sh:
        parts.append(full_prefix(wl, plan, tensor, plan.prefix_of[seq], device)[:n_sh])
    parts.append(private_tokens(wl, tensor, seq, L - n_sh, device))
    return torch.cat(parts, 0) if len(parts) > 1 else parts[0]


def full_prefix(wl: Workload, plan: PagePlan, tensor: str, prefix: int,
                device="cpu") -> torch.Tensor:
    """All tokens of shared prefix ``prefix`` (always drawn at full length,
    so every sequence that shares it sees the same values)."""
    full = len(plan.prefix_pages[prefix]) * wl.page_size
    return prefix_tokens(wl, tensor, prefix, full, device)


def queries(wl: Workload, device="cpu") -> torch.Tensor:
    """bf16 [batch, n_q, num_q_heads, head_dim]."""
    g = wl.group
    return _draw(wl, (wl.batch, wl.n_q, wl.num_q_heads, wl.head_dim), "q", 0, 2,
                 [h // g for h in range(wl.num_q_heads)], device)


def selected_positions(wl: Workload, plan: PagePlan, seq: int, n_groups: int = 512,
                       group: int = 4, recent: int = 3) -> np.ndarray:
    """Synthetic selection for one sequence, in the shape an index cache
    returns: up to ``n_groups`` distinct pooled groups of ``group``
    consecutive history tokens (in a random order, as a top-k list comes)
    plus the last ``recent`` tokens.  int32 token positions."""
    L = int(plan.context_lens[seq])
    rec = min(recent, L)
    n_hist = (L - rec) // group
    g = _gen(wl, "select", seq, "cpu")
    pick = torch.randperm(n_hist, generator=g)[: min(n_groups, n_hist)].numpy()
    pos = (pick[:, None] * group + np.arange(group)[None, :]).reshape(-1)
    return np.concatenate([pos, np.arange(L - rec, L)]).astype(np.int32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def tensor_names(wl: Workload) -> List[str]:
    return ["k"] if wl.kv_shared else ["k", "v"]
