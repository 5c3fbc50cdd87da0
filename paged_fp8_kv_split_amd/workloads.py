"""Seeded synthetic inputs for split-KV verify attention (no attention arithmetic here).

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic, so both the HIP path's tests/benchmark and the CPU oracle
can take their inputs from it.

Shapes follow the microbenchmark setups of aiter PR #5190 ("gfx950 assembly
MTP-verify attention for head_dim 256 fp8 paged KV"), sections Microbenchmark
and Bandwidth sweep, and SGLang PR #37465, section Kernel microbenchmarks:
head_dim 256, page 16 NHD, fp8 e4m3 K/V with per-tensor descales, bf16 Q,
4 query tokens per sequence (1..4 for draft extend / decode), 16 or 8 query
heads per KV head, randomly permuted page tables, rotating replicas for cold L2.

Recipe: Q ~ N(0, 1) rounded to bf16. K and V ~ N(0, 1) in fp32 per tensor,
quantized to e4m3fn with per-tensor scale amax / 448 (aiter PR #7375,
Performance), clamped to +-448 first because torch's cast turns larger values
into NaN. Each sequence's pages are a disjoint slice of a seeded random
permutation of a pool twice the size needed; unused block-table slots point at
a poison page whose bytes are all 0x7F (e4m3fn NaN), which no correct reader
ever touches.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np
import torch

FP8_MAX = 448.0
POISON_BYTE = 0x7F


@dataclass(frozen=True)
class Workload:
    """One verify-attention problem shape (all sequences share the head layout)."""

    name: str
    ctx: Tuple[int, ...]          # KV length of each sequence (includes its query tokens)
    q_lens: Tuple[int, ...]       # query tokens of each sequence, 1..4
    num_q_heads: int
    num_kv_heads: int
    num_segments: Optional[int]   # None: the library's heuristic chooses
    seed: int
    head_dim: int = 256
    page_size: int = 16
    replicas: int = 1             # independent copies rotated for cold-L2 timing
    descale: str = "amax"         # "amax" | "fixed" (scales 0.5 / 2.0) | "override"
    softmax_scale: float = 1.0 / 16.0
    pool_factor: int = 2

    @property
    def num_seqs(self) -> int:
        return len(self.ctx)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def pages_per_seq(self):
        return [-(-c // self.page_size) for c in self.ctx]

    @property
    def kv_bytes(self) -> int:
        """KV bytes one call must read: sum_b L_b * Hkv * D * 2 (K and V, 1 byte each)."""
        return int(sum(self.ctx)) * self.num_kv_heads * self.head_dim * 2


def _uniform(name, n, ctx, q_len, hq, hkv, segs, seed, replicas=1, **kw) -> Workload:
    return Workload(name=name, ctx=(ctx,) * n, q_lens=(q_len,) * n, num_q_heads=hq,
                    num_kv_heads=hkv, num_segments=segs, seed=seed, replicas=replicas, **kw)


def _ragged(seed: int) -> Workload:
    """8 sequences, contexts log-uniform in [6, 105000], q_len uniform in {1..4}."""
    rng = np.random.default_rng(seed)
    q_lens = tuple(int(x) for x in rng.integers(1, 5, size=8))
    ctx = tuple(max(int(round(math.exp(rng.uniform(math.log(6), math.log(105000))))), q)
                for q in q_lens)
    return Workload(name="ragged", ctx=ctx, q_lens=q_lens, num_q_heads=16, num_kv_heads=1,
                    num_segments=None, seed=seed, replicas=16)


WORKLOADS = {
    # tiny verify: 2 x 1000, GQA 16, 4 segments (two descale passes + an extra reading)
    "tiny": _uniform("tiny", 2, 1000, 4, 16, 1, 4, seed=1),
    "tiny_fixed_descale": _uniform("tiny_fixed_descale", 2, 1000, 4, 16, 1, 4, seed=1, descale="fixed"),
    "tiny_override_descale": _uniform("tiny_override_descale", 2, 1000, 4, 16, 1, 4, seed=1,
                                      descale="override"),
    # production verify: 16 x 35000, GQA 16, 16 segments
    "prod": _uniform("prod", 16, 35000, 4, 16, 1, 16, seed=2, replicas=16),
    # the production shape over one-token pages (every key row at a random slot)
    "prod_page1": _uniform("prod_page1", 16, 35000, 4, 16, 1, 16, seed=2, replicas=16, page_size=1),
    # the production shape at head_dim 128 (softmax scale 1 / sqrt(128))
    "prod_hd128": _uniform("prod_hd128", 16, 35000, 4, 16, 1, 16, seed=6, replicas=16, head_dim=128,
                           softmax_scale=1.0 / math.sqrt(128.0)),
    # GQA 8
    "gqa8": _uniform("gqa8", 16, 35000, 4, 8, 1, 16, seed=3, replicas=16),
    # long context and occupancy pair
    "long": _uniform("long", 16, 70000, 4, 16, 1, 16, seed=4, replicas=16),
    "occupancy": _uniform("occupancy", 4, 35000, 4, 16, 1, 64, seed=44, replicas=16),
    # decode: the production shape with one query token per sequence
    "decode": _uniform("decode", 16, 35000, 1, 16, 1, 16, seed=7, replicas=16),
    # ragged draft-extend / decode and the multi-head-group pass
    "ragged": _ragged(5),
    "multigroup": _uniform("multigroup", 2, 777, 4, 32, 2, None, seed=5),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


@dataclass
class Case:
    """Device- or host-resident inputs of one call (torch tensors)."""

    q: torch.Tensor              # bf16 [T, Hq, D]
    k_cache: torch.Tensor        # uint8 e4m3fn codes [num_pages, page, Hkv, D]
    v_cache: torch.Tensor        # uint8 e4m3fn codes [num_pages, page, Hkv, D]
    block_tables: torch.Tensor   # int32 [N, max_pages]
    seq_lens: torch.Tensor       # int32 [N]
    cu_seqlens_q: torch.Tensor   # int32 [N + 1]
    k_descale: torch.Tensor      # float32 [1]
    v_descale: torch.Tensor      # float32 [1]
    softmax_scale: float
    poison_page: int
    workload: Workload = field(repr=False)

    def to(self, device) -> "Case":
        mv = lambda t: t.to(device)
        return Case(mv(self.q), mv(self.k_cache), mv(self.v_cache), mv(self.block_tables),
                    mv(self.seq_lens), mv(self.cu_seqlens_q), mv(self.k_descale),
                    mv(self.v_descale), self.softmax_scale, self.poison_page, self.workload)

    def host_arrays(self):
        """numpy copies in the form the CPU oracle takes (bf16 Q as uint16 bits)."""
        return dict(
            q=self.q.detach().cpu().view(torch.int16).numpy().view(np.uint16),
            k_cache=self.k_cache.detach().cpu().numpy(),
            v_cache=self.v_cache.detach().cpu().numpy(),
            block_tables=self.block_tables.detach().cpu().numpy(),
            seq_lens=self.seq_lens.detach().cpu().numpy(),
            cu_seqlens_q=self.cu_seqlens_q.detach().cpu().numpy(),
            k_descale=float(self.k_descale.item()),
            v_descale=float(self.v_descale.item()),
            softmax_scale=self.softmax_scale,
        )


def _quantize(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Round x / scale to e4m3fn (after clamping to +-448) and return the codes."""
    y = torch.clamp(x / scale, -FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _fill_cache(shape, gen, device, mode, fixed_scale):
    vals = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    amax_scale = float(vals.abs().max().item()) / FP8_MAX
    if mode == "fixed":
        return _quantize(vals, fixed_scale), fixed_scale
    codes = _quantize(vals, amax_scale)
    return codes, (fixed_scale if mode == "override" else amax_scale)


def make_case(w: Workload, device="cpu", replica: int = 0) -> Case:
    """Draw one seeded replica of workload ``w`` directly on ``device``."""
    device = torch.device(device)
    seed = w.seed * 1000 + replica
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    pages = w.pages_per_seq()
    need = int(sum(pages))
    max_pages = max(max(pages), 1)
    pool = w.pool_factor * need + 1          # the last page is the poison page
    poison = pool - 1
    perm = rng.permutation(pool - 1)[:need].astype(np.int32)
    tables = np.full((w.num_seqs, max_pages), poison, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages):
        tables[b, :p] = perm[off:off + p]
        off += p

    shape = (pool - 1, w.page_size, w.num_kv_heads, w.head_dim)
    k_codes, kd = _fill_cache(shape, gen, device, w.descale, 0.5)
    v_codes, vd = _fill_cache(shape, gen, device, w.descale, 2.0)
    poison_block = torch.full((1,) + shape[1:], POISON_BYTE, dtype=torch.uint8, device=device)
    k_cache = torch.cat([k_codes, poison_block], 0)
    v_cache = torch.cat([v_codes, poison_block], 0)

    q = torch.randn((w.total_q, w.num_q_heads, w.head_dim), generator=gen, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    cu = np.zeros(w.num_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(w.q_lens)
    return Case(
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=torch.from_numpy(tables).to(device),
        seq_lens=torch.tensor(w.ctx, dtype=torch.int32, device=device),
        cu_seqlens_q=torch.from_numpy(cu).to(device),
        k_descale=torch.tensor([kd], dtype=torch.float32, device=device),
        v_descale=torch.tensor([vd], dtype=torch.float32, device=device),
        softmax_scale=float(w.softmax_scale),
        poison_page=int(poison),
        workload=w,
    )


def permute_pool(case: Case, seed: int) -> Case:
    """Same problem with the page pool shuffled and the block tables remapped.

    Page ``p`` of the new pool holds what page ``inv[p]`` held; every table entry
    is rewritten accordingly, so each sequence still sees the same bytes.
    """
    n = case.k_cache.shape[0]
    g = np.random.default_rng(seed)
    new_of_old = g.permutation(n)
    old_of_new = np.argsort(new_of_old)
    dev = case.k_cache.device
    idx = torch.from_numpy(old_of_new).to(dev)
    remap = torch.from_numpy(new_of_old.astype(np.int32)).to(dev)
    tables = remap[case.block_tables.long()].to(torch.int32)
    return Case(case.q, case.k_cache[idx].contiguous(), case.v_cache[idx].contiguous(), tables,
                case.seq_lens, case.cu_seqlens_q, case.k_descale, case.v_descale,
                case.softmax_scale, int(new_of_old[case.poison_page]), case.workload)


# ---------------------------------------------------------------- prefill
# Synthetic inputs of the second workload (fp8 varlen prefill, aiter PR #7375,
# Performance): bf16-distributed data quantized per tensor to e4m3 with scale
# amax / 448, packed THD rows, qk head dim 192 and v head dim 128.
@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    lens: tuple                  # ((Lq, Lk), ...) per sequence
    num_q_heads: int
    num_kv_heads: int
    causal: bool
    seed: int
    head_dim_qk: int = 192
    head_dim_v: int = 128

    @property
    def num_seqs(self) -> int:
        return len(self.lens)

    @property
    def total_q(self) -> int:
        return int(sum(a for a, _ in self.lens))

    @property
    def total_k(self) -> int:
        return int(sum(b for _, b in self.lens))

    @property
    def max_seqlen_q(self) -> int:
        return max(max(a for a, _ in self.lens), 1)

    @property
    def flops(self) -> int:
        """Both products over the visible (query, key) pairs: 2 (Dqk + Dv) per pair and head."""
        pairs = 0
        for lq, lk in self.lens:
            if self.causal:
                pairs += sum(max(0, min(lk, lk - lq + i + 1)) for i in range(lq))
            else:
                pairs += lq * lk
        return 2 * (self.head_dim_qk + self.head_dim_v) * pairs * self.num_q_heads


PREFILL_WORKLOADS = {
    # the pages' target shape: one sequence of 12288 queries over 14336 keys, 96 heads
    "prefill_12k": PrefillWorkload("prefill_12k", ((12288, 14336),), 96, 96, False, seed=7),
    "prefill_12k_causal": PrefillWorkload("prefill_12k_causal", ((12288, 14336),), 96, 96, True, seed=8),
    # small varlen parity batch: GQA 4, ragged lengths, fewer keys than queries, empty KV
    "prefill_small": PrefillWorkload("prefill_small", ((300, 300), (129, 517), (64, 40), (17, 0), (1, 77)), 8, 2,
                                     True, seed=9),
}


def prefill_workload(name: str, **overrides) -> PrefillWorkload:
    w = PREFILL_WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


@dataclass
class PrefillCase:
    """Inputs of one prefill call (torch tensors; q/k/v are e4m3fn codes as uint8)."""

    q: torch.Tensor              # [total_q, Hq, 192]
    k: torch.Tensor              # [total_k, Hkv, 192]
    v: torch.Tensor              # [total_k, Hkv, 128]
    cu_seqlens_q: torch.Tensor   # int32 [B + 1]
    cu_seqlens_k: torch.Tensor   # int32 [B + 1]
    q_descale: torch.Tensor      # float32 [1]
    k_descale: torch.Tensor
    v_descale: torch.Tensor
    max_seqlen_q: int
    causal: bool
    workload: PrefillWorkload = field(repr=False)

    def to(self, device) -> "PrefillCase":
        mv = lambda t: t.to(device)
        return PrefillCase(mv(self.q), mv(self.k), mv(self.v), mv(self.cu_seqlens_q), mv(self.cu_seqlens_k),
                           mv(self.q_descale), mv(self.k_descale), mv(self.v_descale), self.max_seqlen_q,
                           self.causal, self.workload)

    def host_arrays(self):
        """numpy inputs in the oracle's argument names."""
        return dict(q=self.q.cpu().numpy(), k=self.k.cpu().numpy(), v=self.v.cpu().numpy(),
                    cu_seqlens_q=self.cu_seqlens_q.cpu().numpy(), cu_seqlens_k=self.cu_seqlens_k.cpu().numpy(),
                    q_descale=float(self.q_descale.item()), k_descale=float(self.k_descale.item()),
                    v_descale=float(self.v_descale.item()), softmax_scale=None, causal=self.causal)


def make_prefill_case(w: PrefillWorkload, device="cpu") -> PrefillCase:
    """Draw workload ``w`` (seeded) directly on ``device``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)

    def quantized(shape):
        vals = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16).float()
        scale = float(vals.abs().max().item()) / FP8_MAX
        return _quantize(vals, scale), scale

    q, qd = quantized((w.total_q, w.num_q_heads, w.head_dim_qk))
    k, kd = quantized((w.total_k, w.num_kv_heads, w.head_dim_qk))
    v, vd = quantized((w.total_k, w.num_kv_heads, w.head_dim_v))
    cq = np.zeros(w.num_seqs + 1, dtype=np.int32)
    ck = np.zeros(w.num_seqs + 1, dtype=np.int32)
    cq[1:] = np.cumsum([a for a, _ in w.lens])
    ck[1:] = np.cumsum([b for _, b in w.lens])
    f32 = lambda x: torch.tensor([x], dtype=torch.float32, device=device)
    return PrefillCase(q, k, v, torch.from_numpy(cq).to(device), torch.from_numpy(ck).to(device), f32(qd), f32(kd),
                       f32(vd), w.max_seqlen_q, w.causal, w)
