"""Seeded synthetic inputs shaped like MiMo-V2-Flash attention workloads.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic, so both the GPU path and the fp64 oracle may use it.

Recipe (all values N(0, 1) unless stated):
  * one ``torch.Generator`` seeded with ``seed`` per call;
  * draw order: Q, K, V (fp32 ``randn``, then rounded to bf16 by ``.to``), then
    the per-head sink logits (fp32 ``randn``);
  * decode caches are drawn after that, in fixed-size chunks, on the device the
    generator lives on;
  * context lengths for the long-context decode workload are
    ``torch.randint(4096, 262145)`` and prompt lengths for the hybrid stack are
    ``round(exp(U(ln 512, ln 32768)))``, each from its own seeded generator.
Shapes follow the model config (model doc, MiMoV2FlashConfig): 64 query heads,
4 KV heads, query/key head dim 192, value head dim 128.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

HQ, HKV, DQK, DV, WINDOW = 64, 4, 192, 128, 129
SOFTMAX_SCALE = 1.0 / math.sqrt(DQK)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn_bf16(shape, gen, device, chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to bf16, generated in fixed-order chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def cu_from_lengths(lengths: Sequence[int], device="cpu") -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32, device=device)


@dataclass
class PrefillInputs:
    q: torch.Tensor          # [T][Hq][Dqk] bf16
    k: torch.Tensor          # [T][Hkv][Dqk] bf16
    v: torch.Tensor          # [T][Hkv][Dv] bf16
    sink: Optional[torch.Tensor]  # [Hq] fp32
    cu_seqlens: torch.Tensor  # [B+1] int32
    lengths: List[int]


def prefill_inputs(lengths: Sequence[int], *, seed: int = 0, device="cpu", with_sink: bool = True,
                   hq: int = HQ, hkv: int = HKV, dqk: int = DQK, dv: int = DV) -> PrefillInputs:
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    g = _gen(seed, device)
    q = _randn_bf16((T, hq, dqk), g, device)
    k = _randn_bf16((T, hkv, dqk), g, device)
    v = _randn_bf16((T, hkv, dv), g, device)
    sink = torch.randn(hq, generator=g, device=device, dtype=torch.float32) if with_sink else None
    return PrefillInputs(q, k, v, sink, cu_from_lengths(lengths, device), lengths)


@dataclass
class DecodeInputs:
    q: torch.Tensor        # [B][Hq][Dqk]
    k_new: torch.Tensor    # [B][Hkv][Dqk]
    v_new: torch.Tensor    # [B][Hkv][Dv]
    sink: Optional[torch.Tensor]
    ctx_lens: torch.Tensor  # [B] int32
    k_cache: torch.Tensor   # SWA ring [B][W-1][Hkv][Dqk] or GA pool [N][Hkv][Dqk]
    v_cache: torch.Tensor
    kv_base: Optional[torch.Tensor]      # GA [B] int64
    kv_capacity: Optional[torch.Tensor]  # GA [B] int64


def decode_inputs(ctx_lens: Sequence[int], layer_type: int, *, seed: int = 0, device="cpu",
                  with_sink: bool = True, window: int = WINDOW, headroom: int = 64,
                  hq: int = HQ, hkv: int = HKV, dqk: int = DQK, dv: int = DV) -> DecodeInputs:
    """Random queries/new tokens and a cache already holding ``ctx_lens[b]``
    random positions per sequence (layer_type 0 = SWA ring, 1 = GA pool)."""
    ctx = [int(x) for x in ctx_lens]
    B = len(ctx)
    g = _gen(seed, device)
    q = _randn_bf16((B, hq, dqk), g, device)
    k_new = _randn_bf16((B, hkv, dqk), g, device)
    v_new = _randn_bf16((B, hkv, dv), g, device)
    sink = torch.randn(hq, generator=g, device=device, dtype=torch.float32) if with_sink else None
    if layer_type == 0:
        R = window - 1
        k_cache = _randn_bf16((B, R, hkv, dqk), g, device)
        v_cache = _randn_bf16((B, R, hkv, dv), g, device)
        kv_base = kv_cap = None
    else:
        caps = [c + headroom for c in ctx]
        base = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
        N = int(sum(caps))
        k_cache = _randn_bf16((N, hkv, dqk), g, device)
        v_cache = _randn_bf16((N, hkv, dv), g, device)
        kv_base = torch.tensor(base, dtype=torch.int64, device=device)
        kv_cap = torch.tensor(caps, dtype=torch.int64, device=device)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=device)
    return DecodeInputs(q, k_new, v_new, sink, ctx_t, k_cache, v_cache, kv_base, kv_cap)


def long_context_lengths(batch: int = 128, lo: int = 4096, hi: int = 262144, seed: int = 0) -> List[int]:
    """Decode context lengths uniform in [lo, hi] (inclusive)."""
    g = _gen(seed, "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (batch,), generator=g)]


def hybrid_prompt_lengths(nseq: int = 32, lo: int = 512, hi: int = 32768, seed: int = 0) -> List[int]:
    """Prompt lengths log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi)))."""
    g = _gen(seed, "cpu")
    u = torch.rand(nseq, generator=g, dtype=torch.float64)
    return [int(round(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo))))) for x in u]


def hybrid_layer_types(num_layers: int = 48, period: int = 6) -> List[int]:
    """5 SWA layers then 1 GA layer, repeated (0 = SWA, 1 = GA)."""
    return [1 if (l % period) == period - 1 else 0 for l in range(num_layers)]


def paged_block_table(ctx_lens: Sequence[int], page_size: int, *, seed: int = 0, extra_tokens: int = 1,
                      spare_pages: int = 3, max_blocks: Optional[int] = None, device="cpu"):
    """Seeded page assignment of a paged GA pool: sequence b gets enough blocks
    for ctx_lens[b] + extra_tokens positions, on distinct pages drawn from a
    random permutation of all pages (spare_pages stay unused).  Unused table
    entries are -1.  Returns (block_table [B][max_blocks] int32, num_pages)."""
    nblk = [(int(c) + extra_tokens + page_size - 1) // page_size for c in ctx_lens]
    mb = max_blocks if max_blocks is not None else max(max(nblk), 1)
    npages = sum(nblk) + spare_pages
    perm = torch.randperm(npages, generator=_gen(seed, "cpu")).to(torch.int32)
    table = torch.full((len(nblk), mb), -1, dtype=torch.int32)
    used = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[used:used + n]
        used += n
    return table.to(device), npages


def random_e4m3_codes(shape, *, seed: int = 0, device="cpu", chunk_elems: int = 1 << 28) -> torch.Tensor:
    """Seeded uniform random OCP E4M3 codes (uint8) with the two NaN codes
    (0x7f, 0xff) replaced by their finite neighbours 0x7e, 0xfe."""
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        part = torch.randint(0, 256, (min(chunk_elems, flat.numel() - s),), generator=g, device=device,
                             dtype=torch.int32)
        part = torch.where((part & 0x7F) == 0x7F, part ^ 1, part)
        flat[s:s + part.numel()] = part.to(torch.uint8)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 view of a bf16 tensor's bit patterns."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
