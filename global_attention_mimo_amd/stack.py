"""Hybrid attention stack driver: the 5 SWA : 1 GA layer pattern over a ragged batch.

Sequences the C-ABI calls of a MiMo-V2-Flash attention stack (model doc
"MiMo-V2-Flash": Key features, 5:1 SWA/GA with a 128-token window;
MiMoV2FlashConfig, num_hidden_layers 48 and layer_types; MiMoV2FlashModel.forward,
past_key_values): a varlen prefill of every layer followed by decode steps,
each step attending and then appending one token per sequence per layer.

There are no weights, so each layer's queries, keys and values come from a
caller-supplied source (seeded synthetic tensors in tests and benchmarks) and
layers are independent.  This module owns the per-layer KV caches (a 128-slot
ring per SWA layer, a pooled region per GA layer) and the per-step context
counters; all attention arithmetic runs in the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from . import binding as B
from . import synth

SWA, GA = 0, 1


@dataclass
class LayerCache:
    layer_type: int
    k: torch.Tensor
    v: torch.Tensor
    kv_base: Optional[torch.Tensor] = None
    kv_capacity: Optional[torch.Tensor] = None


@dataclass
class HybridStack:
    lengths: Sequence[int]
    num_layers: int = 48
    period: int = 6
    decode_steps: int = 64
    device: str = "cuda"
    window: int = synth.WINDOW
    hq: int = synth.HQ
    hkv: int = synth.HKV
    fused: bool = True  # decode steps append through mimo_attn_decode_append
    # Rotary embedding of q and k (prefill: token i of a prompt at position i;
    # decode: the new token at position ctx[b]): None (inputs taken as rotated
    # already), "fused" (mimo_attn_prefill_rope, whose rotated keys are then
    # appended, and mimo_attn_decode_append_rope) or "separate" (mimo_rope_apply
    # in place, then the unfused calls).
    rope_mode: Optional[str] = None
    rope_theta: float = 5e6
    rotary_dim: int = 64
    layer_types: List[int] = field(init=False)
    caches: List[LayerCache] = field(init=False)

    def __post_init__(self):
        self.lengths = [int(x) for x in self.lengths]
        self.layer_types = synth.hybrid_layer_types(self.num_layers, self.period)
        self.batch = len(self.lengths)
        self.total = sum(self.lengths)
        self.max_len = max(self.lengths)
        self.dims = B.make_dims(num_q_heads=self.hq, num_kv_heads=self.hkv, sliding_window=self.window)
        dev = self.device
        self.cu = synth.cu_from_lengths(self.lengths, dev)
        caps = [L + self.decode_steps for L in self.lengths]
        base = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
        self.pool_rows = int(sum(caps))
        self.kv_base = torch.tensor(base, dtype=torch.int64, device=dev)
        self.kv_capacity = torch.tensor(caps, dtype=torch.int64, device=dev)
        R = self.window - 1
        self.caches = []
        for lt in self.layer_types:
            if lt == SWA:
                k = torch.zeros((self.batch, R, self.hkv, synth.DQK), dtype=torch.bfloat16, device=dev)
                v = torch.zeros((self.batch, R, self.hkv, synth.DV), dtype=torch.bfloat16, device=dev)
                self.caches.append(LayerCache(SWA, k, v))
            else:
                k = torch.zeros((self.pool_rows, self.hkv, synth.DQK), dtype=torch.bfloat16, device=dev)
                v = torch.zeros((self.pool_rows, self.hkv, synth.DV), dtype=torch.bfloat16, device=dev)
                self.caches.append(LayerCache(GA, k, v, self.kv_base, self.kv_capacity))
        # Positions already cached once every layer has been prefilled: decode step 0
        # attends at position L_b (prefill appends use zero_ctx).
        self.ctx = torch.tensor(self.lengths, dtype=torch.int32, device=dev)
        self.zero_ctx = torch.zeros(self.batch, dtype=torch.int32, device=dev)
        self.cu_step = torch.arange(self.batch + 1, dtype=torch.int32, device=dev)
        self.max_ctx = self.max_len + self.decode_steps
        self.split = 0  # the library's default GA decode chunking
        self.workspace = None
        ws = B.mimo_attn_decode_workspace_size(self.dims, GA, self.batch, self.max_ctx, self.split)
        if ws:
            self.workspace = torch.empty(ws // 4 + 4, dtype=torch.float32, device=dev)
        # Prefill positions (0 .. L-1 per prompt) and, for the fused rotation, the
        # rotated keys and the (cos, sin) table workspace, allocated on first use.
        self.positions = torch.cat([torch.arange(L, dtype=torch.int32) for L in self.lengths]).to(dev)
        self._k_rot = None
        self._rope_ws = None

    def prefill_layer(self, layer: int, q, k, v, sink, out, lse=None, stream=None):
        """Varlen prefill of one layer, then its KV append (cache positions 0..L-1);
        with rope_mode set, q and k are rotated first (fused: inside the prefill,
        whose rotated keys are what is appended; separate: in place)."""
        lt = self.layer_types[layer]
        c = self.caches[layer]
        if self.rope_mode == "fused":
            if self._k_rot is None:
                self._k_rot = torch.empty_like(k)
                n = B.mimo_attn_prefill_rope_workspace_size(self.dims, self.total, self.rotary_dim)
                self._rope_ws = torch.empty(n // 4 + 4, dtype=torch.float32, device=k.device)
            B.mimo_attn_prefill_rope(self.dims, lt, q, k, v, self.positions, self.cu, self.batch, self.max_len,
                                     self.total, self.rope_theta, self.rotary_dim, sink, out, lse, self._k_rot,
                                     self._rope_ws, stream)
            B.mimo_kv_append(self.dims, lt, self._k_rot, v, self.cu, self.zero_ctx, self.batch, self.total, c.k,
                             c.v, c.kv_base, c.kv_capacity, stream)
            return
        if self.rope_mode == "separate":
            B.mimo_rope_apply(self.dims, q, k, self.positions, self.total, self.rope_theta, self.rotary_dim, stream)
        elif self.rope_mode is not None:
            raise ValueError(f"rope_mode {self.rope_mode!r} is not None, 'fused' or 'separate'")
        B.mimo_attn_prefill(self.dims, lt, q, k, v, self.cu, self.batch, self.max_len, sink, out, lse, stream)
        B.mimo_kv_append(self.dims, lt, k, v, self.cu, self.zero_ctx, self.batch, self.total, c.k, c.v, c.kv_base,
                         c.kv_capacity, stream)

    def decode_layer(self, layer: int, q, k_new, v_new, sink, out, lse=None, stream=None):
        """One decode step of one layer: attend over the cache + new token, then append
        it (one fused library call, or decode then append when `fused` is off); with
        rope_mode set, q and k_new are rotated first (inside that call when "fused",
        in place by a separate pass when "separate")."""
        lt = self.layer_types[layer]
        c = self.caches[layer]
        ws = self.workspace if lt == GA else None
        if self.rope_mode == "fused":
            B.mimo_attn_decode_append_rope(self.dims, lt, q, k_new, v_new, self.ctx, c.k, c.v, c.kv_base,
                                           c.kv_capacity, self.ctx, self.batch, self.max_ctx, self.split,
                                           self.rope_theta, self.rotary_dim, sink, out, lse, ws, stream)
            return
        if self.rope_mode == "separate":
            B.mimo_rope_apply(self.dims, q, k_new, self.ctx, self.batch, self.rope_theta, self.rotary_dim, stream)
        elif self.rope_mode is not None:
            raise ValueError(f"rope_mode {self.rope_mode!r} is not None, 'fused' or 'separate'")
        if self.fused:
            B.mimo_attn_decode_append(self.dims, lt, q, k_new, v_new, c.k, c.v, c.kv_base, c.kv_capacity, self.ctx,
                                      self.batch, self.max_ctx, self.split, sink, out, lse, ws, stream)
            return
        B.mimo_attn_decode(self.dims, lt, q, k_new, v_new, c.k, c.v, c.kv_base, self.ctx, self.batch, self.max_ctx,
                           self.split, sink, out, lse, ws, stream)
        B.mimo_kv_append(self.dims, lt, k_new, v_new, self.cu_step, self.ctx, self.batch, self.batch, c.k, c.v,
                         c.kv_base, c.kv_capacity, stream)

    def advance(self):
        """All layers of a decode step are done: every sequence is one token longer."""
        self.ctx.add_(1)

    def decode_step(self, q, k_new, v_new, sinks, out, lse=None, stream=None):
        """One decode step of every layer (inputs and outputs indexed by layer first),
        then the context advance, all on one stream."""
        for layer in range(self.num_layers):
            self.decode_layer(layer, q[layer], k_new[layer], v_new[layer], sinks[layer], out[layer],
                              None if lse is None else lse[layer], stream)
        self.advance()

    def capture_decode_step(self, q, k_new, v_new, sinks, out, lse=None) -> torch.cuda.CUDAGraph:
        """A HIP graph of `decode_step` over these buffers.  Each replay runs one step
        at the contexts the device holds then (they live in device memory, as do the
        cache positions the appends write) and advances them; replays read whatever
        q / k_new / v_new hold at that time.  The library only launches kernels on
        the stream it is given (no allocation, memset or synchronisation), so the
        step is captured as it is; the context advance is a torch kernel."""
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            self.decode_step(q, k_new, v_new, sinks, out, lse)
        return graph

    def kv_bytes(self) -> dict:
        """KV-cache bytes actually allocated, and what an all-GA stack would need."""
        per_tok = self.hkv * (synth.DQK + synth.DV) * 2
        ga_rows = sum(1 for t in self.layer_types if t == GA) * self.pool_rows
        swa_rows = sum(1 for t in self.layer_types if t == SWA) * self.batch * (self.window - 1)
        return {"hybrid": (ga_rows + swa_rows) * per_tok, "all_ga": self.num_layers * self.pool_rows * per_tok}
