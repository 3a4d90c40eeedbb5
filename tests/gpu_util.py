"""Helpers of the GPU parity tests: device copies of seeded inputs, the oracle
on host copies of the same buffers, and the comparison bars.

Bars (fp32-accumulated bf16 attention against the fp64 oracle): bf16 output
max-abs <= 2e-2 and mean-abs <= 2e-3 over all compared elements; fp32 LSE
max-abs <= 1e-3.  Integer/byte work (cache contents) must match bit for bit.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
DEV = "cuda"


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def orc() -> oracle.Oracle:
    return oracle.get()


def to_dev(x):
    return None if x is None else x.to(DEV).contiguous()


def bits(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits(t)


def sink_array(sink):
    return None if sink is None else sink.detach().cpu().numpy().astype(np.float32)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, what: str):
    """Element-wise comparison against the oracle; returns (max, mean, lse_max)."""
    o = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert o.shape == out_ref.shape, (o.shape, out_ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    d = np.abs(o - out_ref)
    mx, mean = float(d.max()), float(d.mean())
    lmx = 0.0
    if lse_gpu is not None:
        l = lse_gpu.detach().cpu().numpy().astype(np.float64)
        assert np.isfinite(l).all(), f"{what}: non-finite LSE"
        lmx = float(np.abs(l - lse_ref).max())
    log(f"[parity] {what}: out max {mx:.3e} mean {mean:.3e} lse max {lmx:.3e}")
    assert mx <= OUT_MAX, f"{what}: out max-abs {mx:.3e} > {OUT_MAX}"
    assert mean <= OUT_MEAN, f"{what}: out mean-abs {mean:.3e} > {OUT_MEAN}"
    assert lmx <= LSE_MAX, f"{what}: lse max-abs {lmx:.3e} > {LSE_MAX}"
    return mx, mean, lmx


class ParityTally:
    """Element-wise comparison of a whole configuration, chunk by chunk: the
    max-abs and mean-abs bars apply to all compared elements together, so the
    chunks' sums are pooled before the mean is taken."""

    def __init__(self, what: str):
        self.what = what
        self.max = 0.0
        self.sum = 0.0
        self.count = 0
        self.lse_max = 0.0
        self.rows = 0

    def add(self, out_gpu, lse_gpu, out_ref, lse_ref, label: str = ""):
        o = out_gpu.detach().float().cpu().numpy().astype(np.float64)
        assert o.shape == out_ref.shape, (o.shape, out_ref.shape)
        assert np.isfinite(o).all(), f"{self.what} {label}: non-finite output"
        d = np.abs(o - out_ref)
        self.max = max(self.max, float(d.max()))
        self.sum += float(d.sum())
        self.count += d.size
        self.rows += o.shape[0]
        if lse_gpu is not None:
            l = lse_gpu.detach().cpu().numpy().astype(np.float64)
            assert np.isfinite(l).all(), f"{self.what} {label}: non-finite LSE"
            self.lse_max = max(self.lse_max, float(np.abs(l - lse_ref).max()))
        log(f"[parity] {self.what} {label}: chunk max {float(d.max()):.3e} mean {float(d.mean()):.3e}")

    def check(self):
        mean = self.sum / max(self.count, 1)
        log(f"[parity] {self.what}: {self.rows} rows, {self.count} elements: out max {self.max:.3e} "
            f"mean {mean:.3e} lse max {self.lse_max:.3e}")
        assert self.count > 0
        assert self.max <= OUT_MAX, f"{self.what}: out max-abs {self.max:.3e} > {OUT_MAX}"
        assert mean <= OUT_MEAN, f"{self.what}: out mean-abs {mean:.3e} > {OUT_MEAN}"
        assert self.lse_max <= LSE_MAX, f"{self.what}: lse max-abs {self.lse_max:.3e} > {LSE_MAX}"
        return self.max, mean, self.lse_max


def gpu_prefill(x, layer_type, window=129, value_scale=1.0, sink="inputs", lse=True, stream=None):
    s = x.sink if isinstance(sink, str) else sink
    dims = B.make_dims(sliding_window=window, value_scale=value_scale)
    q, k, v, cu = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens)
    out, l = B.prefill(q, k, v, cu, max(x.lengths), layer_type, sink=to_dev(s), dims=dims, want_lse=lse,
                       stream=stream)
    torch.cuda.synchronize()
    return out, l


def oracle_prefill(x, layer_type, window=129, value_scale=1.0, sink="inputs", rows=None):
    s = x.sink if isinstance(sink, str) else sink
    return orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.cpu().numpy(), layer_type=layer_type,
                         window=window, scale=float(np.float32(synth.SOFTMAX_SCALE)), value_scale=value_scale,
                         sink=sink_array(s), rows=rows)


def const_sink(value: float, hq: int = 64):
    return torch.full((hq,), value, dtype=torch.float32)
