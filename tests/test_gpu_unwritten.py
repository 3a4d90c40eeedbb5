"""Cache memory a decode must not read holds NaN and Inf.

A caller's cache is only defined at the positions already appended: SWA ring
slots j < p while the ring is filling (p < W-1), GA pool rows kv_base[b] + j
for j < p.  Here every other slot and row of the cache is filled with NaN and
Inf bit patterns.  A kernel that read them, even with zero weight (0 x NaN),
would turn the output into NaN; the results must instead match the oracle,
which reads positions below p only.
"""
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import compare, log, to_dev
from test_gpu_decode import gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
NAN, INF = 0x7FC0, 0x7F80  # bf16 bit patterns (as int16: both positive)


def _poison(x, layer_type, ctx, window=129):
    """NaN into unwritten K rows, Inf into unwritten V rows."""
    k, v = x.k_cache.view(torch.int16), x.v_cache.view(torch.int16)
    if layer_type == SWA:
        R = window - 1
        for b, p in enumerate(ctx):
            if p < R:
                k[b, p:] = NAN
                v[b, p:] = INF
    else:
        base, cap = x.kv_base.tolist(), x.kv_capacity.tolist()
        for b, p in enumerate(ctx):
            k[base[b] + p:base[b] + cap[b]] = NAN
            v[base[b] + p:base[b] + cap[b]] = INF


@pytest.mark.parametrize("layer_type,ctx,split", [
    (SWA, [0, 1, 5, 100, 127], 0),
    (GA, [0, 1, 63, 300, 4096], 0),
    (GA, [0, 1, 63, 300, 4096], 64),
])
def test_decode_ignores_unwritten_cache(layer_type, ctx, split):
    log(f"[case] unwritten cache layer={layer_type} ctx={ctx} split={split}")
    x = synth.decode_inputs(ctx, layer_type, seed=41)
    _poison(x, layer_type, ctx)
    out, lse = gpu_decode(x, layer_type, split=split)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ro, rl = oracle_decode(x, layer_type)
    compare(out, lse, ro, rl, f"unwritten cache, layer {layer_type}")


@pytest.mark.parametrize("layer_type,ctx", [(SWA, [0, 3, 126, 127]), (GA, [0, 2, 70, 1000])])
def test_decode_append_ignores_unwritten_cache(layer_type, ctx):
    log(f"[case] unwritten cache, fused append, layer={layer_type} ctx={ctx}")
    x = synth.decode_inputs(ctx, layer_type, seed=43)
    _poison(x, layer_type, ctx)
    ro, rl = oracle_decode(x, layer_type)
    dims = B.make_dims()
    bsz = len(ctx)
    d = {name: to_dev(getattr(x, name)) for name in ("q", "k_new", "v_new", "k_cache", "v_cache", "ctx_lens", "sink",
                                                     "kv_base", "kv_capacity")}
    ws = None
    nbytes = B.mimo_attn_decode_workspace_size(dims, layer_type, bsz, max(ctx), 0)
    if nbytes:
        ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty((bsz, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((bsz, 64), dtype=torch.float32, device="cuda")
    B.mimo_attn_decode_append(dims, layer_type, d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                              d["kv_base"], d["kv_capacity"], d["ctx_lens"], bsz, max(ctx), 0, d["sink"], out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    compare(out, lse, ro, rl, f"unwritten cache with append, layer {layer_type}")
    # the new token landed at position p
    kc = d["k_cache"].cpu()
    for b, p in enumerate(ctx):
        row = kc[b, p % 128] if layer_type == SWA else kc[int(x.kv_base[b]) + p]
        assert torch.equal(row, x.k_new[b])


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_chunk_prefill_ignores_unwritten_cache(layer_type):
    """Chunked prefill reads cached positions below ctx_lens[b] only: the rest of
    the ring (while it fills) and of the pool, padding rows included, is NaN/Inf
    in both the GPU caches and the oracle's host copies."""
    import numpy as np
    from test_gpu_chunk import SCALE, _caches, _chunk, _fill
    from gpu_util import bits, orc, sink_array
    lengths = [300, 170, 64, 260]
    cached = [0, 1, 63, 131]
    log(f"[case] unwritten cache, chunked prefill layer={layer_type} cached={cached}")
    x = synth.prefill_inputs(lengths, seed=44)
    kc, vc, base, cap = _caches(layer_type, lengths)
    kh, vh = _fill(x, layer_type, cached, kc, vc, base, cap)
    kd, vd = kc.view(torch.int16), vc.view(torch.int16)
    kh16, vh16 = kh.view(np.int16), vh.view(np.int16)
    if layer_type == SWA:
        spans = [(b, c, 128) for b, c in enumerate(cached) if c < 128]
        for b, lo, hi in spans:
            kd[b, lo:hi] = NAN
            vd[b, lo:hi] = INF
            kh16[b, lo:hi] = NAN
            vh16[b, lo:hi] = INF
    else:
        bl, cl = base.tolist(), cap.tolist()
        spans = [(0, bl[0])] + [(bl[b] + c, bl[b] + cl[b]) for b, c in enumerate(cached)]
        for lo, hi in spans:
            kd[lo:hi] = NAN
            vd[lo:hi] = INF
            kh16[lo:hi] = NAN
            vh16[lo:hi] = INF
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), kh) and np.array_equal(bits(vc), vh)
    out, lse, new, rest, cu_new, ctx = _chunk(x, layer_type, cached, kc, vc, base)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ro, rl = orc().prefill_chunk(bits(x.q[new]), bits(x.k[new]), bits(x.v[new]), cu_new.cpu().numpy(), kh, vh,
                                 ctx.cpu().numpy(), layer_type=layer_type, window=129, scale=SCALE,
                                 sink=sink_array(x.sink), kv_base=None if base is None else base.cpu().numpy())
    compare(out, lse, ro, rl, f"unwritten cache, chunked prefill layer {layer_type}")
