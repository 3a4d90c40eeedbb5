"""Decode and KV append through the C ABI on the GPU against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, const_sink, gpu_prefill, log, orc, oracle_prefill, sink_array, to_dev

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))


def gpu_decode(x, layer_type, max_ctx=None, split=0, sink="inputs", value_scale=1.0, window=129):
    s = x.sink if isinstance(sink, str) else sink
    mc = int(x.ctx_lens.max()) if max_ctx is None else max_ctx
    dims = B.make_dims(value_scale=value_scale, sliding_window=window)
    out, lse = B.decode(to_dev(x.q), to_dev(x.k_new), to_dev(x.v_new), to_dev(x.k_cache), to_dev(x.v_cache),
                        to_dev(x.ctx_lens), mc, layer_type, sink=to_dev(s), kv_base=to_dev(x.kv_base),
                        split_tokens=split, dims=dims)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(x, layer_type, sink="inputs", value_scale=1.0, window=129):
    s = x.sink if isinstance(sink, str) else sink
    return orc().decode(bits(x.q), bits(x.k_new), bits(x.v_new), bits(x.k_cache), bits(x.v_cache),
                        x.ctx_lens.cpu().numpy(), layer_type=layer_type, window=window, scale=SCALE,
                        value_scale=value_scale,
                        sink=sink_array(s), kv_base=None if x.kv_base is None else x.kv_base.cpu().numpy())


CTX = [0, 1, 127, 128, 129, 4096, 300, 5]


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_decode_context_sweep(layer_type):
    log(f"[case] decode sweep layer={layer_type}")
    x = synth.decode_inputs(CTX, layer_type, seed=20)
    out, lse = gpu_decode(x, layer_type)
    ro, rl = oracle_decode(x, layer_type)
    compare(out, lse, ro, rl, f"decode layer {layer_type}")


@pytest.mark.parametrize("window", [2, 33, 97, 225, 226, 257, 258, 300])
def test_swa_decode_ring_sizes(window):
    """Rings of window-1 slots: 1 slot, partial tiles, the two-tile limit (256
    slots: windows 257 and 258 fall on either side of it) and rings long enough
    that waves loop over several tiles."""
    log(f"[case] SWA decode window={window}")
    x = synth.decode_inputs([0, 1, window - 2, window - 1, window, 3 * window + 5, 1000], SWA, seed=29, window=window)
    out, lse = gpu_decode(x, SWA, window=window)
    ro, rl = oracle_decode(x, SWA, window=window)
    compare(out, lse, ro, rl, f"SWA decode window {window}")


@pytest.mark.parametrize("split", [32, 64, 96, 1000, 2048, 8192])
def test_ga_split_sizes(split):
    log(f"[case] GA decode split={split}")
    x = synth.decode_inputs([3000, 31, 32, 33, 4097, 64], GA, seed=21)
    out, lse = gpu_decode(x, GA, split=split)
    ro, rl = oracle_decode(x, GA)
    compare(out, lse, ro, rl, f"GA split {split}")


def test_ga_split_invariance():
    x = synth.decode_inputs([5000, 2100, 77], GA, seed=22)
    ref = gpu_decode(x, GA, split=2048)
    for split in (32, 256, 640):
        o, l = gpu_decode(x, GA, split=split)
        d = (o.float() - ref[0].float()).abs().max().item()
        dl = (l - ref[1]).abs().max().item()
        log(f"[split-invariance] split {split}: out {d:.3e} lse {dl:.3e}")
        assert d <= 1.6e-2 and dl <= 1e-4


@pytest.mark.parametrize("layer_type", [SWA, GA])
@pytest.mark.parametrize("sink", [None, -math.inf, -5.0, 0.0, 5.0, 30.0])
def test_decode_sinks(layer_type, sink):
    x = synth.decode_inputs([130, 20, 0], layer_type, seed=23)
    s = None if sink is None else const_sink(sink)
    out, lse = gpu_decode(x, layer_type, sink=s)
    ro, rl = oracle_decode(x, layer_type, sink=s)
    compare(out, lse, ro, rl, f"decode sink {sink}")


def test_decode_value_scale():
    x = synth.decode_inputs([500, 129], GA, seed=24)
    out, lse = gpu_decode(x, GA, value_scale=0.707)
    ro, rl = oracle_decode(x, GA, value_scale=0.707)
    compare(out, lse, ro, rl, "decode value_scale 0.707")


def test_ga_context_beyond_max_ctx_is_nan():
    """A context longer than the host's max_ctx bound yields NaN, never a silent wrong answer."""
    x = synth.decode_inputs([5000, 10], GA, seed=25)
    out, lse = gpu_decode(x, GA, max_ctx=1000, split=256)
    assert torch.isnan(out[0].float()).all() and torch.isnan(lse[0]).all()
    ro, rl = oracle_decode(x, GA)
    compare(out[1:], lse[1:], ro[1:], rl[1:], "in-bound sequence next to an out-of-bound one")


# ---------------------------------------------------------------------------
def _ring(B_, hkv=4):
    return (torch.zeros((B_, 128, hkv, 192), dtype=torch.bfloat16), torch.zeros((B_, 128, hkv, 128), dtype=torch.bfloat16))


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_append_matches_oracle_bitwise(layer_type):
    """Bulk append of a ragged batch (prefill), then single-token steps."""
    lengths = [0, 1, 127, 128, 129, 300, 5]
    Bn = len(lengths)
    x = synth.prefill_inputs(lengths, seed=26)
    steps = 3
    if layer_type == SWA:
        kc, vc = _ring(Bn)
        base = cap = None
    else:
        caps = [L + steps + (7 if i != 3 else 0) for i, L in enumerate(lengths)]
        caps[5] = lengths[5] - 1  # this sequence does not fit: refused, untouched
        base_l = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
        N = int(sum(caps)) + 8
        kc = torch.zeros((N, 4, 192), dtype=torch.bfloat16)
        vc = torch.zeros((N, 4, 128), dtype=torch.bfloat16)
        base, cap = torch.tensor(base_l), torch.tensor(caps, dtype=torch.int64)
    kc_ref, vc_ref = bits(kc).copy(), bits(vc).copy()
    gk, gv = to_dev(kc), to_dev(vc)
    ctx = torch.zeros(Bn, dtype=torch.int32)
    st = orc().kv_append(bits(x.k), bits(x.v), x.cu_seqlens.numpy(), ctx.numpy(), kc_ref, vc_ref,
                         layer_type=layer_type, kv_base=None if base is None else base.numpy(),
                         kv_capacity=None if cap is None else cap.numpy())
    B.kv_append(to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens), to_dev(ctx), gk, gv, layer_type,
                kv_base=to_dev(base), kv_capacity=to_dev(cap))
    ctx = torch.tensor(lengths, dtype=torch.int32)
    g = torch.Generator().manual_seed(27)
    for step in range(steps):
        kn = torch.randn(Bn, 4, 192, generator=g).to(torch.bfloat16)
        vn = torch.randn(Bn, 4, 128, generator=g).to(torch.bfloat16)
        cu = torch.arange(Bn + 1, dtype=torch.int32)
        orc().kv_append(bits(kn), bits(vn), cu.numpy(), ctx.numpy(), kc_ref, vc_ref, layer_type=layer_type,
                        kv_base=None if base is None else base.numpy(), kv_capacity=None if cap is None else cap.numpy())
        B.kv_append(to_dev(kn), to_dev(vn), to_dev(cu), to_dev(ctx), gk, gv, layer_type, kv_base=to_dev(base),
                    kv_capacity=to_dev(cap))
        ctx += 1
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), kc_ref) and np.array_equal(bits(gv), vc_ref)
    if layer_type == GA:
        assert not bits(gk)[int(base[5]):int(base[5]) + caps[5]].any(), "refused sequence was written"


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_decode_after_append_equals_prefill_row(layer_type):
    """Prefill L+1 tokens; append the first L; decode token L: same row as prefill."""
    lengths = [1, 129, 200, 64]
    xs = synth.prefill_inputs([L + 1 for L in lengths], seed=28)
    Bn = len(lengths)
    cu_full = xs.cu_seqlens.tolist()
    idx_prefix = torch.cat([torch.arange(cu_full[b], cu_full[b] + lengths[b]) for b in range(Bn)])
    idx_last = torch.tensor([cu_full[b] + lengths[b] for b in range(Bn)])
    kp, vp = xs.k[idx_prefix].contiguous(), xs.v[idx_prefix].contiguous()
    cu_p = synth.cu_from_lengths(lengths)
    if layer_type == SWA:
        kc, vc = _ring(Bn)
        base = cap = None
    else:
        caps = [L + 1 for L in lengths]
        base = torch.tensor(np.concatenate([[0], np.cumsum(caps)[:-1]]), dtype=torch.int64)
        cap = torch.tensor(caps, dtype=torch.int64)
        kc = torch.zeros((sum(caps), 4, 192), dtype=torch.bfloat16)
        vc = torch.zeros((sum(caps), 4, 128), dtype=torch.bfloat16)
    gk, gv = to_dev(kc), to_dev(vc)
    B.kv_append(to_dev(kp), to_dev(vp), to_dev(cu_p), to_dev(torch.zeros(Bn, dtype=torch.int32)), gk, gv,
                layer_type, kv_base=to_dev(base), kv_capacity=to_dev(cap))
    ctx = torch.tensor(lengths, dtype=torch.int32)
    out, lse = B.decode(to_dev(xs.q[idx_last]), to_dev(xs.k[idx_last]), to_dev(xs.v[idx_last]), gk, gv, to_dev(ctx),
                        max(lengths), layer_type, sink=to_dev(xs.sink), kv_base=to_dev(base), split_tokens=64)
    pout, plse = gpu_prefill(xs, layer_type)
    torch.cuda.synchronize()
    ro, rl = oracle_prefill(xs, layer_type, rows=idx_last.numpy())
    compare(out, lse, ro, rl, "decode after append vs oracle prefill rows")
    d = (out.float() - pout[idx_last.cuda()].float()).abs().max().item()
    dl = (lse - plse[idx_last.cuda()]).abs().max().item()
    log(f"[decode-vs-prefill] layer {layer_type}: out {d:.3e} lse {dl:.3e}")
    assert d <= 2e-2 and dl <= 1e-3
