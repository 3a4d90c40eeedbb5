"""GPU parity of chunked prefill (new tokens continuing cached sequences) through
the C ABI, against the fp64 oracle on host copies of the same buffers.

The GPU caches are filled by the library's append from the sequences' first
tokens, the oracle's by its own append from host copies of the same tokens
(checked equal byte for byte); the chunk holds the rest.  Bars as in gpu_util.
"""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"


def _split(x, cached):
    """Packed rows of the cached prefixes and of the chunks of a prefill batch."""
    cu = x.cu_seqlens.tolist()
    lengths = x.lengths
    rest = [L - c for L, c in zip(lengths, cached)]
    pre = torch.cat([torch.arange(cu[b], cu[b] + cached[b]) for b in range(len(lengths))]).long()
    new = torch.cat([torch.arange(cu[b] + cached[b], cu[b + 1]) for b in range(len(lengths))]).long()
    return pre, new, rest


def _caches(layer_type, lengths, headroom=8, window=129):
    n = len(lengths)
    if layer_type == SWA:
        return (torch.zeros((n, window - 1, 4, 192), dtype=torch.bfloat16, device=DEV),
                torch.zeros((n, window - 1, 4, 128), dtype=torch.bfloat16, device=DEV), None, None)
    caps = [L + headroom for L in lengths]
    base = torch.tensor(np.concatenate([[3], 3 + np.cumsum(caps)[:-1]]), dtype=torch.int64, device=DEV)
    rows = int(base[-1]) + caps[-1]
    return (torch.zeros((rows, 4, 192), dtype=torch.bfloat16, device=DEV),
            torch.zeros((rows, 4, 128), dtype=torch.bfloat16, device=DEV), base,
            torch.tensor(caps, dtype=torch.int64, device=DEV))


def _fill(x, layer_type, cached, kc, vc, base, cap, window=129):
    """Appends the cached prefixes on the GPU and, with the oracle, into host
    caches of the same shape; returns the host caches after checking that the
    two agree byte for byte."""
    pre, _, _ = _split(x, cached)
    cu_pre = synth.cu_from_lengths(cached, DEV)
    zeros = torch.zeros(len(cached), dtype=torch.int32, device=DEV)
    kh, vh = np.zeros_like(bits(kc)), np.zeros_like(bits(vc))
    if sum(cached):
        B.kv_append(to_dev(x.k[pre]), to_dev(x.v[pre]), cu_pre, zeros, kc, vc, layer_type, kv_base=base,
                    kv_capacity=cap, dims=B.make_dims(sliding_window=window))
        st = orc().kv_append(bits(x.k[pre]), bits(x.v[pre]), cu_pre.cpu().numpy(), zeros.cpu().numpy(), kh, vh,
                             layer_type=layer_type, window=window,
                             kv_base=None if base is None else base.cpu().numpy(),
                             kv_capacity=None if cap is None else cap.cpu().numpy())
        assert st == 0
        torch.cuda.synchronize()
    assert np.array_equal(bits(kc), kh) and np.array_equal(bits(vc), vh), "GPU append differs from the oracle's"
    return kh, vh


def _chunk(x, layer_type, cached, kc, vc, base, max_newlen=None, window=129):
    _, new, rest = _split(x, cached)
    cu_new = synth.cu_from_lengths(rest, DEV)
    ctx = torch.tensor(cached, dtype=torch.int32, device=DEV)
    out, lse = B.prefill_chunk(to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]), cu_new,
                               max(rest) if max_newlen is None else max_newlen, kc, vc, ctx, layer_type,
                               sink=to_dev(x.sink), kv_base=base, dims=B.make_dims(sliding_window=window))
    torch.cuda.synchronize()
    return out, lse, new, rest, cu_new, ctx


@pytest.mark.parametrize("layer_type,window", [(SWA, 129), (SWA, 64), (SWA, 300), (GA, 129)])
def test_chunk_against_oracle_ragged(layer_type, window):
    """Prefixes of 0, 1, 63, 128, 131 and 1000 tokens cached; chunks of 300, 169,
    1, 1, 129 and 500 tokens, in one packed call.  SWA windows up to 145 keys run
    the streaming kernel, wider ones the tiled kernel."""
    lengths = [300, 170, 64, 129, 260, 1500]
    cached = [0, 1, 63, 128, 131, 1000]
    log(f"[case] chunked prefill layer={layer_type} window={window} lengths={lengths} cached={cached}")
    x = synth.prefill_inputs(lengths, seed=40)
    kc, vc, base, cap = _caches(layer_type, lengths, window=window)
    kh, vh = _fill(x, layer_type, cached, kc, vc, base, cap, window=window)
    out, lse, new, rest, cu_new, ctx = _chunk(x, layer_type, cached, kc, vc, base, window=window)
    ro, rl = orc().prefill_chunk(bits(x.q[new]), bits(x.k[new]), bits(x.v[new]), cu_new.cpu().numpy(), kh,
                                 vh, ctx.cpu().numpy(), layer_type=layer_type, window=window, scale=SCALE,
                                 sink=sink_array(x.sink), kv_base=None if base is None else base.cpu().numpy())
    compare(out, lse, ro, rl, f"chunked prefill layer {layer_type} window {window}")


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_chunks_in_sequence_rebuild_prefill(layer_type):
    """One 1000-token sequence fed as chunks of 300, 1, 250 and 449 tokens, each
    attended then appended: equals the oracle's prefill of the whole sequence."""
    L = 1000
    log(f"[case] chunks in sequence layer={layer_type}")
    x = synth.prefill_inputs([L], seed=41)
    kc, vc, base, cap = _caches(layer_type, [L])
    outs, lses, pos = [], [], 0
    for n in (300, 1, 250, 449):
        cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
        ctx = torch.tensor([pos], dtype=torch.int32, device=DEV)
        q, k, v = to_dev(x.q[pos:pos + n]), to_dev(x.k[pos:pos + n]), to_dev(x.v[pos:pos + n])
        o, l = B.prefill_chunk(q, k, v, cu, n, kc, vc, ctx, layer_type, sink=to_dev(x.sink), kv_base=base)
        B.kv_append(k, v, cu, ctx, kc, vc, layer_type, kv_base=base, kv_capacity=cap)
        outs.append(o)
        lses.append(l)
        pos += n
    torch.cuda.synchronize()
    ro, rl = orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.numpy(), layer_type=layer_type, scale=SCALE,
                           sink=sink_array(x.sink))
    compare(torch.cat(outs), torch.cat(lses), ro, rl, f"chunks in sequence layer {layer_type}")


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_chunk_empty_sequences_and_max_newlen(layer_type):
    """Sequences with empty chunks in the batch, and max_newlen below a chunk's
    length: rows past max_newlen stay unwritten, the others are correct."""
    lengths = [200, 50, 90, 130]
    cached = [150, 50, 0, 130]  # chunks of 50, 0, 90, 0 tokens
    log(f"[case] chunk empties/max_newlen layer={layer_type}")
    x = synth.prefill_inputs(lengths, seed=42)
    kc, vc, base, cap = _caches(layer_type, lengths)
    kh, vh = _fill(x, layer_type, cached, kc, vc, base, cap)
    _, new, rest = _split(x, cached)
    ctx = torch.tensor(cached, dtype=torch.int32, device=DEV)
    cu_new = synth.cu_from_lengths(rest, DEV)
    ro, rl = orc().prefill_chunk(bits(x.q[new]), bits(x.k[new]), bits(x.v[new]), cu_new.cpu().numpy(), kh,
                                 vh, ctx.cpu().numpy(), layer_type=layer_type, scale=SCALE,
                                 sink=sink_array(x.sink), kv_base=None if base is None else base.cpu().numpy())
    out, lse, *_ = _chunk(x, layer_type, cached, kc, vc, base)
    compare(out, lse, ro, rl, f"chunk with empty sequences layer {layer_type}")
    out = torch.zeros((len(new), 64, 128), dtype=torch.bfloat16, device=DEV)
    B.mimo_attn_prefill_chunk(B.make_dims(), layer_type, to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]),
                              cu_new, len(lengths), 40, kc, vc, base, ctx, to_dev(x.sink), out, None)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    # chunk rows: sequence 0 owns rows 0..49, sequence 2 rows 50..139
    keep = np.r_[0:40, 50:90]
    assert np.abs(got[keep] - ro[keep]).max() <= 2e-2
    assert not got[40:50].any() and not got[90:140].any()


def test_chunk_ga_long_context_sampled():
    """GA: 28672 positions cached, a 4096-token chunk (the last eighth of a 32K
    prompt); sampled rows against the oracle's prefill of the whole sequence."""
    L, c = 32768, 28672
    log("[case] GA chunk 28672 cached + 4096 new, sampled rows")
    x = synth.prefill_inputs([L], seed=43, device=DEV)
    kc, vc, base, cap = _caches(GA, [L])
    _fill(x, GA, [c], kc, vc, base, cap)
    out, lse, *_ = _chunk(x, GA, [c], kc, vc, base)
    rows_local = [0, 1, 15, 16, 63, 64, 2047, 4094, 4095]
    ro, rl = orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.cpu().numpy(), layer_type=GA, scale=SCALE,
                           sink=sink_array(x.sink), rows=np.array([c + r for r in rows_local], np.int64))
    idx = torch.tensor(rows_local, device=DEV)
    compare(out[idx], lse[idx], ro, rl, "GA chunk 28672+4096 sampled rows")
    assert torch.isfinite(lse).all()


def test_chunk_swa_long_sampled():
    """SWA: 4 sequences with 8192 positions cached (the ring holds the last 128)
    and 8192-token chunks; sampled rows against the whole-sequence oracle."""
    L, c = 16384, 8192
    log("[case] SWA chunk 4 x (8192 cached + 8192 new), sampled rows")
    x = synth.prefill_inputs([L] * 4, seed=44, device=DEV)
    kc, vc, base, cap = _caches(SWA, [L] * 4)
    _fill(x, SWA, [c] * 4, kc, vc, base, cap)
    out, lse, *_ = _chunk(x, SWA, [c] * 4, kc, vc, base)
    local = [0, 1, 127, 128, 129, 5000, 8191]
    rows = [s * L + c + r for s in range(4) for r in local]
    ro, rl = orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.cpu().numpy(), layer_type=SWA,
                           scale=SCALE, sink=sink_array(x.sink), rows=np.array(rows, np.int64))
    idx = torch.tensor([s * (L - c) + r for s in range(4) for r in local], device=DEV)
    compare(out[idx], lse[idx], ro, rl, "SWA chunk 4x(8192+8192) sampled rows")
    assert torch.isfinite(lse).all()
