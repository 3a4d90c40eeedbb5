"""Full-size parity at the benchmark's launch configurations, on sampled outputs.

The GPU computes every output of the workload; the fp64 oracle recomputes the
sampled rows one by one from host copies of the same buffers.  Bars as in
gpu_util (bf16 out max-abs 2e-2 / mean-abs 2e-3, LSE 1e-3).
"""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from global_attention_mimo_amd.stack import HybridStack
from gpu_util import bits, compare, log, orc

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"


def run_prefill(x, layer_type, nseq, max_len):
    out = torch.empty((x.q.shape[0], 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((x.q.shape[0], 64), dtype=torch.float32, device=DEV)
    B.mimo_attn_prefill(B.make_dims(), layer_type, x.q, x.k, x.v, x.cu_seqlens, nseq, max_len, x.sink, out, lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(x, layer_type, rows):
    return orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.cpu().numpy(), layer_type=layer_type,
                         scale=SCALE, sink=x.sink.cpu().numpy(), rows=np.asarray(rows, np.int64))


def test_swa_prefill_4x8192_sampled():
    log("[case] SWA prefill 4x8192 (seed 0), sampled rows")
    x = synth.prefill_inputs([8192] * 4, seed=0, device=DEV)
    out, lse = run_prefill(x, SWA, 4, 8192)
    rows = [s * 8192 + p for s in range(4) for p in (0, 1, 127, 128, 129, 130, 4321, 8190, 8191)]
    ro, rl = oracle_rows(x, SWA, rows)
    idx = torch.tensor(rows, device=DEV)
    compare(out[idx], lse[idx], ro, rl, "SWA 4x8192 sampled rows")
    assert torch.isfinite(lse).all()


def test_ga_prefill_1x32768_sampled():
    log("[case] GA prefill 1x32768 (seed 0), sampled rows")
    x = synth.prefill_inputs([32768], seed=0, device=DEV)
    out, lse = run_prefill(x, GA, 1, 32768)
    g = np.random.default_rng(0)
    rows = sorted(set([0, 1, 2, 15, 16, 63, 64, 4095, 4096, 16383, 32766, 32767] + list(g.integers(0, 32768, 6))))
    ro, rl = oracle_rows(x, GA, rows)
    idx = torch.tensor(rows, device=DEV)
    compare(out[idx], lse[idx], ro, rl, "GA 1x32768 sampled rows")
    assert torch.isfinite(lse).all()


def test_decode_b128_long_contexts():
    """Decode step for 128 sequences with contexts U[4096, 262144] (seed 0): GA over
    the full bf16 pool (default split) for sampled sequences, SWA over the ring for all."""
    ctx = synth.long_context_lengths(128, seed=0)
    log(f"[case] GA decode B=128 ctx U[4096,262144] total {sum(ctx)} tokens")
    x = synth.decode_inputs(ctx, GA, seed=0, device=DEV, headroom=4)
    out, lse = B.decode(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, x.ctx_lens, max(ctx) + 4, GA, sink=x.sink,
                        kv_base=x.kv_base)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    order = np.argsort(ctx)
    pick = [int(order[0]), int(order[-1]), int(order[64])]
    base = x.kv_base.cpu().numpy()
    for b in pick:
        c = ctx[b]
        kc = bits(x.k_cache[base[b]:base[b] + c])
        vc = bits(x.v_cache[base[b]:base[b] + c])
        ro, rl = orc().decode(bits(x.q[b:b + 1]), bits(x.k_new[b:b + 1]), bits(x.v_new[b:b + 1]), kc, vc,
                              np.array([c], np.int32), layer_type=GA, scale=SCALE, sink=x.sink.cpu().numpy(),
                              kv_base=np.zeros(1, np.int64))
        compare(out[b:b + 1], lse[b:b + 1], ro, rl, f"GA decode seq {b} ctx {c}")
    del x
    torch.cuda.empty_cache()
    log("[case] SWA decode B=128 ring")
    y = synth.decode_inputs(ctx, SWA, seed=0, device=DEV)
    out, lse = B.decode(y.q, y.k_new, y.v_new, y.k_cache, y.v_cache, y.ctx_lens, max(ctx), SWA, sink=y.sink)
    torch.cuda.synchronize()
    ro, rl = orc().decode(bits(y.q), bits(y.k_new), bits(y.v_new), bits(y.k_cache), bits(y.v_cache),
                          np.asarray(ctx, np.int32), layer_type=SWA, scale=SCALE, sink=y.sink.cpu().numpy())
    compare(out, lse, ro, rl, "SWA decode B=128 all sequences")


def test_hybrid_stack_48_layers():
    """48 layers (5 SWA : 1 GA), 32 ragged prompts log-uniform in [512, 32768], varlen
    prefill + append, then 64 decode steps (attend, append).  Sampled parity on an SWA
    and a GA layer after prefill and at the last decode step."""
    lengths = synth.hybrid_prompt_lengths(32, seed=0)
    st = HybridStack(lengths, decode_steps=64, device=DEV)
    log(f"[case] hybrid stack: {sum(lengths)} prompt tokens, 48 layers, 64 steps")
    checked = {0: SWA, 5: GA}
    # Host copies of every token appended to the checked layers' caches for the
    # checked sequences: the oracle rebuilds those caches with its own append.
    hist = {}
    order = np.argsort(lengths)
    seqs = [int(order[0]), int(order[-1])]
    cu = st.cu.cpu().numpy()
    out = torch.empty((st.total, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((st.total, 64), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(0)
    sinks = torch.randn((48, 64), generator=gen, device=DEV)
    for layer in range(48):
        x = synth.prefill_inputs(lengths, seed=1000 + layer, device=DEV, with_sink=False)
        st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse)
        if layer in checked:
            torch.cuda.synchronize()
            for b in seqs:
                s0, s1 = int(cu[b]), int(cu[b + 1])
                hist[(layer, b)] = ([bits(x.k[s0:s1])], [bits(x.v[s0:s1])])
                L = s1 - s0
                rows = sorted(set([0, 1, 128, 129, L // 2, L - 1]))
                ro, rl = orc().prefill(bits(x.q[s0:s1]), bits(x.k[s0:s1]), bits(x.v[s0:s1]),
                                       np.array([0, L], np.int32), layer_type=checked[layer], scale=SCALE,
                                       sink=sinks[layer].cpu().numpy(), rows=np.asarray(rows, np.int64))
                idx = torch.tensor([s0 + r for r in rows], device=DEV)
                compare(out[idx], lse[idx], ro, rl, f"stack prefill layer {layer} seq {b} (L={L})")
        del x
    log("[case] hybrid stack: decode steps")
    dout = torch.empty((st.batch, 64, 128), dtype=torch.bfloat16, device=DEV)
    dlse = torch.empty((st.batch, 64), dtype=torch.float32, device=DEV)
    for step in range(64):
        last = step == 63
        for layer in range(48):
            q = torch.randn((st.batch, 64, 192), generator=gen, device=DEV).to(torch.bfloat16)
            kn = torch.randn((st.batch, 4, 192), generator=gen, device=DEV).to(torch.bfloat16)
            vn = torch.randn((st.batch, 4, 128), generator=gen, device=DEV).to(torch.bfloat16)
            if last and layer in checked:
                torch.cuda.synchronize()
                c = st.caches[layer]
                ctx = st.ctx.cpu().numpy()
                snap = []
                for b in seqs:
                    if checked[layer] == GA:
                        b0 = int(st.kv_base[b])
                        gpu = (bits(c.k[b0:b0 + ctx[b]]), bits(c.v[b0:b0 + ctx[b]]))
                        kc = np.zeros((ctx[b], 4, 192), np.uint16)
                        vc = np.zeros((ctx[b], 4, 128), np.uint16)
                        base, cap = np.zeros(1, np.int64), np.array([ctx[b]], np.int64)
                    else:
                        gpu = (bits(c.k[b:b + 1]), bits(c.v[b:b + 1]))
                        kc = np.zeros((1, 128, 4, 192), np.uint16)
                        vc = np.zeros((1, 128, 4, 128), np.uint16)
                        base = cap = None
                    pos = 0
                    for kt, vt in zip(*hist[(layer, b)]):
                        n = kt.shape[0]
                        assert orc().kv_append(kt, vt, np.array([0, n], np.int32), np.array([pos], np.int32), kc, vc,
                                               layer_type=checked[layer], kv_base=base, kv_capacity=cap) == 0
                        pos += n
                    assert pos == ctx[b]
                    assert np.array_equal(gpu[0], kc) and np.array_equal(gpu[1], vc), \
                        f"stack cache of layer {layer} seq {b} differs from the oracle's appends"
                    snap.append((kc, vc))
            st.decode_layer(layer, q, kn, vn, sinks[layer], dout, dlse)
            if layer in checked:
                for b in seqs:
                    hist[(layer, b)][0].append(bits(kn[b:b + 1]))
                    hist[(layer, b)][1].append(bits(vn[b:b + 1]))
            if last and layer in checked:
                torch.cuda.synchronize()
                for (kc, vc), b in zip(snap, seqs):
                    ro, rl = orc().decode(bits(q[b:b + 1]), bits(kn[b:b + 1]), bits(vn[b:b + 1]), kc, vc,
                                          np.array([ctx[b]], np.int32), layer_type=checked[layer], scale=SCALE,
                                          sink=sinks[layer].cpu().numpy(),
                                          kv_base=np.zeros(1, np.int64) if checked[layer] == GA else None)
                    compare(dout[b:b + 1], dlse[b:b + 1], ro, rl,
                            f"stack decode step 64 layer {layer} seq {b} (ctx={ctx[b]})")
        st.advance()
    torch.cuda.synchronize()
    assert int(st.ctx[0]) == lengths[0] + 64
    kv = st.kv_bytes()
    ratio = kv["all_ga"] / kv["hybrid"]
    log(f"[kv] hybrid {kv['hybrid'] / 1e9:.2f} GB vs all-GA {kv['all_ga'] / 1e9:.2f} GB: {ratio:.2f}x")
    assert 5.0 < ratio < 6.0
