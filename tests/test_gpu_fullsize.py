"""Full-size parity at the benchmark's launch configurations.

The GPU computes every output of each workload; the fp64 oracle recomputes, from
host copies of the same buffers:
  * SWA prefill 4 x 8192: every token and head (the whole configuration);
  * GA prefill 1 x 32768: 304 query rows -- one in every 128-token stretch of
    the sequence (cycling through the first, last and inner tokens of 16-token
    query blocks, so every dispatch round of the heaviest-first schedule is
    visited) plus three whole 16-token blocks (first, middle, last);
  * decode B = 128 with contexts U[4096, 262144]: every sequence, GA over the
    bf16 pool and SWA over the ring;
  * the 48-layer hybrid stack: four layers (two SWA, two GA), every sequence,
    sampled prefill rows and the whole last decode step, and the caches those
    layers hold, byte for byte, against the oracle's own appends.
Bars as in gpu_util (bf16 out max-abs 2e-2 / mean-abs 2e-3 over all compared
elements of a configuration, LSE 1e-3).
"""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from global_attention_mimo_amd.stack import HybridStack
from gpu_util import ParityTally, bits, compare, log, orc

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


def ga_prefill_rows(L=32768):
    """One row per 128-token stretch, its offset cycling over first/last/inner
    tokens of a 16-token block, plus whole blocks at the start, middle and end."""
    offsets = (0, 15, 16, 31, 47, 64, 100, 127)
    rows = {128 * k + offsets[k % len(offsets)] for k in range(L // 128)}
    for b0 in (0, L // 2, L - 16):
        rows.update(range(b0, b0 + 16))
    return np.array(sorted(rows), np.int64)


@pytest.mark.timeout(600)
def test_swa_prefill_4x8192_full():
    log("[case] SWA prefill 4x8192 (seed 0), every token")
    x = synth.prefill_inputs([8192] * 4, seed=0, device=DEV)
    out, lse = run_prefill(x, SWA, 4, 8192)
    qb, kb, vb = bits(x.q), bits(x.k), bits(x.v)
    cu = x.cu_seqlens.cpu().numpy()
    tally = ParityTally("SWA prefill 4x8192")
    for s in range(4):
        rows = np.arange(s * 8192, (s + 1) * 8192, dtype=np.int64)
        ro, rl = orc().prefill(qb, kb, vb, cu, layer_type=SWA, scale=SCALE, sink=x.sink.cpu().numpy(), rows=rows)
        tally.add(out[s * 8192:(s + 1) * 8192], lse[s * 8192:(s + 1) * 8192], ro, rl, f"sequence {s}")
    tally.check()
    assert tally.rows == 32768


@pytest.mark.timeout(600)
def test_ga_prefill_1x32768_spread_rows():
    rows = ga_prefill_rows()
    log(f"[case] GA prefill 1x32768 (seed 0), {len(rows)} rows")
    x = synth.prefill_inputs([32768], seed=0, device=DEV)
    out, lse = run_prefill(x, GA, 1, 32768)
    assert torch.isfinite(lse).all()
    qb, kb, vb = bits(x.q), bits(x.k), bits(x.v)
    cu = x.cu_seqlens.cpu().numpy()
    tally = ParityTally("GA prefill 1x32768")
    for part in np.array_split(rows, 4):
        ro, rl = orc().prefill(qb, kb, vb, cu, layer_type=GA, scale=SCALE, sink=x.sink.cpu().numpy(), rows=part)
        idx = torch.tensor(part, device=DEV)
        tally.add(out[idx], lse[idx], ro, rl, f"rows {part[0]}..{part[-1]}")
    tally.check()
    assert tally.rows >= 256


@pytest.mark.timeout(900)
def test_decode_b128_long_contexts_all_sequences():
    """Decode step for 128 sequences with contexts U[4096, 262144] (seed 0): GA over
    the full bf16 pool (default split) and SWA over the ring, every sequence."""
    ctx = synth.long_context_lengths(128, seed=0)
    log(f"[case] GA decode B=128 ctx U[4096,262144] total {sum(ctx)} tokens, every sequence")
    x = synth.decode_inputs(ctx, GA, seed=0, device=DEV, headroom=4)
    out, lse = B.decode(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, x.ctx_lens, max(ctx) + 4, GA, sink=x.sink,
                        kv_base=x.kv_base)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    base = x.kv_base.cpu().numpy()
    sink = x.sink.cpu().numpy()
    qb, knb, vnb = bits(x.q), bits(x.k_new), bits(x.v_new)
    tally = ParityTally("GA decode B=128")
    for b in range(len(ctx)):
        c = ctx[b]
        kc = bits(x.k_cache[base[b]:base[b] + c])
        vc = bits(x.v_cache[base[b]:base[b] + c])
        ro, rl = orc().decode(qb[b:b + 1], knb[b:b + 1], vnb[b:b + 1], kc, vc, np.array([c], np.int32),
                              layer_type=GA, scale=SCALE, sink=sink, kv_base=np.zeros(1, np.int64))
        tally.add(out[b:b + 1], lse[b:b + 1], ro, rl, f"seq {b} ctx {c}")
        del kc, vc
    tally.check()
    assert tally.rows == 128
    del x
    torch.cuda.empty_cache()
    log("[case] SWA decode B=128 ring")
    y = synth.decode_inputs(ctx, SWA, seed=0, device=DEV)
    out, lse = B.decode(y.q, y.k_new, y.v_new, y.k_cache, y.v_cache, y.ctx_lens, max(ctx), SWA, sink=y.sink)
    torch.cuda.synchronize()
    ro, rl = orc().decode(bits(y.q), bits(y.k_new), bits(y.v_new), bits(y.k_cache), bits(y.v_cache),
                          np.asarray(ctx, np.int32), layer_type=SWA, scale=SCALE, sink=y.sink.cpu().numpy())
    compare(out, lse, ro, rl, "SWA decode B=128 all sequences")


@pytest.mark.timeout(900)
def test_hybrid_stack_48_layers():
    """48 layers (5 SWA : 1 GA), 32 ragged prompts log-uniform in [512, 32768], varlen
    prefill + append, then 64 decode steps (attend, append).  Layers 0 and 22 (SWA)
    and 5 and 47 (GA) are checked for every sequence: sampled prefill rows, the
    whole last decode step, and the caches they hold before it."""
    lengths = synth.hybrid_prompt_lengths(32, seed=0)
    st = HybridStack(lengths, decode_steps=64, device=DEV)
    log(f"[case] hybrid stack: {sum(lengths)} prompt tokens, 48 layers, 64 steps")
    checked = {0: SWA, 5: GA, 22: SWA, 47: GA}
    for layer, lt in checked.items():
        assert st.layer_types[layer] == lt
    # Host copies of every token appended to the checked layers' caches: the
    # oracle rebuilds those caches with its own append.
    hist = {}
    seqs = list(range(st.batch))
    cu = st.cu.cpu().numpy()
    out = torch.empty((st.total, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((st.total, 64), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(0)
    sinks = torch.randn((48, 64), generator=gen, device=DEV)
    pre = {layer: ParityTally(f"stack prefill layer {layer}") for layer in checked}
    for layer in range(48):
        x = synth.prefill_inputs(lengths, seed=1000 + layer, device=DEV, with_sink=False)
        st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse)
        if layer in checked:
            torch.cuda.synchronize()
            qb, kb, vb = bits(x.q), bits(x.k), bits(x.v)
            rows = []
            for b in seqs:
                s0, s1 = int(cu[b]), int(cu[b + 1])
                hist[(layer, b)] = ([kb[s0:s1]], [vb[s0:s1]])
                L = s1 - s0
                rows += [s0 + r for r in sorted({0, 1, 15, 16, 127, 128, 129, L // 2, L - 17, L - 16, L - 1})]
            rows = np.asarray(rows, np.int64)
            ro, rl = orc().prefill(qb, kb, vb, cu, layer_type=checked[layer], scale=SCALE,
                                   sink=sinks[layer].cpu().numpy(), rows=rows)
            idx = torch.tensor(rows, device=DEV)
            pre[layer].add(out[idx], lse[idx], ro, rl, f"{len(rows)} rows over {len(seqs)} sequences")
            pre[layer].check()
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
                lt = checked[layer]
                c = st.caches[layer]
                ctx = st.ctx.cpu().numpy()
                if lt == GA:
                    # The oracle's pool: every sequence at the stack's own base rows.
                    rows = st.pool_rows
                    kc = np.zeros((rows, 4, 192), np.uint16)
                    vc = np.zeros((rows, 4, 128), np.uint16)
                    base, cap = st.kv_base.cpu().numpy(), st.kv_capacity.cpu().numpy()
                else:
                    kc = np.zeros((st.batch, 128, 4, 192), np.uint16)
                    vc = np.zeros((st.batch, 128, 4, 128), np.uint16)
                    base = cap = None
                for b in seqs:
                    pos = 0
                    for kt, vt in zip(*hist[(layer, b)]):
                        n = kt.shape[0]
                        bsel = None if base is None else base[b:b + 1]
                        csel = None if cap is None else cap[b:b + 1]
                        kview = kc if lt == GA else kc[b:b + 1]
                        vview = vc if lt == GA else vc[b:b + 1]
                        assert orc().kv_append(kt, vt, np.array([0, n], np.int32), np.array([pos], np.int32), kview,
                                               vview, layer_type=lt, kv_base=bsel, kv_capacity=csel) == 0
                        pos += n
                    assert pos == ctx[b]
                gk, gv = bits(c.k), bits(c.v)
                if lt == GA:
                    for b in seqs:
                        r0, r1 = int(base[b]), int(base[b]) + int(ctx[b])
                        assert np.array_equal(gk[r0:r1], kc[r0:r1]) and np.array_equal(gv[r0:r1], vc[r0:r1]), \
                            f"stack cache of layer {layer} seq {b} differs from the oracle's appends"
                else:
                    assert np.array_equal(gk, kc) and np.array_equal(gv, vc), \
                        f"stack ring of layer {layer} differs from the oracle's appends"
                log(f"[parity] stack layer {layer}: caches of all {len(seqs)} sequences equal the oracle's appends")
                snap = (kc, vc, base)
            st.decode_layer(layer, q, kn, vn, sinks[layer], dout, dlse)
            if layer in checked:
                kb, vb = bits(kn), bits(vn)
                for b in seqs:
                    hist[(layer, b)][0].append(kb[b:b + 1])
                    hist[(layer, b)][1].append(vb[b:b + 1])
            if last and layer in checked:
                torch.cuda.synchronize()
                kc, vc, base = snap
                ro, rl = orc().decode(bits(q), bits(kn), bits(vn), kc, vc, ctx.astype(np.int32),
                                      layer_type=checked[layer], scale=SCALE, sink=sinks[layer].cpu().numpy(),
                                      kv_base=base)
                t = ParityTally(f"stack decode step 64 layer {layer}")
                t.add(dout, dlse, ro, rl, f"all {st.batch} sequences")
                t.check()
        st.advance()
    torch.cuda.synchronize()
    assert int(st.ctx[0]) == lengths[0] + 64
    kv = st.kv_bytes()
    ratio = kv["all_ga"] / kv["hybrid"]
    log(f"[kv] hybrid {kv['hybrid'] / 1e9:.2f} GB vs all-GA {kv['all_ga'] / 1e9:.2f} GB: {ratio:.2f}x")
    assert 5.0 < ratio < 6.0
