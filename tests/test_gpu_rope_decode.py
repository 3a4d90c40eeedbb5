"""A decode step with the rotary embedding fused in (mimo_attn_decode_append_rope)
through the C ABI (model doc "MiMo-V2-Flash", MiMoV2FlashConfig: rope_parameters /
rope_theta; MiMoV2FlashModel.forward: position_ids, past_key_values):
  * bit for bit equal to mimo_rope_apply on copies of q and k_new followed by
    mimo_attn_decode_append over the rotated copies: outputs, LSE and the caches
    afterwards (the appended key is the rotated one), with q and k_new left as
    they were;
  * within the attention bars of the oracle's decode of the oracle's rotation
    rounded to bf16.
Covers the short SWA ring (window 129), a long ring (window 300, the tile-loop
kernel), GA with the default chunking and with 64-key chunks (the new token's
unit in many places of a chunk), rotary dims 64, 128 and 192, positions equal
to ctx_lens and offset from them, a GA sequence with no room for its row, and
the hybrid stack's decode step with the fused rotation replayed from a HIP
graph against the separate rotation issued call by call."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array

pytestmark = pytest.mark.gpu
DEV = "cuda"
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))


def _run(lt, ctx, window, split, rd, theta, offset, full=None, seed=31):
    x = synth.decode_inputs(ctx, lt, seed=seed, device=DEV, window=window)
    bsz = len(ctx)
    max_ctx = max(ctx) + 1
    dims = B.make_dims(sliding_window=window)
    cap = None
    if lt == GA:
        cap = x.kv_capacity.clone()
        if full is not None:
            cap[full] = ctx[full]  # no room for position p: the row stays untouched
    pos = (x.ctx_lens + offset).to(torch.int32)
    nbytes = B.mimo_attn_decode_workspace_size(dims, lt, bsz, max_ctx, split)
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=DEV) if nbytes else None
    q0, k0 = x.q.clone(), x.k_new.clone()
    res = []
    for fused in (True, False):
        kc, vc = x.k_cache.clone(), x.v_cache.clone()
        out = torch.empty((bsz, 64, 128), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((bsz, 64), dtype=torch.float32, device=DEV)
        if fused:
            B.mimo_attn_decode_append_rope(dims, lt, x.q, x.k_new, x.v_new, pos, kc, vc, x.kv_base, cap, x.ctx_lens,
                                           bsz, max_ctx, split, theta, rd, x.sink, out, lse, ws)
        else:
            q2, k2 = x.q.clone(), x.k_new.clone()
            B.rope_apply(q2, k2, pos, theta, rd)
            B.mimo_attn_decode_append(dims, lt, q2, k2, x.v_new, kc, vc, x.kv_base, cap, x.ctx_lens, bsz, max_ctx,
                                      split, x.sink, out, lse, ws)
        torch.cuda.synchronize()
        res.append((out, lse, kc, vc))
    assert torch.equal(x.q, q0) and torch.equal(x.k_new, k0), "the fused call modified q or k_new"
    return x, pos, res


CASES = [
    (SWA, [0, 1, 5, 127, 128, 129, 300, 1000], 129, 0, 64, 1e4, 0),
    (SWA, [0, 3, 298, 299, 300, 4000], 300, 0, 128, 1e6, 0),      # long ring: the tile-loop kernel
    (SWA, [64, 700, 128 * 9 + 5], 129, 0, 192, 5e6, 123456),     # every dim rotates; offset positions
    (GA, [0, 1, 31, 32, 33, 1000, 5000, 70000], 0, 0, 64, 5e6, 0),
    (GA, [0, 1, 63, 64, 65, 300, 2049], 129, 64, 128, 1e4, 7),   # 64-key chunks
    (GA, [4096, 100, 7000], 129, 0, 192, 5e6, 0),
]


@pytest.mark.parametrize("lt,ctx,window,split,rd,theta,offset", CASES)
def test_decode_rope_equals_separate_and_oracle(lt, ctx, window, split, rd, theta, offset):
    log(f"[case] fused decode rope lt={lt} ctx={ctx} W={window} split={split} rd={rd} theta={theta} "
        f"offset={offset}")
    x, pos, ((of, lf, kf, vf), (os_, ls, ks, vs)) = _run(lt, ctx, window if lt == SWA else 129, split, rd, theta,
                                                         offset)
    assert torch.equal(of, os_) and torch.equal(lf, ls), "fused decode differs from rope + decode_append"
    assert torch.equal(kf, ks) and torch.equal(vf, vs), "caches differ from rope + decode_append"
    rq, rk = orc().rope(bits(x.q), bits(x.k_new), pos.cpu().numpy(), theta=float(np.float32(theta)),
                        rotary_dim=rd)
    qb = synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16))
    kb = synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16))
    ro, rl = orc().decode(qb, kb, bits(x.v_new), bits(x.k_cache), bits(x.v_cache), x.ctx_lens.cpu().numpy(),
                          layer_type=lt, window=window if lt == SWA else 129, scale=SCALE, sink=sink_array(x.sink),
                          kv_base=None if x.kv_base is None else x.kv_base.cpu().numpy())
    compare(of, lf, ro, rl, f"fused decode rope lt={lt} rd={rd}")


def test_decode_rope_ga_full_sequence_keeps_its_row():
    ctx = [4096, 100, 7000]
    log("[case] fused decode rope, GA sequence without room")
    x, _, ((of, lf, kf, vf), (os_, ls, ks, vs)) = _run(GA, ctx, 129, 0, 64, 5e6, 0, full=1)
    assert torch.equal(of, os_) and torch.equal(lf, ls)
    assert torch.equal(kf, ks) and torch.equal(vf, vs)
    base = x.kv_base.cpu().tolist()
    assert torch.equal(kf[base[1] + ctx[1]], x.k_cache[base[1] + ctx[1]]), "row past the capacity was written"


def test_stack_step_with_fused_rope_graph_equals_separate_rope():
    """The hybrid stack's decode step with RoPE: one stack replays a captured
    graph of the fused calls, the other issues mimo_rope_apply + the decode call
    per layer; outputs, LSE, caches and contexts agree bit for bit every step."""
    from global_attention_mimo_amd.stack import HybridStack
    from test_gpu_graph import _prefill
    lengths = [300, 77, 128, 129, 1000, 5]
    layers, steps = 12, 4
    log(f"[case] stack decode with fused RoPE: lengths {lengths}, {layers} layers, {steps} steps")
    gen = torch.Generator(device=DEV).manual_seed(9)
    sinks = torch.randn((layers, 64), generator=gen, device=DEV)
    fused = HybridStack(lengths, num_layers=layers, decode_steps=steps + 1, device=DEV, rope_mode="fused")
    sep = HybridStack(lengths, num_layers=layers, decode_steps=steps + 1, device=DEV, rope_mode="separate")
    _prefill(fused, lengths, sinks)
    _prefill(sep, lengths, sinks)
    nb = len(lengths)
    shapes = [(layers, nb, 64, 192), (layers, nb, 4, 192), (layers, nb, 4, 128)]
    static = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    f_out = torch.empty((layers, nb, 64, 128), dtype=torch.bfloat16, device=DEV)
    f_lse = torch.empty((layers, nb, 64), dtype=torch.float32, device=DEV)
    s_out, s_lse = torch.empty_like(f_out), torch.empty_like(f_lse)
    graph = fused.capture_decode_step(*static, sinks, f_out, f_lse)
    for step in range(steps):
        inputs = [torch.randn(s, generator=gen, device=DEV).to(torch.bfloat16) for s in shapes]
        for buf, x in zip(static, inputs):
            buf.copy_(x)
        sep.decode_step(*inputs, sinks, s_out, s_lse)  # rotates its inputs in place
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[case] stack decode with fused RoPE, step {step}")
        assert torch.equal(f_out, s_out) and torch.equal(f_lse, s_lse), f"step {step}: outputs differ"
    for layer in range(layers):
        assert torch.equal(fused.caches[layer].k, sep.caches[layer].k), f"layer {layer}: K cache differs"
        assert torch.equal(fused.caches[layer].v, sep.caches[layer].v), f"layer {layer}: V cache differs"
    assert torch.equal(fused.ctx, sep.ctx)


def test_stack_prefill_with_fused_rope_equals_separate():
    """The hybrid stack's prefill with RoPE (positions 0..L-1): the fused form
    (mimo_attn_prefill_rope, its rotated keys appended) against mimo_rope_apply
    + mimo_attn_prefill + append, bit for bit per layer (outputs, LSE) and in the
    caches afterwards."""
    from global_attention_mimo_amd.stack import HybridStack
    lengths = [300, 77, 128, 129, 1000, 5]
    layers = 12
    log(f"[case] stack prefill with fused RoPE: lengths {lengths}, {layers} layers")
    gen = torch.Generator(device=DEV).manual_seed(11)
    sinks = torch.randn((layers, 64), generator=gen, device=DEV)
    fused = HybridStack(lengths, num_layers=layers, decode_steps=1, device=DEV, rope_mode="fused")
    sep = HybridStack(lengths, num_layers=layers, decode_steps=1, device=DEV, rope_mode="separate")
    T = sum(lengths)
    for layer in range(layers):
        x = synth.prefill_inputs(lengths, seed=700 + layer, device=DEV, with_sink=False)
        outs = []
        for st in (fused, sep):
            out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((T, 64), dtype=torch.float32, device=DEV)
            st.prefill_layer(layer, x.q.clone(), x.k.clone(), x.v.clone(), sinks[layer], out, lse)
            outs.append((out, lse))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), f"layer {layer} differs"
    for layer in range(layers):
        assert torch.equal(fused.caches[layer].k, sep.caches[layer].k), f"layer {layer}: K cache differs"
        assert torch.equal(fused.caches[layer].v, sep.caches[layer].v), f"layer {layer}: V cache differs"
