"""A decode step of the hybrid stack captured in a HIP graph.

Two stacks get identical prompts and decode inputs: one issues every step call by
call, the other replays one captured graph of the step.  Every replay must match
the eager step bit for bit (outputs, LSE), and the caches and contexts must agree
at the end.  Between replays the program does its own eager work (drawing the
next inputs) and synchronises, so a replay that depended on state left by the
capture, or by the previous replay, would show.
"""
import sys

import pytest
import torch

from global_attention_mimo_amd import synth
from global_attention_mimo_amd.stack import HybridStack

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _prefill(st, lengths, sinks):
    out = torch.empty((st.total, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((st.total, 64), dtype=torch.float32, device=DEV)
    for layer in range(st.num_layers):
        x = synth.prefill_inputs(lengths, seed=500 + layer, device=DEV, with_sink=False)
        st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse)
    torch.cuda.synchronize()


def test_decode_step_graph_replays_match_eager():
    # Contexts below, at and past the 128-slot ring, and a GA layer every sixth layer.
    lengths = [300, 77, 128, 129, 1000, 5]
    layers, steps = 12, 6
    log(f"[case] graph decode: lengths {lengths}, {layers} layers, {steps} replays")
    gen = torch.Generator(device=DEV).manual_seed(7)
    sinks = torch.randn((layers, 64), generator=gen, device=DEV)
    eager = HybridStack(lengths, num_layers=layers, decode_steps=steps + 1, device=DEV)
    graphed = HybridStack(lengths, num_layers=layers, decode_steps=steps + 1, device=DEV)
    _prefill(eager, lengths, sinks)
    _prefill(graphed, lengths, sinks)
    nb = len(lengths)
    shapes = [(layers, nb, 64, 192), (layers, nb, 4, 192), (layers, nb, 4, 128)]
    static = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    g_out = torch.empty((layers, nb, 64, 128), dtype=torch.bfloat16, device=DEV)
    g_lse = torch.empty((layers, nb, 64), dtype=torch.float32, device=DEV)
    e_out = torch.empty_like(g_out)
    e_lse = torch.empty_like(g_lse)
    graph = graphed.capture_decode_step(*static, sinks, g_out, g_lse)
    torch.cuda.synchronize()
    assert torch.equal(graphed.ctx, eager.ctx), "capture must not run the step"
    for step in range(steps):
        inputs = [torch.randn(s, generator=gen, device=DEV).to(torch.bfloat16) for s in shapes]
        for buf, x in zip(static, inputs):
            buf.copy_(x)
        eager.decode_step(*inputs, sinks, e_out, e_lse)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[case] graph decode step {step}")
        assert torch.equal(g_out, e_out), f"step {step}: outputs differ"
        assert torch.equal(g_lse, e_lse), f"step {step}: LSE differs"
        assert torch.equal(graphed.ctx, eager.ctx), f"step {step}: contexts differ"
    for layer in range(layers):
        assert torch.equal(graphed.caches[layer].k, eager.caches[layer].k), f"layer {layer}: K cache differs"
        assert torch.equal(graphed.caches[layer].v, eager.caches[layer].v), f"layer {layer}: V cache differs"
    assert torch.equal(graphed.ctx.cpu(), torch.tensor(lengths, dtype=torch.int32) + steps)
