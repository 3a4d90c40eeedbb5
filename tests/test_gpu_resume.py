"""Snapshot and resume of decoding (model doc "MiMo-V2-Flash",
MiMoV2FlashModel.forward: past_key_values holds the keys and values of the
tokens seen so far, and decoding continues from it): the caches and the
context counters are the whole state of a decode.  A 12-layer hybrid stack
(5 SWA : 1 GA) is prefilled and decoded a few steps; its caches and ctx_lens
are copied; k more steps run; the copy is restored and the same k steps run
again, issued call by call and then replayed from a HIP graph: every output,
LSE and cache byte of the second run equals the first."""
import pytest
import torch

from global_attention_mimo_amd import synth
from global_attention_mimo_amd.stack import HybridStack
from gpu_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _snapshot(st):
    return [(c.k.clone(), c.v.clone()) for c in st.caches], st.ctx.clone()


def _restore(st, snap):
    caches, ctx = snap
    for c, (k, v) in zip(st.caches, caches):
        c.k.copy_(k)
        c.v.copy_(v)
    st.ctx.copy_(ctx)


def _inputs(st, steps, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    L, Bd = st.num_layers, st.batch
    return [(torch.randn((L, Bd, 64, 192), generator=g, device=DEV).to(torch.bfloat16),
             torch.randn((L, Bd, 4, 192), generator=g, device=DEV).to(torch.bfloat16),
             torch.randn((L, Bd, 4, 128), generator=g, device=DEV).to(torch.bfloat16)) for _ in range(steps)]


@pytest.mark.parametrize("use_graph", [False, True])
def test_resume_from_snapshot_is_bitwise(use_graph):
    lengths = [300, 1000, 57, 129]
    st = HybridStack(lengths, num_layers=12, decode_steps=16, device=DEV)
    log(f"[case] resume from a cache snapshot, graph={use_graph}")
    sinks = torch.randn((12, 64), generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)
    out = torch.empty((st.total, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((st.total, 64), dtype=torch.float32, device=DEV)
    for layer in range(12):
        x = synth.prefill_inputs(lengths, seed=200 + layer, device=DEV, with_sink=False)
        st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse)
    warm, k = _inputs(st, 3, 7), _inputs(st, 5, 8)
    dout = torch.empty((12, st.batch, 64, 128), dtype=torch.bfloat16, device=DEV)
    dlse = torch.empty((12, st.batch, 64), dtype=torch.float32, device=DEV)
    for q, kn, vn in warm:
        st.decode_step(q, kn, vn, sinks, dout, dlse)
    torch.cuda.synchronize()
    snap = _snapshot(st)

    def run_k():
        outs = []
        for q, kn, vn in k:
            st.decode_step(q, kn, vn, sinks, dout, dlse)
            outs.append((dout.clone(), dlse.clone()))
        torch.cuda.synchronize()
        return outs, _snapshot(st)

    first, end1 = run_k()
    _restore(st, snap)
    if use_graph:
        bq, bk, bv = (torch.empty_like(t) for t in k[0])
        graph = st.capture_decode_step(bq, bk, bv, sinks, dout, dlse)
        _restore(st, snap)  # capture ran nothing, but restore once more to be exact about the state
        second = []
        for q, kn, vn in k:
            bq.copy_(q)
            bk.copy_(kn)
            bv.copy_(vn)
            graph.replay()
            torch.cuda.synchronize()
            second.append((dout.clone(), dlse.clone()))
        end2 = _snapshot(st)
    else:
        second, end2 = run_k()
    for i, ((o1, l1), (o2, l2)) in enumerate(zip(first, second)):
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {i} after the snapshot differs"
    for layer, ((k1, v1), (k2, v2)) in enumerate(zip(end1[0], end2[0])):
        assert torch.equal(k1, k2) and torch.equal(v1, v2), f"layer {layer} cache differs after resuming"
    assert torch.equal(end1[1], end2[1])
    assert torch.equal(end1[1], snap[1] + 5)
    log("[parity] resumed decode: 5 steps x 12 layers bit-identical, caches and contexts equal")
