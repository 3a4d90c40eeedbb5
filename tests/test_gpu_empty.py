"""Zero-length sequences inside a batch, and calls with nothing to compute,
through the C ABI (model doc "MiMo-V2-Flash", MiMoV2FlashModel.forward: a
padded batch of prompts of different lengths becomes packed sequences, and a
sequence may contribute no token to a call):
  * prefill batches with empty sequences between non-empty ones, for the
    streaming SWA kernel (window 129), the tiled SWA kernel (window 300) and GA,
    against the oracle; guard rows past the batch stay untouched;
  * a prefill batch whose every sequence is empty writes nothing;
  * the backward over a batch with empty sequences, against the oracle;
  * a backward call in which no token contributes (max_seqlen 0, or no tokens)
    writes no gradient rows, needs no workspace, and gives dsink = +0 for every
    head (a sum over no tokens), with and without a sink."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev
from test_gpu_backward import SCALE, dout_like, grad_compare, oracle_grads, run

pytestmark = pytest.mark.gpu
DEV = "cuda"
SWA, GA = 0, 1
LENGTHS = [0, 5, 0, 17, 0, 200, 0]
GUARD = 3  # NaN rows after the batch's last token


@pytest.mark.parametrize("layer_type,window", [(SWA, 129), (SWA, 300), (GA, 129)])
def test_prefill_with_empty_sequences(layer_type, window):
    log(f"[case] prefill with empty sequences lt={layer_type} W={window} lengths={LENGTHS}")
    x = synth.prefill_inputs(LENGTHS, seed=61)
    T = x.q.shape[0]
    dims = B.make_dims(sliding_window=window)
    out = torch.full((T + GUARD, 64, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T + GUARD, 64), float("nan"), dtype=torch.float32, device=DEV)
    B.mimo_attn_prefill(dims, layer_type, to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens), len(LENGTHS),
                        max(LENGTHS), to_dev(x.sink), out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(out[T:].float()).all() and torch.isnan(lse[T:]).all(), "rows past the batch were written"
    ro, rl = orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.numpy(), layer_type=layer_type,
                           window=window, scale=SCALE, sink=sink_array(x.sink))
    compare(out[:T], lse[:T], ro, rl, f"prefill with empty sequences lt={layer_type} W={window}")


@pytest.mark.parametrize("layer_type,window", [(SWA, 129), (SWA, 300), (GA, 129)])
def test_prefill_of_empty_sequences_writes_nothing(layer_type, window):
    log(f"[case] prefill of empty sequences only lt={layer_type} W={window}")
    x = synth.prefill_inputs([3], seed=62)  # only for valid buffers
    dims = B.make_dims(sliding_window=window)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)  # three empty sequences
    out = torch.full((GUARD, 64, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((GUARD, 64), float("nan"), dtype=torch.float32, device=DEV)
    for max_seqlen in (0, 16):
        B.mimo_attn_prefill(dims, layer_type, to_dev(x.q), to_dev(x.k), to_dev(x.v), cu, 3, max_seqlen,
                            to_dev(x.sink), out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


@pytest.mark.parametrize("layer_type", [SWA, GA])
def test_backward_with_empty_sequences(layer_type):
    log(f"[case] backward with empty sequences lt={layer_type} lengths={LENGTHS}")
    x = synth.prefill_inputs(LENGTHS, seed=63)
    dout = dout_like(x.q.shape[0], 64)
    dq, dk, dv, ds = run(x, dout, layer_type)
    rq, rk, rv, rs = oracle_grads(x, dout, layer_type)
    grad_compare(dq, rq, "dq")
    grad_compare(dk, rk, "dk")
    grad_compare(dv, rv, "dv")
    grad_compare(ds, rs, "dsink")


@pytest.mark.parametrize("with_sink", [True, False])
def test_backward_without_contributing_tokens_zeroes_dsink(with_sink):
    log(f"[case] backward with nothing to compute, sink={with_sink}")
    x = synth.prefill_inputs([7, 9], seed=65)
    dims = B.make_dims()
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    sink = to_dev(x.sink) if with_sink else None
    out = torch.zeros((16, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((16, 64), dtype=torch.float32, device=DEV)
    dout = to_dev(dout_like(16, 66))
    for what, cu, nseq, max_seqlen, total in (
            ("max_seqlen 0", to_dev(x.cu_seqlens), 2, 0, 16),
            ("no tokens", torch.zeros(3, dtype=torch.int32, device=DEV), 2, 8, 0)):
        dq = torch.full_like(q, float("nan"))
        dk = torch.full_like(k, float("nan"))
        dv = torch.full_like(v, float("nan"))
        ds = torch.full((64,), float("nan"), dtype=torch.float32, device=DEV)
        B.mimo_attn_prefill_backward(dims, GA, q, k, v, out, lse, dout, cu, nseq, max_seqlen, total, sink, dq, dk, dv,
                                     ds, None)
        torch.cuda.synchronize()
        assert torch.isnan(dq.float()).all() and torch.isnan(dk.float()).all() and torch.isnan(dv.float()).all(), \
            f"{what}: gradient rows were written"
        assert (ds.view(torch.int32) == 0).all(), f"{what}: dsink is not +0: {ds[:4].tolist()}"
