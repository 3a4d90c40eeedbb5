"""GPU parity of the prefill backward (dq, dk, dv, dsink) through the C ABI
against the fp64 oracle, which recomputes the forward from the inputs (the GPU
backward reads the GPU forward's out and lse).

The backward is handed the forward's output, which is stored in bf16, and
D = dO.out is taken from it; the oracle's gradients are therefore taken with D
from its own forward output rounded once to bf16 (stored_out).  Against the
exact gradients, that rounding alone moves dk by up to ~1.4e-3 R in the mean on
one- and two-token sequences: where one key holds most of a row's weight,
dS = P (dP - D) is a small difference and D's rounding is a large part of it.

Bar (gradients are sums over many rows, so it is relative to the tensor's
largest magnitude R = max|ref|): max-abs error <= 1e-2 R and mean-abs error
<= 1e-3 R for dq, dk, dv (bf16 outputs: half an ulp is 2^-9 R at most; P and dS
enter the MFMAs rounded to bf16, relative 2^-9 per term with random signs, and
the GPU forward's own output differs from the rounded exact one by its P
rounding); dsink (fp32) within 1e-2 of max_h |dsink_ref[h]|.
"""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"


def grad_compare(got, ref, what, max_rel=1e-2, mean_rel=1e-3):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite"
    R = max(float(np.abs(ref).max()), 1e-30)
    d = np.abs(g - ref)
    mx, mean = float(d.max()) / R, float(d.mean()) / R
    log(f"[parity] {what}: max {mx:.2e} R, mean {mean:.2e} R (R = {R:.3e})")
    assert mx <= max_rel, f"{what}: max-abs error {mx:.2e} R > {max_rel}"
    assert mean <= mean_rel, f"{what}: mean-abs error {mean:.2e} R > {mean_rel}"


def run(x, dout, layer_type, window=129, value_scale=1.0, sink="inputs", max_seqlen=None):
    s = x.sink if isinstance(sink, str) else sink
    dims = B.make_dims(sliding_window=window, value_scale=value_scale)
    q, k, v, cu = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens)
    ml = max(x.lengths) if max_seqlen is None else max_seqlen
    out, lse = B.prefill(q, k, v, cu, ml, layer_type, sink=to_dev(s), dims=dims)
    dq, dk, dv, ds = B.prefill_backward(q, k, v, out, lse, to_dev(dout), cu, ml, layer_type, sink=to_dev(s), dims=dims)
    torch.cuda.synchronize()
    return dq, dk, dv, ds


def oracle_grads(x, dout, layer_type, window=129, value_scale=1.0, sink="inputs", **kw):
    s = x.sink if isinstance(sink, str) else sink
    return orc().prefill_backward(bits(x.q), bits(x.k), bits(x.v), bits(dout), x.cu_seqlens.cpu().numpy(),
                                  layer_type=layer_type, window=window, scale=SCALE,
                                  value_scale=float(np.float32(value_scale)), sink=sink_array(s), stored_out=True,
                                  **kw)


def dout_like(T, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((T, 64, 128), generator=g).to(torch.bfloat16)


CASES = [(SWA, 129, 1.0), (SWA, 17, 1.0), (SWA, 300, 0.707), (GA, 129, 1.0), (GA, 129, 0.707)]


@pytest.mark.parametrize("layer_type,window,vs", CASES)
def test_backward_ragged(layer_type, window, vs):
    """Ragged batch {1, 2, 17, 100, 300, 33}: every gradient row and dsink."""
    lengths = [1, 2, 17, 100, 300, 33]
    log(f"[case] backward layer={layer_type} window={window} value_scale={vs} lengths={lengths}")
    x = synth.prefill_inputs(lengths, seed=90)
    dout = dout_like(sum(lengths), 91)
    dq, dk, dv, ds = run(x, dout, layer_type, window, vs)
    rq, rk, rv, rs = oracle_grads(x, dout, layer_type, window, vs)
    grad_compare(dq, rq, "dq")
    grad_compare(dk, rk, "dk")
    grad_compare(dv, rv, "dv")
    grad_compare(ds, rs, "dsink")


@pytest.mark.parametrize("sink", [None, float("-inf")])
def test_backward_without_sink(sink):
    lengths = [64, 130]
    log(f"[case] backward without sink ({sink})")
    x = synth.prefill_inputs(lengths, seed=92)
    dout = dout_like(sum(lengths), 93)
    sk = None if sink is None else torch.full((64,), sink, dtype=torch.float32)
    for lt in (SWA, GA):
        dq, dk, dv, ds = run(x, dout, lt, sink=sk)
        rq, rk, rv, rs = oracle_grads(x, dout, lt, sink=sk)
        grad_compare(dq, rq, f"dq lt={lt}")
        grad_compare(dk, rk, f"dk lt={lt}")
        grad_compare(dv, rv, f"dv lt={lt}")
        assert not ds.any(), "dsink without a sink must be 0"


def test_backward_max_seqlen_bounds_rows():
    """Tokens past max_seqlen are left unwritten and contribute nothing."""
    lengths = [40, 90]
    log("[case] backward max_seqlen 48")
    x = synth.prefill_inputs(lengths, seed=94)
    dout = dout_like(130, 95)
    dims = B.make_dims()
    q, k, v, cu = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens)
    out, lse = B.prefill(q, k, v, cu, 48, GA, sink=to_dev(x.sink))
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ds = torch.empty(64, dtype=torch.float32, device=DEV)
    ws = torch.empty(B.mimo_attn_prefill_backward_workspace_size(dims, 130) // 4 + 4, dtype=torch.float32, device=DEV)
    B.mimo_attn_prefill_backward(dims, GA, q, k, v, out, lse, to_dev(dout), cu, 2, 48, 130, to_dev(x.sink), dq, dk, dv,
                                 ds, ws)
    torch.cuda.synchronize()
    keep = torch.tensor(list(range(0, 40)) + list(range(40, 88)))
    drop = torch.tensor(list(range(88, 130)))
    assert torch.isnan(dq[drop.to(DEV)].float()).all() and torch.isnan(dk[drop.to(DEV)].float()).all()
    # the oracle on the truncated sequences (40 and 48 tokens)
    y = synth.PrefillInputs(x.q[keep], x.k[keep], x.v[keep], x.sink, synth.cu_from_lengths([40, 48]), [40, 48])
    rq, rk, rv, rs = oracle_grads(y, dout[keep], GA)
    kd = keep.to(DEV)
    grad_compare(dq[kd], rq, "dq max_seqlen")
    grad_compare(dk[kd], rk, "dk max_seqlen")
    grad_compare(dv[kd], rv, "dv max_seqlen")
    grad_compare(ds, rs, "dsink max_seqlen")


def assert_vanishing(x, dout, dq, dk, what=""):
    """dq and dk of one-token sequences without a sink at value_scale 1, whose
    exact values are zero: the only weight is exactly 1 and the output is v, so
    dS = dP - D = 0.  What is left is the fp32 rounding of two 128-term dot
    products of bf16 values (dP by the MFMA, D by the row-dot kernel), each
    within 128 u sum|dO v| with u = 2^-24 (the bound below allows twice both)."""
    q, k, v, do = (t.float().numpy().astype(np.float64) for t in (x.q, x.k, x.v, dout))
    T = q.shape[0]
    g = np.arange(64) // 16
    ds_bound = 4 * 128 * 2.0 ** -24 * np.abs(do * v[:, g]).sum(-1)            # [T][64]
    q_bound = SCALE * ds_bound[..., None] * np.abs(k[:, g])                     # dq = scale dS k
    k_bound = SCALE * (ds_bound[..., None] * np.abs(q)).reshape(T, 4, 16, 192).sum(2)
    got_q = dq.float().cpu().numpy().astype(np.float64)
    got_k = dk.float().cpu().numpy().astype(np.float64)
    log(f"[parity] {what}one key: |dq| max {np.abs(got_q).max():.2e} (bound {q_bound.max():.2e}), "
        f"|dk| max {np.abs(got_k).max():.2e} (bound {k_bound.max():.2e})")
    assert (np.abs(got_q) <= q_bound).all(), "dq of a lone key does not vanish"
    assert (np.abs(got_k) <= k_bound).all(), "dk of a lone key does not vanish"


def test_backward_one_key_without_sink_vanishes():
    """One-token sequences without a sink and value_scale 1: dq and dk vanish
    (within the rounding bound of assert_vanishing); dv = sum over the group of
    dO, against the oracle."""
    lengths = [1, 1, 1, 1, 1]
    log(f"[case] backward one key, no sink: lengths {lengths}")
    x = synth.prefill_inputs(lengths, seed=98)
    dout = dout_like(len(lengths), 99)
    dq, dk, dv, ds = run(x, dout, GA, value_scale=1.0, sink=None)
    rq, rk, rv, _ = oracle_grads(x, dout, GA, value_scale=1.0, sink=None)
    assert not rq.any() and not rk.any(), "the oracle's dq and dk of lone keys are not zero"
    grad_compare(dv, rv, "dv one key")
    assert not ds.any(), "dsink without a sink must be 0"
    assert_vanishing(x, dout, dq, dk)


def test_backward_ga_1x32768_sampled():
    """GA 1 x 32768 (the prefill benchmark input): sampled dq rows, and dk/dv
    rows near the end of the sequence (whose receivers the oracle can afford)."""
    L = 32768
    log("[case] backward GA 1x32768 sampled")
    x = synth.prefill_inputs([L], seed=0, device=DEV)
    dout = torch.randn((L, 64, 128), generator=torch.Generator(device=DEV).manual_seed(96), device=DEV).to(torch.bfloat16)
    out, lse = B.prefill(x.q, x.k, x.v, x.cu_seqlens, L, GA, sink=x.sink)
    dq, dk, dv, ds = B.prefill_backward(x.q, x.k, x.v, out, lse, dout, x.cu_seqlens, L, GA, sink=x.sink)
    torch.cuda.synchronize()
    qr = np.array([0, 1, 15, 16, 31, 32, 4095, 16383, 32766, 32767])
    kr = np.array([32704, 32735, 32736, 32767])
    rq, rk, rv, _ = orc().prefill_backward(bits(x.q), bits(x.k), bits(x.v), bits(dout), x.cu_seqlens.cpu().numpy(),
                                           layer_type=GA, scale=SCALE, sink=sink_array(x.sink), q_rows=qr, kv_rows=kr,
                                           want_dsink=False, stored_out=True)
    grad_compare(dq[torch.tensor(qr, device=DEV)], rq, "GA 32K dq sampled")
    grad_compare(dk[torch.tensor(kr, device=DEV)], rk, "GA 32K dk sampled")
    grad_compare(dv[torch.tensor(kr, device=DEV)], rv, "GA 32K dv sampled")
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dq.float()).all() and torch.isfinite(ds).all()


def test_backward_swa_4x8192_sampled():
    """SWA 4 x 8192 (the prefill benchmark input): sampled rows and dsink."""
    L = 8192
    log("[case] backward SWA 4x8192 sampled")
    x = synth.prefill_inputs([L] * 4, seed=0, device=DEV)
    dout = torch.randn((4 * L, 64, 128), generator=torch.Generator(device=DEV).manual_seed(97),
                       device=DEV).to(torch.bfloat16)
    out, lse = B.prefill(x.q, x.k, x.v, x.cu_seqlens, L, SWA, sink=x.sink)
    dq, dk, dv, ds = B.prefill_backward(x.q, x.k, x.v, out, lse, dout, x.cu_seqlens, L, SWA, sink=x.sink)
    torch.cuda.synchronize()
    rows = np.array([s * L + p for s in range(4) for p in (0, 1, 127, 128, 129, 4000, 8063, 8064, 8191)])
    rq, rk, rv, rs = orc().prefill_backward(bits(x.q), bits(x.k), bits(x.v), bits(dout), x.cu_seqlens.cpu().numpy(),
                                            layer_type=SWA, scale=SCALE, sink=sink_array(x.sink), q_rows=rows,
                                            kv_rows=rows, want_dsink=True, stored_out=True)
    idx = torch.tensor(rows, device=DEV)
    grad_compare(dq[idx], rq, "SWA 4x8192 dq sampled")
    grad_compare(dk[idx], rk, "SWA 4x8192 dk sampled")
    grad_compare(dv[idx], rv, "SWA 4x8192 dv sampled")
    grad_compare(ds, rs, "SWA 4x8192 dsink")
