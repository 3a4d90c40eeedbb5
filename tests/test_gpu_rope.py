"""GPU parity of the rotary embedding (mimo_rope_apply) through the C ABI
against the fp64 oracle.

Bar per element of a rotated pair (x, y): |gpu - ref| <= 2^-8 |ref| +
2^-20 (|x| + |y|) -- the bf16 rounding of the exact value (half an ulp, 2^-9
relative) with room for the fp32 products when the two terms cancel; the
dims past rotary_dim must come back bit for bit.
"""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = float(np.float32(synth.SOFTMAX_SCALE))


def check_rope(got, x, ref, rd, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    xin = synth.bf16_bits(x).astype(np.uint32)
    xf = (xin << 16).view(np.float32).astype(np.float64)
    half = rd // 2
    pair = np.concatenate([xf[..., half:rd], xf[..., :half]], axis=-1)  # the partner of each rotated element
    bound = 2.0 ** -8 * np.abs(ref[..., :rd]) + 2.0 ** -20 * (np.abs(xf[..., :rd]) + np.abs(pair))
    err = np.abs(g[..., :rd] - ref[..., :rd])
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    log(f"[parity] {what}: worst error / bound = {worst:.3f}")
    assert (err <= bound).all(), f"{what}: rotated dims outside the bar ({worst:.3f} x bound)"
    assert np.array_equal(synth.bf16_bits(got)[..., rd:], synth.bf16_bits(x)[..., rd:]), f"{what}: pass-through dims"


POS = [0, 1, 2, 127, 128, 129, 4095, 32767, 131071, 262143]


@pytest.mark.parametrize("rd,theta", [(64, 1e4), (64, 5e6), (192, 1e4), (16, 1e6)])
def test_rope_against_oracle(rd, theta):
    T = 257
    log(f"[case] rope rd={rd} theta={theta}")
    g = torch.Generator().manual_seed(rd)
    q = torch.randn((T, 64, 192), generator=g).to(torch.bfloat16)
    k = torch.randn((T, 4, 192), generator=g).to(torch.bfloat16)
    pos = np.array(POS + list(torch.randint(0, 262144, (T - len(POS),), generator=g).numpy()), np.int32)
    qd, kd = to_dev(q), to_dev(k)
    B.rope_apply(qd, kd, torch.tensor(pos, device=DEV), theta, rd)
    torch.cuda.synchronize()
    rq, rk = orc().rope(bits(q), bits(k), pos, theta=float(np.float32(theta)), rotary_dim=rd)
    check_rope(qd, q, rq, rd, f"q rd={rd} theta={theta}")
    check_rope(kd, k, rk, rd, f"k rd={rd} theta={theta}")


def test_rope_q_only_and_k_only():
    T = 40
    log("[case] rope q only / k only")
    g = torch.Generator().manual_seed(5)
    q = torch.randn((T, 64, 192), generator=g).to(torch.bfloat16)
    k = torch.randn((T, 4, 192), generator=g).to(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int32) * 1000
    qd, kd = to_dev(q), to_dev(k)
    B.rope_apply(qd, None, to_dev(pos), 1e4, 64)
    B.rope_apply(None, kd, to_dev(pos), 1e4, 64)
    torch.cuda.synchronize()
    rq, rk = orc().rope(bits(q), bits(k), pos.numpy(), theta=1e4, rotary_dim=64)
    check_rope(qd, q, rq, 64, "q only")
    check_rope(kd, k, rk, 64, "k only")


@pytest.mark.parametrize("layer_type", [0, 1])
def test_rope_then_prefill(layer_type):
    """q and k rotated at their positions, then prefill: against the oracle's
    prefill of the oracle's rotation rounded to bf16."""
    lengths = [300, 129, 17]
    log(f"[case] rope then prefill layer={layer_type}")
    x = synth.prefill_inputs(lengths, seed=98)
    pos = np.concatenate([np.arange(L) for L in lengths]).astype(np.int32)
    theta = 5e6 if layer_type == 1 else 1e4
    qd, kd = to_dev(x.q), to_dev(x.k)
    B.rope_apply(qd, kd, torch.tensor(pos, device=DEV), theta, 64)
    out, lse = B.prefill(qd, kd, to_dev(x.v), to_dev(x.cu_seqlens), max(lengths), layer_type, sink=to_dev(x.sink))
    torch.cuda.synchronize()
    rq, rk = orc().rope(bits(x.q), bits(x.k), pos, theta=theta, rotary_dim=64)
    qb = synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16))
    kb = synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16))
    ro, rl = orc().prefill(qb, kb, bits(x.v), x.cu_seqlens.numpy(), layer_type=layer_type, scale=SCALE,
                           sink=sink_array(x.sink))
    compare(out, lse, ro, rl, f"rope + prefill layer {layer_type}")


def test_rope_ga_1x32768_sampled():
    """The GA prefill input (1 x 32768), rotary dims 64, theta 5e6: sampled rows."""
    L = 32768
    log("[case] rope 1x32768 sampled")
    x = synth.prefill_inputs([L], seed=0, device=DEV)
    q0, k0 = x.q.clone(), x.k.clone()
    B.rope_apply(x.q, x.k, torch.arange(L, dtype=torch.int32, device=DEV), 5e6, 64)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2, 100, 4095, 16384, 32766, 32767])
    idx = torch.tensor(rows, device=DEV)
    rq, rk = orc().rope(bits(q0[idx]), bits(k0[idx]), rows.astype(np.int32), theta=5e6, rotary_dim=64)
    check_rope(x.q[idx], q0[idx], rq, 64, "q 32K sampled")
    check_rope(x.k[idx], k0[idx], rk, 64, "k 32K sampled")
