"""GPU parity of the FP8 (OCP E4M3) GA cache through the C ABI: quantised append
bit for bit against the oracle, decode against the fp64 oracle over the
oracle's own copy of the pool.  Bars as in gpu_util."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
GA = 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"
# Per-KV-head scales: an amax calibration of N(0,1) values (about 4.5 / 448) and
# values that are not powers of two.
K_SCALE = np.float32([0.01, 0.0173, 0.0071, 0.031])
V_SCALE = np.float32([0.0105, 0.0063, 0.022, 0.0149])
# Uniform random codes span +-448: scales that keep keys within +-9 and values
# within +-4.5, the magnitudes of N(0,1) data the output bar is derived for.
RAND_K_SCALE = np.float32([1 / 64, 1 / 90, 1 / 50, 1 / 70])
RAND_V_SCALE = np.float32([1 / 120, 1 / 160, 1 / 100, 1 / 200])


def _pools(rows):
    return (torch.zeros((rows, 4, 192), dtype=torch.uint8, device=DEV),
            torch.zeros((rows, 4, 128), dtype=torch.uint8, device=DEV))


def test_fp8_append_bytes():
    """Ragged bulk append, then decode-step appends, with elements that
    saturate; a sequence past its capacity is skipped.  Codes bit for bit."""
    lengths = [1, 37, 300, 5]
    caps = [8, 40, 310, 4]  # the last sequence does not fit
    log(f"[case] FP8 append lengths {lengths}")
    x = synth.prefill_inputs(lengths, seed=70)
    k = x.k.clone()
    k[3, 2, :4] = torch.tensor([1e4, -1e4, 500.0, 448.0 * 0.0173], dtype=torch.bfloat16)
    base = np.concatenate([[3], 3 + np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(base[-1]) + caps[-1]
    kc, vc = _pools(rows)
    ks, vs = torch.tensor(K_SCALE, device=DEV), torch.tensor(V_SCALE, device=DEV)
    base_d, cap_d = torch.tensor(base, device=DEV), torch.tensor(caps, dtype=torch.int64, device=DEV)
    zeros = torch.zeros(len(lengths), dtype=torch.int32, device=DEV)
    B.kv_append_fp8(to_dev(k), to_dev(x.v), to_dev(x.cu_seqlens), zeros, kc, vc, base_d, cap_d, ks, vs)
    kr, vr = np.zeros((rows, 4, 192), np.uint8), np.zeros((rows, 4, 128), np.uint8)
    st = orc().kv_append_fp8(bits(k), bits(x.v), x.cu_seqlens.numpy(), np.zeros(len(lengths), np.int32), kr, vr,
                             base, np.asarray(caps, np.int64), K_SCALE, V_SCALE)
    assert st == 2
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr), "FP8 bulk append codes"
    # three decode-step appends at positions L_b, L_b + 1, L_b + 2 (the last sequence stays refused)
    for step in range(3):
        d = synth.decode_inputs([0] * len(lengths), GA, seed=71 + step)
        ctx = np.asarray(lengths, np.int32) + step
        cu = np.arange(len(lengths) + 1, dtype=np.int32)
        B.kv_append_fp8(to_dev(d.k_new), to_dev(d.v_new), torch.tensor(cu, device=DEV), torch.tensor(ctx, device=DEV),
                        kc, vc, base_d, cap_d, ks, vs)
        orc().kv_append_fp8(bits(d.k_new), bits(d.v_new), cu, ctx, kr, vr, base, np.asarray(caps, np.int64),
                            K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr), "FP8 step append codes"
    # packed token 3 is position 2 of sequence 1
    assert kr[base[1] + 2, 2, 0] == 0x7E and kr[base[1] + 2, 2, 1] == 0xFE  # saturated


def _every_bf16_token_rows(width):
    """Every finite bf16 bit pattern (the 254 NaN patterns left out), laid out
    row-major in [T][4][width] tokens (zero-padded)."""
    pats = np.arange(65536, dtype=np.uint32)
    exp, man = (pats >> 7) & 0xFF, pats & 0x7F
    pats = pats[~((exp == 0xFF) & (man != 0))].astype(np.uint16)
    T = -(-pats.size // (4 * width))
    a = np.zeros(T * 4 * width, np.uint16)
    a[:pats.size] = pats
    return a.reshape(T, 4, width)


@pytest.mark.parametrize("k_scale,v_scale", [
    ([1.0, 0.01, 4.5 / 448, 0.7], [448.0, 3.0, 1.0 / 448, 0.1]),
    ([1e-30, 3e38, 1e-38, 1.9999999], [0.0173, 7.0, 1e-20, 1e20]),
])
def test_fp8_append_every_bf16_value(k_scale, v_scale):
    """Every finite bf16 value through the quantising append (as K and as V),
    under ordinary, tiny and huge per-head scales: codes bit for bit against
    the oracle's E4M3(clamp(x / scale)) with the fp32 IEEE quotient."""
    ks, vs = np.float32(k_scale), np.float32(v_scale)
    kb, vb = _every_bf16_token_rows(192), _every_bf16_token_rows(128)
    T = max(kb.shape[0], vb.shape[0])
    kh = np.zeros((T, 4, 192), np.uint16)
    vh = np.zeros((T, 4, 128), np.uint16)
    kh[:kb.shape[0]], vh[:vb.shape[0]] = kb, vb
    log(f"[case] FP8 append of every bf16 value: {T} tokens, K scales {ks.tolist()}, V scales {vs.tolist()}")
    as_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    kc, vc = _pools(T)
    cu = np.array([0, T], np.int32)
    base, caps = np.zeros(1, np.int64), np.array([T], np.int64)
    B.kv_append_fp8(as_dev(kh), as_dev(vh), torch.tensor(cu, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV),
                    kc, vc, torch.tensor(base, device=DEV), torch.tensor(caps, device=DEV), torch.tensor(ks, device=DEV),
                    torch.tensor(vs, device=DEV))
    kr, vr = np.zeros((T, 4, 192), np.uint8), np.zeros((T, 4, 128), np.uint8)
    orc().kv_append_fp8(kh, vh, cu, np.zeros(1, np.int32), kr, vr, base, caps, ks, vs)
    torch.cuda.synchronize()
    gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
    nk, nv = int((gk != kr).sum()), int((gv != vr).sum())
    assert nk == 0 and nv == 0, f"{nk} K and {nv} V codes differ from the oracle's"


@pytest.mark.parametrize("split", [0, 96])
def test_fp8_decode_against_oracle(split):
    """Contexts on and around tile and split boundaries; the pool holds N(0,1)
    keys and values quantised by the append (the oracle quantises its own copy)."""
    ctx = [0, 1, 31, 32, 33, 95, 96, 97, 2047, 2048, 2049, 5000]
    log(f"[case] FP8 decode ctx {ctx} split {split}")
    lengths = [max(c, 1) for c in ctx]
    x = synth.prefill_inputs(lengths, seed=72)
    d = synth.decode_inputs(ctx, GA, seed=73)
    caps = [c + 2 for c in lengths]
    base = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(sum(caps))
    kc, vc = _pools(rows)
    kr, vr = np.zeros((rows, 4, 192), np.uint8), np.zeros((rows, 4, 128), np.uint8)
    ks, vs = torch.tensor(K_SCALE, device=DEV), torch.tensor(V_SCALE, device=DEV)
    base_d, cap_d = torch.tensor(base, device=DEV), torch.tensor(caps, dtype=torch.int64, device=DEV)
    cached = np.asarray(ctx, np.int32)
    cu = x.cu_seqlens.numpy()
    pre = np.concatenate([np.arange(cu[b], cu[b] + c) for b, c in enumerate(ctx)]).astype(np.int64)
    cu_pre = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    zeros = np.zeros(len(ctx), np.int32)
    B.kv_append_fp8(to_dev(x.k[pre]), to_dev(x.v[pre]), torch.tensor(cu_pre, device=DEV),
                    torch.tensor(zeros, device=DEV), kc, vc, base_d, cap_d, ks, vs)
    assert orc().kv_append_fp8(bits(x.k[pre]), bits(x.v[pre]), cu_pre, zeros, kr, vr, base,
                               np.asarray(caps, np.int64), K_SCALE, V_SCALE) == 0
    out, lse = B.decode_fp8(to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), kc, vc, base_d, ks, vs,
                            torch.tensor(cached, device=DEV), max(ctx), sink=to_dev(d.sink), split_tokens=split)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr)
    ro, rl = orc().decode_fp8(bits(d.q), bits(d.k_new), bits(d.v_new), kr, vr, base, K_SCALE, V_SCALE, cached,
                              scale=SCALE, sink=sink_array(d.sink))
    compare(out, lse, ro, rl, f"FP8 decode split {split}")


@pytest.mark.parametrize("sink", [None, 30.0])
def test_fp8_decode_sinks_and_value_scale(sink):
    """No sink, and a dominating sink; value_scale 0.707."""
    ctx = [0, 17, 600]
    log(f"[case] FP8 decode sink {sink}")
    d = synth.decode_inputs(ctx, GA, seed=74)
    rows = int(d.k_cache.shape[0])
    kr = synth.random_e4m3_codes((rows, 4, 192), seed=75)
    vr = synth.random_e4m3_codes((rows, 4, 128), seed=76)
    ks, vs = RAND_K_SCALE, RAND_V_SCALE
    sk = None if sink is None else torch.full((64,), sink, dtype=torch.float32)
    dims = B.make_dims(value_scale=0.707)
    out, lse = B.decode_fp8(to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(kr), to_dev(vr),
                            to_dev(d.kv_base), torch.tensor(ks, device=DEV), torch.tensor(vs, device=DEV),
                            to_dev(d.ctx_lens), max(ctx), sink=to_dev(sk), dims=dims)
    torch.cuda.synchronize()
    ro, rl = orc().decode_fp8(bits(d.q), bits(d.k_new), bits(d.v_new), kr.numpy(), vr.numpy(), d.kv_base.numpy(),
                              ks, vs, d.ctx_lens.numpy(), scale=SCALE, value_scale=float(np.float32(0.707)),
                              sink=sink_array(sk))
    compare(out, lse, ro, rl, f"FP8 decode sink {sink}")


def test_fp8_decode_b128_long_contexts_sampled():
    """Decode step for 128 sequences with contexts U[4096, 262144] (seed 0) over an
    FP8 pool of random codes (22 GB): sampled sequences against the oracle."""
    ctx = synth.long_context_lengths(128, seed=0)
    log(f"[case] FP8 GA decode B=128 ctx U[4096,262144] total {sum(ctx)} tokens")
    d = synth.decode_inputs([0] * 128, GA, seed=0, device=DEV)  # queries, new tokens, sinks
    caps = [c + 4 for c in ctx]
    base = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(sum(caps))
    kc = synth.random_e4m3_codes((rows, 4, 192), seed=1, device=DEV)
    vc = synth.random_e4m3_codes((rows, 4, 128), seed=2, device=DEV)
    ks, vs = RAND_K_SCALE, RAND_V_SCALE
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    out, lse = B.decode_fp8(d.q, d.k_new, d.v_new, kc, vc, torch.tensor(base, device=DEV),
                            torch.tensor(ks, device=DEV), torch.tensor(vs, device=DEV), ctx_d, max(ctx) + 4,
                            sink=d.sink)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    order = np.argsort(ctx)
    for b in (int(order[0]), int(order[-1]), int(order[64])):
        c = ctx[b]
        kr = kc[base[b]:base[b] + c].cpu().numpy()
        vr = vc[base[b]:base[b] + c].cpu().numpy()
        ro, rl = orc().decode_fp8(bits(d.q[b:b + 1]), bits(d.k_new[b:b + 1]), bits(d.v_new[b:b + 1]), kr, vr,
                                  np.zeros(1, np.int64), ks, vs, np.array([c], np.int32), scale=SCALE,
                                  sink=d.sink.cpu().numpy())
        compare(out[b:b + 1], lse[b:b + 1], ro, rl, f"FP8 GA decode seq {b} ctx {c}")
