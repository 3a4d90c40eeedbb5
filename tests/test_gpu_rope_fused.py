"""Prefill with the rotary embedding fused in (mimo_attn_prefill_rope) through
the C ABI (model doc "MiMo-V2-Flash", MiMoV2FlashConfig: rope_parameters /
rope_theta; MiMoV2FlashModel.forward: position_ids):
  * bit for bit equal to mimo_rope_apply on copies of q and k followed by
    mimo_attn_prefill (outputs, LSE, and k_rot against the rotated k);
  * within the attention bars of the oracle's prefill of the oracle's
    rotation (oracle_rope, pinned to Transformers' rotary code) rounded to bf16;
  * decode after appending k_rot equals the fused prefill's row at that
    position (the caches hold post-RoPE keys).
Covers the streaming SWA kernel (window 129), the tiled SWA kernel (window
300) and GA, rotary dims 32, 64 and 192, position ids that are not 0..L-1, and
k_rot aliasing k."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = float(np.float32(synth.SOFTMAX_SCALE))


def positions_for(lengths, offset=0):
    return np.concatenate([np.arange(L) + offset for L in lengths]).astype(np.int32)


def run_fused_and_separate(x, lt, window, pos, theta, rd):
    dims = B.make_dims(sliding_window=window)
    q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
    posd = torch.tensor(pos, device=DEV)
    of, lf, krot = B.prefill_rope(q, k, v, posd, cu, max(x.lengths), lt, theta, rd, sink=sink, dims=dims)
    q2, k2 = q.clone(), k.clone()
    B.rope_apply(q2, k2, posd, theta, rd)
    os_, ls = B.prefill(q2, k2, v, cu, max(x.lengths), lt, sink=sink, dims=dims)
    torch.cuda.synchronize()
    assert torch.equal(q, to_dev(x.q)) and torch.equal(k, to_dev(x.k)), "fused RoPE modified q or k"
    return (of, lf, krot), (os_, ls, k2)


@pytest.mark.parametrize("lt,window,rd,theta,offset", [
    (0, 129, 64, 1e4, 0),      # streaming SWA kernel, the library's SWA theta
    (0, 129, 32, 1e4, 7000),   # position ids offset from the token order
    (0, 300, 64, 1e4, 0),      # tiled SWA kernel
    (1, 129, 64, 5e6, 0),      # GA, the library's GA theta
    (1, 129, 192, 1e6, 0),     # every dim rotates
    (1, 129, 64, 5e6, 100000),
])
def test_fused_equals_separate_and_oracle(lt, window, rd, theta, offset):
    lengths = [1, 130, 257, 600, 16]
    log(f"[case] fused rope lt={lt} W={window} rd={rd} theta={theta} offset={offset}")
    x = synth.prefill_inputs(lengths, seed=120 + rd + lt)
    pos = positions_for(lengths, offset)
    (of, lf, krot), (os_, ls, k2) = run_fused_and_separate(x, lt, window, pos, theta, rd)
    assert torch.equal(krot, k2), "k_rot differs from mimo_rope_apply's k"
    assert torch.equal(of, os_) and torch.equal(lf, ls), "fused prefill differs from rope + prefill"
    rq, rk = orc().rope(bits(x.q), bits(x.k), pos, theta=float(np.float32(theta)), rotary_dim=rd)
    qb = synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16))
    kb = synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16))
    ro, rl = orc().prefill(qb, kb, bits(x.v), x.cu_seqlens.numpy(), layer_type=lt, window=window, scale=SCALE,
                           sink=sink_array(x.sink))
    compare(of, lf, ro, rl, f"fused rope lt={lt} W={window} rd={rd}")


def test_k_rot_may_alias_k():
    lengths = [200, 77]
    x = synth.prefill_inputs(lengths, seed=130)
    pos = positions_for(lengths)
    log("[case] fused rope, k_rot == k")
    q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
    posd = torch.tensor(pos, device=DEV)
    of, lf, krot = B.prefill_rope(q, k, v, posd, cu, 200, 1, 5e6, 64, sink=sink, k_rot=k)
    q2, k2 = to_dev(x.q), to_dev(x.k)
    B.rope_apply(q2, k2, posd, 5e6, 64)
    os_, ls = B.prefill(q2, k2, v, cu, 200, 1, sink=sink)
    torch.cuda.synchronize()
    assert krot.data_ptr() == k.data_ptr() and torch.equal(k, k2)
    assert torch.equal(of, os_) and torch.equal(lf, ls)


@pytest.mark.parametrize("lt", [0, 1])
def test_decode_after_fused_prefill_and_append(lt):
    """Prefill positions 0..p-1 with fused RoPE, append k_rot, rotate the decode
    token's q and k at position p (mimo_rope_apply), decode: equals row p of a
    fused prefill over 0..p."""
    L = 333
    theta = 5e6 if lt == 1 else 1e4
    x = synth.prefill_inputs([L], seed=131 + lt)
    log(f"[case] fused rope prefill, append, decode lt={lt}")
    pos = np.arange(L, dtype=np.int32)
    q, k, v, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.sink))
    full, _, _ = B.prefill_rope(q, k, v, torch.tensor(pos, device=DEV), to_dev(x.cu_seqlens), L, lt, theta, 64,
                                sink=sink)
    flse = B.prefill_rope(q, k, v, torch.tensor(pos, device=DEV), to_dev(x.cu_seqlens), L, lt, theta, 64,
                          sink=sink)[1]
    p = L - 1
    cu_p = torch.tensor([0, p], dtype=torch.int32, device=DEV)
    _, _, krot = B.prefill_rope(q[:p].contiguous(), k[:p].contiguous(), v[:p].contiguous(),
                                torch.tensor(pos[:p], device=DEV), cu_p, p, lt, theta, 64, sink=sink)
    if lt == 0:
        kc = torch.zeros((1, 128, 4, 192), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros((1, 128, 4, 128), dtype=torch.bfloat16, device=DEV)
        base = cap = None
    else:
        kc = torch.zeros((L + 4, 4, 192), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros((L + 4, 4, 128), dtype=torch.bfloat16, device=DEV)
        base = torch.zeros(1, dtype=torch.int64, device=DEV)
        cap = torch.full((1,), L + 4, dtype=torch.int64, device=DEV)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.kv_append(krot, v[:p].contiguous(), cu_p, zero, kc, vc, lt, kv_base=base, kv_capacity=cap)
    qn, kn = q[p:p + 1].clone(), k[p:p + 1].clone()
    B.rope_apply(qn, kn, torch.tensor([p], dtype=torch.int32, device=DEV), theta, 64)
    out, lse = B.decode(qn, kn, v[p:p + 1].contiguous(), kc, vc, torch.tensor([p], dtype=torch.int32, device=DEV), p,
                        lt, sink=sink, kv_base=base)
    torch.cuda.synchronize()
    compare(out, lse, full[p:p + 1].double().cpu().numpy(), flse[p:p + 1].double().cpu().numpy(),
            f"decode after fused prefill lt={lt}")
