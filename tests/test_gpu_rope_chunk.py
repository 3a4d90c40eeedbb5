"""Chunked prefill with the rotary embedding fused in (mimo_attn_prefill_chunk_rope)
through the C ABI (model doc "MiMo-V2-Flash", MiMoV2FlashConfig: rope_parameters
/ rope_theta; MiMoV2FlashModel.forward: position_ids, past_key_values):
  * bit for bit equal to mimo_rope_apply on copies of the chunk's q and k
    followed by mimo_attn_prefill_chunk(_paged) (outputs, LSE, and k_rot
    against the rotated k), wherever both run the same kernel (a streaming-
    window SWA chunk rotating more than 64 dims runs the tiled kernel instead);
  * within the attention bars of the oracle's chunked prefill of the oracle's
    rotation rounded to bf16, over caches filled with seeded keys (a cache holds
    post-RoPE keys; their values are arbitrary here).
Covers the streaming SWA kernel (window 129, rotary dims up to 64), the tiled SWA
kernel (window 300, and rotary dim 192 at window 129), GA over the contiguous
and the paged pool, positions ctx + i and positions offset from them, and
k_rot aliasing k."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev
from test_gpu_chunk import _caches, _fill, _split

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"
LENGTHS = [300, 170, 64, 129, 260, 600]
CACHED = [0, 1, 63, 128, 131, 512]


def _positions(cached, rest, offset):
    return np.concatenate([np.arange(n) + c + offset for c, n in zip(cached, rest)]).astype(np.int32)


def _paged(x, kh, vh, base, lengths, P=16, seed=3):
    """The contiguous pool's rows of each sequence on shuffled pages (GPU and host copies)."""
    table, npages = synth.paged_block_table(lengths, P, seed=seed)
    tb = table.numpy()
    kp = np.zeros((npages * P, 4, 192), np.uint16)
    vp = np.zeros((npages * P, 4, 128), np.uint16)
    b0 = base.cpu().numpy()
    for b, L in enumerate(lengths):
        for j0 in range(0, L, P):
            n = min(P, L - j0)
            page = int(tb[b, j0 // P])
            kp[page * P:page * P + n] = kh[b0[b] + j0:b0[b] + j0 + n]
            vp[page * P:page * P + n] = vh[b0[b] + j0:b0[b] + j0 + n]
    as_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return as_dev(kp), as_dev(vp), table, kp, vp


@pytest.mark.parametrize("lt,window,rd,theta,offset,paged", [
    (SWA, 129, 64, 1e4, 0, False),      # streaming SWA kernel
    (SWA, 129, 32, 1e4, 5000, False),   # position ids offset from ctx + i
    (SWA, 300, 64, 1e4, 0, False),      # tiled SWA kernel
    (SWA, 129, 192, 1e6, 0, False),     # every dim rotates: tiled SWA kernel
    (GA, 129, 64, 5e6, 0, False),
    (GA, 129, 64, 5e6, 0, True),        # paged pool
    (GA, 129, 128, 5e6, 100000, True),
])
def test_chunk_rope_equals_separate_and_oracle(lt, window, rd, theta, offset, paged):
    log(f"[case] chunked fused rope lt={lt} W={window} rd={rd} theta={theta} offset={offset} paged={paged}")
    x = synth.prefill_inputs(LENGTHS, seed=140 + rd + lt)
    dims = B.make_dims(sliding_window=window)
    kc, vc, base, cap = _caches(lt, LENGTHS, window=window)
    kh, vh = _fill(x, lt, CACHED, kc, vc, base, cap, window=window)
    table = None
    if paged:
        kc, vc, table, kh, vh = _paged(x, kh, vh, base, LENGTHS)
    _, new, rest = _split(x, CACHED)
    cu_new = synth.cu_from_lengths(rest, DEV)
    ctx = torch.tensor(CACHED, dtype=torch.int32, device=DEV)
    pos = _positions(CACHED, rest, offset)
    posd = torch.tensor(pos, device=DEV)
    q, k, v, sink = to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]), to_dev(x.sink)
    kw = dict(block_table=table.to(DEV), page_size=16) if paged else dict(kv_base=base)
    of, lf, krot = B.prefill_chunk_rope(q, k, v, posd, cu_new, max(rest), kc, vc, ctx, lt, theta, rd, sink=sink,
                                        dims=dims, **kw)
    q2, k2 = q.clone(), k.clone()
    B.rope_apply(q2, k2, posd, theta, rd)
    if paged:
        os_, ls = B.prefill_chunk_paged(q2, k2, v, cu_new, max(rest), kc, vc, table.to(DEV), 16, ctx, sink=sink,
                                        dims=dims)
    else:
        os_, ls = B.prefill_chunk(q2, k2, v, cu_new, max(rest), kc, vc, ctx, lt, sink=sink, kv_base=base, dims=dims)
    torch.cuda.synchronize()
    assert torch.equal(q, to_dev(x.q[new])) and torch.equal(k, to_dev(x.k[new])), "fused RoPE modified q or k"
    assert torch.equal(krot, k2), "k_rot differs from mimo_rope_apply's k"
    # Windows up to 145 keys run the streaming SWA kernel, which rotates at most 64 dims in its blocks; a wider
    # rotation there goes to the tiled kernel, so the separate path (streaming) sums in another order.
    if not (lt == SWA and window <= 145 and rd > 64):
        assert torch.equal(of, os_) and torch.equal(lf, ls), "fused chunk differs from rope + chunk"
    rq, rk = orc().rope(bits(x.q[new]), bits(x.k[new]), pos, theta=float(np.float32(theta)), rotary_dim=rd)
    qb = synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16))
    kb = synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16))
    if paged:
        ro, rl = orc().prefill_chunk_paged(qb, kb, bits(x.v[new]), cu_new.cpu().numpy(), kh, vh, table.numpy(), 16,
                                           ctx.cpu().numpy(), scale=SCALE, sink=sink_array(x.sink))
    else:
        ro, rl = orc().prefill_chunk(qb, kb, bits(x.v[new]), cu_new.cpu().numpy(), kh, vh, ctx.cpu().numpy(),
                                     layer_type=lt, window=window, scale=SCALE, sink=sink_array(x.sink),
                                     kv_base=None if base is None else base.cpu().numpy())
    compare(of, lf, ro, rl, f"chunked fused rope lt={lt} W={window} rd={rd} paged={paged}")


def test_chunk_rope_k_rot_may_alias_k():
    log("[case] chunked fused rope, k_rot == k")
    x = synth.prefill_inputs(LENGTHS, seed=150)
    kc, vc, base, cap = _caches(GA, LENGTHS)
    _fill(x, GA, CACHED, kc, vc, base, cap)
    _, new, rest = _split(x, CACHED)
    cu_new = synth.cu_from_lengths(rest, DEV)
    ctx = torch.tensor(CACHED, dtype=torch.int32, device=DEV)
    posd = torch.tensor(_positions(CACHED, rest, 0), device=DEV)
    q, k, v, sink = to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]), to_dev(x.sink)
    of, lf, krot = B.prefill_chunk_rope(q, k, v, posd, cu_new, max(rest), kc, vc, ctx, GA, 5e6, 64, sink=sink,
                                        kv_base=base, k_rot=k)
    q2, k2 = to_dev(x.q[new]), to_dev(x.k[new])
    B.rope_apply(q2, k2, posd, 5e6, 64)
    os_, ls = B.prefill_chunk(q2, k2, v, cu_new, max(rest), kc, vc, ctx, GA, sink=sink, kv_base=base)
    torch.cuda.synchronize()
    assert krot.data_ptr() == k.data_ptr() and torch.equal(k, k2)
    assert torch.equal(of, os_) and torch.equal(lf, ls)
