"""mimo_attn_decode_append against mimo_attn_decode followed by mimo_kv_append.

The fused call must give the same outputs and LSE bit for bit (same kernels and
arithmetic) and leave the caches byte-identical to the two-call sequence: the
SWA ring slot p mod 128 overwritten only after the attention read it, the GA
pool row kv_base[b] + p written only when p < kv_capacity[b].  Parity of the
attention itself with the oracle is covered by the decode tests; this file
pins the fused form to it.
"""
import sys

import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SWA, GA = 0, 1


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _both(lt, ctx, split, full_seq=None):
    x = synth.decode_inputs(ctx, lt, seed=11, device=DEV)
    bsz = len(ctx)
    max_ctx = max(ctx) + 1
    dims = B.make_dims()
    cap = None
    if lt == GA:
        cap = x.kv_capacity.clone()
        if full_seq is not None:
            cap[full_seq] = ctx[full_seq]  # no room for position p: the row must stay untouched
    ws = None
    nbytes = B.mimo_attn_decode_workspace_size(dims, lt, bsz, max_ctx, split)
    if nbytes:
        ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=DEV)
    outs = []
    for fused in (False, True):
        kc, vc = x.k_cache.clone(), x.v_cache.clone()
        out = torch.empty((bsz, 64, 128), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((bsz, 64), dtype=torch.float32, device=DEV)
        if fused:
            B.mimo_attn_decode_append(dims, lt, x.q, x.k_new, x.v_new, kc, vc, x.kv_base, cap, x.ctx_lens, bsz,
                                      max_ctx, split, x.sink, out, lse, ws)
        else:
            B.mimo_attn_decode(dims, lt, x.q, x.k_new, x.v_new, kc, vc, x.kv_base, x.ctx_lens, bsz, max_ctx, split,
                               x.sink, out, lse, ws)
            cu = torch.arange(bsz + 1, dtype=torch.int32, device=DEV)
            B.mimo_kv_append(dims, lt, x.k_new, x.v_new, cu, x.ctx_lens, bsz, bsz, kc, vc, x.kv_base, cap)
        torch.cuda.synchronize()
        outs.append((out, lse, kc, vc))
    return x, outs


@pytest.mark.parametrize("lt,ctx,split,full", [
    (SWA, [0, 1, 127, 128, 129, 300], 0, None),
    (SWA, [5000, 4097, 128 * 40 + 17], 0, None),
    (GA, [0, 1, 63, 64, 65, 300, 2049], 64, None),
    (GA, [4096, 100, 7000], 0, 1),
])
def test_decode_append_equals_decode_then_append(lt, ctx, split, full):
    log(f"[case] decode_append layer={'SWA' if lt == SWA else 'GA'} ctx={ctx} split={split} full={full}")
    x, ((o0, l0, k0, v0), (o1, l1, k1, v1)) = _both(lt, ctx, split, full)
    assert torch.equal(o0, o1), "outputs differ"
    assert torch.equal(l0, l1), "LSE differs"
    assert torch.equal(k0, k1), "K cache differs"
    assert torch.equal(v0, v1), "V cache differs"
    # The new token did land where the append puts it (and nowhere else changed).
    changed = (k1 != x.k_cache).flatten(start_dim=1).any(dim=1) if lt == GA else None
    if lt == GA:
        base = x.kv_base.cpu().tolist()
        rows = {base[b] + c for b, c in enumerate(ctx) if b != full}
        assert set(torch.nonzero(changed).flatten().tolist()) <= rows
        for b, c in enumerate(ctx):
            if b == full:
                assert torch.equal(k1[base[b] + c], x.k_cache[base[b] + c])
            else:
                assert torch.equal(k1[base[b] + c], x.k_new[b]) and torch.equal(v1[base[b] + c], x.v_new[b])
    else:
        for b, c in enumerate(ctx):
            assert torch.equal(k1[b, c % 128], x.k_new[b]) and torch.equal(v1[b, c % 128], x.v_new[b])
