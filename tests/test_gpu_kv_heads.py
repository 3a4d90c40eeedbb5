"""KV-head counts other than the model's 4 (MiMoV2FlashConfig: num_key_value_heads,
grouped-query attention with 16 query heads per KV head): one KV head (a
single wave of the GA decode split workgroup) and five (the split workgroup's
second z-slice holds one working wave and three that exit).  Prefill, decode
and append through the C ABI against the fp64 oracle; appends bit for bit; the
fused decode step with RoPE bit for bit against the rotation and the unfused
step."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, to_dev

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))


@pytest.mark.parametrize("hkv", [1, 5])
@pytest.mark.parametrize("lt", [SWA, GA])
def test_prefill_kv_heads(hkv, lt):
    hq = 16 * hkv
    lengths = [1, 130, 257, 40]
    log(f"[case] prefill lt={lt} hkv={hkv} lengths={lengths}")
    x = synth.prefill_inputs(lengths, seed=70 + hkv, hq=hq, hkv=hkv)
    dims = B.make_dims(num_q_heads=hq, num_kv_heads=hkv)
    out, lse = B.prefill(to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens), max(lengths), lt,
                         sink=to_dev(x.sink), dims=dims)
    torch.cuda.synchronize()
    ro, rl = orc().prefill(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.numpy(), layer_type=lt, scale=SCALE,
                           sink=x.sink.numpy())
    compare(out, lse, ro, rl, f"prefill lt={lt} hkv={hkv}")


@pytest.mark.parametrize("hkv", [1, 5])
@pytest.mark.parametrize("lt", [SWA, GA])
def test_decode_and_append_kv_heads(hkv, lt):
    hq = 16 * hkv
    ctx = [0, 1, 127, 128, 700, 3000]
    log(f"[case] decode + append lt={lt} hkv={hkv} ctx={ctx}")
    x = synth.decode_inputs(ctx, lt, seed=80 + hkv, hq=hq, hkv=hkv, headroom=3)
    dims = B.make_dims(num_q_heads=hq, num_kv_heads=hkv)
    d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "kv_capacity",
                                            "ctx_lens", "sink")}
    for split in (0, 64):
        out, lse = B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], max(ctx), lt,
                            sink=d["sink"], kv_base=d["kv_base"], split_tokens=split, dims=dims)
        torch.cuda.synchronize()
        base = None if x.kv_base is None else x.kv_base.numpy()
        ro, rl = orc().decode(bits(x.q), bits(x.k_new), bits(x.v_new), bits(x.k_cache), bits(x.v_cache),
                              x.ctx_lens.numpy(), layer_type=lt, scale=SCALE, sink=x.sink.numpy(), kv_base=base)
        compare(out, lse, ro, rl, f"decode lt={lt} hkv={hkv} split={split}")
    # Append the new tokens (attend, then append) and compare the caches byte for byte.
    cu = torch.arange(len(ctx) + 1, dtype=torch.int32)
    B.kv_append(d["k_new"], d["v_new"], to_dev(cu), d["ctx_lens"], d["k_cache"], d["v_cache"], lt,
                kv_base=d["kv_base"], kv_capacity=d["kv_capacity"], dims=dims)
    torch.cuda.synchronize()
    kc, vc = bits(x.k_cache).copy(), bits(x.v_cache).copy()
    cap = None if x.kv_capacity is None else x.kv_capacity.numpy()
    assert orc().kv_append(bits(x.k_new), bits(x.v_new), cu.numpy(), x.ctx_lens.numpy(), kc, vc, layer_type=lt,
                           kv_base=base, kv_capacity=cap) == 0
    assert np.array_equal(bits(d["k_cache"]), kc) and np.array_equal(bits(d["v_cache"]), vc), \
        f"append lt={lt} hkv={hkv} differs from the oracle's"
    log(f"[parity] append lt={lt} hkv={hkv}: caches bit-exact")


@pytest.mark.parametrize("hkv", [1, 5])
@pytest.mark.parametrize("lt", [SWA, GA])
def test_decode_append_rope_kv_heads(hkv, lt):
    """The fused decode step with RoPE at one and five KV heads: bit for bit
    against mimo_rope_apply + mimo_attn_decode_append (outputs and caches)."""
    hq = 16 * hkv
    ctx = [0, 1, 127, 128, 700, 3000]
    log(f"[case] decode_append_rope lt={lt} hkv={hkv} ctx={ctx}")
    x = synth.decode_inputs(ctx, lt, seed=90 + hkv, hq=hq, hkv=hkv, headroom=3)
    dims = B.make_dims(num_q_heads=hq, num_kv_heads=hkv)
    d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "kv_capacity",
                                            "ctx_lens", "sink")}
    bsz, max_ctx = len(ctx), max(ctx) + 1
    nbytes = B.mimo_attn_decode_workspace_size(dims, lt, bsz, max_ctx, 64)
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device="cuda") if nbytes else None
    pos = (d["ctx_lens"] + 11).to(torch.int32)
    res = []
    for fused in (True, False):
        kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
        out = torch.empty((bsz, hq, 128), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((bsz, hq), dtype=torch.float32, device="cuda")
        if fused:
            B.mimo_attn_decode_append_rope(dims, lt, d["q"], d["k_new"], d["v_new"], pos, kc, vc, d["kv_base"],
                                           d["kv_capacity"], d["ctx_lens"], bsz, max_ctx, 64, 5e6, 128, d["sink"],
                                           out, lse, ws)
        else:
            q2, k2 = d["q"].clone(), d["k_new"].clone()
            B.rope_apply(q2, k2, pos, 5e6, 128, dims=dims)
            B.mimo_attn_decode_append(dims, lt, q2, k2, d["v_new"], kc, vc, d["kv_base"], d["kv_capacity"],
                                      d["ctx_lens"], bsz, max_ctx, 64, d["sink"], out, lse, ws)
        torch.cuda.synchronize()
        res.append((out, lse, kc, vc))
    (of, lf, kf, vf), (os_, ls, ks, vs) = res
    assert torch.equal(of, os_) and torch.equal(lf, ls), f"lt={lt} hkv={hkv}: outputs differ"
    assert torch.equal(kf, ks) and torch.equal(vf, vs), f"lt={lt} hkv={hkv}: caches differ"
