"""The no-allocation decode entry point (mimo_attn_decode_noalloc) against
mimo_attn_decode with a caller workspace, through the C ABI: two calls in a
row on the same GPU (the second with a smaller batch, so it runs over what the
first left in the library's scratch array), GA and SWA, and a batch large
enough that the scratch caps the chunk count.  Bars as in gpu_util; where the
chunking is the same the outputs are bit-identical."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import compare, log, to_dev

pytestmark = pytest.mark.gpu
SWA, GA = 0, 1


def _run_both(ctx, lt, seed, split=0):
    x = synth.decode_inputs(ctx, lt, seed=seed, headroom=2)
    d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "ctx_lens",
                                            "sink")}
    dims = B.make_dims()
    Bd, mc = len(ctx), max(ctx)
    o_ws, l_ws = B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], mc, lt,
                          sink=d["sink"], kv_base=d["kv_base"], split_tokens=split)
    o_na = torch.full((Bd, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_na = torch.full((Bd, 64), float("nan"), dtype=torch.float32, device="cuda")
    B.mimo_attn_decode_noalloc(dims, lt, d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["kv_base"],
                               d["ctx_lens"], Bd, mc, split, d["sink"], o_na, l_na)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


def _check(ctx, lt, seed, what, bitwise=True, split=0):
    o_ws, l_ws, o_na, l_na = _run_both(ctx, lt, seed, split)
    compare(o_na, l_na, o_ws.double().cpu().numpy(), l_ws.double().cpu().numpy(), what)
    if bitwise:
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), f"{what}: not bit-identical"


@pytest.mark.parametrize("lt", [GA, SWA])
def test_noalloc_two_calls_second_smaller(lt):
    log(f"[case] no-alloc decode lt={lt}: two calls, the second smaller")
    _check([5000, 70000, 33, 129000, 1, 260000, 4096, 17], lt, 110, f"no-alloc lt={lt} call 1 (8 sequences)")
    _check([300, 9000, 0], lt, 111, f"no-alloc lt={lt} call 2 (3 sequences)")


def test_noalloc_scratch_caps_the_chunks():
    """900 sequences at 64 query heads leave room for about 100 chunks in the
    32 MiB scratch instead of the 256 a workspace gives: results agree within
    the bars (fp32 rounding order), not bit for bit."""
    g = np.random.default_rng(5)
    ctx = [int(c) for c in g.integers(100, 3000, 900)]
    log("[case] no-alloc decode: 900 sequences, capped chunk count")
    _check(ctx, GA, 112, "no-alloc 900 sequences", bitwise=False)
    _check(ctx[:20], GA, 113, "no-alloc 20 sequences after 900")


def test_noalloc_rejects_batch_beyond_scratch():
    ctx = torch.zeros(2000, dtype=torch.int32, device="cuda")
    dims = B.make_dims()
    q = torch.zeros((2000, 64, 192), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((2000, 4, 192), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros((2000, 4, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((2000, 4, 192), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((2000, 4, 128), dtype=torch.bfloat16, device="cuda")
    base = torch.arange(2000, dtype=torch.int64, device="cuda")
    out = torch.empty((2000, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MimoError) as e:
        B.mimo_attn_decode_noalloc(dims, GA, q, kn, vn, kc, vc, base, ctx, 2000, 0, 0, None, out, None)
    assert e.value.status == B.MIMO_ERR_UNSUPPORTED
    assert "scratch" in B.mimo_last_error()
