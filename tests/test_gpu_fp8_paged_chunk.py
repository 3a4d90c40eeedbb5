"""The FP8 GA pool in the paged layout and as the cache of chunked prefill,
through the C ABI, against the fp64 oracle (model doc "MiMo-V2-Flash",
MiMoV2FlashModel.forward: past_key_values; the E4M3 storage format is a
reading, see include/mimo_attn.h):
  * paged FP8 append: codes bit for bit equal to the oracle's, bulk then
    decode-step appends, refusals past max_blocks and unmapped blocks;
  * paged FP8 decode: bit-identical to the contiguous FP8 decode over the same
    codes, and within the attention bars of the oracle, with chunks longer than
    the 128 pages a split preloads at a time;
  * FP8 chunked prefill (contiguous and paged): within the bars of the oracle,
    cached prefixes on and off the 64-key tile edges (tiles wholly from the
    cache, tiles across ctx_lens, tiles of chunk keys only), and the paged
    form bit-identical to the contiguous one.
Cached values are random E4M3 codes with per-head scales that keep keys within
+-9 and values within +-4.5 (the magnitudes of N(0,1) data)."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
GA = 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
K_SCALE = np.float32([0.01, 0.0173, 0.0071, 0.031])  # for quantised N(0,1) data
V_SCALE = np.float32([0.0105, 0.0063, 0.022, 0.0149])
RAND_K_SCALE = np.float32([1 / 64, 1 / 90, 1 / 50, 1 / 70])  # for uniform random codes
RAND_V_SCALE = np.float32([1 / 120, 1 / 160, 1 / 100, 1 / 200])


def _dev_scales(ks, vs):
    return torch.tensor(ks, device=DEV), torch.tensor(vs, device=DEV)


def _flat_to_paged(kc, vc, base, lengths, P, seed, extra=0):
    """Scatters each sequence's code rows of a flat pool onto shuffled pages (numpy)."""
    table, npages = synth.paged_block_table(lengths, P, seed=seed, extra_tokens=extra)
    tb = table.numpy()
    kp = np.zeros((npages * P,) + kc.shape[1:], np.uint8)
    vp = np.zeros((npages * P,) + vc.shape[1:], np.uint8)
    for b, L in enumerate(lengths):
        for j0 in range(0, L, P):
            n = min(P, L - j0)
            page = int(tb[b, j0 // P])
            kp[page * P:page * P + n] = kc[base[b] + j0:base[b] + j0 + n]
            vp[page * P:page * P + n] = vc[base[b] + j0:base[b] + j0 + n]
    return kp, vp, table


@pytest.mark.parametrize("page_size", [16, 64])
def test_fp8_paged_append_codes(page_size):
    lengths = [1, 37, 300, 5]
    log(f"[case] paged FP8 append lengths {lengths} page {page_size}")
    x = synth.prefill_inputs(lengths, seed=170)
    k = x.k.clone()
    k[3, 2, :3] = torch.tensor([1e4, -1e4, 500.0], dtype=torch.bfloat16)  # saturate
    table, npages = synth.paged_block_table(lengths, page_size, seed=page_size, extra_tokens=3)
    table[3, 0] = -1  # sequence 3's only block is unmapped: its tokens are not written
    kp = torch.zeros((npages * page_size, 4, 192), dtype=torch.uint8, device=DEV)
    vp = torch.zeros((npages * page_size, 4, 128), dtype=torch.uint8, device=DEV)
    kr, vr = np.zeros(tuple(kp.shape), np.uint8), np.zeros(tuple(vp.shape), np.uint8)
    ks, vs = _dev_scales(K_SCALE, V_SCALE)
    zeros = np.zeros(len(lengths), np.int32)
    tb_d = table.to(DEV)
    B.kv_append_fp8_paged(to_dev(k), to_dev(x.v), to_dev(x.cu_seqlens), torch.tensor(zeros, device=DEV), kp, vp,
                          tb_d, page_size, ks, vs)
    st = orc().kv_append_fp8_paged(bits(k), bits(x.v), x.cu_seqlens.numpy(), zeros, kr, vr, table.numpy(),
                                   page_size, K_SCALE, V_SCALE)
    assert st != 0  # the unmapped block
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), kr) and np.array_equal(vp.cpu().numpy(), vr), "bulk paged FP8 append"
    # a decode step: one token per sequence at position lengths[b]; sequence 2 is refused past max_blocks
    d = synth.decode_inputs(lengths, GA, seed=171)
    ctx = np.asarray(lengths, np.int32)
    mb = table.shape[1]
    ctx[2] = mb * page_size  # exactly full: the new token does not fit
    step = np.arange(len(lengths) + 1, dtype=np.int32)
    B.kv_append_fp8_paged(to_dev(d.k_new), to_dev(d.v_new), torch.tensor(step, device=DEV),
                          torch.tensor(ctx, device=DEV), kp, vp, tb_d, page_size, ks, vs)
    orc().kv_append_fp8_paged(bits(d.k_new), bits(d.v_new), step, ctx, kr, vr, table.numpy(), page_size, K_SCALE,
                              V_SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), kr) and np.array_equal(vp.cpu().numpy(), vr), "step paged FP8 append"


@pytest.mark.parametrize("page_size,split", [(16, 0), (16, 6000), (64, 0), (256, 96)])
def test_fp8_paged_decode(page_size, split):
    """Contexts around tile, page and split edges plus long ones; split 6000
    over 16-row pages gives chunks of 375 pages (three preload spans)."""
    ctx = [0, 1, 15, 16, 17, 31, 33, 255, 2047, 2049, 5000, 9000]
    log(f"[case] paged FP8 decode page {page_size} split {split}")
    d = synth.decode_inputs(ctx, GA, seed=172, headroom=2)
    rows = int(d.k_cache.shape[0])
    kc = synth.random_e4m3_codes((rows, 4, 192), seed=173).numpy()
    vc = synth.random_e4m3_codes((rows, 4, 128), seed=174).numpy()
    base = d.kv_base.numpy()
    kp, vp, table = _flat_to_paged(kc, vc, base, ctx, page_size, seed=175, extra=1)
    ks, vs = _dev_scales(RAND_K_SCALE, RAND_V_SCALE)
    q, kn, vn, sink, ctx_d = (to_dev(t) for t in (d.q, d.k_new, d.v_new, d.sink, d.ctx_lens))
    op, lp = B.decode_fp8_paged(q, kn, vn, to_dev(torch.from_numpy(kp)), to_dev(torch.from_numpy(vp)), table.to(DEV),
                                page_size, ks, vs, ctx_d, max(ctx), sink=sink, split_tokens=split)
    of, lf = B.decode_fp8(q, kn, vn, to_dev(torch.from_numpy(kc)), to_dev(torch.from_numpy(vc)), to_dev(d.kv_base),
                          ks, vs, ctx_d, max(ctx), sink=sink, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf), "paged FP8 decode differs from the contiguous FP8 pool"
    ro, rl = orc().decode_fp8_paged(bits(d.q), bits(d.k_new), bits(d.v_new), kp, vp, table.numpy(), page_size,
                                    RAND_K_SCALE, RAND_V_SCALE, d.ctx_lens.numpy(), scale=SCALE,
                                    sink=sink_array(d.sink))
    compare(op, lp, ro, rl, f"paged FP8 decode page {page_size} split {split}")


def _chunk_case(cached, new, seed):
    """FP8 pool of random codes for the cached prefixes (rows base[b] ..), and
    bf16 chunk tokens packed by cu."""
    x = synth.prefill_inputs(new, seed=seed)
    caps = [c + 8 for c in cached]
    base = np.concatenate([[5], 5 + np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(base[-1]) + caps[-1]
    kc = synth.random_e4m3_codes((rows, 4, 192), seed=seed + 1).numpy()
    vc = synth.random_e4m3_codes((rows, 4, 128), seed=seed + 2).numpy()
    return x, base, kc, vc


CHUNK_CASES = [
    # cached prefixes on and off 64-key tile edges; chunk lengths ragged
    ([0, 33, 64, 100, 128, 1000], [40, 1, 300, 64, 65, 129]),
    ([5000, 63, 2], [300, 200, 17]),
]


@pytest.mark.parametrize("cached,new", CHUNK_CASES)
def test_fp8_chunk_prefill_against_oracle(cached, new):
    log(f"[case] FP8 chunked prefill cached {cached} new {new}")
    x, base, kc, vc = _chunk_case(cached, new, 180 + len(cached))
    ks, vs = _dev_scales(RAND_K_SCALE, RAND_V_SCALE)
    q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
    ctx_d = torch.tensor(cached, dtype=torch.int32, device=DEV)
    kcd, vcd = to_dev(torch.from_numpy(kc)), to_dev(torch.from_numpy(vc))
    out, lse = B.prefill_chunk_fp8(q, k, v, cu, max(new), kcd, vcd, ks, vs, ctx_d, kv_base=to_dev(
        torch.from_numpy(base)), sink=sink)
    # the same cache on shuffled 16-row pages
    kp, vp, table = _flat_to_paged(kc, vc, base, cached, 16, seed=181)
    op, lp = B.prefill_chunk_fp8(q, k, v, cu, max(new), to_dev(torch.from_numpy(kp)), to_dev(torch.from_numpy(vp)),
                                 ks, vs, ctx_d, block_table=table.to(DEV), page_size=16, sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(op, out) and torch.equal(lp, lse), "paged FP8 chunk differs from the contiguous FP8 pool"
    ro, rl = orc().prefill_chunk_fp8(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.numpy(), kc, vc, RAND_K_SCALE,
                                     RAND_V_SCALE, np.asarray(cached, np.int32), kv_base=base, scale=SCALE,
                                     sink=sink_array(x.sink))
    compare(out, lse, ro, rl, f"FP8 chunk cached {cached}")


def test_fp8_chunk_prefill_value_scale_and_no_sink():
    cached, new = [70, 0, 200], [33, 64, 5]
    log("[case] FP8 chunked prefill, value_scale 0.707, no sink")
    x, base, kc, vc = _chunk_case(cached, new, 190)
    # other per-head scales than above; values stay within +-4.5, the magnitude the output bar is derived for
    ks, vs = _dev_scales(np.float32([1 / 40, 1 / 90, 1 / 50, 1 / 33]),
                         np.float32([1 / 110, 1 / 160, 1 / 100, 1 / 130]))
    dims = B.make_dims(value_scale=0.707)
    out, lse = B.prefill_chunk_fp8(to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_seqlens), max(new),
                                   to_dev(torch.from_numpy(kc)), to_dev(torch.from_numpy(vc)), ks, vs,
                                   torch.tensor(cached, dtype=torch.int32, device=DEV),
                                   kv_base=to_dev(torch.from_numpy(base)), dims=dims)
    torch.cuda.synchronize()
    ro, rl = orc().prefill_chunk_fp8(bits(x.q), bits(x.k), bits(x.v), x.cu_seqlens.numpy(), kc, vc,
                                     ks.cpu().numpy(), vs.cpu().numpy(), np.asarray(cached, np.int32), kv_base=base,
                                     scale=SCALE, value_scale=float(np.float32(0.707)))
    compare(out, lse, ro, rl, "FP8 chunk value_scale 0.707, no sink")
