"""GPU parity of the paged GA pool (block table of fixed-size pages) through the
C ABI: append placement bit for bit against the oracle, decode and chunked
prefill against the fp64 oracle, and bit-identical to the same calls over a
contiguous pool holding the same rows.  Bars as in gpu_util."""
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


def _pools(num_pages, page_size):
    rows = num_pages * page_size
    return (torch.zeros((rows, 4, 192), dtype=torch.bfloat16, device=DEV),
            torch.zeros((rows, 4, 128), dtype=torch.bfloat16, device=DEV))


def _flat(lengths, headroom=8):
    caps = [L + headroom for L in lengths]
    base = torch.tensor(np.concatenate([[5], 5 + np.cumsum(caps)[:-1]]), dtype=torch.int64, device=DEV)
    rows = int(base[-1]) + caps[-1]
    return (torch.zeros((rows, 4, 192), dtype=torch.bfloat16, device=DEV),
            torch.zeros((rows, 4, 128), dtype=torch.bfloat16, device=DEV), base,
            torch.tensor(caps, dtype=torch.int64, device=DEV))


@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_paged_append_and_decode(page_size):
    """Contexts on and around page and split boundaries; the cache is written by
    the paged append (bulk prefix, then the decode token), decode reads it."""
    ctx = [0, 1, 15, 16, 17, 255, 2047, 2048, 2049, 5000]
    log(f"[case] paged append + decode, page {page_size}, ctx {ctx}")
    x = synth.decode_inputs(ctx, GA, seed=50)
    table, npages = synth.paged_block_table(ctx, page_size, seed=page_size)
    table_d = table.to(DEV)
    kp, vp = _pools(npages, page_size)
    kf, vf, base, cap = _flat(ctx)
    # Cached prefixes: the first ctx[b] rows of each sequence's region of the seeded flat pool.
    rows = torch.cat([torch.arange(int(x.kv_base[b]), int(x.kv_base[b]) + c) for b, c in enumerate(ctx)]).long()
    k_pre, v_pre = to_dev(x.k_cache[rows]), to_dev(x.v_cache[rows])
    cu = synth.cu_from_lengths(ctx, DEV)
    zeros = torch.zeros(len(ctx), dtype=torch.int32, device=DEV)
    B.kv_append_paged(k_pre, v_pre, cu, zeros, kp, vp, table_d, page_size)
    B.kv_append(k_pre, v_pre, cu, zeros, kf, vf, GA, kv_base=base, kv_capacity=cap)
    torch.cuda.synchronize()
    kp_ref, vp_ref = np.zeros_like(bits(kp)), np.zeros_like(bits(vp))
    st = orc().kv_append_paged(bits(k_pre), bits(v_pre), cu.cpu().numpy(), zeros.cpu().numpy(), kp_ref, vp_ref,
                               table.numpy(), page_size)
    assert st == 0
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref), "paged append bytes"

    q, kn, vn, sink = to_dev(x.q), to_dev(x.k_new), to_dev(x.v_new), to_dev(x.sink)
    ctx_d = to_dev(x.ctx_lens)
    op, lp = B.decode_paged(q, kn, vn, kp, vp, table_d, page_size, ctx_d, max(ctx), sink=sink)
    of, lf = B.decode(q, kn, vn, kf, vf, ctx_d, max(ctx), GA, sink=sink, kv_base=base)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf), "paged decode is not bit-identical to the contiguous pool"
    ro, rl = orc().decode_paged(bits(x.q), bits(x.k_new), bits(x.v_new), kp_ref, vp_ref, table.numpy(),
                                page_size, x.ctx_lens.numpy(), scale=SCALE, sink=sink_array(x.sink))
    compare(op, lp, ro, rl, f"paged decode page {page_size}")

    # Decode-step append of the new tokens at positions ctx[b].
    step = torch.arange(len(ctx) + 1, dtype=torch.int32, device=DEV)
    B.kv_append_paged(kn, vn, step, ctx_d, kp, vp, table_d, page_size)
    torch.cuda.synchronize()
    st = orc().kv_append_paged(bits(x.k_new), bits(x.v_new), step.cpu().numpy(), x.ctx_lens.numpy(), kp_ref, vp_ref,
                               table.numpy(), page_size)
    assert st == 0
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref), "paged decode-step append bytes"


@pytest.mark.parametrize("page_size", [16, 128])
def test_paged_chunk_prefill(page_size):
    """Ragged cached prefixes (0, 1, 63, 128, 131, 1000) in a paged pool and
    packed chunks: against the oracle and bit-identical to the contiguous pool."""
    lengths = [300, 170, 64, 129, 260, 1500]
    cached = [0, 1, 63, 128, 131, 1000]
    log(f"[case] paged chunked prefill page {page_size}")
    x = synth.prefill_inputs(lengths, seed=51)
    cu = x.cu_seqlens.tolist()
    pre = torch.cat([torch.arange(cu[b], cu[b] + c) for b, c in enumerate(cached)]).long()
    new = torch.cat([torch.arange(cu[b] + c, cu[b + 1]) for b, c in enumerate(cached)]).long()
    rest = [L - c for L, c in zip(lengths, cached)]
    table, npages = synth.paged_block_table(cached, page_size, seed=7, extra_tokens=0)
    table_d = table.to(DEV)
    kp, vp = _pools(npages, page_size)
    kf, vf, base, cap = _flat(lengths)
    cu_pre = synth.cu_from_lengths(cached, DEV)
    zeros = torch.zeros(len(lengths), dtype=torch.int32, device=DEV)
    B.kv_append_paged(to_dev(x.k[pre]), to_dev(x.v[pre]), cu_pre, zeros, kp, vp, table_d, page_size)
    B.kv_append(to_dev(x.k[pre]), to_dev(x.v[pre]), cu_pre, zeros, kf, vf, GA, kv_base=base, kv_capacity=cap)
    kp_ref, vp_ref = np.zeros_like(bits(kp)), np.zeros_like(bits(vp))
    assert orc().kv_append_paged(bits(x.k[pre]), bits(x.v[pre]), cu_pre.cpu().numpy(), zeros.cpu().numpy(), kp_ref,
                                 vp_ref, table.numpy(), page_size) == 0
    cu_new = synth.cu_from_lengths(rest, DEV)
    ctx = torch.tensor(cached, dtype=torch.int32, device=DEV)
    q, k, v, sink = to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]), to_dev(x.sink)
    op, lp = B.prefill_chunk_paged(q, k, v, cu_new, max(rest), kp, vp, table_d, page_size, ctx, sink=sink)
    of, lf = B.prefill_chunk(q, k, v, cu_new, max(rest), kf, vf, ctx, GA, sink=sink, kv_base=base)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf), "paged chunk is not bit-identical to the contiguous pool"
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref), "paged append bytes"
    ro, rl = orc().prefill_chunk_paged(bits(x.q[new]), bits(x.k[new]), bits(x.v[new]), cu_new.cpu().numpy(),
                                       kp_ref, vp_ref, table.numpy(), page_size, np.asarray(cached, np.int32),
                                       scale=SCALE, sink=sink_array(x.sink))
    compare(op, lp, ro, rl, f"paged chunk page {page_size}")


def test_paged_append_refusals_and_unmapped_blocks():
    """A sequence needing more than max_blocks pages is skipped whole; tokens on
    an unmapped block (-1) are skipped; bytes match the oracle.  A decode whose
    table has an unmapped block below the context reads zero keys there and
    leaves the other sequences bit-identical to a clean table."""
    P = 16
    table = torch.tensor([[3, 0, -1, 5], [1, 2, 4, 6]], dtype=torch.int32)
    npages = 8
    log("[case] paged append refusals / unmapped blocks")
    x = synth.prefill_inputs([70, 40], seed=52)
    kp, vp = _pools(npages, P)
    cu = x.cu_seqlens.to(DEV)
    ctx0 = torch.zeros(2, dtype=torch.int32, device=DEV)
    # sequence 0: 70 positions need 5 blocks > max_blocks 4 -> refused whole
    B.kv_append_paged(to_dev(x.k), to_dev(x.v), cu, ctx0, kp, vp, table.to(DEV), P)
    torch.cuda.synchronize()
    kr, vr = np.zeros_like(bits(kp)), np.zeros_like(bits(vp))
    st = orc().kv_append_paged(bits(x.k), bits(x.v), x.cu_seqlens.numpy(), np.zeros(2, np.int32), kr, vr,
                               table.numpy(), P)
    assert st == 2 and np.array_equal(bits(kp), kr) and np.array_equal(bits(vp), vr)
    assert not bits(kp)[3 * P:4 * P].any(), "refused sequence was written"
    # sequence 0 again with 40 positions: block 2 (positions 32..39) is unmapped
    cu2 = torch.tensor([0, 40, 80], dtype=torch.int32, device=DEV)
    kk = torch.cat([to_dev(x.k[:40]), to_dev(x.k[70:110])])
    vv = torch.cat([to_dev(x.v[:40]), to_dev(x.v[70:110])])
    kp.zero_()
    vp.zero_()
    B.kv_append_paged(kk, vv, cu2, ctx0, kp, vp, table.to(DEV), P)
    torch.cuda.synchronize()
    kr[:] = 0
    vr[:] = 0
    st = orc().kv_append_paged(bits(kk), bits(vv), cu2.cpu().numpy(), np.zeros(2, np.int32), kr, vr, table.numpy(), P)
    assert st == 2 and np.array_equal(bits(kp), kr) and np.array_equal(bits(vp), vr)

    # decode at positions 40 and 40 with sequence 0's block 2 unmapped
    d = synth.decode_inputs([40, 40], GA, seed=53)
    q, kn, vn, sink = to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(d.sink)
    ctx = torch.tensor([40, 40], dtype=torch.int32, device=DEV)
    o1, l1 = B.decode_paged(q, kn, vn, kp, vp, table.to(DEV), P, ctx, 40, sink=sink)
    clean = table.clone()
    clean[0, 2] = 7
    o2, l2 = B.decode_paged(q, kn, vn, kp, vp, clean.to(DEV), P, ctx, 40, sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(o1[1], o2[1]) and torch.equal(l1[1], l2[1])
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    # page 7 was never written (zeros), so the unmapped block reads the same zero keys
    assert torch.equal(o1[0], o2[0]) and torch.equal(l1[0], l2[0])


def test_paged_decode_b128_long_contexts_equals_contiguous():
    """Decode step for 128 sequences with contexts U[4096, 262144] (seed 0), GA
    pool in pages of 16 (random page order): bit-identical to the contiguous
    pool, whose outputs the full-size test checks against the oracle."""
    ctx = synth.long_context_lengths(128, seed=0)
    P = 16
    log(f"[case] paged GA decode b128 long contexts, page {P}")
    x = synth.decode_inputs(ctx, GA, seed=0, device=DEV)
    table, npages = synth.paged_block_table(ctx, P, seed=1, device=DEV)
    kp = torch.empty((npages * P, 4, 192), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty((npages * P, 4, 128), dtype=torch.bfloat16, device=DEV)
    for b, c in enumerate(ctx):  # rearrange each sequence's rows onto its pages
        j = torch.arange(c, device=DEV)
        dst = table[b, j // P].long() * P + j % P
        src = int(x.kv_base[b]) + j
        kp[dst] = x.k_cache[src]
        vp[dst] = x.v_cache[src]
    op, lp = B.decode_paged(x.q, x.k_new, x.v_new, kp, vp, table, P, x.ctx_lens, max(ctx), sink=x.sink)
    of, lf = B.decode(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, x.ctx_lens, max(ctx), GA, sink=x.sink,
                      kv_base=x.kv_base)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf)
    assert torch.isfinite(lp).all()
