"""Seeded random cases across the three attention entry points, against the oracle.

Each case draws its own shape from a generator seeded with the case number:
prefill over 1-5 ragged sequences (lengths at tile edges 15/16/17 or anywhere
up to 700) with SWA windows from 1 to 300 (streaming and tiled kernels) or GA;
decode over 1-9 sequences with contexts at ring and tile edges or up to 3000,
ring sizes from 1 to 299 slots and GA splits of 32 to 1024 keys; chunked
prefill with random cached prefixes.  Sinks are the seeded ones, absent, -inf
on every third head, or six times larger; value_scale is 1 or 0.7071.  The
bars are those of every other parity test.  Two more families: the prefill
backward on seeded ragged batches (gradient bars of the backward tests), and
the fused decode + append against decode followed by append (bit for bit),
some GA sequences with no room left for the new token; and the paged GA pool
(page sizes 16-1024, splits 32-2048, contexts to 6000) against the oracle and
bit for bit against the contiguous pool; the FP8 E4M3 pool (append codes
bit for bit, decode within the bars); and the fused-RoPE prefill, chunked
prefill and decode step (rotary dims 32-192, position offsets) bit for bit
against the rotation followed by the unfused call and within the bars of the
oracle.
"""
import random

import pytest

from global_attention_mimo_amd import synth
from gpu_util import bits, compare, gpu_prefill, log, oracle_prefill, orc, sink_array
from test_gpu_chunk import _caches, _chunk, _fill
from test_gpu_decode import SCALE, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu
N_CASES = 96


def _sink(rng, x):
    c = rng.choice(["inputs", "none", "neginf", "big"])
    if c == "inputs":
        return c, "inputs"
    if c == "none":
        return c, None
    s = x.sink.clone()
    if c == "neginf":
        s[::3] = float("-inf")
    else:
        s = s * 6.0
    return c, s


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case(case):
    rng = random.Random(7919 * case + 17)
    kind = ("prefill", "decode", "chunk")[case % 3]
    lt = rng.choice([0, 1])
    seed = 2000 + case
    if kind == "prefill":
        lengths = [rng.choice([1, 2, 15, 16, 17, rng.randint(1, 700)]) for _ in range(rng.randint(1, 5))]
        window = rng.choice([1, 2, 17, 64, 128, 129, 130, 145, 146, 300]) if lt == 0 else 129
        vs = rng.choice([1.0, 0.7071])
        x = synth.prefill_inputs(lengths, seed=seed)
        sc, s = _sink(rng, x)
        log(f"[case {case}] prefill layer={lt} lengths={lengths} window={window} value_scale={vs} sink={sc}")
        out, lse = gpu_prefill(x, lt, window=window, value_scale=vs, sink=s)
        ro, rl = oracle_prefill(x, lt, window=window, value_scale=vs, sink=s)
    elif kind == "decode":
        ctx = [rng.choice([0, 1, 2, 127, 128, 129, 255, 256, rng.randint(0, 3000)]) for _ in range(rng.randint(1, 9))]
        window = rng.choice([2, 17, 129, 130, 200, 225, 300]) if lt == 0 else 129
        split = rng.choice([0, 32, 64, 96, 256, 1024]) if lt == 1 else 0
        vs = rng.choice([1.0, 0.7071])
        x = synth.decode_inputs(ctx, lt, seed=seed, window=window)
        sc, s = _sink(rng, x)
        log(f"[case {case}] decode layer={lt} ctx={ctx} window={window} split={split} value_scale={vs} sink={sc}")
        out, lse = gpu_decode(x, lt, split=split, sink=s, value_scale=vs, window=window)
        ro, rl = oracle_decode(x, lt, sink=s, value_scale=vs, window=window)
    else:
        lengths = [rng.randint(1, 600) for _ in range(rng.randint(1, 5))]
        cached = [rng.choice([0, 1, L - 1, rng.randint(0, L - 1)]) for L in lengths]
        window = rng.choice([2, 17, 129, 145, 146, 300]) if lt == 0 else 129
        x = synth.prefill_inputs(lengths, seed=seed)
        log(f"[case {case}] chunked prefill layer={lt} lengths={lengths} cached={cached} window={window}")
        kc, vc, base, cap = _caches(lt, lengths, window=window)
        kh, vh = _fill(x, lt, cached, kc, vc, base, cap, window=window)
        out, lse, new, rest, cu_new, ctxd = _chunk(x, lt, cached, kc, vc, base, window=window)
        ro, rl = orc().prefill_chunk(bits(x.q[new]), bits(x.k[new]), bits(x.v[new]), cu_new.cpu().numpy(), kh, vh,
                                     ctxd.cpu().numpy(), layer_type=lt, window=window, scale=SCALE,
                                     sink=sink_array(x.sink), kv_base=None if base is None else base.cpu().numpy())
    compare(out, lse, ro, rl, f"random case {case} ({kind})")


N_BACKWARD = 40


@pytest.mark.parametrize("case", range(N_BACKWARD))
def test_random_backward_case(case):
    """Prefill backward over a seeded ragged batch against the oracle's gradients."""
    from test_gpu_backward import assert_vanishing, dout_like, grad_compare, oracle_grads, run
    rng = random.Random(104729 * case + 3)
    lt = rng.choice([0, 1])
    lengths = [rng.choice([1, 2, 16, 17, 32, 33, rng.randint(1, 400)]) for _ in range(rng.randint(1, 4))]
    window = rng.choice([2, 17, 64, 129, 130, 300]) if lt == 0 else 129
    vs = rng.choice([1.0, 0.7071])
    x = synth.prefill_inputs(lengths, seed=3000 + case)
    sc, s = _sink(rng, x)
    log(f"[case {case}] backward layer={lt} lengths={lengths} window={window} value_scale={vs} sink={sc}")
    dout = dout_like(sum(lengths), 4000 + case)
    dq, dk, dv, ds = run(x, dout, lt, window, vs, sink=s)
    rq, rk, rv, rs = oracle_grads(x, dout, lt, window, vs, sink=s)
    if not rq.any() and not rk.any():
        # Every sequence is one token, without a sink, at value_scale 1: the
        # exact dq and dk are zero and a bar relative to their size is empty.
        assert all(n == 1 for n in lengths) and vs == 1.0
        assert_vanishing(x, dout, dq, dk, f"case {case} ")
    else:
        grad_compare(dq, rq, "dq")
        grad_compare(dk, rk, "dk")
    grad_compare(dv, rv, "dv")
    grad_compare(ds, rs, "dsink")


N_APPEND = 16


@pytest.mark.parametrize("case", range(N_APPEND))
def test_random_decode_append_case(case):
    """Fused decode + append equals decode then append, bit for bit, on seeded contexts."""
    import torch
    from test_gpu_decode_append import _both
    rng = random.Random(1299709 * case + 11)
    lt = case % 2
    ctx = [rng.choice([0, 1, 127, 128, 129, 255, 256, rng.randint(0, 5000)]) for _ in range(rng.randint(1, 9))]
    split = rng.choice([0, 32, 64, 256]) if lt == 1 else 0
    full = rng.randrange(len(ctx)) if lt == 1 and rng.random() < 0.5 else None
    log(f"[case {case}] decode_append layer={lt} ctx={ctx} split={split} full={full}")
    _, ((o0, l0, k0, v0), (o1, l1, k1, v1)) = _both(lt, ctx, split, full)
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "outputs differ"
    assert torch.equal(k0, k1) and torch.equal(v0, v1), "caches differ"


N_PAGED = 16


@pytest.mark.parametrize("case", range(N_PAGED))
def test_random_paged_decode_case(case):
    """Paged GA pool with seeded page sizes, splits and contexts: the paged append
    matches the oracle's bytes, and the paged decode equals the contiguous pool's
    decode bit for bit (same split) and the oracle within the bars."""
    import numpy as np
    import torch
    from global_attention_mimo_amd import binding as B
    from gpu_util import to_dev
    from test_gpu_paged import _flat, _pools
    rng = random.Random(15485863 * case + 5)
    ctx = [rng.choice([0, 1, 15, 16, 17, 255, 256, 2047, 2048, rng.randint(0, 6000)])
           for _ in range(rng.randint(1, 9))]
    page = rng.choice([16, 32, 64, 128, 256, 1024])
    split = rng.choice([0, 32, 64, 256, 2048])
    log(f"[case {case}] paged decode ctx={ctx} page={page} split={split}")
    x = synth.decode_inputs(ctx, 1, seed=5000 + case)
    table, npages = synth.paged_block_table(ctx, page, seed=case)
    table_d = table.to("cuda")
    kp, vp = _pools(npages, page)
    kf, vf, base, cap = _flat(ctx)
    rows = torch.cat([torch.arange(int(x.kv_base[b]), int(x.kv_base[b]) + c) for b, c in enumerate(ctx)]).long()
    k_pre, v_pre = to_dev(x.k_cache[rows]), to_dev(x.v_cache[rows])
    cu = synth.cu_from_lengths(ctx, "cuda")
    zeros = torch.zeros(len(ctx), dtype=torch.int32, device="cuda")
    if sum(ctx):
        B.kv_append_paged(k_pre, v_pre, cu, zeros, kp, vp, table_d, page)
        B.kv_append(k_pre, v_pre, cu, zeros, kf, vf, 1, kv_base=base, kv_capacity=cap)
    torch.cuda.synchronize()
    kp_ref, vp_ref = np.zeros_like(bits(kp)), np.zeros_like(bits(vp))
    if sum(ctx):
        assert orc().kv_append_paged(bits(k_pre), bits(v_pre), cu.cpu().numpy(), zeros.cpu().numpy(), kp_ref, vp_ref,
                                     table.numpy(), page) == 0
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref), "paged append bytes"
    q, kn, vn, sink = to_dev(x.q), to_dev(x.k_new), to_dev(x.v_new), to_dev(x.sink)
    ctx_d = to_dev(x.ctx_lens)
    op, lp = B.decode_paged(q, kn, vn, kp, vp, table_d, page, ctx_d, max(ctx), sink=sink, split_tokens=split)
    of, lf = B.decode(q, kn, vn, kf, vf, ctx_d, max(ctx), 1, sink=sink, kv_base=base, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf), "paged decode differs from the contiguous pool's"
    ro, rl = orc().decode_paged(bits(x.q), bits(x.k_new), bits(x.v_new), kp_ref, vp_ref, table.numpy(), page,
                                x.ctx_lens.numpy(), scale=float(np.float32(synth.SOFTMAX_SCALE)),
                                sink=sink_array(x.sink))
    compare(op, lp, ro, rl, f"random paged decode case {case}")


N_FP8 = 12


@pytest.mark.parametrize("case", range(N_FP8))
def test_random_fp8_decode_case(case):
    """FP8 E4M3 GA pool over seeded contexts and splits: the quantising append
    matches the oracle's codes bit for bit, the decode the oracle within the bars."""
    import numpy as np
    import torch
    from global_attention_mimo_amd import binding as B
    from gpu_util import to_dev
    from test_gpu_fp8 import K_SCALE, V_SCALE, _pools
    rng = random.Random(32452843 * case + 7)
    ctx = [rng.choice([0, 1, 31, 32, 33, 255, 256, rng.randint(0, 4000)]) for _ in range(rng.randint(1, 8))]
    split = rng.choice([0, 32, 96, 256, 1024])
    log(f"[case {case}] FP8 decode ctx={ctx} split={split}")
    lengths = [max(c, 1) for c in ctx]
    x = synth.prefill_inputs(lengths, seed=6000 + case)
    d = synth.decode_inputs(ctx, 1, seed=7000 + case)
    sc, s = _sink(rng, d)
    caps = [c + 2 for c in lengths]
    base = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    rows = int(sum(caps))
    kc, vc = _pools(rows)
    kr, vr = np.zeros((rows, 4, 192), np.uint8), np.zeros((rows, 4, 128), np.uint8)
    ks, vs = torch.tensor(K_SCALE, device="cuda"), torch.tensor(V_SCALE, device="cuda")
    base_d, cap_d = torch.tensor(base, device="cuda"), torch.tensor(caps, dtype=torch.int64, device="cuda")
    cached = np.asarray(ctx, np.int32)
    cu = x.cu_seqlens.numpy()
    pre = np.concatenate([np.arange(cu[b], cu[b] + c) for b, c in enumerate(ctx)]).astype(np.int64)
    cu_pre = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    zeros = np.zeros(len(ctx), np.int32)
    if sum(ctx):
        B.kv_append_fp8(to_dev(x.k[pre]), to_dev(x.v[pre]), torch.tensor(cu_pre, device="cuda"),
                        torch.tensor(zeros, device="cuda"), kc, vc, base_d, cap_d, ks, vs)
        assert orc().kv_append_fp8(bits(x.k[pre]), bits(x.v[pre]), cu_pre, zeros, kr, vr, base,
                                   np.asarray(caps, np.int64), K_SCALE, V_SCALE) == 0
    sd = d.sink if isinstance(s, str) else s
    out, lse = B.decode_fp8(to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), kc, vc, base_d, ks, vs,
                            torch.tensor(cached, device="cuda"), max(ctx), sink=to_dev(sd), split_tokens=split)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr), "FP8 append codes"
    ro, rl = orc().decode_fp8(bits(d.q), bits(d.k_new), bits(d.v_new), kr, vr, base, K_SCALE, V_SCALE, cached,
                              scale=SCALE, sink=sink_array(sd))
    compare(out, lse, ro, rl, f"random FP8 decode case {case} (sink {sc})")


N_ROPE = 18


@pytest.mark.parametrize("case", range(N_ROPE))
def test_random_rope_case(case):
    """The fused-RoPE entry points on seeded shapes, rotary dims and position
    offsets: prefill, chunked prefill and the decode step, each bit for bit
    against mimo_rope_apply on copies followed by the unfused call (where both
    run the same kernel) and within the bars of the oracle's rotation followed
    by the oracle's attention."""
    import numpy as np
    import torch
    from global_attention_mimo_amd import binding as B
    from gpu_util import to_dev
    rng = random.Random(15485863 * case + 3)
    kind = ("prefill", "chunk", "decode")[case % 3]
    lt = rng.choice([0, 1])
    window = rng.choice([17, 129, 145, 146, 300]) if lt == 0 else 129
    theta = rng.choice([1e4, 1e6, 5e6])
    dims = B.make_dims(sliding_window=window)
    dev = "cuda"
    if kind == "decode":
        from test_gpu_rope_decode import _run
        rd = rng.choice([64, 128, 192])
        ctx = [rng.choice([0, 1, window - 2, window - 1, window, rng.randint(0, 4000)]) for _ in
               range(rng.randint(1, 7))]
        split = rng.choice([0, 32, 64]) if lt == 1 else 0
        offset = rng.choice([0, 0, rng.randint(1, 100000)])
        log(f"[case {case}] decode rope layer={lt} W={window} ctx={ctx} split={split} rd={rd} theta={theta} "
            f"offset={offset}")
        x, pos, ((of, lf, kf, vf), (os_, ls, ks, vs)) = _run(lt, ctx, window, split, rd, theta, offset,
                                                             seed=6000 + case)
        assert torch.equal(of, os_) and torch.equal(lf, ls), "fused decode differs from rope + decode_append"
        assert torch.equal(kf, ks) and torch.equal(vf, vs), "caches differ"
        rq, rk = orc().rope(bits(x.q), bits(x.k_new), pos.cpu().numpy(), theta=float(np.float32(theta)),
                            rotary_dim=rd)
        ro, rl = orc().decode(synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16)),
                              synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16)), bits(x.v_new),
                              bits(x.k_cache), bits(x.v_cache), x.ctx_lens.cpu().numpy(), layer_type=lt,
                              window=window, scale=SCALE, sink=sink_array(x.sink),
                              kv_base=None if x.kv_base is None else x.kv_base.cpu().numpy())
        compare(of, lf, ro, rl, f"random decode rope case {case}")
        return
    rd = rng.choice([32, 64, 128, 192])
    lengths = [rng.choice([1, 16, 17, 64, 65, rng.randint(1, 600)]) for _ in range(rng.randint(1, 4))]
    x = synth.prefill_inputs(lengths, seed=6100 + case)
    # the same kernel on both sides unless a streaming-window SWA call rotates more than 64 dims
    same_kernel = not (lt == 0 and window <= 145 and rd > 64)
    if kind == "prefill":
        offs = [rng.choice([0, rng.randint(1, 50000)]) for _ in lengths]
        pos = np.concatenate([np.arange(L) + o for L, o in zip(lengths, offs)]).astype(np.int32)
        posd = torch.tensor(pos, device=dev)
        q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
        log(f"[case {case}] prefill rope layer={lt} W={window} lengths={lengths} rd={rd} theta={theta}")
        of, lf, krot = B.prefill_rope(q, k, v, posd, cu, max(lengths), lt, theta, rd, sink=sink, dims=dims)
        q2, k2 = q.clone(), k.clone()
        B.rope_apply(q2, k2, posd, theta, rd)
        os_, ls = B.prefill(q2, k2, v, cu, max(lengths), lt, sink=sink, dims=dims)
        torch.cuda.synchronize()
        assert torch.equal(krot, k2), "k_rot differs from mimo_rope_apply's k"
        if same_kernel:
            assert torch.equal(of, os_) and torch.equal(lf, ls), "fused prefill differs from rope + prefill"
        rq, rk = orc().rope(bits(x.q), bits(x.k), pos, theta=float(np.float32(theta)), rotary_dim=rd)
        ro, rl = orc().prefill(synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16)),
                               synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16)), bits(x.v),
                               x.cu_seqlens.numpy(), layer_type=lt, window=window, scale=SCALE,
                               sink=sink_array(x.sink))
        compare(of, lf, ro, rl, f"random prefill rope case {case}")
        return
    from test_gpu_chunk import _split
    cached = [rng.randint(0, L - 1) if rng.random() < 0.8 else 0 for L in lengths]
    kc, vc, base, cap = _caches(lt, lengths, window=window)
    kh, vh = _fill(x, lt, cached, kc, vc, base, cap, window=window)
    _, new, rest = _split(x, cached)
    cu_new = synth.cu_from_lengths(rest, dev)
    ctx = torch.tensor(cached, dtype=torch.int32, device=dev)
    offset = rng.choice([0, rng.randint(1, 50000)])
    pos = np.concatenate([np.arange(n) + c + offset for c, n in zip(cached, rest)]).astype(np.int32)
    posd = torch.tensor(pos, device=dev)
    q, k, v, sink = to_dev(x.q[new]), to_dev(x.k[new]), to_dev(x.v[new]), to_dev(x.sink)
    log(f"[case {case}] chunk rope layer={lt} W={window} lengths={lengths} cached={cached} rd={rd} theta={theta}")
    of, lf, krot = B.prefill_chunk_rope(q, k, v, posd, cu_new, max(rest), kc, vc, ctx, lt, theta, rd, sink=sink,
                                        kv_base=base, dims=dims)
    q2, k2 = q.clone(), k.clone()
    B.rope_apply(q2, k2, posd, theta, rd)
    os_, ls = B.prefill_chunk(q2, k2, v, cu_new, max(rest), kc, vc, ctx, lt, sink=sink, kv_base=base, dims=dims)
    torch.cuda.synchronize()
    assert torch.equal(krot, k2), "k_rot differs from mimo_rope_apply's k"
    if same_kernel:
        assert torch.equal(of, os_) and torch.equal(lf, ls), "fused chunk differs from rope + chunk"
    rq, rk = orc().rope(bits(x.q[new]), bits(x.k[new]), pos, theta=float(np.float32(theta)), rotary_dim=rd)
    ro, rl = orc().prefill_chunk(synth.bf16_bits(torch.from_numpy(rq).to(torch.bfloat16)),
                                 synth.bf16_bits(torch.from_numpy(rk).to(torch.bfloat16)), bits(x.v[new]),
                                 cu_new.cpu().numpy(), kh, vh, ctx.cpu().numpy(), layer_type=lt, window=window,
                                 scale=SCALE, sink=sink_array(x.sink),
                                 kv_base=None if base is None else base.cpu().numpy())
    compare(of, lf, ro, rl, f"random chunk rope case {case}")
