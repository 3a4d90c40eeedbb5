"""Pins that tie the fp64 oracle to facts other than its own code.

Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises AssertionError when
the oracle disagrees with:
  * a structurally different brute force (dense masked score matrix with the
    sink appended as an extra zero-value column, softmax by torch);
  * torch's fp64 scaled_dot_product_attention in the special cases that reduce
    to it (no sink; sink as an extra key with zero key and value vectors and an
    additive mask of sigma);
  * closed forms (first query of a sequence; all-equal scores);
  * invariants (weights plus sink mass sum to one; a sink of -inf is no sink;
    SWA equals GA when the window covers the sequence; GQA equals MHA with the
    K/V heads repeated; value_scale is linear; decode at position p equals row
    p of prefill; ring-slot contents after appends);
  * for the backward pass: torch fp64 autograd through a dense brute force of
    the same attention (sink as an extra logit with no value), and the closed
    form of one-token sequences;
  * for the rotary embedding: Transformers' own MiMo-V2-Flash rotate-half
    application and default inverse frequencies (a library implementation of
    the same convention), and the invariants of a rotation (norms, dependence
    of q.k on the position difference only, identity at position 0);
  * for the FP8 (OCP E4M3) GA cache: the format's own table
    (tests/golden/ocp_e4m3.json) and torch's float8_e4m3fn conversions (a
    library implementation of the same format); FP8 decode equals bf16 decode
    where the dequantised values are exact in bf16, and a dense numpy brute
    force elsewhere.

The attention definition pinned here is the one from the Hugging Face
Transformers model doc "MiMo-V2-Flash" (Key features: 5:1 SWA/GA, 128-token
window, learnable attention sink bias; MiMoV2FlashConfig: 64/4 heads, head_dim
192, v_head_dim 128, sliding_window 129, attention_value_scale 0.707).

``run_all(path)`` runs every pin against the library at ``path`` and returns
the names of the pins that failed; the mutation test uses it, stopping at the
first failure, on planted-mistake builds of the oracle.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from global_attention_mimo_amd import synth  # noqa: E402

SWA, GA = oracle.SWA, oracle.GA


def _bits(t):
    return synth.bf16_bits(t)


def _f64(t):
    return t.detach().to(torch.float64)


def _make(lengths, seed=0, hq=64, hkv=4, dqk=192, dv=128, sink=True):
    return synth.prefill_inputs(lengths, seed=seed, hq=hq, hkv=hkv, dqk=dqk, dv=dv, with_sink=sink)


def _run_prefill(orc, x, layer_type, window, scale, value_scale=1.0, sink="inputs", **kw):
    s = x.sink if isinstance(sink, str) else sink
    s = None if s is None else np.asarray(s.numpy() if torch.is_tensor(s) else s, dtype=np.float32)
    return orc.prefill(_bits(x.q), _bits(x.k), _bits(x.v), x.cu_seqlens.numpy(), layer_type=layer_type,
                       window=window, scale=scale, value_scale=value_scale, sink=s, **kw)


def _allowed(L, layer_type, window):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    ok = j <= i
    if layer_type == SWA:
        ok &= j >= i - (window - 1)
    return ok


def _brute(x, layer_type, window, scale, value_scale, sink):
    """Dense brute force: full LxL score matrix per head, masked with -inf, the
    sink appended as one more column whose value row is zero, torch.softmax."""
    hq, hkv = x.q.shape[1], x.k.shape[1]
    G = hq // hkv
    outs, lses = [], []
    cu = x.cu_seqlens.tolist()
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        q = _f64(x.q[s0:s1])  # [L][Hq][D]
        k = _f64(x.k[s0:s1])
        v = _f64(x.v[s0:s1])
        ok = torch.from_numpy(_allowed(L, layer_type, window))
        o_b = torch.empty(L, hq, v.shape[2], dtype=torch.float64)
        l_b = torch.empty(L, hq, dtype=torch.float64)
        for h in range(hq):
            g = h // G
            S = float(scale) * (q[:, h, :] @ k[:, g, :].T)
            S = S.masked_fill(~ok, -math.inf)
            sig = -math.inf if sink is None else float(sink[h])
            S_aug = torch.cat([S, torch.full((L, 1), sig, dtype=torch.float64)], dim=1)
            P = torch.softmax(S_aug, dim=1)
            V_aug = torch.cat([v[:, g, :], torch.zeros(1, v.shape[2], dtype=torch.float64)], dim=0)
            o_b[:, h, :] = float(value_scale) * (P @ V_aug)
            l_b[:, h] = torch.logsumexp(S_aug, dim=1)
        outs.append(o_b)
        lses.append(l_b)
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
def pin_bruteforce_small(orc):
    """Small shapes, two ragged sequences, SWA and GA, with and without sink."""
    x = _make([7, 11], seed=1, hq=4, hkv=2, dqk=8, dv=4)
    sink = x.sink.clone()
    sink[3] = -math.inf
    for lt in (SWA, GA):
        for W in (1, 3, 5):
            for s in (sink, None):
                o, l = _run_prefill(orc, x, lt, W, 0.37, 0.9, sink=s)
                bo, bl = _brute(x, lt, W, np.float32(0.37), np.float32(0.9), None if s is None else s.numpy())
                _close(o, bo, 1e-12, f"brute out lt={lt} W={W}")
                _close(l, bl, 1e-12, f"brute lse lt={lt} W={W}")


def pin_bruteforce_full_dims(orc):
    """Model dims (64/4 heads, 192/128), window 129 reached (L = 140)."""
    x = _make([140, 16], seed=2)
    scale = np.float32(synth.SOFTMAX_SCALE)
    for lt in (SWA, GA):
        o, l = _run_prefill(orc, x, lt, 129, float(scale))
        bo, bl = _brute(x, lt, 129, scale, np.float32(1.0), x.sink.numpy())
        _close(o, bo, 1e-12, f"brute full out lt={lt}")
        _close(l, bl, 1e-12, f"brute full lse lt={lt}")


def _sdpa_rows(x, layer_type, window, scale, sink):
    """torch fp64 SDPA per sequence: boolean mask, KV repeated per group; with a
    sink, one extra key (k = 0, v = 0) whose additive mask entry is sigma."""
    hq, hkv = x.q.shape[1], x.k.shape[1]
    G = hq // hkv
    cu = x.cu_seqlens.tolist()
    outs, lses = [], []
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        q = _f64(x.q[s0:s1]).transpose(0, 1)  # [Hq][L][D]
        k = _f64(x.k[s0:s1]).repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        v = _f64(x.v[s0:s1]).repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        ok = torch.from_numpy(_allowed(L, layer_type, window))
        if sink is None:
            mask = ok.unsqueeze(0).expand(hq, L, L)
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(scale))
            sc = (q @ k.transpose(1, 2)) * float(scale)
            lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=2)
        else:
            kz = torch.cat([k, torch.zeros(hq, 1, k.shape[2], dtype=torch.float64)], dim=1)
            vz = torch.cat([v, torch.zeros(hq, 1, v.shape[2], dtype=torch.float64)], dim=1)
            add = torch.zeros(hq, L, L + 1, dtype=torch.float64)
            add[:, :, :L] = add[:, :, :L].masked_fill(~ok, -math.inf)
            add[:, :, L] = torch.as_tensor(sink, dtype=torch.float64)[:, None]
            o = torch.nn.functional.scaled_dot_product_attention(q, kz, vz, attn_mask=add, scale=float(scale))
            sc = (q @ kz.transpose(1, 2)) * float(scale) + add
            lse = torch.logsumexp(sc, dim=2)
        outs.append(o.transpose(0, 1))
        lses.append(lse.transpose(0, 1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def pin_sdpa_no_sink(orc):
    x = _make([50, 33], seed=3)
    scale = np.float32(synth.SOFTMAX_SCALE)
    for lt, W in ((SWA, 129), (SWA, 17), (GA, 129)):
        ref_o, ref_l = _sdpa_rows(x, lt, W, scale, None)
        for s in (None, np.full(64, -np.inf, np.float32)):
            o, l = _run_prefill(orc, x, lt, W, float(scale), sink=s)
            _close(o, ref_o, 1e-10, f"sdpa no-sink out lt={lt} W={W}")
            _close(l, ref_l, 1e-10, f"sdpa no-sink lse lt={lt} W={W}")


def pin_sdpa_sink_as_extra_key(orc):
    x = _make([45, 21], seed=4)
    scale = np.float32(synth.SOFTMAX_SCALE)
    sink = (x.sink * 3.0).numpy().astype(np.float32)  # spread: some sinks dominate
    for lt, W in ((SWA, 129), (SWA, 9), (GA, 129)):
        ref_o, ref_l = _sdpa_rows(x, lt, W, scale, sink)
        o, l = _run_prefill(orc, x, lt, W, float(scale), sink=sink)
        _close(o, ref_o, 1e-10, f"sdpa sink out lt={lt} W={W}")
        _close(l, ref_l, 1e-10, f"sdpa sink lse lt={lt} W={W}")


def pin_first_query_closed_form(orc):
    """Position 0 sees only itself: o = vs * v0 / (1 + exp(sigma - s0)),
    lse = ln(exp(s0) + exp(sigma))."""
    x = _make([5, 9, 3], seed=5)
    scale = float(np.float32(synth.SOFTMAX_SCALE))
    vs = 0.707
    o, l = _run_prefill(orc, x, SWA, 129, scale, vs)
    cu = x.cu_seqlens.tolist()
    q, k, v, sk = _f64(x.q), _f64(x.k), _f64(x.v), x.sink.double()
    for b in range(3):
        t = cu[b]
        for h in range(64):
            g = h // 16
            s0 = scale * float(torch.dot(q[t, h], k[t, g]))
            sig = float(sk[h])
            exp_o = float(np.float32(vs)) * v[t, g].numpy() / (1.0 + math.exp(sig - s0))
            exp_l = max(s0, sig) + math.log1p(math.exp(-abs(s0 - sig)))
            _close(o[t, h], exp_o, 1e-12, "first-query out")
            _close(l[t, h], exp_l, 1e-12, "first-query lse")


def pin_equal_scores_closed_form(orc):
    """K = 0 makes every score 0: o = vs * sum_J v_j / (|J| + e^sigma),
    lse = ln(|J| + e^sigma); |J| = min(p+1, W) for SWA, p+1 for GA."""
    x = _make([300], seed=6)
    x.k.zero_()
    vs = 0.5
    v = _f64(x.v)[:, :, :].numpy()
    csum = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v, axis=0)])
    sk = x.sink.double().numpy()
    for lt, W in ((SWA, 129), (GA, 129), (SWA, 2)):
        o, l = _run_prefill(orc, x, lt, W, 0.25, vs)
        for p in (0, 1, 2, 127, 128, 129, 130, 200, 299):
            lo = max(0, p - (W - 1)) if lt == SWA else 0
            n = p + 1 - lo
            vsum = csum[p + 1] - csum[lo]  # [Hkv][Dv]
            for h in (0, 15, 16, 40, 63):
                den = n + math.exp(sk[h])
                _close(o[p, h], vs * vsum[h // 16] / den, 1e-12, f"equal-scores out lt={lt} W={W} p={p}")
                _close(l[p, h], math.log(den), 1e-12, f"equal-scores lse lt={lt} W={W} p={p}")


def pin_weights_normalised(orc):
    """Per query: weights + sink mass = 1, and weights vanish outside [lo, p]."""
    x = _make([40, 140], seed=7)
    for lt, W in ((SWA, 129), (SWA, 10), (GA, 129)):
        o, l, w = _run_prefill(orc, x, lt, W, float(np.float32(synth.SOFTMAX_SCALE)), want_weights=True)
        tot = w.sum(axis=2)
        _close(tot, np.ones_like(tot), 1e-12, f"weights sum lt={lt} W={W}")
        cu = x.cu_seqlens.tolist()
        for b in range(2):
            L = cu[b + 1] - cu[b]
            for p in range(L):
                lo = max(0, p - (W - 1)) if lt == SWA else 0
                row = w[cu[b] + p]
                assert np.all(row[:, :lo] == 0.0), "weight on a key left of the window"
                assert np.all(row[:, p + 1:-1] == 0.0), "weight on a future key"
                assert np.all(row[:, lo:p + 1] > 0.0), "a key in the set got zero weight"
                assert np.all(row[:, -1] > 0.0), "sink mass missing"


def pin_sink_neg_inf_is_no_sink(orc):
    x = _make([70], seed=8)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    for lt in (SWA, GA):
        o0, l0 = _run_prefill(orc, x, lt, 129, sc, sink=None)
        o1, l1 = _run_prefill(orc, x, lt, 129, sc, sink=np.full(64, -np.inf, np.float32))
        o2, l2 = _run_prefill(orc, x, lt, 129, sc, sink=np.full(64, -1e30, np.float32))
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), "-inf sink differs from no sink"
        assert np.array_equal(o0, o2) and np.array_equal(l0, l2), "-1e30 sink differs from no sink"
        o3, l3 = _run_prefill(orc, x, lt, 129, sc)
        assert not np.array_equal(l0, l3), "a finite sink changed nothing"


def pin_swa_equals_ga_when_window_covers(orc):
    x = _make([60, 100], seed=9)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    og, lg = _run_prefill(orc, x, GA, 129, sc)
    os_, ls = _run_prefill(orc, x, SWA, 129, sc)  # 129 >= 100
    assert np.array_equal(og, os_) and np.array_equal(lg, ls), "SWA(W>=L) != GA"
    os2, _ = _run_prefill(orc, x, SWA, 30, sc)
    assert not np.array_equal(og, os2), "a narrow window changed nothing"


def pin_gqa_equals_repeated_mha(orc):
    x = _make([37, 12], seed=10)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    rep = synth.PrefillInputs(x.q, x.k.repeat_interleave(16, dim=1).contiguous(),
                              x.v.repeat_interleave(16, dim=1).contiguous(), x.sink, x.cu_seqlens, x.lengths)
    for lt in (SWA, GA):
        o, l = _run_prefill(orc, x, lt, 20, sc)
        o2, l2 = _run_prefill(orc, rep, lt, 20, sc)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), "GQA != MHA with repeated K/V"


def pin_value_scale_linear(orc):
    x = _make([90], seed=11)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    o1, l1 = _run_prefill(orc, x, SWA, 129, sc, 1.0)
    o2, l2 = _run_prefill(orc, x, SWA, 129, sc, 0.707)
    assert np.array_equal(l1, l2), "value_scale changed the LSE"
    _close(o2, float(np.float32(0.707)) * o1, 1e-14, "value_scale linearity")
    assert abs(math.sqrt(4096 / (64 * 128)) - 0.707) < 5e-4


def _append_positions(orc, kc, vc, k_tok, v_tok, chunks, layer_type, window=129, base=None, cap=None):
    """Appends the tokens of one sequence in the given chunk sizes."""
    pos = 0
    for n in chunks:
        cu = np.array([0, n], np.int32)
        st = orc.kv_append(k_tok[pos:pos + n], v_tok[pos:pos + n], cu, np.array([pos], np.int32), kc, vc,
                           layer_type=layer_type, window=window, kv_base=base, kv_capacity=cap)
        assert st == oracle.OK, f"append status {st}"
        pos += n
    return pos


def pin_decode_equals_prefill_row(orc):
    """Cache positions 0..p-1 (bulk, then single tokens), decode token p: equals
    row p of prefill over the first p+1 tokens.  SWA rings of W-1 slots for
    windows 300, 129, 17 and 2 (a ring reader or writer that assumed 128 slots
    reads the wrong positions at every window but 129)."""
    L = 300
    x = _make([L], seed=12)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    kb, vb, qb = _bits(x.k), _bits(x.v), _bits(x.q)
    sink = x.sink.numpy()
    for lt, W in ((SWA, 300), (SWA, 129), (SWA, 17), (SWA, 2), (GA, 129)):
        R = W - 1
        ofull, lfull = _run_prefill(orc, x, lt, W, sc)
        for p in sorted({0, 1, R - 1, R, R + 1, 127, 128, 129, 200, 299} & set(range(1 if R == 0 else 0, L))):
            if lt == SWA:
                kc = np.zeros((1, R, 4, 192), np.uint16)
                vc = np.zeros((1, R, 4, 128), np.uint16)
                base = cap = None
            else:
                kc = np.zeros((L + 5, 4, 192), np.uint16)
                vc = np.zeros((L + 5, 4, 128), np.uint16)
                base = np.array([3], np.int64)
                cap = np.array([L], np.int64)
            chunks = [p // 2, p - p // 2 - min(3, p - p // 2)] + [1] * min(3, p - p // 2)
            chunks = [c for c in chunks if c > 0]
            _append_positions(orc, kc, vc, kb, vb, chunks, lt, W, base, cap)
            o, l = orc.decode(qb[p:p + 1], kb[p:p + 1], vb[p:p + 1], kc, vc, np.array([p], np.int32),
                              layer_type=lt, window=W, scale=sc, sink=sink, kv_base=base)
            _close(o[0], ofull[p], 1e-13, f"decode vs prefill out lt={lt} W={W} p={p}")
            _close(l[0], lfull[p], 1e-13, f"decode vs prefill lse lt={lt} W={W} p={p}")


def pin_ring_contents(orc):
    """After positions 0..p-1 are appended, ring slot r of a ring of R = W-1
    slots holds the unique position t = r (mod R) with p-R <= t <= p-1 (rings
    of 299, 128, 16 and 1 slots, i.e. windows 300, 129, 17 and 2)."""
    for R in (299, 128, 16, 1):
        for p, chunks in ((5, [5]), (R, [R]), (R + 1, [R + 1]), (128, [100, 28]), (300, [250, 1, 1, 48]),
                          (129, [129]), (2 * R + 3, [R, 2, R + 1])):
            tok = np.zeros((p, 1, 2), np.uint16)
            tok[:, 0, 0] = np.arange(p) + 1  # position tag (non-zero)
            kc = np.zeros((1, R, 1, 2), np.uint16)
            vc = np.zeros((1, R, 1, 2), np.uint16)
            pos = 0
            for n in chunks:
                st = orc.kv_append(tok[pos:pos + n], tok[pos:pos + n], np.array([0, n], np.int32),
                                   np.array([pos], np.int32), kc, vc, layer_type=SWA, window=R + 1)
                assert st == oracle.OK
                pos += n
            for r in range(R):
                want = [t for t in range(max(0, p - R), p) if t % R == r]
                got = int(kc[0, r, 0, 0])
                assert got == (want[0] + 1 if want else 0), f"ring slot {r} of {R} after {p}: {got}"


def pin_ga_capacity(orc):
    tok = np.ones((4, 1, 2), np.uint16)
    kc = np.zeros((10, 1, 2), np.uint16)
    vc = np.zeros((10, 1, 2), np.uint16)
    st = orc.kv_append(tok, tok, np.array([0, 4], np.int32), np.array([3], np.int32), kc, vc, layer_type=GA,
                       kv_base=np.array([2], np.int64), kv_capacity=np.array([6], np.int64))
    assert st == oracle.ECAPACITY and not kc.any(), "capacity overflow not refused"
    st = orc.kv_append(tok, tok, np.array([0, 4], np.int32), np.array([2], np.int32), kc, vc, layer_type=GA,
                       kv_base=np.array([2], np.int64), kv_capacity=np.array([6], np.int64))
    assert st == oracle.OK and kc[4:8].all() and not kc[:4].any() and not kc[8:].any()


def _caches(layer_type, batch, rows, window=129):
    if layer_type == SWA:
        R = window - 1
        return np.zeros((batch, R, 4, 192), np.uint16), np.zeros((batch, R, 4, 128), np.uint16)
    return np.zeros((rows, 4, 192), np.uint16), np.zeros((rows, 4, 128), np.uint16)


def _pack(a, lengths, starts):
    """Rows [starts[b], starts[b] + lengths[b]) of each sequence of a packed array."""
    return np.concatenate([a[s:s + n] for s, n in zip(starts, lengths)]) if sum(lengths) else a[:0]


def pin_chunk_without_cache_is_prefill(orc):
    """Chunked prefill with nothing cached is plain prefill."""
    x = _make([1, 40, 300, 129], seed=30)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    for lt in (SWA, GA):
        of, lf = _run_prefill(orc, x, lt, 129, sc)
        kc, vc = _caches(lt, 4, 8)
        base = np.zeros(4, np.int64) if lt == GA else None
        o, l = orc.prefill_chunk(_bits(x.q), _bits(x.k), _bits(x.v), x.cu_seqlens.numpy(), kc, vc,
                                 np.zeros(4, np.int32), layer_type=lt, scale=sc, sink=x.sink.numpy(), kv_base=base)
        _close(o, of, 1e-13, f"chunk without cache out lt={lt}")
        _close(l, lf, 1e-13, f"chunk without cache lse lt={lt}")


def pin_chunk_continues_prefill(orc):
    """Sequences of a ragged batch with their first c_b tokens cached (appended
    to the ring or pool) and the rest passed as one packed chunk: the chunk's
    rows equal rows c_b..L_b-1 of prefill over the whole sequences.  SWA over
    rings of W-1 slots for windows 300, 129, 17 and 2."""
    lengths = [300, 170, 64, 129, 260]
    cached = [0, 1, 63, 128, 131]
    x = _make(lengths, seed=31)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    qb, kb, vb = _bits(x.q), _bits(x.k), _bits(x.v)
    cu = x.cu_seqlens.numpy()
    rest = [L - c for L, c in zip(lengths, cached)]
    starts = [int(cu[b]) + cached[b] for b in range(len(lengths))]
    cu_new = np.concatenate([[0], np.cumsum(rest)]).astype(np.int32)
    for lt, W in ((SWA, 300), (SWA, 129), (SWA, 17), (SWA, 2), (GA, 129)):
        of, lf = _run_prefill(orc, x, lt, W, sc)
        kc, vc = _caches(lt, len(lengths), sum(lengths) + 7, W)
        base = cap = None
        if lt == GA:
            base = np.concatenate([[5], 5 + np.cumsum(lengths)[:-1]]).astype(np.int64)
            cap = np.asarray(lengths, np.int64)
        pre_cu = np.concatenate([[0], np.cumsum(cached)]).astype(np.int32)
        pre_k, pre_v = _pack(kb, cached, cu[:-1]), _pack(vb, cached, cu[:-1])
        st = orc.kv_append(pre_k, pre_v, pre_cu, np.zeros(len(lengths), np.int32), kc, vc, layer_type=lt,
                           window=W, kv_base=base, kv_capacity=cap)
        assert st == oracle.OK
        o, l = orc.prefill_chunk(_pack(qb, rest, starts), _pack(kb, rest, starts), _pack(vb, rest, starts), cu_new,
                                 kc, vc, np.asarray(cached, np.int32), layer_type=lt, window=W, scale=sc,
                                 sink=x.sink.numpy(), kv_base=base)
        rows = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, rest)])
        _close(o, of[rows], 1e-13, f"chunk vs prefill out lt={lt} W={W}")
        _close(l, lf[rows], 1e-13, f"chunk vs prefill lse lt={lt} W={W}")


def pin_chunk_of_one_token_is_decode(orc):
    """A chunk of one token per sequence is a decode step."""
    ctx = [0, 5, 127, 128, 400]
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    for lt in (SWA, GA):
        x = synth.decode_inputs(ctx, lt, seed=32)
        args = (_bits(x.q), _bits(x.k_new), _bits(x.v_new))
        base = None if x.kv_base is None else x.kv_base.numpy()
        od, ld = orc.decode(*args, _bits(x.k_cache), _bits(x.v_cache), x.ctx_lens.numpy(), layer_type=lt,
                            scale=sc, sink=x.sink.numpy(), kv_base=base)
        oc, lc = orc.prefill_chunk(*args, np.arange(len(ctx) + 1, dtype=np.int32), _bits(x.k_cache),
                                   _bits(x.v_cache), x.ctx_lens.numpy(), layer_type=lt, scale=sc,
                                   sink=x.sink.numpy(), kv_base=base)
        _close(oc, od, 1e-13, f"one-token chunk vs decode out lt={lt}")
        _close(lc, ld, 1e-13, f"one-token chunk vs decode lse lt={lt}")


def pin_chunks_in_sequence_rebuild_prefill(orc):
    """One sequence fed as chunks [50, 1, 100, 149], each attended and then
    appended: the concatenated chunk outputs equal the whole prefill."""
    L = 300
    x = _make([L], seed=33)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    qb, kb, vb = _bits(x.q), _bits(x.k), _bits(x.v)
    for lt in (SWA, GA):
        of, lf = _run_prefill(orc, x, lt, 129, sc)
        kc, vc = _caches(lt, 1, L + 3)
        base = np.array([3], np.int64) if lt == GA else None
        cap = np.array([L], np.int64) if lt == GA else None
        pos, outs, lses = 0, [], []
        for n in (50, 1, 100, 149):
            cu = np.array([0, n], np.int32)
            ctx = np.array([pos], np.int32)
            o, l = orc.prefill_chunk(qb[pos:pos + n], kb[pos:pos + n], vb[pos:pos + n], cu, kc, vc, ctx,
                                     layer_type=lt, scale=sc, sink=x.sink.numpy(), kv_base=base)
            outs.append(o)
            lses.append(l)
            assert orc.kv_append(kb[pos:pos + n], vb[pos:pos + n], cu, ctx, kc, vc, layer_type=lt, kv_base=base,
                                 kv_capacity=cap) == oracle.OK
            pos += n
        _close(np.concatenate(outs), of, 1e-13, f"chunks in sequence out lt={lt}")
        _close(np.concatenate(lses), lf, 1e-13, f"chunks in sequence lse lt={lt}")



def _paged_from_flat(flats, starts, lengths, page_size, max_blocks, rng, spare=3):
    """Rearranges flat pools (sequence b at rows starts[b] .. + lengths[b]-1) into
    paged pools with the blocks on randomly permuted pages (plus spare pages),
    by plain numpy slicing, one table for all.  Returns (paged pools, block
    table); unused table entries are -1."""
    nblk = [(L + page_size - 1) // page_size for L in lengths]
    npages = sum(nblk) + spare
    perm = rng.permutation(npages)
    table = np.full((len(lengths), max_blocks), -1, np.int32)
    pools = [np.zeros((npages * page_size,) + f.shape[1:], f.dtype) for f in flats]
    used = 0
    for b, (s0, L) in enumerate(zip(starts, lengths)):
        for i in range(nblk[b]):
            page = int(perm[used])
            used += 1
            table[b, i] = page
            n = min(page_size, L - i * page_size)
            for pool, f in zip(pools, flats):
                pool[page * page_size:page * page_size + n] = f[s0 + i * page_size:s0 + i * page_size + n]
    return pools, table


def pin_paged_decode_is_flat_decode(orc):
    """GA decode over a paged pool whose pages hold the flat pool's rows in a
    shuffled order equals decode over the flat pool, for page sizes 1, 3, 16
    and 64 and contexts on and around page boundaries."""
    ctx = [0, 1, 15, 16, 17, 64, 200]
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    x = synth.decode_inputs(ctx, GA, seed=34)
    base = x.kv_base.numpy()
    args = (_bits(x.q), _bits(x.k_new), _bits(x.v_new))
    kc, vc = _bits(x.k_cache), _bits(x.v_cache)
    od, ld = orc.decode(*args, kc, vc, x.ctx_lens.numpy(), layer_type=GA, scale=sc, sink=x.sink.numpy(),
                        kv_base=base)
    rng = np.random.default_rng(34)
    for P in (1, 3, 16, 64):
        mb = max((c + P - 1) // P for c in ctx) + 1
        (kp, vp), tb = _paged_from_flat([kc, vc], base, ctx, P, mb, rng)
        op, lp = orc.decode_paged(*args, kp, vp, tb, P, x.ctx_lens.numpy(), scale=sc, sink=x.sink.numpy())
        assert np.array_equal(op, od) and np.array_equal(lp, ld), f"paged decode differs from flat (page {P})"


def pin_paged_chunk_is_flat_chunk(orc):
    """GA chunked prefill with the cached prefixes in a shuffled paged pool
    equals chunked prefill over the flat pool."""
    lengths = [40, 170, 64, 33]
    cached = [0, 33, 64, 32]
    x = _make(lengths, seed=35)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    qb, kb, vb = _bits(x.q), _bits(x.k), _bits(x.v)
    cu = x.cu_seqlens.numpy()
    rest = [L - c for L, c in zip(lengths, cached)]
    starts = [int(cu[b]) + cached[b] for b in range(len(lengths))]
    cu_new = np.concatenate([[0], np.cumsum(rest)]).astype(np.int32)
    # flat pool: the cached prefix of sequence b sits at its packed rows cu[b] ..
    base = cu[:-1].astype(np.int64)
    of, lf = orc.prefill_chunk(_pack(qb, rest, starts), _pack(kb, rest, starts), _pack(vb, rest, starts), cu_new,
                               kb, vb, np.asarray(cached, np.int32), layer_type=GA, scale=sc, sink=x.sink.numpy(),
                               kv_base=base)
    for P in (1, 16, 32):
        mb = max((c + P - 1) // P for c in cached) + 2
        rng = np.random.default_rng(P)
        (kp, vp), tb = _paged_from_flat([kb, vb], base, cached, P, mb, rng)
        op, lp = orc.prefill_chunk_paged(_pack(qb, rest, starts), _pack(kb, rest, starts), _pack(vb, rest, starts),
                                         cu_new, kp, vp, tb, P, np.asarray(cached, np.int32), scale=sc,
                                         sink=x.sink.numpy())
        assert np.array_equal(op, of) and np.array_equal(lp, lf), f"paged chunk differs from flat (page {P})"


def pin_paged_append_places_positions(orc):
    """Appending to a paged pool (bulk, then single tokens) puts position j of
    sequence b at row table[b][j // P] * P + j % P, checked against a position
    tag; nothing else is written.  A sequence that would need more than
    max_blocks blocks is refused whole (filling exactly max_blocks * P is
    accepted), and a token on an unmapped block is not written."""
    P, mb = 4, 3
    table = np.array([[5, 0, 2], [1, -1, 3]], np.int32)  # page -1: unmapped
    npages = 7
    kc = np.zeros((npages * P, 1, 2), np.uint16)
    vc = np.zeros((npages * P, 1, 2), np.uint16)
    lengths = [12, 6]
    tags = [np.arange(L, dtype=np.uint16) + 1 + 100 * b for b, L in enumerate(lengths)]
    pos = [0, 0]
    for chunk in ((7, 3), (1, 1), (4, 2)):
        tok = np.zeros((sum(chunk), 1, 2), np.uint16)
        tok[:, 0, 0] = np.concatenate([tags[b][pos[b]:pos[b] + n] for b, n in enumerate(chunk)])
        cu = np.array([0, chunk[0], sum(chunk)], np.int32)
        st = orc.kv_append_paged(tok, tok, cu, np.array(pos, np.int32), kc, vc, table, P)
        # sequence 1's positions 4..7 sit on the unmapped block 1
        want = oracle.ECAPACITY if any(4 <= p < 8 for p in range(pos[1], pos[1] + chunk[1])) else oracle.OK
        assert st == want, f"append status {st}, expected {want}"
        pos = [p + n for p, n in zip(pos, chunk)]
    expect = np.zeros(npages * P, np.uint16)
    for b, L in enumerate(lengths):
        for j in range(L):
            page = table[b, j // P]
            if page >= 0:
                expect[page * P + j % P] = tags[b][j]
    assert np.array_equal(kc[:, 0, 0], expect) and np.array_equal(vc[:, 0, 0], expect), "paged append placement"
    assert not kc[:, 0, 1].any()
    before = kc.copy()
    one = np.ones((1, 1, 2), np.uint16)
    st = orc.kv_append_paged(one, one, np.array([0, 1, 1], np.int32), np.array([12, 0], np.int32), kc, vc, table, P)
    assert st == oracle.ECAPACITY and np.array_equal(kc, before), "append past max_blocks * page_size not refused"



# -- backward ------------------------------------------------------------------

def _torch_grads(x, dout, layer_type, window, scale, value_scale, sink):
    """Gradients of sum(dout * out) by torch fp64 autograd through a dense masked
    attention per sequence, the sink appended as one more logit with no value."""
    q = _f64(x.q).clone().requires_grad_(True)
    k = _f64(x.k).clone().requires_grad_(True)
    v = _f64(x.v).clone().requires_grad_(True)
    sg = None if sink is None else torch.tensor(np.float64(sink)).requires_grad_(True)
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    cu = x.cu_seqlens.tolist()
    loss = 0.0
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        if L == 0:
            continue
        qs = q[s0:s1].transpose(0, 1)                                   # [H, L, Dqk]
        ks = k[s0:s1].transpose(0, 1).repeat_interleave(G, dim=0)       # [H, L, Dqk]
        vs = v[s0:s1].transpose(0, 1).repeat_interleave(G, dim=0)       # [H, L, Dv]
        sc = float(scale) * (qs @ ks.transpose(1, 2))
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        ok = j <= i
        if layer_type == SWA:
            ok = ok & (j >= i - (window - 1))
        sc = sc.masked_fill(~ok, float("-inf"))
        if sg is not None:
            sc = torch.cat([sc, sg[:, None, None].expand(hq, L, 1)], dim=2)
        pr = torch.softmax(sc, dim=2)[:, :, :L]
        out = float(value_scale) * (pr @ vs)                              # [H, L, Dv]
        loss = loss + (out * _f64(dout[s0:s1]).transpose(0, 1)).sum()
    loss.backward()
    ds = None if sg is None else sg.grad.numpy()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), ds


def _rel_close(a, b, tol, what):
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b)))
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e} > {tol:.1e} x {scale:.3e}"


def pin_backward_torch_autograd(orc):
    """Oracle gradients (dq, dk, dv, dsink) equal torch fp64 autograd of a dense
    brute force, for SWA windows 5 and 129, GA, value_scale 0.707, with and
    without a sink, over a ragged batch."""
    x = _make([1, 9, 40], seed=80)
    dout = torch.randn((50, 64, 128), generator=torch.Generator().manual_seed(81)).to(torch.bfloat16)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    vsc = float(np.float32(0.707))
    for lt, win, sink in ((SWA, 5, x.sink.numpy()), (SWA, 129, x.sink.numpy()), (GA, 129, x.sink.numpy()),
                          (GA, 129, None)):
        dq, dk, dv, ds = orc.prefill_backward(_bits(x.q), _bits(x.k), _bits(x.v), _bits(dout), x.cu_seqlens.numpy(),
                                              layer_type=lt, window=win, scale=sc, value_scale=vsc, sink=sink)
        tq, tk, tv, ts = _torch_grads(x, dout, lt, win, sc, vsc, sink)
        _rel_close(dq, tq, 1e-12, f"dq lt={lt} W={win}")
        _rel_close(dk, tk, 1e-12, f"dk lt={lt} W={win}")
        _rel_close(dv, tv, 1e-12, f"dv lt={lt} W={win}")
        if sink is None:
            assert not ds.any(), "dsink without a sink must be 0"
        else:
            _rel_close(ds, ts, 1e-12, f"dsink lt={lt} W={win}")


def pin_backward_one_token_closed_form(orc):
    """One-token sequences: with s = scale q.k and P = 1 / (1 + exp(sigma - s)),
    out = value_scale P v, so d/dv = value_scale P dO, d/dsigma =
    -value_scale P (1 - P) dO.v, d/dq = scale value_scale P (1 - P) (dO.v) k and
    d/dk likewise with q (GQA: dk and dv sum the 16 heads of a group)."""
    x = _make([1, 1, 1], seed=82)
    dout = torch.randn((3, 64, 128), generator=torch.Generator().manual_seed(83)).to(torch.bfloat16)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    vsc = float(np.float32(0.707))
    sink = x.sink.numpy()
    dq, dk, dv, ds = orc.prefill_backward(_bits(x.q), _bits(x.k), _bits(x.v), _bits(dout), x.cu_seqlens.numpy(),
                                          layer_type=GA, scale=sc, value_scale=vsc, sink=sink)
    q, k, v, do = _f64(x.q).numpy(), _f64(x.k).numpy(), _f64(x.v).numpy(), _f64(dout).numpy()
    want_ds = np.zeros(64)
    for t in range(3):
        for h in range(64):
            g = h // 16
            s = sc * float(q[t, h] @ k[t, g])
            P = 1.0 / (1.0 + math.exp(float(sink[h]) - s))
            dov = float(do[t, h] @ v[t, g])
            _close(dq[t, h], sc * vsc * P * (1 - P) * dov * k[t, g], 1e-12, f"one-token dq t={t} h={h}")
            want_ds[h] -= vsc * P * (1 - P) * dov
        for g in range(4):
            hs = range(16 * g, 16 * g + 16)
            Ps = [1.0 / (1.0 + math.exp(float(sink[h]) - sc * float(q[t, h] @ k[t, g]))) for h in hs]
            wk = sum(sc * vsc * P * (1 - P) * float(do[t, h] @ v[t, g]) * q[t, h] for P, h in zip(Ps, hs))
            wv = sum(vsc * P * do[t, h] for P, h in zip(Ps, hs))
            _close(dk[t, g], wk, 1e-11, f"one-token dk t={t} g={g}")
            _close(dv[t, g], wv, 1e-12, f"one-token dv t={t} g={g}")
    _close(ds, want_ds, 1e-11, "one-token dsink")


def _bf16_nearest_even(x):
    """float64 array -> nearest bf16 values (as float64), ties to the even bit
    pattern, decided by exact rational distances among torch's conversion and
    its two bf16 neighbours (torch converts through float32, which can round
    twice)."""
    from fractions import Fraction
    flat = np.asarray(x, np.float64).ravel()
    b = torch.from_numpy(flat).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
    out = np.empty_like(flat)
    for i, (xv, bv) in enumerate(zip(flat, b)):
        cands = []
        for c in (bv - 1, bv, bv + 1):
            val = float(torch.tensor([c], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double())
            cands.append((abs(Fraction(val) - Fraction(float(xv))), c & 1, val))
        out[i] = min(cands)[2]
    return out.reshape(np.shape(x))


def pin_backward_stored_output_closed_form(orc):
    """With stored_out, D takes the forward output as a bf16 forward stores it.
    One-token sequences: out = bf16(value_scale P v) elementwise (rounded once,
    to nearest, ties to even), D' = dO.out, dS = P (value_scale dO.v - D'), so
    d/dq = scale dS k, d/dk sums scale dS q over the group, d/dsigma =
    -(1 - P) D', and d/dv is value_scale P dO as without the option.  Where the
    output is exact in bf16 (value_scale 1, no sink: out = v) the option changes
    nothing."""
    x = _make([1, 1, 1], seed=86)
    dout = torch.randn((3, 64, 128), generator=torch.Generator().manual_seed(87)).to(torch.bfloat16)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    vsc = float(np.float32(0.707))
    sink = x.sink.numpy()
    args = (_bits(x.q), _bits(x.k), _bits(x.v), _bits(dout), x.cu_seqlens.numpy())
    dq, dk, dv, ds = orc.prefill_backward(*args, layer_type=GA, scale=sc, value_scale=vsc, sink=sink,
                                          stored_out=True)
    exact = orc.prefill_backward(*args, layer_type=GA, scale=sc, value_scale=vsc, sink=sink)
    assert np.array_equal(dv, exact[2]), "dv depends on D"
    assert not np.array_equal(dk, exact[1]), "the stored output's rounding did not reach dk"
    q, k, v, do = _f64(x.q).numpy(), _f64(x.k).numpy(), _f64(x.v).numpy(), _f64(dout).numpy()
    want_ds = np.zeros(64)
    wk = np.zeros((3, 4, 192))
    for t in range(3):
        for h in range(64):
            g = h // 16
            P = 1.0 / (1.0 + math.exp(float(sink[h]) - sc * float(q[t, h] @ k[t, g])))
            out = _bf16_nearest_even(vsc * P * v[t, g])
            Dp = float(do[t, h] @ out)
            dS = P * (vsc * float(do[t, h] @ v[t, g]) - Dp)
            _close(dq[t, h], sc * dS * k[t, g], 1e-12, f"stored-out one-token dq t={t} h={h}")
            wk[t, g] += sc * dS * q[t, h]
            want_ds[h] -= (1.0 - P) * Dp
    _close(dk, wk, 1e-11, "stored-out one-token dk")
    _close(ds, want_ds, 1e-11, "stored-out one-token dsink")
    for lt in (SWA, GA):
        a = orc.prefill_backward(*args, layer_type=lt, scale=sc, sink=None, stored_out=True)
        b = orc.prefill_backward(*args, layer_type=lt, scale=sc, sink=None)
        for u, w in zip(a[:3], b[:3]):
            assert np.array_equal(u, w), "an exact bf16 output changed the gradients"


def pin_backward_rows_and_neg_inf_sink(orc):
    """Sampled rows equal the full computation, and a sink of -inf gives the
    no-sink gradients with dsink 0."""
    x = _make([30, 64], seed=84)
    dout = torch.randn((94, 64, 128), generator=torch.Generator().manual_seed(85)).to(torch.bfloat16)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    args = (_bits(x.q), _bits(x.k), _bits(x.v), _bits(dout), x.cu_seqlens.numpy())
    for lt in (SWA, GA):
        full = orc.prefill_backward(*args, layer_type=lt, window=17, scale=sc, sink=x.sink.numpy())
        qr, kr = np.array([0, 29, 30, 77, 93]), np.array([3, 30, 31, 90, 93])
        part = orc.prefill_backward(*args, layer_type=lt, window=17, scale=sc, sink=x.sink.numpy(), q_rows=qr,
                                    kv_rows=kr, want_dsink=False)
        assert np.array_equal(part[0], full[0][qr]) and np.array_equal(part[1], full[1][kr])
        assert np.array_equal(part[2], full[2][kr]) and part[3] is None
        none = orc.prefill_backward(*args, layer_type=lt, window=17, scale=sc, sink=None)
        ninf = orc.prefill_backward(*args, layer_type=lt, window=17, scale=sc,
                                    sink=np.full(64, -np.inf, np.float32))
        for a, b in zip(none[:3], ninf[:3]):
            assert np.array_equal(a, b), "sink -inf differs from no sink"
        assert not ninf[3].any()


def _transformers_attention(layer_type, window, q, k, v, sinks, value_scale, scale):
    """One sequence through the installed Transformers MiMo-V2-Flash attention
    module (MiMoV2FlashAttention.forward, eager path, fp64): its projections are
    selection matrices that hand it q, k and v unchanged, the rotary embedding is
    the identity (cos 1, sin 0), the additive mask is the library's own causal or
    sliding-window mask for `window`, and the output projection reads the heads'
    outputs back.  Returns out [L][Hq][Dv]."""
    from transformers.masking_utils import causal_mask_function, eager_mask, sliding_window_causal_mask_function
    from transformers.models.mimo_v2_flash import modeling_mimo_v2_flash as mm
    from transformers.models.mimo_v2_flash.configuration_mimo_v2_flash import MiMoV2FlashConfig
    L, hq, dqk = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    swa = layer_type == SWA
    nq, nk, nv, no = hq * dqk, hkv * dqk, hkv * dv, hq * dv
    hidden = nq + nk + nv
    cfg = MiMoV2FlashConfig(hidden_size=hidden, num_attention_heads=hq,
                            num_key_value_heads=hkv // 2 if swa else hkv,  # the library doubles SWA's KV heads
                            head_dim=dqk, v_head_dim=dv, num_hidden_layers=1, sliding_window=window,
                            layer_types=["sliding_attention" if swa else "full_attention"],
                            attention_value_scale=value_scale)
    cfg._attn_implementation = "eager"
    mod = mm.MiMoV2FlashAttention(cfg, 0).double().eval()
    assert mod.num_key_value_groups == hq // hkv and (mod.sinks is not None) == swa
    eye = torch.eye(hidden, dtype=torch.float64)
    with torch.no_grad():
        mod.q_proj.weight.copy_(eye[:nq])
        mod.k_proj.weight.copy_(eye[nq:nq + nk])
        mod.v_proj.weight.copy_(eye[nq + nk:])
        mod.o_proj.weight.copy_(torch.eye(hidden, no, dtype=torch.float64))
        if swa:
            mod.sinks.copy_(torch.as_tensor(sinks, dtype=torch.float64))
    mod.scaling = scale
    x = torch.cat([q.reshape(L, nq), k.reshape(L, nk), v.reshape(L, nv)], dim=1)[None]
    cos = torch.ones((1, L, dqk), dtype=torch.float64)
    sin = torch.zeros((1, L, dqk), dtype=torch.float64)
    fn = sliding_window_causal_mask_function(window) if swa else causal_mask_function
    mask = eager_mask(1, L, L, mask_function=fn, dtype=torch.float64)
    with torch.no_grad():
        out, _ = mod(x, (cos, sin), attention_mask=mask)
    return out[0, :, :no].reshape(L, hq, dv).numpy()


def pin_prefill_equals_transformers_attention_module(orc):
    """The oracle's prefill equals the installed Transformers MiMo-V2-Flash
    attention module run on the same q, k, v in fp64: its sink is one more logit
    per head, taken unscaled and dropped after the softmax (reading: denominator
    only), its value scale multiplies V before the attention (the same as scaling
    the output), its GQA repeats each KV head for a contiguous group of query
    heads, and its sliding-window mask for window W keeps the W keys up to and
    including the query.  SWA layers with a sink (windows 1, 4, 129 > L) and a GA
    layer without one, 4 query heads over 2 KV heads."""
    vs = float(np.float32(0.707))
    scale = float(np.float32(8 ** -0.5))
    for lt, window, seed in ((SWA, 4, 90), (SWA, 1, 91), (SWA, 129, 92), (GA, 129, 93)):
        x = _make([23], seed=seed, hq=4, hkv=2, dqk=8, dv=6)
        sink = x.sink.numpy() * 3.0 if lt == SWA else None
        o, _ = orc.prefill(_bits(x.q), _bits(x.k), _bits(x.v), x.cu_seqlens.numpy(), layer_type=lt, window=window,
                           scale=scale, value_scale=vs, sink=None if sink is None else sink.astype(np.float32))
        ref = _transformers_attention(lt, window, _f64(x.q), _f64(x.k), _f64(x.v),
                                      None if sink is None else sink.astype(np.float32).astype(np.float64), vs, scale)
        _close(o, ref, 1e-12, f"transformers module lt={lt} W={window}")


# -- rotary embedding ---------------------------------------------------------

def _rope_inputs(T, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, 64, 192), generator=g).to(torch.bfloat16)
    k = torch.randn((T, 4, 192), generator=g).to(torch.bfloat16)
    return q, k


def pin_rope_transformers_convention(orc):
    """The oracle's rotation equals Transformers' MiMo-V2-Flash apply_rotary_pos_emb
    (run in fp64) on cos/sin built from its default inverse frequencies, for
    rotary dims 64 (the library's 0.334 factor) and 192 and both of its thetas."""
    from types import SimpleNamespace
    from transformers.models.mimo_v2_flash import modeling_mimo_v2_flash as mm
    q, k = _rope_inputs(40, 70)
    pos = np.array(list(range(20)) + [1000 + 37 * i for i in range(20)], np.int32)
    for theta, factor in ((1e4, 0.334), (5e6, 0.334), (1e4, 1.0)):
        cfg = SimpleNamespace(rope_parameters={"x": {"rope_theta": theta, "partial_rotary_factor": factor}},
                              head_dim=192, hidden_size=4096, num_attention_heads=64)
        inv, _ = mm.MiMoV2FlashRotaryEmbedding.compute_default_rope_parameters(cfg, "cpu", layer_type="x")
        rd = 2 * inv.shape[0]
        assert rd == int(192 * factor) // 2 * 2
        ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv.to(torch.float64)[None, :]
        emb = torch.cat([ang, ang], dim=-1)
        cos, sin = emb.cos()[None], emb.sin()[None]  # [1, T, rd]
        lq, lk = mm.apply_rotary_pos_emb(_f64(q).transpose(0, 1)[None], _f64(k).transpose(0, 1)[None], cos, sin)
        oq, ok = orc.rope(_bits(q), _bits(k), pos, theta=theta, rotary_dim=rd)
        # the library's inverse frequencies are fp32: angles agree to ~1e-7 relative
        tol = 2e-7 * float(pos.max()) * 8 + 1e-12
        _close(oq, lq[0].transpose(0, 1).numpy(), tol, f"rope q theta={theta} rd={rd}")
        _close(ok, lk[0].transpose(0, 1).numpy(), tol, f"rope k theta={theta} rd={rd}")


def pin_rope_rotation_invariants(orc):
    """Rotation invariants: each head vector keeps its norm, dims past the rotary
    dims are untouched, position 0 is the identity, and q.k depends only on the
    difference of the two positions."""
    q, k = _rope_inputs(6, 71)
    qf, kf = _f64(q).numpy(), _f64(k).numpy()
    pos = np.array([0, 5, 129, 4096, 70000, 262143], np.int32)
    for rd in (64, 192):
        oq, ok = orc.rope(_bits(q), _bits(k), pos, theta=1e4, rotary_dim=rd)
        _close(np.linalg.norm(oq, axis=-1), np.linalg.norm(qf, axis=-1), 1e-12, "rope keeps norms")
        assert np.array_equal(oq[:, :, rd:], qf[:, :, rd:]) and np.array_equal(ok[:, :, rd:], kf[:, :, rd:])
        assert np.array_equal(oq[0], qf[0]) and np.array_equal(ok[0], kf[0]), "position 0 is the identity"
        # same q and k vectors at positions (p, j) and (p + c, j + c)
        qq = np.repeat(_bits(q)[1:2], 4, axis=0)
        kk = np.repeat(_bits(k)[1:2], 4, axis=0)
        rq, _ = orc.rope(qq, None, np.array([300, 1300, 60300, 300], np.int32), theta=1e4, rotary_dim=rd)
        _, rk = orc.rope(None, kk, np.array([100, 1100, 60100, 299], np.int32), theta=1e4, rotary_dim=rd)
        dots = np.einsum("thd,tgd->thg", rq, rk)
        _close(dots[1], dots[0], 1e-9, "rope shift invariance")
        _close(dots[2], dots[0], 1e-8, "rope shift invariance (far)")
        assert np.abs(dots[3] - dots[0]).max() > 1e-3, "a different offset must change q.k"

# -- FP8 (OCP E4M3) GA cache -------------------------------------------------

def _torch_e4m3_codes(x):
    """Codes of float32 values through torch's float8_e4m3fn (nearest, ties to even)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_probe_values():
    """Every rounding midpoint between neighbouring positive codes, 1-3 float32
    ulps either side, the codes themselves, both signs, plus random values."""
    grid = _torch_decode_all()[:0x7f]
    xs = []
    for a, b in zip(grid[:-1], grid[1:]):
        for v in (np.float32(a), np.float32((a + b) / 2)):
            xs.append(v)
            up = dn = v
            for _ in range(3):
                up = np.nextafter(up, np.float32(np.inf), dtype=np.float32)
                dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
                xs += [up, dn]
    xs = np.array(xs, np.float32)
    rng = np.random.default_rng(60)
    r = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000) * rng.choice([1e-3, 0.1, 10], 20000)])
    return np.concatenate([xs, -xs, r.astype(np.float32), np.float32([0.0, -0.0])])


def _torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_e4m3_decode_spec_table_and_torch(orc):
    """Decoding every code agrees with torch's float8_e4m3fn, and the named values
    of the format's table (largest/smallest normal and subnormal, NaN, zeros)."""
    import json
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    t = _torch_decode_all()
    assert np.all((d == t) | (np.isnan(d) & np.isnan(t))), "E4M3 decode differs from torch float8_e4m3fn"
    spec = json.load(open(os.path.join(HERE, "golden", "ocp_e4m3.json")))
    for key in ("max_normal", "min_normal", "max_subnormal", "min_subnormal"):
        c = int(spec[key]["code"], 16)
        assert d[c] == spec[key]["value"] and d[c | 0x80] == -spec[key]["value"], key
    assert all(np.isnan(d[int(c, 16)]) for c in spec["nan"]["codes"])
    assert int(np.isnan(d).sum()) == 2 and not np.isinf(d).any()
    assert all(d[int(c, 16)] == 0.0 for c in spec["zeros"]["codes"])
    assert d[0x38] == 1.0 and (0x38 >> 3) == spec["exponent_bias"]["value"]


def pin_e4m3_encode_nearest_even_saturating(orc):
    """Encoding equals torch's float8_e4m3fn rounding (nearest, ties to even) on
    every midpoint and its neighbouring floats, and saturates beyond +-448."""
    x = _e4m3_probe_values()
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3_codes(x)), "E4M3 encode differs from torch"
    big = np.float32([448.0, 449.0, 463.9, 464.0, 500.0, 1e9, -449.0, -1e30])
    assert np.array_equal(orc.e4m3_encode(big), np.uint8([0x7e] * 6 + [0xfe] * 2)), "no saturation at 448"
    c = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(orc.e4m3_decode(c))
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(c[finite]).astype(np.float32)), c[finite]), "round trip"


def _fp8_pool_case(ctx, seed, k_scale, v_scale, exact_bf16):
    """Random E4M3 code pools (no NaN codes) for GA decode, and the bf16 pools of
    their values when those are exact in bf16 (power-of-two scales)."""
    x = synth.decode_inputs(ctx, GA, seed=seed)
    rng = np.random.default_rng(seed)
    n = x.k_cache.shape[0]
    kc = rng.integers(0, 256, (n, 4, 192)).astype(np.uint8)
    vc = rng.integers(0, 256, (n, 4, 128)).astype(np.uint8)
    kc[(kc & 0x7f) == 0x7f] ^= 1   # NaN codes -> neighbouring finite codes
    vc[(vc & 0x7f) == 0x7f] ^= 1
    pools = None
    if exact_bf16:
        dec = _torch_decode_all()
        kf = (dec[kc] * np.asarray(k_scale)[None, :, None]).astype(np.float32)
        vf = (dec[vc] * np.asarray(v_scale)[None, :, None]).astype(np.float32)
        kb = torch.from_numpy(kf).to(torch.bfloat16)
        vb = torch.from_numpy(vf).to(torch.bfloat16)
        assert np.array_equal(kb.float().numpy(), kf) and np.array_equal(vb.float().numpy(), vf)
        pools = (_bits(kb), _bits(vb))
    return x, kc, vc, pools


def pin_fp8_decode_equals_bf16_where_exact(orc):
    """With power-of-two scales (different per head, for K and V) every
    dequantised value is exact in bf16: FP8 decode over the codes equals bf16
    decode over those values, for contexts 0, 1, 31, 32, 33, 300."""
    ctx = [0, 1, 31, 32, 33, 300]
    ks, vs = np.float32([0.5, 1.0, 2.0, 0.25]), np.float32([2.0, 0.125, 1.0, 4.0])
    x, kc, vc, (kb, vb) = _fp8_pool_case(ctx, 61, ks, vs, True)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    args = (_bits(x.q), _bits(x.k_new), _bits(x.v_new))
    o8, l8 = orc.decode_fp8(*args, kc, vc, x.kv_base.numpy(), ks, vs, x.ctx_lens.numpy(), scale=sc,
                            sink=x.sink.numpy())
    ob, lb = orc.decode(*args, kb, vb, x.ctx_lens.numpy(), layer_type=GA, scale=sc, sink=x.sink.numpy(),
                        kv_base=x.kv_base.numpy())
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb), "FP8 decode differs from bf16 decode on exact values"


def pin_fp8_decode_brute_force(orc):
    """Scales that are not powers of two: FP8 decode against a dense numpy brute
    force (dequantise, scores, sink-seeded softmax, weighted values)."""
    ctx = [0, 5, 64]
    ks, vs = np.float32([0.37, 0.011, 1.7, 0.05]), np.float32([0.021, 0.9, 0.33, 3.1])
    x, kc, vc, _ = _fp8_pool_case(ctx, 62, ks, vs, False)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    sink = x.sink.numpy()
    o8, l8 = orc.decode_fp8(_bits(x.q), _bits(x.k_new), _bits(x.v_new), kc, vc, x.kv_base.numpy(), ks, vs,
                            x.ctx_lens.numpy(), scale=sc, value_scale=0.707, sink=sink)
    dec = _torch_decode_all()
    q, kn, vn = _f64(x.q).numpy(), _f64(x.k_new).numpy(), _f64(x.v_new).numpy()
    base = x.kv_base.numpy()
    for b, p in enumerate(ctx):
        for h in range(64):
            g = h // 16
            K = np.concatenate([dec[kc[base[b]:base[b] + p, g]] * float(ks[g]), kn[b, g][None]])
            V = np.concatenate([dec[vc[base[b]:base[b] + p, g]] * float(vs[g]), vn[b, g][None]])
            s = np.float64(sc) * (K @ q[b, h])
            allv = np.append(s, float(sink[h]))
            mx = allv.max()
            lse = mx + np.log(np.exp(allv - mx).sum())
            o = float(np.float32(0.707)) * (np.exp(s - lse) @ V)
            # fp64 rounding-order differences scale with the value magnitudes (|V| up to ~1400 here)
            _close(o8[b, h], o, 1e-13 * (1 + np.abs(V).max()), f"fp8 decode brute force b={b} h={h}")
            assert abs(l8[b, h] - lse) < 1e-13 * (1 + np.abs(s).max())


def pin_fp8_append_codes(orc):
    """Appending to an FP8 pool stores torch's E4M3 code of (bf16 value / head
    scale) computed in float32, clamped to +-448, at row kv_base + position; a
    sequence past its capacity is skipped whole."""
    lengths = [5, 3]
    x = _make(lengths, seed=63)
    ks, vs = np.float32([0.37, 0.011, 1.7, 0.05]), np.float32([0.021, 0.9, 0.33, 3.1])
    kb, vb = _bits(x.k).copy(), _bits(x.v).copy()
    big = torch.tensor([1000.0, -3e5, 7.0], dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb[0, 1, :3] = big  # beyond 448 after scaling: saturates
    vb[1, 3, :3] = big
    kc = np.zeros((20, 4, 192), np.uint8)
    vc = np.zeros((20, 4, 128), np.uint8)
    base, cap = np.array([2, 12], np.int64), np.array([8, 4], np.int64)
    st = orc.kv_append_fp8(kb, vb, x.cu_seqlens.numpy(), np.array([1, 2], np.int32), kc, vc, base, cap, ks, vs)
    assert st == oracle.ECAPACITY  # sequence 1: 2 + 3 > 4
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vf = (vb.astype(np.uint32) << 16).view(np.float32)
    want_k = _torch_e4m3_codes(np.clip(kf[:5] / ks[None, :, None], -448, 448))
    want_v = _torch_e4m3_codes(np.clip(vf[:5] / vs[None, :, None], -448, 448))
    assert np.array_equal(kc[3:8], want_k) and np.array_equal(vc[3:8], want_v), "FP8 append codes"
    assert not kc[:3].any() and not kc[8:].any() and not vc[8:].any(), "FP8 append wrote outside its rows"
    assert kc[3, 1, 0] == 0x7e and kc[3, 1, 1] == 0xfe, "saturation"

def pin_fp8_paged_decode_is_flat_decode(orc):
    """FP8 decode over a paged pool whose pages hold the flat FP8 pool's code
    rows in a shuffled order equals FP8 decode over the flat pool (page sizes 1,
    16, 64; contexts around page boundaries)."""
    ctx = [0, 1, 15, 16, 17, 64, 200]
    ks, vs = np.float32([0.37, 0.011, 1.7, 0.05]), np.float32([0.021, 0.9, 0.33, 3.1])
    x, kc, vc, _ = _fp8_pool_case(ctx, 64, ks, vs, False)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    base, cl = x.kv_base.numpy(), x.ctx_lens.numpy()
    args = (_bits(x.q), _bits(x.k_new), _bits(x.v_new))
    of, lf = orc.decode_fp8(*args, kc, vc, base, ks, vs, cl, scale=sc, sink=x.sink.numpy())
    rng = np.random.default_rng(64)
    for P in (1, 16, 64):
        mb = max((c + P - 1) // P for c in ctx) + 1
        (kp, vp), tb = _paged_from_flat([kc, vc], base, ctx, P, mb, rng)
        op, lp = orc.decode_fp8_paged(*args, kp, vp, tb, P, ks, vs, cl, scale=sc, sink=x.sink.numpy())
        assert np.array_equal(op, of) and np.array_equal(lp, lf), f"paged FP8 decode differs from flat (page {P})"


def _fp8_chunk_case(seed, k_scale, v_scale, exact_bf16):
    """Chunked-prefill inputs over an FP8 pool: sequence b has cached[b]
    positions (code rows at base[b] ..) and brings rest[b] new bf16 tokens."""
    lengths = [40, 170, 64, 33]
    cached = [0, 33, 64, 32]
    rest = [L - c for L, c in zip(lengths, cached)]
    x = _make(rest, seed=seed)
    rng = np.random.default_rng(seed)
    base = np.array([3, 50, 120, 300], np.int64)
    rows = 340
    kc = rng.integers(0, 256, (rows, 4, 192)).astype(np.uint8)
    vc = rng.integers(0, 256, (rows, 4, 128)).astype(np.uint8)
    kc[(kc & 0x7f) == 0x7f] ^= 1
    vc[(vc & 0x7f) == 0x7f] ^= 1
    pools = None
    if exact_bf16:
        dec = _torch_decode_all()
        kf = (dec[kc] * np.asarray(k_scale)[None, :, None]).astype(np.float32)
        vf = (dec[vc] * np.asarray(v_scale)[None, :, None]).astype(np.float32)
        kb = torch.from_numpy(kf).to(torch.bfloat16)
        vb = torch.from_numpy(vf).to(torch.bfloat16)
        assert np.array_equal(kb.float().numpy(), kf) and np.array_equal(vb.float().numpy(), vf)
        pools = (_bits(kb), _bits(vb))
    return x, np.asarray(cached, np.int32), base, kc, vc, pools


def pin_fp8_chunk_equals_bf16_where_exact(orc):
    """With power-of-two scales every dequantised cached value is exact in
    bf16: chunked prefill over the FP8 codes equals chunked prefill over a bf16
    pool of those values (cached prefixes 0, 33, 64, 32)."""
    ks, vs = np.float32([0.5, 1.0, 2.0, 0.25]), np.float32([2.0, 0.125, 1.0, 4.0])
    x, cached, base, kc, vc, (kb, vb) = _fp8_chunk_case(65, ks, vs, True)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    args = (_bits(x.q), _bits(x.k), _bits(x.v), x.cu_seqlens.numpy())
    o8, l8 = orc.prefill_chunk_fp8(*args, kc, vc, ks, vs, cached, kv_base=base, scale=sc, sink=x.sink.numpy())
    ob, lb = orc.prefill_chunk(*args, kb, vb, cached, layer_type=GA, scale=sc, sink=x.sink.numpy(), kv_base=base)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb), "FP8 chunk differs from bf16 chunk on exact values"


def pin_fp8_chunk_brute_force_and_paged(orc):
    """Scales that are not powers of two: FP8 chunked prefill against a dense
    numpy brute force on sampled tokens (dequantised cached keys, then the
    chunk's own keys up to the token, sink-seeded softmax); the same cache in a
    shuffled paged pool gives the same results."""
    ks, vs = np.float32([0.37, 0.011, 1.7, 0.05]), np.float32([0.021, 0.9, 0.33, 3.1])
    x, cached, base, kc, vc, _ = _fp8_chunk_case(66, ks, vs, False)
    sc = float(np.float32(synth.SOFTMAX_SCALE))
    sink = x.sink.numpy()
    cu = x.cu_seqlens.numpy()
    args = (_bits(x.q), _bits(x.k), _bits(x.v), cu)
    o8, l8 = orc.prefill_chunk_fp8(*args, kc, vc, ks, vs, cached, kv_base=base, scale=sc, value_scale=0.707,
                                   sink=sink)
    dec = _torch_decode_all()
    q, k, v = _f64(x.q).numpy(), _f64(x.k).numpy(), _f64(x.v).numpy()
    for b in range(len(cached)):
        c, n = int(cached[b]), int(cu[b + 1] - cu[b])
        for i in sorted({0, n // 2, n - 1}) if n else ():
            t = int(cu[b]) + i
            for h in (0, 17, 38, 63):
                g = h // 16
                K = np.concatenate([dec[kc[base[b]:base[b] + c, g]] * float(ks[g]), k[cu[b]:t + 1, g]])
                V = np.concatenate([dec[vc[base[b]:base[b] + c, g]] * float(vs[g]), v[cu[b]:t + 1, g]])
                s = np.float64(sc) * (K @ q[t, h])
                allv = np.append(s, float(sink[h]))
                mx = allv.max()
                lse = mx + np.log(np.exp(allv - mx).sum())
                o = float(np.float32(0.707)) * (np.exp(s - lse) @ V)
                _close(o8[t, h], o, 1e-13 * (1 + np.abs(V).max()), f"fp8 chunk brute force t={t} h={h}")
                assert abs(l8[t, h] - lse) < 1e-13 * (1 + np.abs(s).max())
    rng = np.random.default_rng(66)
    for P in (1, 16, 32):
        mb = max((int(c) + P - 1) // P for c in cached) + 2
        (kp, vp), tb = _paged_from_flat([kc, vc], base, [int(c) for c in cached], P, mb, rng)
        op, lp = orc.prefill_chunk_fp8(*args, kp, vp, ks, vs, cached, block_table=tb, page_size=P, scale=sc,
                                       value_scale=0.707, sink=sink)
        assert np.array_equal(op, o8) and np.array_equal(lp, l8), f"paged FP8 chunk differs from flat (page {P})"


def pin_fp8_paged_append_places_codes(orc):
    """Appending to a paged FP8 pool writes, for every mapped position, the
    codes the flat FP8 append writes for it (bulk, then single tokens); a
    sequence that would need more than max_blocks blocks is refused whole, and
    a token on an unmapped block is not written."""
    P, mb = 4, 3
    table = np.array([[5, 0, 2], [1, -1, 3]], np.int32)
    npages = 7
    ks, vs = np.float32([0.37, 0.011, 1.7, 0.05]), np.float32([0.021, 0.9, 0.33, 3.1])
    lengths = [12, 6]
    x = _make(lengths, seed=67)
    kb, vb = _bits(x.k), _bits(x.v)
    cu = x.cu_seqlens.numpy()
    flat_k = np.zeros((40, 4, 192), np.uint8)
    flat_v = np.zeros((40, 4, 128), np.uint8)
    base = np.array([0, 20], np.int64)
    st = orc.kv_append_fp8(kb, vb, cu, np.zeros(2, np.int32), flat_k, flat_v, base, np.array([20, 20], np.int64),
                           ks, vs)
    assert st == oracle.OK
    kp = np.zeros((npages * P, 4, 192), np.uint8)
    vp = np.zeros((npages * P, 4, 128), np.uint8)
    pos = [0, 0]
    for chunk in ((7, 3), (1, 1), (4, 2)):
        sel = np.concatenate([np.arange(cu[b] + pos[b], cu[b] + pos[b] + n) for b, n in enumerate(chunk)])
        cu_c = np.array([0, chunk[0], sum(chunk)], np.int32)
        st = orc.kv_append_fp8_paged(kb[sel], vb[sel], cu_c, np.array(pos, np.int32), kp, vp, table, P, ks, vs)
        want = oracle.ECAPACITY if any(4 <= p < 8 for p in range(pos[1], pos[1] + chunk[1])) else oracle.OK
        assert st == want, f"append status {st}, expected {want}"
        pos = [p + n for p, n in zip(pos, chunk)]
    ek, ev = np.zeros_like(kp), np.zeros_like(vp)
    for b, L in enumerate(lengths):
        for j in range(L):
            page = table[b, j // P]
            if page >= 0:
                ek[page * P + j % P] = flat_k[base[b] + j]
                ev[page * P + j % P] = flat_v[base[b] + j]
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev), "paged FP8 append placement"
    full = np.zeros((2, 1, 192), np.uint16), np.zeros((2, 1, 128), np.uint16)
    kq = np.zeros((npages * P, 1, 192), np.uint8)
    vq = np.zeros((npages * P, 1, 128), np.uint8)
    st = orc.kv_append_fp8_paged(*full, np.array([0, 1, 2], np.int32), np.array([12, 11], np.int32), kq, vq,
                                 table, P, ks[:1], vs[:1])
    assert st == oracle.ECAPACITY and not kq.any(), "past max_blocks * P: sequence 0 refused whole"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]


# The slowest pins (seconds each); the mutation check runs them last.
SLOW_PINS = ("pin_rope_transformers_convention", "pin_chunk_continues_prefill", "pin_chunk_without_cache_is_prefill",
             "pin_chunks_in_sequence_rebuild_prefill")


def run_all(path: str, first_failure: bool = False):
    """Names of the pins that fail against the oracle build at `path` (all of them,
    or only the first, trying the slow pins last)."""
    orc = oracle.Oracle(path)
    pins = ALL_PINS
    if first_failure:
        pins = [p for p in ALL_PINS if p.__name__ not in SLOW_PINS] + \
               [p for p in ALL_PINS if p.__name__ in SLOW_PINS]
    failed = []
    for pin in pins:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
            if first_failure:
                break
    return failed


if __name__ == "__main__":  # used by the mutation test: prints failing pin names
    torch.set_num_threads(2)
    names = run_all(sys.argv[1], first_failure="--first" in sys.argv[2:])
    print("FAILED:" + ",".join(names))
