"""Check mode on the GPU, through the C ABI:
  * valid calls of every checked entry point give bit-identical outputs and
    caches with check mode on and off, and leave the device's check word 0;
  * a call whose device-resident arguments break a rule returns
    MIMO_ERR_PRECONDITION with that rule's bit, and its outputs and caches keep
    their previous bytes (none of its kernels ran);
  * under HIP graph capture the check joins the graph: each replay records its
    findings in the sticky word, and the captured kernels run as documented.
The violations used here are ones the kernels tolerate by contract (a context
past max_ctx gives NaN outputs, unmapped blocks are never dereferenced, a
sequence past its capacity is skipped, a sink or scale that is not finite only
yields non-finite numbers, a short max_seqlen leaves rows unwritten), so no
case depends on the gate to stay in bounds."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
SWA, GA = 0, 1
C = B.CHECK_BITS


@pytest.fixture
def check_on():
    B.mimo_attn_set_check(True)
    B.mimo_attn_check_flags(clear=True)
    yield
    torch.cuda.synchronize()
    B.mimo_attn_set_check(False)
    B.mimo_attn_check_flags(clear=True)


def both_modes(run):
    """run() -> tuple of tensors, once with check mode off and once on."""
    B.mimo_attn_set_check(False)
    off = [t.clone() for t in run()]
    torch.cuda.synchronize()
    B.mimo_attn_set_check(True)
    on = [t.clone() for t in run()]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(off, on)):
        assert torch.equal(a, b), f"result {i} differs under check mode"
    assert B.mimo_attn_check_flags(clear=True) == 0


def decode_setup(ctx, lt, seed):
    x = synth.decode_inputs(ctx, lt, seed=seed, headroom=2)
    return {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "ctx_lens",
                                               "sink")}


def test_valid_calls_unchanged(check_on):
    log("[case] check mode: valid calls of every checked entry point")
    lengths = [1, 130, 257]
    x = synth.prefill_inputs(lengths, seed=140)
    q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
    T = q.shape[0]
    for lt in (SWA, GA):
        both_modes(lambda: B.prefill(q, k, v, cu, max(lengths), lt, sink=sink))
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    both_modes(lambda: B.prefill_rope(q, k, v, pos, cu, max(lengths), GA, 5e6, 64, sink=sink))
    out, lse = B.prefill(q, k, v, cu, max(lengths), GA, sink=sink)
    dout = torch.randn_like(out.float()).to(torch.bfloat16)
    both_modes(lambda: B.prefill_backward(q, k, v, out, lse, dout, cu, max(lengths), GA, sink=sink))

    for lt in (SWA, GA):
        d = decode_setup([0, 5, 300, 129], lt, 141 + lt)
        both_modes(lambda: B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], 300,
                                    lt, sink=d["sink"], kv_base=d["kv_base"]))
        cap = torch.full((4,), 400, dtype=torch.int64, device=DEV) if lt == GA else None

        def step_rope(d=d, lt=lt, cap=cap):
            kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
            out, lse = B.decode_append_rope(d["q"], d["k_new"], d["v_new"], d["ctx_lens"], kc, vc, d["ctx_lens"], 300,
                                            lt, 5e6, 64, sink=d["sink"], kv_base=d["kv_base"], kv_capacity=cap)
            return out, lse, kc, vc
        both_modes(step_rope)
    # GA append, then chunked prefill over what it wrote
    base = torch.tensor([0, 300, 700], dtype=torch.int64, device=DEV)
    cap = torch.tensor([300, 400, 300], dtype=torch.int64, device=DEV)
    kc = torch.zeros((1000, 4, 192), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((1000, 4, 128), dtype=torch.bfloat16, device=DEV)
    zeros = torch.zeros(3, dtype=torch.int32, device=DEV)

    def append():
        kc.zero_()
        vc.zero_()
        B.kv_append(k, v, cu, zeros, kc, vc, GA, kv_base=base, kv_capacity=cap)
        return kc, vc
    both_modes(append)
    ctx = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    both_modes(lambda: B.prefill_chunk(q, k, v, cu, max(lengths), kc, vc, ctx, GA, sink=sink, kv_base=base))

    # paged pool: append, decode, chunk
    P = 16
    table, npages = synth.paged_block_table(lengths, P, seed=4, extra_tokens=200)
    table = table.to(DEV)
    kp = torch.zeros((npages * P, 4, 192), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros((npages * P, 4, 128), dtype=torch.bfloat16, device=DEV)

    def append_paged():
        kp.zero_()
        vp.zero_()
        B.kv_append_paged(k, v, cu, zeros, kp, vp, table, P)
        return kp, vp
    both_modes(append_paged)
    d = decode_setup(lengths, GA, 143)
    both_modes(lambda: B.decode_paged(d["q"], d["k_new"], d["v_new"], kp, vp, table, P, ctx, max(lengths),
                                      sink=d["sink"]))
    both_modes(lambda: B.prefill_chunk_paged(q, k, v, cu, max(lengths), kp, vp, table, P, ctx, sink=sink))

    # FP8 pool: append and decode
    ks = torch.tensor([0.01, 0.0173, 0.0071, 0.031], device=DEV)
    vs = torch.tensor([0.0105, 0.0063, 0.022, 0.0149], device=DEV)
    k8 = torch.zeros((1000, 4, 192), dtype=torch.uint8, device=DEV)
    v8 = torch.zeros((1000, 4, 128), dtype=torch.uint8, device=DEV)

    def append_fp8():
        k8.zero_()
        v8.zero_()
        B.kv_append_fp8(k, v, cu, zeros, k8, v8, base, cap, ks, vs)
        return k8, v8
    both_modes(append_fp8)
    both_modes(lambda: B.decode_fp8(d["q"], d["k_new"], d["v_new"], k8, v8, base, ks, vs, ctx, max(lengths),
                                    sink=d["sink"]))


def refused(bit, call, *untouched):
    before = [t.clone() for t in untouched]
    B.mimo_attn_check_flags(clear=True)
    with pytest.raises(B.MimoError) as e:
        call()
    torch.cuda.synchronize()
    assert e.value.status == B.MIMO_ERR_PRECONDITION, str(e.value)
    assert B.mimo_attn_check_flags(clear=True) == bit
    for a, b in zip(before, untouched):
        assert torch.equal(a, b), "a refused call changed a buffer"
    log(f"[check] refused with 0x{bit:03x}: {e.value}")


def test_violations_are_refused_before_any_kernel(check_on):
    log("[case] check mode: violations refused")
    lengths = [1, 130, 257]
    x = synth.prefill_inputs(lengths, seed=150)
    q, k, v, cu, sink = (to_dev(t) for t in (x.q, x.k, x.v, x.cu_seqlens, x.sink))
    T = q.shape[0]
    out = torch.full((T, 64, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, 64), 7.0, device=DEV)
    # a sequence longer than max_seqlen
    refused(C["CU_LENGTH"], lambda: B.prefill(q, k, v, cu, 200, GA, sink=sink, out=out, lse=lse), out, lse)
    # a NaN sink
    bad_sink = sink.clone()
    bad_sink[9] = float("nan")
    refused(C["SINK"], lambda: B.prefill(q, k, v, cu, 257, SWA, sink=bad_sink, out=out, lse=lse), out, lse)
    # backward with cu_seqlens ending before total_tokens
    dq = torch.full_like(q, 1.0)
    dk, dv = torch.full_like(k, 1.0), torch.full_like(v, 1.0)
    dsink = torch.full((64,), 1.0, device=DEV)
    nbytes = B.mimo_attn_prefill_backward_workspace_size(B.make_dims(), T)
    ws = torch.empty(nbytes // 4 + 4, device=DEV)
    short_cu = torch.tensor([0, 1, 131], dtype=torch.int32, device=DEV)
    refused(C["CU_TOTAL"], lambda: B.mimo_attn_prefill_backward(
        B.make_dims(), GA, q, k, v, out, lse, out, short_cu, 2, 130, T, sink, dq, dk, dv, dsink, ws), dq, dk, dv,
        dsink)

    # GA decode: a context past max_ctx
    d = decode_setup([10, 400, 20], GA, 151)
    dout = torch.full((3, 64, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    dlse = torch.full((3, 64), 7.0, device=DEV)
    refused(C["CTX_RANGE"], lambda: B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                             d["ctx_lens"], 300, GA, sink=d["sink"], kv_base=d["kv_base"], out=dout,
                                             lse=dlse), dout, dlse)

    # the fused decode step with RoPE: a context past max_ctx
    kd, vd = d["k_cache"].clone(), d["v_cache"].clone()
    capd = torch.full((3,), 500, dtype=torch.int64, device=DEV)
    refused(C["CTX_RANGE"], lambda: B.decode_append_rope(d["q"], d["k_new"], d["v_new"], d["ctx_lens"], kd, vd,
                                                         d["ctx_lens"], 300, GA, 5e6, 64, sink=d["sink"],
                                                         kv_base=d["kv_base"], kv_capacity=capd, out=dout, lse=dlse),
            dout, dlse, kd, vd)

    # append past a sequence's capacity
    base = torch.tensor([0, 300, 700], dtype=torch.int64, device=DEV)
    cap = torch.tensor([300, 100, 300], dtype=torch.int64, device=DEV)
    kc = torch.full((1000, 4, 192), 2.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full((1000, 4, 128), 2.0, dtype=torch.bfloat16, device=DEV)
    zeros = torch.zeros(3, dtype=torch.int32, device=DEV)
    refused(C["CAPACITY"], lambda: B.kv_append(k, v, cu, zeros, kc, vc, GA, kv_base=base, kv_capacity=cap), kc, vc)

    # FP8 append with a zero scale
    k8 = torch.full((1000, 4, 192), 5, dtype=torch.uint8, device=DEV)
    v8 = torch.full((1000, 4, 128), 5, dtype=torch.uint8, device=DEV)
    ks = torch.tensor([0.01, 0.0, 0.0071, 0.031], device=DEV)
    vs = torch.ones(4, device=DEV)
    cap_ok = torch.tensor([300, 400, 300], dtype=torch.int64, device=DEV)
    refused(C["FP8_SCALE"], lambda: B.kv_append_fp8(k, v, cu, zeros, k8, v8, base, cap_ok, ks, vs), k8, v8)

    # paged decode reading a block mapped outside the pool
    P = 16
    ctx = [40, 7, 100]
    table, npages = synth.paged_block_table(ctx, P, seed=5)
    table[2, 3] = npages + 4  # positions 48..63 of sequence 2
    table = table.to(DEV)
    kp = torch.zeros((npages * P, 4, 192), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros((npages * P, 4, 128), dtype=torch.bfloat16, device=DEV)
    dp = decode_setup(ctx, GA, 152)
    refused(C["BLOCK_TABLE"], lambda: B.decode_paged(dp["q"], dp["k_new"], dp["v_new"], kp, vp, table, P,
                                                     dp["ctx_lens"], 100, out=dout, lse=dlse), dout, dlse)


def test_graph_capture_records_findings(check_on):
    """A GA decode captured with check mode on: one capture whose context
    passes max_ctx (the check records it on every replay; the sequence's
    outputs are NaN by contract), one that is valid (word stays 0)."""
    log("[case] check mode under HIP graph capture")
    d = decode_setup([10, 400, 20], GA, 160)
    out = torch.empty((3, 64, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((3, 64), device=DEV)
    ws = torch.empty(B.mimo_attn_decode_workspace_size(B.make_dims(), GA, 3, 500, 0) // 4 + 4, device=DEV)

    def call(max_ctx):
        B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], max_ctx, GA,
                 sink=d["sink"], kv_base=d["kv_base"], out=out, lse=lse, workspace=ws)

    B.mimo_attn_set_check(False)
    refs = {}
    for max_ctx in (300, 500):
        call(max_ctx)
        torch.cuda.synchronize()
        refs[max_ctx] = out.clone(), lse.clone()
    B.mimo_attn_set_check(True)
    call(500)  # an eager checked call first: the check word's address is looked up outside capture
    torch.cuda.synchronize()
    assert B.mimo_attn_check_flags(clear=True) == 0
    for max_ctx, want in ((300, C["CTX_RANGE"]), (500, 0)):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call(max_ctx)
        torch.cuda.synchronize()
        assert B.mimo_attn_check_flags(clear=True) == 0, "capture ran the check"
        ref_out, ref_lse = refs[max_ctx]
        keep = [0, 2] if want else [0, 1, 2]
        for r in range(3):
            out.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert B.mimo_attn_check_flags(clear=True) == want, f"replay {r}, max_ctx {max_ctx}"
            assert torch.equal(out[keep], ref_out[keep]) and torch.equal(lse[keep], ref_lse[keep])
            if want:
                assert torch.isnan(out[1].float()).all()
        del g
    log("[check] captured decode: findings recorded on every replay")
