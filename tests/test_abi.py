"""The C-ABI library on the CPU: it loads, exports every function include/*.h
declares, and rejects misuse on the host with the documented status before
anything is enqueued.  Every call below carries at least one invalid argument,
so no kernel is ever launched; the pointer values are never dereferenced."""
import ctypes
import glob
import os
import re

import pytest

from global_attention_mimo_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte-aligned stand-in pointer; validation never reads it
FAKE_ODD = 0x10008  # 8-byte aligned only


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(mimo_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIBRARY):
        from global_attention_mimo_amd import build
        build.build()
    return B.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert names == set(B.ENTRY_POINTS), names
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_version_and_status_strings(L):
    assert B.mimo_abi_version() == 14
    assert B.mimo_status_string(0) == "MIMO_OK"
    assert B.mimo_status_string(3) == "MIMO_ERR_WORKSPACE"
    assert B.mimo_status_string(99) == "MIMO_ERR_UNKNOWN"


def prefill_call(L, dims=None, layer=0, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, nseq=1, maxlen=16, out=FAKE):
    d = dims if dims is not None else B.make_dims()
    return L.mimo_attn_prefill(ctypes.byref(d) if d is not False else None, layer, q, k, v, cu, nseq, maxlen, None,
                               out, None, None)


@pytest.mark.parametrize("case,status", [
    (dict(dims=False), B.MIMO_ERR_INVALID_ARG),
    (dict(layer=2), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(out=None), B.MIMO_ERR_INVALID_ARG),
    (dict(cu=None), B.MIMO_ERR_INVALID_ARG),
    (dict(k=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=0), B.MIMO_ERR_INVALID_ARG),
    (dict(maxlen=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(num_q_heads=64, num_kv_heads=8)), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(num_q_heads=60, num_kv_heads=8)), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(head_dim_qk=128)), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(head_dim_v=192)), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(num_kv_heads=0)), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(num_q_heads=16 * 4096, num_kv_heads=4096)), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(sliding_window=0)), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(softmax_scale=float("nan"))), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(value_scale=float("inf"))), B.MIMO_ERR_INVALID_ARG),
])
def test_prefill_rejects(L, case, status):
    assert prefill_call(L, **case) == status
    assert B.mimo_last_error() != ""


def test_prefill_empty_is_ok_without_launch(L):
    assert prefill_call(L, maxlen=0) == B.MIMO_OK


def chunk_call(L, dims=None, layer=1, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, nseq=2, maxlen=16, kc=FAKE, vc=FAKE,
               base=FAKE, ctx=FAKE, out=FAKE):
    d = dims if dims is not None else B.make_dims()
    return L.mimo_attn_prefill_chunk(ctypes.byref(d) if d is not False else None, layer, q, k, v, cu, nseq, maxlen,
                                     kc, vc, base, ctx, None, out, None, None)


@pytest.mark.parametrize("case,status", [
    (dict(dims=False), B.MIMO_ERR_INVALID_ARG),
    (dict(layer=2), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(cu=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(vc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
    (dict(out=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=0), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=70000), B.MIMO_ERR_INVALID_ARG),
    (dict(maxlen=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(layer=0, dims=B.make_dims(sliding_window=1)), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(head_dim_v=64)), B.MIMO_ERR_UNSUPPORTED),
])
def test_prefill_chunk_rejects(L, case, status):
    assert chunk_call(L, **case) == status
    assert B.mimo_last_error() != ""


def test_prefill_chunk_empty_is_ok_and_swa_needs_no_base(L):
    assert chunk_call(L, maxlen=0) == B.MIMO_OK
    assert chunk_call(L, layer=0, base=None, maxlen=0) == B.MIMO_OK


def decode_call(L, dims=None, layer=1, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, base=FAKE, ctx=FAKE, batch=2,
                max_ctx=100, split=0, out=FAKE, ws=None, ws_bytes=0):
    d = dims or B.make_dims()
    return L.mimo_attn_decode(ctypes.byref(d), layer, q, kn, vn, kc, vc, base, ctx, batch, max_ctx, split, None, out,
                              None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(layer=5), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(vn=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(max_ctx=-3), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=100), B.MIMO_ERR_WORKSPACE),
    (dict(layer=0, dims=B.make_dims(sliding_window=1)), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(head_dim_qk=64)), B.MIMO_ERR_UNSUPPORTED),
    (dict(max_ctx=1_400_000), B.MIMO_ERR_UNSUPPORTED),  # > 2 GiB of K rows for one sequence
    (dict(layer=0, dims=B.make_dims(sliding_window=2_000_000)), B.MIMO_ERR_UNSUPPORTED),
])
def test_decode_rejects(L, case, status):
    assert decode_call(L, **case) == status


def noalloc_call(L, dims=None, layer=1, batch=2, max_ctx=100):
    d = dims or B.make_dims()
    return L.mimo_attn_decode_noalloc(ctypes.byref(d), layer, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, batch, max_ctx,
                                      0, None, FAKE, None, None)


@pytest.mark.parametrize("case,status", [
    (dict(layer=5), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(head_dim_qk=64)), B.MIMO_ERR_UNSUPPORTED),
    (dict(batch=1008), B.MIMO_ERR_UNSUPPORTED),                                   # scratch holds 1007 slots of 64 heads
    (dict(batch=300, dims=B.make_dims(num_q_heads=256, num_kv_heads=16)), B.MIMO_ERR_UNSUPPORTED),
])
def test_noalloc_rejects_before_touching_the_device(L, case, status):
    """Checks that need no GPU: the scratch capacity (32 MiB) is a host-side bound."""
    assert noalloc_call(L, **case) == status
    assert B.mimo_last_error() != ""


def decode_append_call(L, layer=1, q=FAKE, kc=FAKE, base=FAKE, cap=FAKE, ctx=FAKE, batch=2):
    d = B.make_dims()
    return L.mimo_attn_decode_append(ctypes.byref(d), layer, q, FAKE, FAKE, kc, FAKE, base, cap, ctx, batch, 100, 0,
                                     None, FAKE, None, None, 0, None)


@pytest.mark.parametrize("case,status", [
    (dict(layer=5), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(cap=None), B.MIMO_ERR_INVALID_ARG),   # GA append needs the capacities
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
])
def test_decode_append_rejects(L, case, status):
    assert decode_append_call(L, **case) == status


def decode_append_rope_call(L, layer=1, q=FAKE, pos=FAKE, kc=FAKE, base=FAKE, cap=FAKE, ctx=FAKE, batch=2,
                            theta=1e4, rd=64):
    d = B.make_dims()
    return L.mimo_attn_decode_append_rope(ctypes.byref(d), layer, q, FAKE, FAKE, pos, kc, FAKE, base, cap, ctx,
                                          batch, 100, 0, theta, rd, None, FAKE, None, None, 0, None)


@pytest.mark.parametrize("case,status", [
    (dict(layer=5), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(pos=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(cap=None), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=1.0), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=float("inf")), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=float("nan")), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=32), B.MIMO_ERR_UNSUPPORTED),      # the pair would sit in another lane: use mimo_rope_apply
    (dict(rd=96), B.MIMO_ERR_UNSUPPORTED),
    (dict(rd=0), B.MIMO_ERR_UNSUPPORTED),
    (dict(rd=256), B.MIMO_ERR_UNSUPPORTED),
    (dict(layer=0, rd=100), B.MIMO_ERR_UNSUPPORTED),
])
def test_decode_append_rope_rejects(L, case, status):
    assert decode_append_rope_call(L, **case) == status
    assert B.mimo_last_error() != ""


def ga_workspace_expected(batch, max_ctx, split, hq=64):
    """The GA decode workspace as the header states it: a header of batch + 2
    int64 padded to 256 bytes, then (chunks + batch) slots of hq x 130 fp32,
    chunks = the split grid for batch sequences of max_ctx cached keys (units of
    32 keys plus one per new token, chunks of at least max(1, ceil(split/32))
    units, default 8, in whole rounds of 256 up to 4 rounds)."""
    units = batch * (-(-max_ctx // 32) + 1)
    mu = 8 if split <= 0 else -(-min(split, 1 << 30) // 32)
    by_len = -(-units // mu)
    chunks = max(1, min(by_len, 256))
    header = -(-8 * (batch + 2) // 256) * 256
    return header + (chunks + batch) * hq * 130 * 4


def test_workspace_size(L):
    d = B.make_dims()
    ws = lambda b, c, s: B.mimo_attn_decode_workspace_size(d, 1, b, c, s)
    for b, c, s in [(3, 4095, 2048), (3, 4096, 2048), (1, 0, 0), (2, 100, 33), (128, 262207, 0), (32, 32832, 0),
                    (32, 32832, 384), (1, 262143, 0), (4, 65535, 1024), (3, 4095, 256), (7, 5, 32)]:
        assert ws(b, c, s) == ga_workspace_expected(b, c, s), (b, c, s)
    # Worked values: one short sequence needs one chunk; the long-context batch
    # of 128 sequences caps at 256 chunks (12.8 MB, not per split).
    assert ws(1, 0, 0) == 256 + 2 * 64 * 130 * 4
    assert ws(128, 262207, 0) == 1280 + (256 + 128) * 64 * 130 * 4
    assert ws(128, 262207, 0) == ws(128, 100000, 0)          # bounded by the chunk cap, not by max_ctx
    big = (1 << 31) - 2                                       # largest accepted max_ctx
    assert ws(65535, big, 0) == ga_workspace_expected(65535, big, 0)
    assert ws(65536, 10, 0) == 0 and ws(1, (1 << 31) - 1, 0) == 0   # what decode rejects
    assert B.mimo_attn_decode_workspace_size(d, 0, 128, 262144, 0) == 0
    assert B.mimo_attn_decode_workspace_size(d, 1, 0, 10, 0) == 0
    assert B.mimo_attn_decode_workspace_size(B.make_dims(head_dim_v=64), 1, 1, 10, 0) == 0


def append_call(L, dims=None, layer=1, k=FAKE, v=FAKE, cu=FAKE, ctx=FAKE, batch=1, total=4, kc=FAKE, vc=FAKE,
                base=FAKE, cap=FAKE):
    d = dims or B.make_dims()
    return L.mimo_kv_append(ctypes.byref(d), layer, k, v, cu, ctx, batch, total, kc, vc, base, cap, None)


@pytest.mark.parametrize("case,status", [
    (dict(k=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(cap=None), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(vc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(layer=0, dims=B.make_dims(sliding_window=1)), B.MIMO_ERR_INVALID_ARG),
    (dict(dims=B.make_dims(num_q_heads=32)), B.MIMO_ERR_UNSUPPORTED),
])
def test_append_rejects(L, case, status):
    assert append_call(L, **case) == status


def test_append_nothing_is_ok_without_launch(L):
    assert append_call(L, total=0) == B.MIMO_OK


def pages(table=FAKE, max_blocks=8, page_size=16, num_pages=100):
    return B.mimo_kv_pages(table, max_blocks, page_size, num_pages)


PAGES_BAD = [
    (dict(table=None), B.MIMO_ERR_INVALID_ARG),
    (dict(max_blocks=0), B.MIMO_ERR_INVALID_ARG),
    (dict(num_pages=0), B.MIMO_ERR_INVALID_ARG),
    (dict(page_size=0), B.MIMO_ERR_INVALID_ARG),
    (dict(page_size=8), B.MIMO_ERR_UNSUPPORTED),
    (dict(page_size=48), B.MIMO_ERR_UNSUPPORTED),
    (dict(page_size=1 << 17), B.MIMO_ERR_UNSUPPORTED),
]


def paged_decode_call(L, pg=None, q=FAKE, kc=FAKE, ctx=FAKE, batch=2, max_ctx=100, split=0, ws=FAKE,
                      ws_bytes=1 << 30, dims=None):
    d = dims or B.make_dims()
    pref = None if pg is False else ctypes.byref(pg or pages())
    return L.mimo_attn_decode_paged(ctypes.byref(d), q, FAKE, FAKE, kc, FAKE, pref, ctx, batch, max_ctx, split, None,
                                    FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [(dict(pg=pages(**c)), st) for c, st in PAGES_BAD] + [
    (dict(pg=False), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(ws_bytes=100), B.MIMO_ERR_WORKSPACE),
    (dict(dims=B.make_dims(head_dim_qk=64)), B.MIMO_ERR_UNSUPPORTED),
])
def test_decode_paged_rejects(L, case, status):
    assert paged_decode_call(L, **case) == status
    assert B.mimo_last_error() != ""


def paged_chunk_call(L, pg=None, q=FAKE, kc=FAKE, ctx=FAKE, nseq=2, maxlen=16):
    pref = None if pg is False else ctypes.byref(pg or pages())
    return L.mimo_attn_prefill_chunk_paged(ctypes.byref(B.make_dims()), q, FAKE, FAKE, FAKE, nseq, maxlen, kc, FAKE,
                                           pref, ctx, None, FAKE, None, None)


@pytest.mark.parametrize("case,status", [(dict(pg=pages(**c)), st) for c, st in PAGES_BAD] + [
    (dict(pg=False), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=0), B.MIMO_ERR_INVALID_ARG),
    (dict(maxlen=-1), B.MIMO_ERR_INVALID_ARG),
])
def test_prefill_chunk_paged_rejects(L, case, status):
    assert paged_chunk_call(L, **case) == status


def paged_append_call(L, pg=None, k=FAKE, kc=FAKE, batch=1, total=4):
    pref = None if pg is False else ctypes.byref(pg or pages())
    return L.mimo_kv_append_paged(ctypes.byref(B.make_dims()), k, FAKE, FAKE, FAKE, batch, total, kc, FAKE, pref,
                                  None)


@pytest.mark.parametrize("case,status", [(dict(pg=pages(**c)), st) for c, st in PAGES_BAD] + [
    (dict(pg=False), B.MIMO_ERR_INVALID_ARG),
    (dict(k=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
])
def test_append_paged_rejects(L, case, status):
    assert paged_append_call(L, **case) == status


def test_paged_empty_calls_are_ok(L):
    assert paged_chunk_call(L, maxlen=0) == B.MIMO_OK
    assert paged_append_call(L, total=0) == B.MIMO_OK


def fp8_decode_call(L, q=FAKE, kc=FAKE, base=FAKE, ks=FAKE, vs=FAKE, ctx=FAKE, batch=2, max_ctx=100, ws=FAKE,
                    ws_bytes=1 << 30, dims=None):
    d = dims or B.make_dims()
    return L.mimo_attn_decode_fp8(ctypes.byref(d), q, FAKE, FAKE, kc, FAKE, base, ks, vs, ctx, batch, max_ctx, 0,
                                  None, FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ks=None), B.MIMO_ERR_INVALID_ARG),
    (dict(vs=FAKE + 2), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(max_ctx=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(max_ctx=2_800_000), B.MIMO_ERR_UNSUPPORTED),  # > 2 GiB of K codes for one sequence
    (dict(dims=B.make_dims(head_dim_v=64)), B.MIMO_ERR_UNSUPPORTED),
])
def test_decode_fp8_rejects(L, case, status):
    assert fp8_decode_call(L, **case) == status
    assert B.mimo_last_error() != ""


def fp8_append_call(L, k=FAKE, kc=FAKE, base=FAKE, cap=FAKE, ks=FAKE, vs=FAKE, batch=1, total=4):
    return L.mimo_kv_append_fp8(ctypes.byref(B.make_dims()), k, FAKE, FAKE, FAKE, batch, total, kc, FAKE, base, cap,
                                ks, vs, None)


@pytest.mark.parametrize("case,status", [
    (dict(k=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),
    (dict(cap=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ks=None), B.MIMO_ERR_INVALID_ARG),
    (dict(vs=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
])
def test_append_fp8_rejects(L, case, status):
    assert fp8_append_call(L, **case) == status


def test_append_fp8_nothing_is_ok(L):
    assert fp8_append_call(L, total=0) == B.MIMO_OK


def fp8_paged_decode_call(L, pg=None, kc=FAKE, ks=FAKE, vs=FAKE, ctx=FAKE, batch=2, max_ctx=100, ws=FAKE,
                          ws_bytes=1 << 30):
    pref = None if pg is False else ctypes.byref(pg or pages())
    return L.mimo_attn_decode_fp8_paged(ctypes.byref(B.make_dims()), FAKE, FAKE, FAKE, kc, FAKE, pref, ks, vs, ctx,
                                        batch, max_ctx, 0, None, FAKE, None, ws, ws_bytes, None)


def fp8_paged_append_call(L, pg=None, kc=FAKE, ks=FAKE, vs=FAKE, batch=1, total=4):
    pref = None if pg is False else ctypes.byref(pg or pages())
    return L.mimo_kv_append_fp8_paged(ctypes.byref(B.make_dims()), FAKE, FAKE, FAKE, FAKE, batch, total, kc, FAKE,
                                      pref, ks, vs, None)


def fp8_chunk_call(L, paged=False, pg=None, kc=FAKE, base=FAKE, ks=FAKE, vs=FAKE, ctx=FAKE, nseq=2, maxlen=16):
    d = ctypes.byref(B.make_dims())
    if paged:
        pref = None if pg is False else ctypes.byref(pg or pages())
        return L.mimo_attn_prefill_chunk_fp8_paged(d, FAKE, FAKE, FAKE, FAKE, nseq, maxlen, kc, FAKE, pref, ks, vs,
                                                   ctx, None, FAKE, None, None)
    return L.mimo_attn_prefill_chunk_fp8(d, FAKE, FAKE, FAKE, FAKE, nseq, maxlen, kc, FAKE, base, ks, vs, ctx, None,
                                         FAKE, None, None)


FP8_COMMON_BAD = [
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(ks=None), B.MIMO_ERR_INVALID_ARG),
    (dict(vs=FAKE + 2), B.MIMO_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("case,status", FP8_COMMON_BAD + [(dict(pg=pages(**c)), st) for c, st in PAGES_BAD] + [
    (dict(pg=False), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
])
def test_decode_fp8_paged_rejects(L, case, status):
    assert fp8_paged_decode_call(L, **case) == status
    assert B.mimo_last_error() != ""


@pytest.mark.parametrize("case,status", FP8_COMMON_BAD + [(dict(pg=pages(**c)), st) for c, st in PAGES_BAD] + [
    (dict(pg=False), B.MIMO_ERR_INVALID_ARG),
    (dict(batch=0), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
])
def test_append_fp8_paged_rejects(L, case, status):
    assert fp8_paged_append_call(L, **case) == status


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("case,status", FP8_COMMON_BAD + [
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=0), B.MIMO_ERR_INVALID_ARG),
    (dict(maxlen=-1), B.MIMO_ERR_INVALID_ARG),
])
def test_prefill_chunk_fp8_rejects(L, paged, case, status):
    assert fp8_chunk_call(L, paged=paged, **case) == status


def test_fp8_layout_rejects_and_empty_calls(L):
    assert fp8_chunk_call(L, base=None) == B.MIMO_ERR_INVALID_ARG  # contiguous GA needs kv_base
    assert fp8_chunk_call(L, paged=True, pg=False) == B.MIMO_ERR_INVALID_ARG
    assert fp8_chunk_call(L, maxlen=0) == B.MIMO_OK
    assert fp8_chunk_call(L, paged=True, maxlen=0) == B.MIMO_OK
    assert fp8_paged_append_call(L, total=0) == B.MIMO_OK


def bwd_call(L, dims=None, layer=1, q=FAKE, out=FAKE, lse=FAKE, do=FAKE, cu=FAKE, nseq=2, maxlen=16, total=32,
             dq=FAKE, dk=FAKE, ws=FAKE, ws_bytes=1 << 30):
    d = dims or B.make_dims()
    return L.mimo_attn_prefill_backward(ctypes.byref(d), layer, q, FAKE, FAKE, out, lse, do, cu, nseq, maxlen, total,
                                        None, dq, dk, FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(layer=3), B.MIMO_ERR_INVALID_ARG),
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(out=None), B.MIMO_ERR_INVALID_ARG),
    (dict(lse=None), B.MIMO_ERR_INVALID_ARG),
    (dict(do=None), B.MIMO_ERR_INVALID_ARG),
    (dict(do=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(cu=None), B.MIMO_ERR_INVALID_ARG),
    (dict(dq=None), B.MIMO_ERR_INVALID_ARG),
    (dict(dk=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(nseq=0), B.MIMO_ERR_INVALID_ARG),
    (dict(maxlen=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(ws_bytes=100), B.MIMO_ERR_WORKSPACE),
    (dict(dims=B.make_dims(head_dim_qk=128)), B.MIMO_ERR_UNSUPPORTED),
])
def test_backward_rejects(L, case, status):
    assert bwd_call(L, **case) == status
    assert B.mimo_last_error() != ""


def test_backward_empty_and_workspace_size(L):
    assert bwd_call(L, maxlen=0, ws=None) == B.MIMO_OK
    assert bwd_call(L, total=0, ws=None) == B.MIMO_OK
    assert B.mimo_attn_prefill_backward_workspace_size(B.make_dims(), 1000) == 1000 * 64 * 4
    assert B.mimo_attn_prefill_backward_workspace_size(B.make_dims(head_dim_v=64), 1000) == 0


def rope_call(L, q=FAKE, k=FAKE, pos=FAKE, total=8, theta=1e4, rd=64, dims=None):
    d = dims or B.make_dims()
    return L.mimo_rope_apply(ctypes.byref(d), q, k, pos, total, theta, rd, None)


@pytest.mark.parametrize("case,status", [
    (dict(q=None, k=None), B.MIMO_ERR_INVALID_ARG),
    (dict(pos=None), B.MIMO_ERR_INVALID_ARG),
    (dict(q=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=1.0), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=float("inf")), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=-16), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=208), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=24), B.MIMO_ERR_UNSUPPORTED),
    (dict(dims=B.make_dims(head_dim_qk=128)), B.MIMO_ERR_UNSUPPORTED),
])
def test_rope_rejects(L, case, status):
    assert rope_call(L, **case) == status
    assert B.mimo_last_error() != ""


def test_rope_nothing_to_do_is_ok(L):
    assert rope_call(L, total=0) == B.MIMO_OK
    assert rope_call(L, rd=0) == B.MIMO_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.lib()


def rope_prefill_call(L, dims=None, layer=0, k_rot=FAKE, pos=FAKE, total=64, theta=1e4, rd=64, ws=FAKE,
                      ws_bytes=1 << 20, maxlen=16):
    d = dims or B.make_dims()
    return L.mimo_attn_prefill_rope(ctypes.byref(d), layer, FAKE, FAKE, FAKE, pos, FAKE, 1, maxlen, total, theta, rd,
                                    None, FAKE, None, k_rot, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(k_rot=None), B.MIMO_ERR_INVALID_ARG),
    (dict(pos=None), B.MIMO_ERR_INVALID_ARG),
    (dict(k_rot=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=1.0), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=float("inf")), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=16), B.MIMO_ERR_UNSUPPORTED),      # pairs across half-waves: use mimo_rope_apply
    (dict(rd=0), B.MIMO_ERR_UNSUPPORTED),
    (dict(rd=224), B.MIMO_ERR_UNSUPPORTED),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(ws_bytes=64 * 32 * 8 - 1), B.MIMO_ERR_WORKSPACE),
    (dict(layer=3), B.MIMO_ERR_INVALID_ARG),
])
def test_prefill_rope_rejects(L, case, status):
    assert rope_prefill_call(L, **case) == status
    assert B.mimo_last_error() != ""


def chunk_rope_call(L, layer=1, q=FAKE, pos=FAKE, kc=FAKE, base=FAKE, pg=None, ctx=FAKE, total=64, maxlen=16,
                    theta=1e4, rd=64, krot=FAKE, ws=FAKE, ws_bytes=64 * 32 * 8):
    pref = ctypes.byref(pg) if pg is not None else None
    return L.mimo_attn_prefill_chunk_rope(ctypes.byref(B.make_dims()), layer, q, FAKE, FAKE, pos, FAKE, 2, maxlen,
                                          total, kc, FAKE, base, pref, ctx, theta, rd, None, FAKE, None, krot, ws,
                                          ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(q=None), B.MIMO_ERR_INVALID_ARG),
    (dict(pos=None), B.MIMO_ERR_INVALID_ARG),
    (dict(krot=None), B.MIMO_ERR_INVALID_ARG),
    (dict(krot=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(kc=None), B.MIMO_ERR_INVALID_ARG),
    (dict(ctx=None), B.MIMO_ERR_INVALID_ARG),
    (dict(base=None), B.MIMO_ERR_INVALID_ARG),            # contiguous GA needs kv_base
    (dict(layer=0, pg=pages()), B.MIMO_ERR_INVALID_ARG),  # a paged pool is GA only
    (dict(pg=pages(page_size=8)), B.MIMO_ERR_UNSUPPORTED),
    (dict(total=-1), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=1.0), B.MIMO_ERR_INVALID_ARG),
    (dict(theta=float("nan")), B.MIMO_ERR_INVALID_ARG),
    (dict(rd=48), B.MIMO_ERR_UNSUPPORTED),
    (dict(rd=224), B.MIMO_ERR_UNSUPPORTED),
    (dict(ws=None), B.MIMO_ERR_WORKSPACE),
    (dict(ws_bytes=64 * 32 * 8 - 1), B.MIMO_ERR_WORKSPACE),
    (dict(ws=FAKE_ODD), B.MIMO_ERR_INVALID_ARG),
    (dict(layer=2), B.MIMO_ERR_INVALID_ARG),
])
def test_prefill_chunk_rope_rejects(L, case, status):
    assert chunk_rope_call(L, **case) == status
    assert B.mimo_last_error() != ""


def test_prefill_chunk_rope_empty(L):
    assert chunk_rope_call(L, total=0, ws=None) == B.MIMO_OK
    assert chunk_rope_call(L, maxlen=0, ws=None) == B.MIMO_OK
    assert chunk_rope_call(L, layer=0, base=None, total=0) == B.MIMO_OK  # SWA ignores kv_base


def test_prefill_rope_workspace_and_empty(L):
    d = B.make_dims()
    assert B.mimo_attn_prefill_rope_workspace_size(d, 32768, 64) == 32768 * 32 * 2 * 4
    assert B.mimo_attn_prefill_rope_workspace_size(d, 10, 192) == 10 * 96 * 8
    assert B.mimo_attn_prefill_rope_workspace_size(d, 10, 48) == 0
    assert rope_prefill_call(L, total=0) == B.MIMO_OK
    assert rope_prefill_call(L, maxlen=0) == B.MIMO_OK
