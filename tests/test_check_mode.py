"""Check mode on the CPU: the C-ABI layer (global_attention_mimo_amd/csrc/api.cpp)
built with host-only launcher stand-ins (tests/sanitize/launch_stub.cpp) whose
check pass evaluates the library's own rules (csrc/check_rules.hpp) on HOST
arrays.  For every entry point that reads device-resident sizes, offsets,
block tables, sinks or FP8 scales, each rule is broken on its own and the call
must return MIMO_ERR_PRECONDITION with exactly that rule's bit, without
reaching its launch; the same call with valid arrays reaches the launch (which
the stand-ins report as MIMO_ERR_HIP: there is no device).  The rules restate
the argument contracts of include/mimo_attn.h; the expected bits below are
worked out from those contracts, not from the rules' code.

MIMO_ATTN_HOST_STUB names a prebuilt stand-in library (the sanitizer test
passes its ASan/UBSan build); otherwise one is built here with g++."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

from global_attention_mimo_amd import binding as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
FAKE = 0x10000  # 16-byte aligned stand-in for buffers the check never reads
HUGE_WS = 1 << 40
C = B.CHECK_BITS


def build_stub(path):
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "global_attention_mimo_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "sanitize", "launch_stub.cpp"), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
           "-lamdhip64", "-o", path]
    subprocess.run(cmd, check=True)
    return path


@pytest.fixture(scope="module")
def L(tmp_path_factory):
    path = os.environ.get("MIMO_ATTN_HOST_STUB") or build_stub(str(tmp_path_factory.mktemp("stub") / "stub.so"))
    lib = B.load(path)
    lib.mimo_attn_set_check(1)
    yield lib
    lib.mimo_attn_set_check(0)


def p(a):
    return a.ctypes.data


def i32(*v):
    return np.array(v, dtype=np.int32)


def i64(*v):
    return np.array(v, dtype=np.int64)


def sinks(n=64, bad=None):
    s = np.zeros(n, dtype=np.float32)
    s[5] = -np.inf  # "no sink" for head 5: legal
    if bad is not None:
        s[17] = bad
    return s


def expect(L, status, bits):
    """status is what the call returned; bits the rules it must report (0: none, the launch was reached)."""
    msg = L.mimo_last_error()
    w = ctypes.c_uint32(0)
    assert L.mimo_attn_check_flags(ctypes.byref(w), 1) == B.MIMO_OK
    if bits:
        assert status == B.MIMO_ERR_PRECONDITION, (status, msg)
        assert w.value == bits, (hex(w.value), msg)
        assert b"check mode found 0x%03x" % bits in msg, msg
    else:
        assert status == B.MIMO_ERR_HIP, (status, msg)
        assert w.value == 0, hex(w.value)


def dims(window=129):
    return ctypes.byref(B.make_dims(sliding_window=window))


def pages(table, max_blocks, page_size=16, num_pages=8):
    pg = B.mimo_kv_pages(p(table), max_blocks, page_size, num_pages)
    pages.keep.append((pg, table))
    return ctypes.byref(pg)


pages.keep = []


# --------------------------------------------------------------------------- prefill family
@pytest.mark.parametrize("cu,maxlen,sink,bits", [
    (i32(0, 5, 9), 5, sinks(), 0),
    (i32(1, 5, 9), 5, None, C["CU_START"]),
    (i32(0, 5, 3, 9), 6, None, C["CU_ORDER"]),
    (i32(0, 6, 9), 5, None, C["CU_LENGTH"]),
    (i32(0, 5, 9), 5, sinks(bad=np.nan), C["SINK"]),
    (i32(0, 5, 9), 5, sinks(bad=np.inf), C["SINK"]),
    (i32(2, 9, 4), 5, sinks(bad=np.inf), C["CU_START"] | C["CU_ORDER"] | C["CU_LENGTH"] | C["SINK"]),
])
@pytest.mark.parametrize("layer", [0, 1])
def test_prefill(L, cu, maxlen, sink, bits, layer):
    st = L.mimo_attn_prefill(dims(), layer, FAKE, FAKE, FAKE, p(cu), len(cu) - 1, maxlen,
                             p(sink) if sink is not None else None, FAKE, None, None)
    expect(L, st, bits)


@pytest.mark.parametrize("total,bits", [(7, 0), (8, C["CU_TOTAL"])])
def test_chunked_fused_rope_total(L, total, bits):
    cu, ctx, base = i32(0, 4, 7), i32(100, 0), i64(0, 4096)
    pos = np.arange(total, dtype=np.int32)
    st = L.mimo_attn_prefill_chunk_rope(dims(), 1, FAKE, FAKE, FAKE, p(pos), p(cu), 2, 4, total, FAKE, FAKE, p(base),
                                        None, p(ctx), 1e4, 64, None, FAKE, None, FAKE, FAKE, HUGE_WS, None)
    expect(L, st, bits)


@pytest.mark.parametrize("total,bits", [(9, 0), (10, C["CU_TOTAL"]), (8, C["CU_TOTAL"])])
def test_backward_and_fused_rope_total(L, total, bits):
    cu = i32(0, 5, 9)
    st = L.mimo_attn_prefill_backward(dims(), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, p(cu), 2, 5, total, None, FAKE,
                                      FAKE, FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)
    pos = np.arange(total, dtype=np.int32)
    st = L.mimo_attn_prefill_rope(dims(), 0, FAKE, FAKE, FAKE, p(pos), p(cu), 2, 5, total, 1e4, 64, None, FAKE,
                                  None, FAKE, FAKE, HUGE_WS, None)
    expect(L, st, bits)


# --------------------------------------------------------------------------- chunked prefill
@pytest.mark.parametrize("layer,ctx,base,bits", [
    (1, i32(100, 0), i64(0, 4096), 0),
    (1, i32(-1, 0), i64(0, 4096), C["CTX_RANGE"]),
    (1, i32(100, 0), i64(0, -16), C["KV_BASE"]),
    (0, i32(100, 0), i64(0, -16), 0),  # SWA ignores kv_base
    (1, i32(2**31 - 3, 0), i64(0, 0), C["CTX_RANGE"]),  # positions ctx .. ctx+4 pass INT32_MAX
])
def test_chunk(L, layer, ctx, base, bits):
    cu = i32(0, 4, 7)
    st = L.mimo_attn_prefill_chunk(dims(), layer, FAKE, FAKE, FAKE, p(cu), 2, 4, FAKE, FAKE, p(base), p(ctx), None,
                                   FAKE, None, None)
    expect(L, st, bits)


@pytest.mark.parametrize("ctx,table,bits", [
    # page 16 tokens, 4 blocks per sequence; a chunk reads positions < ctx only
    (i32(40, 16), i32(0, 1, 2, -1, 3, 9, 9, 9), 0),        # seq 0 reads blocks 0-2, seq 1 block 0
    (i32(40, 16), i32(0, 1, 8, -1, 3, 9, 9, 9), C["BLOCK_TABLE"]),  # block 2 of seq 0 past num_pages
    (i32(40, 17), i32(0, 1, 2, -1, 3, 9, 9, 9), C["BLOCK_TABLE"]),  # seq 1 now reads block 1 (entry 9)
    (i32(65, 0), i32(0, 1, 2, 4, 3, 9, 9, 9), C["CAPACITY"]),      # 65 positions > 4 blocks x 16
    (i32(0, 0), i32(-1, -1, -1, -1, -1, -1, -1, -1), 0),            # nothing cached: no entry read
])
def test_chunk_paged(L, ctx, table, bits):
    cu = i32(0, 3, 5)
    st = L.mimo_attn_prefill_chunk_paged(dims(), FAKE, FAKE, FAKE, p(cu), 2, 3, FAKE, FAKE, pages(table, 4), p(ctx),
                                         None, FAKE, None, None)
    expect(L, st, bits)


# --------------------------------------------------------------------------- decode
@pytest.mark.parametrize("layer,ctx,max_ctx,base,sink,bits", [
    (1, i32(0, 300, 17), 300, i64(0, 1000, 5000), sinks(), 0),
    (0, i32(0, 300, 17), 300, i64(0, 0, 0), sinks(), 0),
    (1, i32(0, 301, 17), 300, i64(0, 1000, 5000), None, C["CTX_RANGE"]),
    (0, i32(0, 301, 17), 300, i64(0, 0, 0), None, C["CTX_RANGE"]),
    (1, i32(0, -5, 17), 300, i64(0, 1000, 5000), None, C["CTX_RANGE"]),
    (1, i32(0, 3, 17), 300, i64(0, -1000, 5000), None, C["KV_BASE"]),
    (1, i32(0, 3, 17), 300, i64(0, 1000, 5000), sinks(bad=np.nan), C["SINK"]),
])
def test_decode(L, layer, ctx, max_ctx, base, sink, bits):
    st = L.mimo_attn_decode(dims(), layer, FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(ctx), 3, max_ctx, 0,
                            p(sink) if sink is not None else None, FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)


def test_noalloc_decode_is_checked(L):
    """The no-allocation entry point shares the decode path.  Its SWA form
    needs no scratch and meets the gate; the GA form looks its scratch up
    first, which the stand-ins fail."""
    ctx, base = i32(0, 301), i64(0, 1000)
    st = L.mimo_attn_decode_noalloc(dims(), 1, FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(ctx), 2, 300, 0, None, FAKE,
                                    None, None)
    assert st == B.MIMO_ERR_HIP
    expect(L, L.mimo_attn_decode_noalloc(dims(), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, p(ctx), 2, 300, 0, None,
                                         FAKE, None, None), C["CTX_RANGE"])


@pytest.mark.parametrize("ctx,cap,bits", [
    (i32(10, 99), i64(11, 100), 0),              # p = ctx fits below the capacity
    (i32(10, 100), i64(11, 100), C["CAPACITY"]),  # row 100 of a 100-row reservation
])
def test_decode_append_capacity(L, ctx, cap, bits):
    base = i64(0, 4096)
    st = L.mimo_attn_decode_append(dims(), 1, FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(cap), p(ctx), 2, 200, 0, None,
                                   FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)
    # the same step with the rotation fused in is checked alike
    st = L.mimo_attn_decode_append_rope(dims(), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(cap), p(ctx), 2,
                                        200, 0, 1e4, 64, None, FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)
    # without append, the capacity does not enter
    st = L.mimo_attn_decode(dims(), 1, FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(ctx), 2, 200, 0, None, FAKE, None,
                            FAKE, HUGE_WS, None)
    expect(L, st, 0)


@pytest.mark.parametrize("ctx,table,bits", [
    (i32(33, 0), i32(5, 6, 7, 99), 0),                         # positions 0..32: blocks 0-2; block 3 unused
    (i32(33, 0), i32(5, 6, -7, 99), C["BLOCK_TABLE"]),
    (i32(64, 0), i32(5, 6, 7, 0), 0),
    (i32(65, 0), i32(5, 6, 7, 0), C["CAPACITY"] | C["CTX_RANGE"]),  # also past max_ctx 64
])
def test_decode_paged(L, ctx, table, bits):
    table = np.concatenate([table, i32(-1, -1, -1, -1)])  # sequence 1 has nothing cached
    st = L.mimo_attn_decode_paged(dims(), FAKE, FAKE, FAKE, FAKE, FAKE, pages(table, 4), p(ctx), 2, 64, 0, None,
                                  FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)


@pytest.mark.parametrize("kscale,vscale,bits", [
    (np.full(4, 0.01, np.float32), np.full(4, 2.0, np.float32), 0),
    (np.array([0.01, 0, 1, 1], np.float32), np.ones(4, np.float32), C["FP8_SCALE"]),
    (np.ones(4, np.float32), np.array([1, 1, -2, 1], np.float32), C["FP8_SCALE"]),
    (np.ones(4, np.float32), np.array([1, 1, 1, np.inf], np.float32), C["FP8_SCALE"]),
    (np.array([1, np.nan, 1, 1], np.float32), np.ones(4, np.float32), C["FP8_SCALE"]),
])
def test_fp8_scales(L, kscale, vscale, bits):
    ctx, base, cap = i32(5, 9), i64(0, 100), i64(100, 100)
    st = L.mimo_attn_decode_fp8(dims(), FAKE, FAKE, FAKE, FAKE, FAKE, p(base), p(kscale), p(vscale), p(ctx), 2, 9, 0,
                                None, FAKE, None, FAKE, HUGE_WS, None)
    expect(L, st, bits)
    cu = i32(0, 2, 3)
    st = L.mimo_kv_append_fp8(dims(), FAKE, FAKE, p(cu), p(ctx), 2, 3, FAKE, FAKE, p(base), p(cap), p(kscale),
                              p(vscale), None)
    expect(L, st, bits)


def test_fp8_paged_and_chunk_entry_points(L):
    ks, vs = np.full(4, 0.01, np.float32), np.full(4, 2.0, np.float32)
    bad_vs = np.array([2.0, 0.0, 2.0, 2.0], np.float32)
    ctx, table = i32(33, 0), i32(5, 6, 7, 99, -1, -1, -1, -1)
    bad_table = i32(5, 6, 70, 99, -1, -1, -1, -1)  # block 2 of sequence 0 outside the 8-page pool
    for tb, scale_v, bits in ((table, vs, 0), (bad_table, vs, C["BLOCK_TABLE"]), (table, bad_vs, C["FP8_SCALE"])):
        st = L.mimo_attn_decode_fp8_paged(dims(), FAKE, FAKE, FAKE, FAKE, FAKE, pages(tb, 4), p(ks), p(scale_v),
                                          p(ctx), 2, 64, 0, None, FAKE, None, FAKE, HUGE_WS, None)
        expect(L, st, bits)
        cu = i32(0, 3, 5)
        st = L.mimo_attn_prefill_chunk_fp8_paged(dims(), FAKE, FAKE, FAKE, p(cu), 2, 3, FAKE, FAKE, pages(tb, 4), p(ks),
                                                 p(scale_v), p(ctx), None, FAKE, None, None)
        expect(L, st, bits)
    base = i64(0, 100)
    st = L.mimo_attn_prefill_chunk_fp8(dims(), FAKE, FAKE, FAKE, p(i32(0, 3, 5)), 2, 3, FAKE, FAKE, p(base), p(ks),
                                       p(bad_vs), p(ctx), None, FAKE, None, None)
    expect(L, st, C["FP8_SCALE"])
    st = L.mimo_attn_prefill_chunk_fp8(dims(), FAKE, FAKE, FAKE, p(i32(0, 3, 5)), 2, 3, FAKE, FAKE, p(i64(0, -4)),
                                       p(ks), p(vs), p(ctx), None, FAKE, None, None)
    expect(L, st, C["KV_BASE"])
    # paged FP8 append: sequence 0 writes positions 62..64 of a 4 x 16 table
    st = L.mimo_kv_append_fp8_paged(dims(), FAKE, FAKE, p(i32(0, 3, 5)), p(i32(62, 0)), 2, 5, FAKE, FAKE,
                                    pages(i32(0, 1, 2, 3, 4, 9, 9, 9), 4), p(ks), p(vs), None)
    expect(L, st, C["CAPACITY"])


# --------------------------------------------------------------------------- append
@pytest.mark.parametrize("layer,cu,total,ctx,cap,bits", [
    (1, i32(0, 3, 5), 5, i32(10, 0), i64(13, 2), 0),
    (1, i32(0, 3, 5), 5, i32(10, 0), i64(12, 2), C["CAPACITY"]),      # 10 + 3 > 12
    (1, i32(0, 3, 5), 6, i32(10, 0), i64(13, 2), C["CU_TOTAL"]),
    (1, i32(0, 3, 2), 2, i32(10, 0), i64(13, 2), C["CU_ORDER"]),
    (0, i32(0, 3, 5), 5, i32(10, 0), i64(0, 0), 0),                    # SWA: no pool capacity
    (0, i32(0, 3, 5), 5, i32(-1, 0), i64(0, 0), C["CTX_RANGE"]),
])
def test_append(L, layer, cu, total, ctx, cap, bits):
    base = i64(0, 64)
    st = L.mimo_kv_append(dims(), layer, FAKE, FAKE, p(cu), p(ctx), 2, total, FAKE, FAKE, p(base), p(cap), None)
    expect(L, st, bits)


@pytest.mark.parametrize("ctx,table,bits", [
    # 16-token pages, 4 blocks; sequence 0 appends 3 tokens at ctx, sequence 1 two at 0
    (i32(14, 0), i32(1, 2, 9, 9, 4, 9, 9, 9), 0),                   # seq 0 writes blocks 0-1, seq 1 block 0
    (i32(14, 0), i32(-1, 2, 9, 9, 4, 9, 9, 9), C["BLOCK_TABLE"]),   # position 14 lies in block 0
    (i32(16, 0), i32(-1, 2, 9, 9, 4, 9, 9, 9), 0),                  # positions 16-18: block 1 only
    (i32(62, 0), i32(0, 1, 2, 3, 4, 9, 9, 9), C["CAPACITY"]),       # 62 + 3 > 4 x 16
])
def test_append_paged(L, ctx, table, bits):
    cu = i32(0, 3, 5)
    st = L.mimo_kv_append_paged(dims(), FAKE, FAKE, p(cu), p(ctx), 2, 5, FAKE, FAKE, pages(table, 4), None)
    expect(L, st, bits)


# --------------------------------------------------------------------------- switch and word
def test_check_off_reaches_every_launch(L):
    L.mimo_attn_set_check(0)
    try:
        cu = i32(3, 1)
        st = L.mimo_attn_prefill(dims(), 0, FAKE, FAKE, FAKE, p(cu), 1, 5, None, FAKE, None, None)
        assert st == B.MIMO_ERR_HIP
    finally:
        assert L.mimo_attn_set_check(1) == 0


def test_sticky_word_accumulates_until_cleared(L):
    w = ctypes.c_uint32(0)
    L.mimo_attn_check_flags(ctypes.byref(w), 1)
    bad_cu, bad_ctx = i32(1, 4), i32(-3)
    L.mimo_attn_prefill(dims(), 1, FAKE, FAKE, FAKE, p(bad_cu), 1, 5, None, FAKE, None, None)
    L.mimo_attn_decode(dims(), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, p(bad_ctx), 1, 10, 0, None, FAKE, None, None, 0,
                       None)
    assert L.mimo_attn_check_flags(ctypes.byref(w), 0) == B.MIMO_OK
    assert w.value == C["CU_START"] | C["CTX_RANGE"]
    assert L.mimo_attn_check_flags(ctypes.byref(w), 1) == B.MIMO_OK and w.value == C["CU_START"] | C["CTX_RANGE"]
    assert L.mimo_attn_check_flags(ctypes.byref(w), 0) == B.MIMO_OK and w.value == 0
    assert L.mimo_attn_check_flags(None, 0) == B.MIMO_ERR_INVALID_ARG


def test_host_errors_come_before_the_check(L):
    """Misuse detectable on the host keeps its own status in check mode."""
    bad_cu = i32(1, 4)
    w = ctypes.c_uint32(0)
    L.mimo_attn_check_flags(ctypes.byref(w), 1)
    st = L.mimo_attn_prefill(dims(window=0), 0, FAKE, FAKE, FAKE, p(bad_cu), 1, 5, None, FAKE, None, None)
    assert st == B.MIMO_ERR_INVALID_ARG
    assert L.mimo_attn_check_flags(ctypes.byref(w), 0) == B.MIMO_OK and w.value == 0  # nothing was checked


def test_environment_switch(L, tmp_path):
    """MIMO_ATTN_CHECK=1 switches check mode on at the first call; other values leave it off."""
    path = L._name
    code = ("import sys; from global_attention_mimo_amd import binding as B; L = B.load(sys.argv[1]); "
            "print(L.mimo_attn_set_check(0))")
    for value, want in (("1", "1"), ("0", "0"), ("", "0"), ("yes", "0")):
        env = dict(os.environ, MIMO_ATTN_CHECK=value)
        out = subprocess.run([sys.executable, "-c", code, path], cwd=ROOT, env=env, capture_output=True, text=True,
                             check=True).stdout.strip()
        assert out == want, (value, out)
