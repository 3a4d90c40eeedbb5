"""fp64 CPU oracle for MiMo-V2-Flash hybrid SWA/GA attention with a per-head sink.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the GPU library: the arithmetic lives in ``mimo_oracle.c`` (plain C, double
precision, libm ``exp``/``log``), built with gcc into ``libmimo_oracle.so`` next
to this file.  The definition it follows is written out in the header comment
of ``mimo_oracle.c`` with its citations (Hugging Face Transformers model doc
"MiMo-V2-Flash": Key features; MiMoV2FlashConfig; MiMoV2FlashModel.forward).

Arrays are numpy.  bf16 tensors travel as their uint16 bit patterns; the C code
widens them exactly to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "mimo_oracle.c")
LIBRARY = os.path.join(HERE, "libmimo_oracle.so")

SWA = 0
GA = 1

OK = 0
EINVAL = 1
ECAPACITY = 2


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = f"{output}.{os.getpid()}.tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", *extra_flags,
           "-o", tmp, source, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_I64 = ctypes.c_int64


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built; run oracle.build()")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_prefill.restype = _I
        lib.oracle_prefill.argtypes = [_I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _I, _P,
                                       _P, _I64, _P, _P, _P, _I, _I]
        lib.oracle_decode.restype = _I
        lib.oracle_decode.argtypes = [_I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _I,
                                      _P, _P, _I, _P, _P, _P, _I]
        lib.oracle_prefill_chunk.restype = _I
        lib.oracle_prefill_chunk.argtypes = [_I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _I, _P, _P, _I,
                                             _P, _P, _P, _P, _P, _I]
        lib.oracle_kv_append.restype = _I
        lib.oracle_kv_append.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P]
        lib.oracle_decode_paged.restype = _I
        lib.oracle_decode_paged.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I64, _P, _I,
                                            _P, _P, _P, _I]
        lib.oracle_prefill_chunk_paged.restype = _I
        lib.oracle_prefill_chunk_paged.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I,
                                                   _I64, _P, _P, _P, _P, _I]
        lib.oracle_prefill_backward.restype = _I
        lib.oracle_prefill_backward.argtypes = [_I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _I, _P, _P,
                                                _I64, _P, _I64, _P, _P, _P, _P, _I, _I]
        lib.oracle_rope.restype = _I
        lib.oracle_rope.argtypes = [_I, _I, _I, _P, _P, _P, _I64, ctypes.c_double, _I, _P, _P]
        lib.oracle_decode_fp8.restype = _I
        lib.oracle_decode_fp8.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                          _P, _I]
        lib.oracle_kv_append_fp8.restype = _I
        lib.oracle_kv_append_fp8.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P]
        lib.oracle_decode_fp8_paged.restype = _I
        lib.oracle_decode_fp8_paged.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I64, _P,
                                                _P, _P, _I, _P, _P, _P, _I]
        lib.oracle_prefill_chunk_fp8.restype = _I
        lib.oracle_prefill_chunk_fp8.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, _P, _I]
        lib.oracle_prefill_chunk_fp8_paged.restype = _I
        lib.oracle_prefill_chunk_fp8_paged.argtypes = [_I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _I, _P, _P, _P, _I,
                                                       _I, _I64, _P, _P, _P, _P, _P, _P, _I]
        lib.oracle_kv_append_fp8_paged.restype = _I
        lib.oracle_kv_append_fp8_paged.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I64, _P,
                                                   _P]
        lib.oracle_e4m3_encode.restype = None
        lib.oracle_e4m3_encode.argtypes = [_P, _P, _I64]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_e4m3_decode.argtypes = [_P, _P, _I64]
        lib.oracle_kv_append_paged.restype = _I
        lib.oracle_kv_append_paged.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I64]
        lib.oracle_default_threads.restype = _I
        lib.oracle_default_threads.argtypes = []
        self.lib = lib

    def default_threads(self) -> int:
        return int(self.lib.oracle_default_threads())

    # -- helpers ----------------------------------------------------------
    @staticmethod
    def _u16(a: np.ndarray, shape_tail) -> np.ndarray:
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint16:
            raise TypeError("bf16 tensors are passed as uint16 bit patterns")
        if tuple(a.shape[1:]) != tuple(shape_tail):
            raise ValueError(f"shape {a.shape} does not end in {shape_tail}")
        return a

    @staticmethod
    def _ptr(a: Optional[np.ndarray]):
        return None if a is None else a.ctypes.data

    def prefill(self, q, k, v, cu_seqlens, *, layer_type: int, window: int = 129,
                scale: float, value_scale: float = 1.0, sink=None, rows=None,
                want_weights: bool = False, nthreads: int = 0):
        """Attention of packed varlen sequences.

        q [T][Hq][Dqk], k [T][Hkv][Dqk], v [T][Hkv][Dv] as uint16 bf16 bits;
        cu_seqlens [B+1] int32; sink [Hq] float32 or None; rows: optional int64
        packed token indices.  Returns (out [R][Hq][Dv] f64, lse [R][Hq] f64)
        and, if want_weights, weights [R][Hq][maxlen+1] (sink mass last).
        """
        q = np.ascontiguousarray(q)
        hq, dqk = q.shape[1], q.shape[2]
        hkv, dv = k.shape[1], v.shape[2]
        q = self._u16(q, (hq, dqk))
        k = self._u16(k, (hkv, dqk))
        v = self._u16(v, (hkv, dv))
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        nseq = cu.shape[0] - 1
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        rw = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = int(cu[-1]) if rw is None else int(rw.shape[0])
        out = np.empty((nrows, hq, dv), np.float64)
        lse = np.empty((nrows, hq), np.float64)
        maxlen = int(np.max(np.diff(cu))) if nseq > 0 else 0
        wstride = maxlen + 1
        wts = np.empty((nrows, hq, wstride), np.float64) if want_weights else None
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_prefill(hq, hkv, dqk, dv, layer_type, window, scale, value_scale,
                                     self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(cu), nseq,
                                     self._ptr(sk), self._ptr(rw), nrows, self._ptr(out),
                                     self._ptr(lse), self._ptr(wts), wstride, nth)
        if rc != OK:
            raise ValueError(f"oracle_prefill rejected its arguments (status {rc})")
        return (out, lse, wts) if want_weights else (out, lse)

    def decode(self, q, k_new, v_new, k_cache, v_cache, ctx_lens, *, layer_type: int,
               window: int = 129, scale: float, value_scale: float = 1.0, sink=None,
               kv_base=None, nthreads: int = 0):
        """One new token per sequence; SWA reads ring [B][W-1][Hkv][D], GA reads
        pool [N][Hkv][D] at kv_base[b] + position.  Returns (out [B][Hq][Dv], lse [B][Hq])."""
        q = np.ascontiguousarray(q)
        batch, hq, dqk = q.shape
        hkv, dv = v_new.shape[1], v_new.shape[2]
        q = self._u16(q, (hq, dqk))
        kn = self._u16(k_new, (hkv, dqk))
        vn = self._u16(v_new, (hkv, dv))
        kc = None if k_cache is None else np.ascontiguousarray(k_cache)
        vc = None if v_cache is None else np.ascontiguousarray(v_cache)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        base = None if kv_base is None else np.ascontiguousarray(kv_base, dtype=np.int64)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        ring = window - 1 if layer_type == SWA else 0
        out = np.empty((batch, hq, dv), np.float64)
        lse = np.empty((batch, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_decode(hq, hkv, dqk, dv, layer_type, window, scale, value_scale,
                                    self._ptr(q), self._ptr(kn), self._ptr(vn), self._ptr(kc),
                                    self._ptr(vc), ring, self._ptr(base), self._ptr(ctx), batch,
                                    self._ptr(sk), self._ptr(out), self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_decode rejected its arguments (status {rc})")
        return out, lse

    def prefill_chunk(self, q, k, v, cu_newlens, k_cache, v_cache, ctx_lens, *, layer_type: int,
                      window: int = 129, scale: float, value_scale: float = 1.0, sink=None, kv_base=None,
                      nthreads: int = 0):
        """Chunked prefill: new tokens (packed by cu_newlens) at positions ctx_lens[b] + i attend
        to the cached positions (SWA ring [B][W-1][Hkv][D] / GA pool at kv_base[b] + j) and to
        the chunk's own earlier tokens.  Returns (out [Tn][Hq][Dv], lse [Tn][Hq])."""
        q = np.ascontiguousarray(q)
        hq, dqk = q.shape[1], q.shape[2]
        hkv, dv = k.shape[1], v.shape[2]
        q = self._u16(q, (hq, dqk))
        k = self._u16(k, (hkv, dqk))
        v = self._u16(v, (hkv, dv))
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        batch = cu.shape[0] - 1
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        kc = None if k_cache is None else np.ascontiguousarray(k_cache)
        vc = None if v_cache is None else np.ascontiguousarray(v_cache)
        base = None if kv_base is None else np.ascontiguousarray(kv_base, dtype=np.int64)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        ring = window - 1 if layer_type == SWA else 0
        tn = int(cu[-1])
        out = np.empty((tn, hq, dv), np.float64)
        lse = np.empty((tn, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_prefill_chunk(hq, hkv, dqk, dv, layer_type, window, scale, value_scale,
                                           self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(cu), batch,
                                           self._ptr(kc), self._ptr(vc), ring, self._ptr(base), self._ptr(ctx),
                                           self._ptr(sk), self._ptr(out), self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_prefill_chunk rejected its arguments (status {rc})")
        return out, lse

    def kv_append(self, k, v, cu_newlens, ctx_lens, k_cache, v_cache, *, layer_type: int,
                  window: int = 129, kv_base=None, kv_capacity=None) -> int:
        """Writes new tokens into the caches in place; returns the status code."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        hkv, dqk, dv = k.shape[1], k.shape[2], v.shape[2]
        for c in (k_cache, v_cache):
            if not (c.flags["C_CONTIGUOUS"] and c.dtype == np.uint16):
                raise TypeError("caches must be C-contiguous uint16 arrays")
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        base = None if kv_base is None else np.ascontiguousarray(kv_base, dtype=np.int64)
        cap = None if kv_capacity is None else np.ascontiguousarray(kv_capacity, dtype=np.int64)
        ring = window - 1 if layer_type == SWA else 0
        return int(self.lib.oracle_kv_append(hkv, dqk, dv, layer_type, ring, self._ptr(k),
                                             self._ptr(v), self._ptr(cu), self._ptr(ctx),
                                             cu.shape[0] - 1, self._ptr(k_cache), self._ptr(v_cache),
                                             self._ptr(base), self._ptr(cap)))


    def prefill_backward(self, q, k, v, dout, cu_seqlens, *, layer_type: int, window: int = 129, scale: float,
                         value_scale: float = 1.0, sink=None, q_rows=None, kv_rows=None, want_dsink: bool = True,
                         stored_out: bool = False, nthreads: int = 0):
        """Gradients of sum(dout * prefill(q, k, v)) (bf16 bits in, float64 out).

        Returns (dq [nq][Hq][Dqk], dk [nkv][Hkv][Dqk], dv [nkv][Hkv][Dv], dsink [Hq] or None) for the
        packed tokens q_rows / kv_rows (default: all tokens).  stored_out: take D = dO . o from the output
        rounded to bf16 as a forward stores it, instead of the exact output."""
        q = np.ascontiguousarray(q)
        hq, dqk = q.shape[1], q.shape[2]
        hkv, dv = k.shape[1], v.shape[2]
        q = self._u16(q, (hq, dqk))
        k = self._u16(k, (hkv, dqk))
        v = self._u16(v, (hkv, dv))
        do = self._u16(dout, (hq, dv))
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        nseq = cu.shape[0] - 1
        T = int(cu[-1])
        qr = np.arange(T, dtype=np.int64) if q_rows is None else np.ascontiguousarray(q_rows, dtype=np.int64)
        kr = np.arange(T, dtype=np.int64) if kv_rows is None else np.ascontiguousarray(kv_rows, dtype=np.int64)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        dq = np.empty((qr.shape[0], hq, dqk), np.float64)
        dk = np.empty((kr.shape[0], hkv, dqk), np.float64)
        dvv = np.empty((kr.shape[0], hkv, dv), np.float64)
        ds = np.empty(hq, np.float64) if want_dsink else None
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_prefill_backward(hq, hkv, dqk, dv, layer_type, window, scale, value_scale,
                                              self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(do), self._ptr(cu),
                                              nseq, self._ptr(sk), self._ptr(qr), qr.shape[0], self._ptr(kr),
                                              kr.shape[0], self._ptr(dq), self._ptr(dk), self._ptr(dvv),
                                              self._ptr(ds), int(bool(stored_out)), nth)
        if rc != OK:
            raise ValueError(f"oracle_prefill_backward rejected its arguments (status {rc})")
        return dq, dk, dvv, ds

    def rope(self, q, k, positions, *, theta: float, rotary_dim: int):
        """Rotary embedding of q [T][Hq][D] and k [T][Hkv][D] (bf16 bits, either may be None) at
        positions [T]; returns float64 (q_out, k_out)."""
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        T = pos.shape[0]
        qq = None if q is None else np.ascontiguousarray(q)
        kk = None if k is None else np.ascontiguousarray(k)
        ref = qq if qq is not None else kk
        d = ref.shape[2]
        hq = 0 if qq is None else qq.shape[1]
        hkv = 0 if kk is None else kk.shape[1]
        if qq is not None:
            qq = self._u16(qq, (hq, d))
        if kk is not None:
            kk = self._u16(kk, (hkv, d))
        qo = None if qq is None else np.empty(qq.shape, np.float64)
        ko = None if kk is None else np.empty(kk.shape, np.float64)
        rc = self.lib.oracle_rope(hq, hkv, d, self._ptr(qq), self._ptr(kk), self._ptr(pos), T, float(theta),
                                  rotary_dim, self._ptr(qo), self._ptr(ko))
        if rc != OK:
            raise ValueError(f"oracle_rope rejected its arguments (status {rc})")
        return qo, ko

    # -- paged GA pool ----------------------------------------------------
    @staticmethod
    def _table(block_table, page_size, k_cache):
        tb = np.ascontiguousarray(block_table, dtype=np.int32)
        if tb.ndim != 2:
            raise ValueError("block_table is [batch][max_blocks]")
        if k_cache.shape[0] % page_size:
            raise ValueError("a paged pool holds whole pages")
        return tb, tb.shape[1], k_cache.shape[0] // page_size

    def decode_paged(self, q, k_new, v_new, k_pool, v_pool, block_table, page_size: int, ctx_lens, *,
                     scale: float, value_scale: float = 1.0, sink=None, nthreads: int = 0):
        """GA decode over a paged pool [num_pages*page_size][Hkv][D]: position j of sequence b is row
        block_table[b][j // page_size] * page_size + j % page_size.  Returns (out, lse) as decode."""
        q = np.ascontiguousarray(q)
        batch, hq, dqk = q.shape
        hkv, dv = v_new.shape[1], v_new.shape[2]
        q = self._u16(q, (hq, dqk))
        kn = self._u16(k_new, (hkv, dqk))
        vn = self._u16(v_new, (hkv, dv))
        kc = self._u16(k_pool, (hkv, dqk))
        vc = self._u16(v_pool, (hkv, dv))
        tb, mb, npages = self._table(block_table, page_size, kc)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        out = np.empty((batch, hq, dv), np.float64)
        lse = np.empty((batch, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_decode_paged(hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(kn),
                                          self._ptr(vn), self._ptr(kc), self._ptr(vc), self._ptr(tb), mb,
                                          page_size, npages, self._ptr(ctx), batch, self._ptr(sk), self._ptr(out),
                                          self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_decode_paged rejected its arguments (status {rc})")
        return out, lse

    def prefill_chunk_paged(self, q, k, v, cu_newlens, k_pool, v_pool, block_table, page_size: int, ctx_lens, *,
                            scale: float, value_scale: float = 1.0, sink=None, nthreads: int = 0):
        """GA chunked prefill whose cached positions live in a paged pool (as decode_paged)."""
        q = np.ascontiguousarray(q)
        hq, dqk = q.shape[1], q.shape[2]
        hkv, dv = k.shape[1], v.shape[2]
        q = self._u16(q, (hq, dqk))
        k = self._u16(k, (hkv, dqk))
        v = self._u16(v, (hkv, dv))
        kc = self._u16(k_pool, (hkv, dqk))
        vc = self._u16(v_pool, (hkv, dv))
        tb, mb, npages = self._table(block_table, page_size, kc)
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        batch = cu.shape[0] - 1
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        tn = int(cu[-1])
        out = np.empty((tn, hq, dv), np.float64)
        lse = np.empty((tn, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_prefill_chunk_paged(hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(k),
                                                 self._ptr(v), self._ptr(cu), batch, self._ptr(kc), self._ptr(vc),
                                                 self._ptr(tb), mb, page_size, npages, self._ptr(ctx), self._ptr(sk),
                                                 self._ptr(out), self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_prefill_chunk_paged rejected its arguments (status {rc})")
        return out, lse

    def kv_append_paged(self, k, v, cu_newlens, ctx_lens, k_pool, v_pool, block_table, page_size: int) -> int:
        """Writes new tokens into a paged pool in place; returns the status code."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        hkv, dqk, dv = k.shape[1], k.shape[2], v.shape[2]
        for c in (k_pool, v_pool):
            if not (c.flags["C_CONTIGUOUS"] and c.dtype == np.uint16):
                raise TypeError("caches must be C-contiguous uint16 arrays")
        tb, mb, npages = self._table(block_table, page_size, k_pool)
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        return int(self.lib.oracle_kv_append_paged(hkv, dqk, dv, self._ptr(k), self._ptr(v), self._ptr(cu),
                                                   self._ptr(ctx), cu.shape[0] - 1, self._ptr(k_pool),
                                                   self._ptr(v_pool), self._ptr(tb), mb, page_size, npages))

    # -- FP8 (OCP E4M3) GA pool ----------------------------------------------
    def e4m3_encode(self, x) -> np.ndarray:
        """E4M3 codes (uint8) of float32 values: |x| clamped to 448, nearest, ties to even."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint8)
        self.lib.oracle_e4m3_encode(self._ptr(x), self._ptr(out), x.size)
        return out

    def e4m3_decode(self, codes) -> np.ndarray:
        """Values (float64) of E4M3 codes."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, np.float64)
        self.lib.oracle_e4m3_decode(self._ptr(c), self._ptr(out), c.size)
        return out

    @staticmethod
    def _scales(s, hkv):
        s = np.ascontiguousarray(s, dtype=np.float32)
        if s.shape != (hkv,):
            raise ValueError(f"scales must have shape ({hkv},)")
        return s

    def decode_fp8(self, q, k_new, v_new, k_pool, v_pool, kv_base, k_scale, v_scale, ctx_lens, *, scale: float,
                   value_scale: float = 1.0, sink=None, nthreads: int = 0):
        """GA decode over an FP8 pool of E4M3 codes [N][Hkv][D] (uint8): cached position j of sequence b
        is code[kv_base[b] + j] * scale[g]; the new token comes from k_new / v_new (bf16)."""
        q = np.ascontiguousarray(q)
        batch, hq, dqk = q.shape
        hkv, dv = v_new.shape[1], v_new.shape[2]
        q = self._u16(q, (hq, dqk))
        kn = self._u16(k_new, (hkv, dqk))
        vn = self._u16(v_new, (hkv, dv))
        kc = np.ascontiguousarray(k_pool, dtype=np.uint8)
        vc = np.ascontiguousarray(v_pool, dtype=np.uint8)
        if kc.shape[1:] != (hkv, dqk) or vc.shape[1:] != (hkv, dv):
            raise ValueError("FP8 pools are [N][Hkv][D] uint8")
        base = np.ascontiguousarray(kv_base, dtype=np.int64)
        ks, vs = self._scales(k_scale, hkv), self._scales(v_scale, hkv)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        out = np.empty((batch, hq, dv), np.float64)
        lse = np.empty((batch, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_decode_fp8(hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(kn),
                                        self._ptr(vn), self._ptr(kc), self._ptr(vc), self._ptr(base), self._ptr(ks),
                                        self._ptr(vs), self._ptr(ctx), batch, self._ptr(sk), self._ptr(out),
                                        self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_decode_fp8 rejected its arguments (status {rc})")
        return out, lse

    def kv_append_fp8(self, k, v, cu_newlens, ctx_lens, k_pool, v_pool, kv_base, kv_capacity, k_scale,
                      v_scale) -> int:
        """Quantises new tokens into an FP8 GA pool in place; returns the status code."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        hkv, dqk, dv = k.shape[1], k.shape[2], v.shape[2]
        for c in (k_pool, v_pool):
            if not (c.flags["C_CONTIGUOUS"] and c.dtype == np.uint8):
                raise TypeError("FP8 pools must be C-contiguous uint8 arrays")
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        base = np.ascontiguousarray(kv_base, dtype=np.int64)
        cap = np.ascontiguousarray(kv_capacity, dtype=np.int64)
        ks, vs = self._scales(k_scale, hkv), self._scales(v_scale, hkv)
        return int(self.lib.oracle_kv_append_fp8(hkv, dqk, dv, self._ptr(k), self._ptr(v), self._ptr(cu),
                                                 self._ptr(ctx), cu.shape[0] - 1, self._ptr(k_pool),
                                                 self._ptr(v_pool), self._ptr(base), self._ptr(cap), self._ptr(ks),
                                                 self._ptr(vs)))

    @staticmethod
    def _codes(pool, hkv, d):
        c = np.ascontiguousarray(pool, dtype=np.uint8)
        if c.shape[1:] != (hkv, d):
            raise ValueError("FP8 pools are [N][Hkv][D] uint8")
        return c

    def decode_fp8_paged(self, q, k_new, v_new, k_pool, v_pool, block_table, page_size: int, k_scale, v_scale,
                         ctx_lens, *, scale: float, value_scale: float = 1.0, sink=None, nthreads: int = 0):
        """GA decode over a paged FP8 pool: cached position j of sequence b is the code row
        block_table[b][j // page_size] * page_size + j % page_size, read as code * scale[g]."""
        q = np.ascontiguousarray(q)
        batch, hq, dqk = q.shape
        hkv, dv = v_new.shape[1], v_new.shape[2]
        q = self._u16(q, (hq, dqk))
        kn = self._u16(k_new, (hkv, dqk))
        vn = self._u16(v_new, (hkv, dv))
        kc, vc = self._codes(k_pool, hkv, dqk), self._codes(v_pool, hkv, dv)
        tb, mb, npages = self._table(block_table, page_size, kc)
        ks, vs = self._scales(k_scale, hkv), self._scales(v_scale, hkv)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        out = np.empty((batch, hq, dv), np.float64)
        lse = np.empty((batch, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        rc = self.lib.oracle_decode_fp8_paged(hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(kn),
                                              self._ptr(vn), self._ptr(kc), self._ptr(vc), self._ptr(tb), mb,
                                              page_size, npages, self._ptr(ks), self._ptr(vs), self._ptr(ctx), batch,
                                              self._ptr(sk), self._ptr(out), self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_decode_fp8_paged rejected its arguments (status {rc})")
        return out, lse

    def prefill_chunk_fp8(self, q, k, v, cu_newlens, k_pool, v_pool, k_scale, v_scale, ctx_lens, *,
                          kv_base=None, block_table=None, page_size: int = 0, scale: float,
                          value_scale: float = 1.0, sink=None, nthreads: int = 0):
        """GA chunked prefill whose cached positions are FP8 codes, in a contiguous pool (kv_base) or a
        paged one (block_table, page_size), read as code * scale[g]; the chunk's k, v are bf16."""
        q = np.ascontiguousarray(q)
        hq, dqk = q.shape[1], q.shape[2]
        hkv, dv = k.shape[1], v.shape[2]
        q = self._u16(q, (hq, dqk))
        k = self._u16(k, (hkv, dqk))
        v = self._u16(v, (hkv, dv))
        kc, vc = self._codes(k_pool, hkv, dqk), self._codes(v_pool, hkv, dv)
        ks, vs = self._scales(k_scale, hkv), self._scales(v_scale, hkv)
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        batch = cu.shape[0] - 1
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        tn = int(cu[-1])
        out = np.empty((tn, hq, dv), np.float64)
        lse = np.empty((tn, hq), np.float64)
        nth = nthreads if nthreads > 0 else self.default_threads()
        if block_table is not None:
            tb, mb, npages = self._table(block_table, page_size, kc)
            rc = self.lib.oracle_prefill_chunk_fp8_paged(
                hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(cu), batch,
                self._ptr(kc), self._ptr(vc), self._ptr(tb), mb, page_size, npages, self._ptr(ks), self._ptr(vs),
                self._ptr(ctx), self._ptr(sk), self._ptr(out), self._ptr(lse), nth)
        else:
            base = np.ascontiguousarray(kv_base, dtype=np.int64)
            rc = self.lib.oracle_prefill_chunk_fp8(
                hq, hkv, dqk, dv, scale, value_scale, self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(cu), batch,
                self._ptr(kc), self._ptr(vc), self._ptr(base), self._ptr(ks), self._ptr(vs), self._ptr(ctx),
                self._ptr(sk), self._ptr(out), self._ptr(lse), nth)
        if rc != OK:
            raise ValueError(f"oracle_prefill_chunk_fp8 rejected its arguments (status {rc})")
        return out, lse

    def kv_append_fp8_paged(self, k, v, cu_newlens, ctx_lens, k_pool, v_pool, block_table, page_size: int, k_scale,
                            v_scale) -> int:
        """Quantises new tokens into a paged FP8 pool in place; returns the status code."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        hkv, dqk, dv = k.shape[1], k.shape[2], v.shape[2]
        for c in (k_pool, v_pool):
            if not (c.flags["C_CONTIGUOUS"] and c.dtype == np.uint8):
                raise TypeError("FP8 pools must be C-contiguous uint8 arrays")
        tb, mb, npages = self._table(block_table, page_size, k_pool)
        cu = np.ascontiguousarray(cu_newlens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        ks, vs = self._scales(k_scale, hkv), self._scales(v_scale, hkv)
        return int(self.lib.oracle_kv_append_fp8_paged(hkv, dqk, dv, self._ptr(k), self._ptr(v), self._ptr(cu),
                                                       self._ptr(ctx), cu.shape[0] - 1, self._ptr(k_pool),
                                                       self._ptr(v_pool), self._ptr(tb), mb, page_size, npages,
                                                       self._ptr(ks), self._ptr(vs)))


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
