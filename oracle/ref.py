"""ctypes front end of the CPU oracle (oracle/pagedkv_ref.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it to check and to time the HIP path.  It imports nothing from
the product package and the product never imports it.  All arithmetic is in the
C file; this module only marshals numpy arrays.

Dtype codes: 0 = float32, 1 = float16, 2 = bfloat16.  16-bit buffers are passed
as numpy uint16 arrays holding the raw bits (numpy has no bfloat16).

``Oracle(path)`` wraps one build of the library; the module-level functions use
the default build (oracle/libpagedkv_ref.so, compiled on first use if missing
or stale).  Tests also load deliberately broken builds through ``Oracle`` to
show that the pins catch planted mistakes.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

F32, F16, BF16 = 0, 1, 2


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _check_store(a, dtype):
    want = np.float32 if dtype == F32 else np.uint16
    if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
        raise ValueError("expected a C-contiguous %s array for dtype code %d" % (want.__name__, dtype))


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class Oracle:
    def __init__(self, path):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.ref_f16_bits_to_double.argtypes = [ctypes.c_uint16]
        L.ref_f16_bits_to_double.restype = dbl
        L.ref_bf16_bits_to_double.argtypes = [ctypes.c_uint16]
        L.ref_bf16_bits_to_double.restype = dbl
        L.ref_double_to_f16_bits.argtypes = [dbl]
        L.ref_double_to_f16_bits.restype = ctypes.c_uint16
        L.ref_double_to_bf16_bits.argtypes = [dbl]
        L.ref_double_to_bf16_bits.restype = ctypes.c_uint16
        L.ref_to_double.argtypes = [P, i64, ctypes.c_int, P]
        L.ref_to_double.restype = ctypes.c_int
        L.ref_cast.argtypes = [P, i64, ctypes.c_int, P]
        L.ref_cast.restype = ctypes.c_int
        L.ref_physical_slot.argtypes = [P, i32, i64]
        L.ref_physical_slot.restype = i64
        L.ref_append.argtypes = [P, P, P, P, i32, i32, i32, i32, ctypes.c_int, P, i32, P, i32]
        L.ref_append.restype = ctypes.c_int
        L.ref_gather.argtypes = [P, i32, i32, i32, ctypes.c_int, P, i32, P]
        L.ref_copy_blocks.argtypes = [P, P, i32, i32, i32, i32, ctypes.c_int, P, P, P, i32]
        L.ref_copy_blocks.restype = ctypes.c_int
        L.ref_append_tokens.argtypes = [P, P, P, P, i32, i32, i32, i32, ctypes.c_int, P, i32, P, P, i32]
        L.ref_append_tokens.restype = ctypes.c_int
        L.ref_swap.argtypes = [P, P, i32, i32, i32, i32, ctypes.c_int, P, i32, P, P, ctypes.c_int]
        L.ref_swap.restype = ctypes.c_int
        L.ref_attention_prefill.argtypes = [P, P, P, i32, i32, i32, ctypes.c_int, P, i32, P, P, i32, i32, dbl,
                                            P, i32, P]
        L.ref_attention_prefill.restype = ctypes.c_int
        L.ref_gather.restype = ctypes.c_int
        L.ref_attention_decode.argtypes = [P, P, P, i32, i32, i32, ctypes.c_int, P, i32, P, i32,
                                           i32, dbl, P, i32, i32, P]
        L.ref_attention_decode.restype = ctypes.c_int
        L.ref_num_threads.argtypes = []
        L.ref_num_threads.restype = ctypes.c_int
        self.L = L
        self.path = path

    # -- storage formats ---------------------------------------------------
    def f16_bits_to_double(self, bits):
        return self.L.ref_f16_bits_to_double(int(bits))

    def bf16_bits_to_double(self, bits):
        return self.L.ref_bf16_bits_to_double(int(bits))

    def double_to_f16_bits(self, x):
        return self.L.ref_double_to_f16_bits(float(x))

    def double_to_bf16_bits(self, x):
        return self.L.ref_double_to_bf16_bits(float(x))

    def to_double(self, a, dtype):
        """Decode a storage array (float32, or uint16 bits) to float64."""
        _check_store(a, dtype)
        out = np.empty(a.shape, dtype=np.float64)
        rc = self.L.ref_to_double(_ptr(a), a.size, dtype, _ptr(out))
        if rc:
            raise ValueError("ref_to_double failed (%d)" % rc)
        return out

    def cast(self, x, dtype):
        """Round a float64 array to `dtype` (RNE); returns float32 or uint16 bits."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.float32 if dtype == F32 else np.uint16)
        rc = self.L.ref_cast(_ptr(x), x.size, dtype, _ptr(out))
        if rc:
            raise ValueError("ref_cast failed (%d)" % rc)
        return out

    # -- the path ----------------------------------------------------------
    def physical_slot(self, table_row, block_size, i):
        t = _i32(table_row)
        return self.L.ref_physical_slot(_ptr(t), block_size, i)

    def append(self, k_new, v_new, k_cache, v_cache, block_tables, positions, dtype):
        """In place on k_cache / v_cache ([num_blocks][B][Hkv][D] stores)."""
        for a in (k_new, v_new, k_cache, v_cache):
            _check_store(a, dtype)
        nb, B, Hkv, D = k_cache.shape
        bt, pos = _i32(block_tables), _i32(positions)
        S = pos.shape[0]
        if k_new.shape != (S, Hkv, D) or v_new.shape != (S, Hkv, D) or v_cache.shape != k_cache.shape:
            raise ValueError("shape mismatch")
        rc = self.L.ref_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), nb, B, Hkv,
                               D, dtype, _ptr(bt), bt.shape[1], _ptr(pos), S)
        if rc:
            raise ValueError("ref_append rejected its arguments (%d)" % rc)

    def copy_blocks(self, k_cache, v_cache, src, dst, n_rows, dtype):
        """In place: rows [0, n_rows[i]) of block src[i] to block dst[i], both caches."""
        for a in (k_cache, v_cache):
            _check_store(a, dtype)
        nb, B, Hkv, D = k_cache.shape
        if v_cache.shape != k_cache.shape:
            raise ValueError("shape mismatch")
        s, d, n = _i32(src), _i32(dst), _i32(n_rows)
        if not (s.shape == d.shape == n.shape) or s.ndim != 1:
            raise ValueError("src, dst and n_rows must be equal-length vectors")
        rc = self.L.ref_copy_blocks(_ptr(k_cache), _ptr(v_cache), nb, B, Hkv, D, dtype, _ptr(s), _ptr(d),
                                    _ptr(n), s.shape[0])
        if rc:
            raise ValueError("ref_copy_blocks rejected its arguments (%d)" % rc)

    def append_tokens(self, k_new, v_new, k_cache, v_cache, block_tables, cu_new, start_pos, dtype):
        """In place: rows cu_new[s]..cu_new[s+1]-1 of k_new/v_new to positions start_pos[s], ..."""
        for a in (k_new, v_new, k_cache, v_cache):
            _check_store(a, dtype)
        nb, B, Hkv, D = k_cache.shape
        bt, cu, sp = _i32(block_tables), _i32(cu_new), _i32(start_pos)
        S = sp.shape[0]
        if cu.shape != (S + 1,) or k_new.shape != (int(cu[-1]), Hkv, D) or v_new.shape != k_new.shape:
            raise ValueError("shape mismatch")
        rc = self.L.ref_append_tokens(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), nb, B, Hkv, D,
                                      dtype, _ptr(bt), bt.shape[1], _ptr(cu), _ptr(sp), S)
        if rc:
            raise ValueError("ref_append_tokens rejected its arguments (%d)" % rc)

    def attention_prefill(self, q, k_cache, v_cache, block_tables, cu_q, context_lens, scale, dtype,
                          row_ids=None):
        """float64 [total][Hq][D] chunked-prefill attention (causal inside each chunk).
        With row_ids, only those query rows are computed (the rest are NaN)."""
        for a in (q, k_cache, v_cache):
            _check_store(a, dtype)
        nb, B, Hkv, D = k_cache.shape
        bt, cu, lens = _i32(block_tables), _i32(cu_q), _i32(context_lens)
        S = lens.shape[0]
        total, Hq = q.shape[0], q.shape[1]
        if cu.shape != (S + 1,) or int(cu[-1]) != total or q.shape[2] != D:
            raise ValueError("shape mismatch")
        out = np.full((total, Hq, D), np.nan)
        ids = None if row_ids is None else _i32(row_ids)
        rc = self.L.ref_attention_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), B, Hkv, D, dtype, _ptr(bt),
                                          bt.shape[1], _ptr(cu), _ptr(lens), S, Hq, float(scale),
                                          None if ids is None else _ptr(ids), 0 if ids is None else ids.shape[0],
                                          _ptr(out))
        if rc:
            raise ValueError("ref_attention_prefill rejected its arguments (%d)" % rc)
        return out

    def swap_out(self, k_cache, v_cache, blocks, dtype):
        """Host copies [n][B][Hkv][D] of blocks `blocks` of both caches."""
        for a in (k_cache, v_cache):
            _check_store(a, dtype)
        b = _i32(blocks)
        hk = np.empty((b.shape[0],) + k_cache.shape[1:], k_cache.dtype)
        hv = np.empty_like(hk)
        nb, B, Hkv, D = k_cache.shape
        rc = self.L.ref_swap(_ptr(k_cache), _ptr(v_cache), nb, B, Hkv, D, dtype, _ptr(b), b.shape[0], _ptr(hk),
                             _ptr(hv), 0)
        if rc:
            raise ValueError("ref_swap rejected its arguments (%d)" % rc)
        return hk, hv

    def swap_in(self, k_cache, v_cache, blocks, host_k, host_v, dtype):
        """In place: block blocks[i] of both caches = host slot i."""
        for a in (k_cache, v_cache, host_k, host_v):
            _check_store(a, dtype)
        b = _i32(blocks)
        nb, B, Hkv, D = k_cache.shape
        if host_k.shape != (b.shape[0], B, Hkv, D) or host_v.shape != host_k.shape:
            raise ValueError("host buffers must be [n][B][Hkv][D]")
        rc = self.L.ref_swap(_ptr(k_cache), _ptr(v_cache), nb, B, Hkv, D, dtype, _ptr(b), b.shape[0],
                             _ptr(host_k), _ptr(host_v), 1)
        if rc:
            raise ValueError("ref_swap rejected its arguments (%d)" % rc)

    def gather(self, cache, table_row, length, dtype):
        """Contiguous [Hkv][length][D] float64 copy of one sequence's cache."""
        _check_store(cache, dtype)
        nb, B, Hkv, D = cache.shape
        t = _i32(table_row)
        out = np.empty((Hkv, length, D), dtype=np.float64)
        rc = self.L.ref_gather(_ptr(cache), B, Hkv, D, dtype, _ptr(t), length, _ptr(out))
        if rc:
            raise ValueError("ref_gather failed (%d)" % rc)
        return out

    def attention_decode(self, q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                         seq_ids=None, part_tokens=0):
        """float64 [S][Hq][D] decode attention through the block tables.

        seq_ids: compute only these sequences (the other rows are NaN).
        part_tokens: 0 = plain two-pass softmax; > 0 = split-K with that partition.
        """
        for a in (q, k_cache, v_cache):
            _check_store(a, dtype)
        nb, B, Hkv, D = k_cache.shape
        S, Hq, Dq = q.shape
        if Dq != D or v_cache.shape != k_cache.shape:
            raise ValueError("shape mismatch")
        bt, lens = _i32(block_tables), _i32(context_lens)
        if bt.shape[0] != S or lens.shape[0] != S:
            raise ValueError("block_tables / context_lens must have one row per sequence")
        ids = None if seq_ids is None else _i32(seq_ids)
        out = np.full((S, Hq, D), np.nan, dtype=np.float64)
        rc = self.L.ref_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), B, Hkv, D, dtype,
                                         _ptr(bt), bt.shape[1], _ptr(lens), S, Hq, float(scale),
                                         _ptr(ids), 0 if ids is None else ids.shape[0],
                                         part_tokens, _ptr(out))
        if rc:
            raise ValueError("ref_attention_decode rejected its arguments (%d)" % rc)
        return out

    def num_threads(self):
        return self.L.ref_num_threads()


_default = None


def default():
    """The oracle built from oracle/pagedkv_ref.c (compiled if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(build_oracle.LIB) or (
                os.path.getmtime(build_oracle.LIB) < os.path.getmtime(build_oracle.SRC)):
            build_oracle.build()
        _default = Oracle(build_oracle.LIB)
    return _default


def f16_bits_to_double(bits):
    return default().f16_bits_to_double(bits)


def bf16_bits_to_double(bits):
    return default().bf16_bits_to_double(bits)


def double_to_f16_bits(x):
    return default().double_to_f16_bits(x)


def double_to_bf16_bits(x):
    return default().double_to_bf16_bits(x)


def to_double(a, dtype):
    return default().to_double(a, dtype)


def cast(x, dtype):
    return default().cast(x, dtype)


def physical_slot(table_row, block_size, i):
    return default().physical_slot(table_row, block_size, i)


def append(*a, **k):
    return default().append(*a, **k)


def copy_blocks(*a, **k):
    return default().copy_blocks(*a, **k)


def append_tokens(*a, **k):
    return default().append_tokens(*a, **k)


def attention_prefill(*a, **k):
    return default().attention_prefill(*a, **k)


def swap_out(*a, **k):
    return default().swap_out(*a, **k)


def swap_in(*a, **k):
    return default().swap_in(*a, **k)


def gather(*a, **k):
    return default().gather(*a, **k)


def attention_decode(*a, **k):
    return default().attention_decode(*a, **k)


def num_threads():
    return default().num_threads()
