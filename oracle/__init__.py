"""ctypes front-end of the CPU oracle for paged-attention decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
All arrays are host numpy arrays; fp16 data is passed as raw 16-bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16/uint16 data, got {a.dtype}")
    return a


class Oracle:
    """Handle on one compiled oracle library (the default one, or a variant)."""

    def __init__(self, path=None):
        path = path or _build.LIB
        if not os.path.exists(path):
            _build.build(quiet=True)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_array_to_double.argtypes = [_P, _P, _I64]
        lib.oracle_half_array_to_double.restype = None
        lib.oracle_gather.argtypes = [_P, _P, _P, _P, _P, _P] + [_I32] * 7
        lib.oracle_gather.restype = ctypes.c_int
        lib.oracle_decode_pairs.argtypes = ([_P, _P, _I32, _P, _P, _P, _P, _P] + [_I32] * 6
                                            + [ctypes.c_double, _P])
        lib.oracle_decode_pairs.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [_P] * 6 + [_I32] * 6 + [ctypes.c_double, _P]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_reshape_and_cache.argtypes = [_P] * 5 + [_I32] * 5
        lib.oracle_reshape_and_cache.restype = ctypes.c_int
        lib.oracle_copy_blocks.argtypes = [_P, _P, _P, _I32, _I32, _I64]
        lib.oracle_copy_blocks.restype = ctypes.c_int
        lib.oracle_swap_blocks.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I64]
        lib.oracle_swap_blocks.restype = ctypes.c_int
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_float_to_e4m3.argtypes = [ctypes.c_float]
        lib.oracle_float_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_quantize_e4m3.argtypes = [_P, _P, _I64, ctypes.c_float]
        lib.oracle_quantize_e4m3.restype = None
        lib.oracle_reshape_and_cache_fp8.argtypes = [_P] * 5 + [_I32] * 5 + [ctypes.c_float] * 2
        lib.oracle_reshape_and_cache_fp8.restype = ctypes.c_int
        lib.oracle_decode_fp8_pairs.argtypes = ([_P, _P, _I32, _P, _P, _P, _P, _P] + [_I32] * 6
                                                + [ctypes.c_double, ctypes.c_float, ctypes.c_float,
                                                   _P])
        lib.oracle_decode_fp8_pairs.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [_P] * 7 + [_I32] * 7 + [ctypes.c_double, _P]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill_fp8.argtypes = ([_P] * 7 + [_I32] * 7
                                           + [ctypes.c_double, ctypes.c_float, ctypes.c_float, _P])
        lib.oracle_prefill_fp8.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        self.lib = lib
        self.threads_used = 1

    def set_threads(self, n):
        """Host threads for later calls (n <= 0: the OpenMP default); timing
        plumbing only.  Returns the count now in effect."""
        return int(self.lib.oracle_set_threads(int(n)))

    # -- binary16 decoding -------------------------------------------------
    def half_to_double(self, bits):
        src = _u16(np.asarray(bits))
        out = np.empty(src.shape, dtype=np.float64)
        self.lib.oracle_half_array_to_double(_ptr(src), _ptr(out), src.size)
        return out

    # -- gather ---------------------------------------------------------------
    def gather(self, k_cache, v_cache, block_tables, context_lens, seq, head):
        k_cache, v_cache = _u16(k_cache), _u16(v_cache)
        nb, bs, nh, hd = k_cache.shape
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        L = int(cl[seq])
        K = np.empty((max(L, 1), hd), dtype=np.float64)
        V = np.empty((max(L, 1), hd), dtype=np.float64)
        rc = self.lib.oracle_gather(_ptr(K), _ptr(V), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                    _ptr(cl), seq, head, nh, hd, nb, bs, bt.shape[1])
        if rc < 0:
            raise ValueError(f"oracle_gather failed ({rc})")
        return K[:L], V[:L]

    # -- decode ---------------------------------------------------------------
    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale):
        """fp64 [S, H, D] attention output for every (sequence, head)."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        S, H, D = q.shape
        nb, bs, nh, hd = k_cache.shape
        assert (nh, hd) == (H, D) and v_cache.shape == k_cache.shape
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.empty((S, H, D), dtype=np.float64)
        used = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                    _ptr(cl), S, H, D, nb, bs, bt.shape[1], float(scale),
                                    _ptr(used))
        if rc:
            raise ValueError(f"oracle_decode failed ({rc})")
        self.threads_used = int(used[0])
        return out

    def decode_pairs(self, pairs, q, k_cache, v_cache, block_tables, context_lens, scale):
        """fp64 [len(pairs), D] outputs for the listed (sequence, head) pairs."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        S, H, D = q.shape
        nb, bs, nh, hd = k_cache.shape
        assert (nh, hd) == (H, D) and v_cache.shape == k_cache.shape
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.empty((pr.shape[0], D), dtype=np.float64)
        used = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_decode_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                                          S, H, D, nb, bs, bt.shape[1], float(scale), _ptr(used))
        if rc:
            raise ValueError(f"oracle_decode_pairs failed ({rc})")
        self.threads_used = int(used[0])
        return out

    # -- reshape_and_cache ----------------------------------------------------
    def reshape_and_cache(self, key, value, k_cache, v_cache, slot_mapping):
        """Writes into k_cache / v_cache in place (uint16 or float16 arrays)."""
        key, value = _u16(key), _u16(value)
        kc = k_cache.view(np.uint16) if k_cache.dtype == np.float16 else k_cache
        vc = v_cache.view(np.uint16) if v_cache.dtype == np.float16 else v_cache
        assert kc.flags.c_contiguous and vc.flags.c_contiguous
        T, H, D = key.shape
        nb, bs, nh, hd = kc.shape
        assert (nh, hd) == (H, D)
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        rc = self.lib.oracle_reshape_and_cache(_ptr(key), _ptr(value), _ptr(kc), _ptr(vc),
                                               _ptr(sm), T, H, D, nb, bs)
        if rc:
            raise ValueError(f"oracle_reshape_and_cache failed ({rc})")

    # -- block copies -----------------------------------------------------------
    def copy_blocks(self, k_cache, v_cache, block_mapping):
        """In place: block dst of both caches becomes a copy of block src, for
        each (src, dst) row of block_mapping [N, 2]."""
        kc = k_cache.view(np.uint16) if k_cache.dtype == np.float16 else k_cache
        vc = v_cache.view(np.uint16) if v_cache.dtype == np.float16 else v_cache
        assert kc.flags.c_contiguous and vc.flags.c_contiguous and kc.shape == vc.shape
        m = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
        nb = kc.shape[0]
        rc = self.lib.oracle_copy_blocks(_ptr(kc), _ptr(vc), _ptr(m), m.shape[0], nb,
                                         int(np.prod(kc.shape[1:])))
        if rc:
            raise ValueError(f"oracle_copy_blocks failed ({rc})")

    def swap_blocks(self, src, dst, block_mapping):
        """In place on dst: block b of dst becomes a copy of block a of src for
        each (a, b) row of block_mapping [N, 2]."""
        s_ = _u16(src)
        d_ = dst.view(np.uint16) if dst.dtype == np.float16 else dst
        assert d_.flags.c_contiguous and s_.shape[1:] == d_.shape[1:]
        m = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
        rc = self.lib.oracle_swap_blocks(_ptr(s_), _ptr(d_), _ptr(m), m.shape[0], s_.shape[0],
                                         d_.shape[0], int(np.prod(s_.shape[1:])))
        if rc:
            raise ValueError(f"oracle_swap_blocks failed ({rc})")

    # -- FP8 (OCP E4M3) ------------------------------------------------------------
    def e4m3_to_double(self, codes):
        return np.array([self.lib.oracle_e4m3_to_double(int(c)) for c in np.asarray(codes).ravel()],
                        dtype=np.float64).reshape(np.shape(codes))

    def float_to_e4m3(self, values):
        v = np.asarray(values, dtype=np.float32)
        return np.array([self.lib.oracle_float_to_e4m3(float(x)) for x in v.ravel()],
                        dtype=np.uint8).reshape(v.shape)

    def quantize_e4m3(self, x_f16, scale):
        x = _u16(np.asarray(x_f16))
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_quantize_e4m3(_ptr(x), _ptr(out), x.size, float(scale))
        return out

    def reshape_and_cache_fp8(self, key, value, k_cache8, v_cache8, slot_mapping, k_scale,
                              v_scale):
        key, value = _u16(key), _u16(value)
        assert k_cache8.dtype == np.uint8 and v_cache8.dtype == np.uint8
        assert k_cache8.flags.c_contiguous and v_cache8.flags.c_contiguous
        T, H, D = key.shape
        nb, bs, nh, hd = k_cache8.shape
        assert (nh, hd) == (H, D)
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        rc = self.lib.oracle_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(k_cache8),
                                                   _ptr(v_cache8), _ptr(sm), T, H, D, nb, bs,
                                                   float(k_scale), float(v_scale))
        if rc:
            raise ValueError(f"oracle_reshape_and_cache_fp8 failed ({rc})")

    def decode_fp8(self, q, k_cache8, v_cache8, block_tables, context_lens, scale, k_scale,
                   v_scale, pairs=None):
        q = _u16(q)
        S, H, D = q.shape
        nb, bs, nh, hd = k_cache8.shape
        assert (nh, hd) == (H, D) and k_cache8.dtype == np.uint8 and v_cache8.shape == k_cache8.shape
        kc = np.ascontiguousarray(k_cache8)
        vc = np.ascontiguousarray(v_cache8)
        whole = pairs is None
        if whole:
            pairs = [(s, h) for s in range(S) for h in range(H)]
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.empty((pr.shape[0], D), dtype=np.float64)
        used = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_decode_fp8_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q), _ptr(kc),
                                              _ptr(vc), _ptr(bt), _ptr(cl), S, H, D, nb, bs,
                                              bt.shape[1], float(scale), float(k_scale),
                                              float(v_scale), _ptr(used))
        if rc:
            raise ValueError(f"oracle_decode_fp8_pairs failed ({rc})")
        self.threads_used = int(used[0])
        return out.reshape(S, H, D) if whole else out

    # -- multi-query (chunked prefill) ------------------------------------------
    def prefill(self, q, k_cache, v_cache, block_tables, context_lens, query_start, scale):
        """fp64 [T, H, D]: causal attention of each sequence's last n_s positions."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        T, H, D = q.shape
        nb, bs, nh, hd = k_cache.shape
        assert (nh, hd) == (H, D) and v_cache.shape == k_cache.shape
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        S = cl.shape[0]
        out = np.zeros((T, H, D), dtype=np.float64)
        used = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                     _ptr(cl), _ptr(qs), S, T, H, D, nb, bs, bt.shape[1],
                                     float(scale), _ptr(used))
        if rc:
            raise ValueError(f"oracle_prefill failed ({rc})")
        self.threads_used = int(used[0])
        return out

    def prefill_fp8(self, q, k_cache8, v_cache8, block_tables, context_lens, query_start, scale,
                    k_scale, v_scale):
        """fp64 [T, H, D]: prefill over FP8 caches (values = code * scale)."""
        q = _u16(q)
        T, H, D = q.shape
        nb, bs, nh, hd = k_cache8.shape
        assert (nh, hd) == (H, D) and k_cache8.dtype == np.uint8 and v_cache8.shape == k_cache8.shape
        kc = np.ascontiguousarray(k_cache8)
        vc = np.ascontiguousarray(v_cache8)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        S = cl.shape[0]
        out = np.zeros((T, H, D), dtype=np.float64)
        used = np.zeros(1, dtype=np.int32)
        rc = self.lib.oracle_prefill_fp8(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                                         _ptr(cl), _ptr(qs), S, T, H, D, nb, bs, bt.shape[1],
                                         float(scale), float(k_scale), float(v_scale), _ptr(used))
        if rc:
            raise ValueError(f"oracle_prefill_fp8 failed ({rc})")
        self.threads_used = int(used[0])
        return out


_default = None


def get():
    """The oracle built from oracle/pa_oracle.c (built on first use if absent)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
