"""CPU oracle for the stable merge of two sorted arrays.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``ordered_merge_sorted_amd``) never imports, links or calls it, and
this package imports nothing from the product: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc into
``liboracle.so`` next to it); this module only marshals numpy arrays.  See the
header of ``oracle.c`` for what each routine computes and which passage of the
pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-Wall", "-Werror", "-shared", "-fPIC"]


def compile_c(src: str, out: str) -> str:
    """Compile one C source into a shared library with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (no GPU needed)."""
    if force or not os.path.exists(LIB):
        compile_c(SRC, LIB)
    return LIB


def _i32(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.int32:
        raise TypeError("oracle keys must be int32, got %s" % x.dtype)
    return x


def _u32(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint32:
        raise TypeError("oracle payloads must be uint32, got %s" % x.dtype)
    return x


KIND_I32, KIND_U32, KIND_F32, KIND_I64, KIND_U64, KIND_F64 = 0, 1, 2, 3, 4, 5
ORDER_DESCENDING = 8
_KIND = {np.dtype(np.int32): KIND_I32, np.dtype(np.uint32): KIND_U32,
         np.dtype(np.float32): KIND_F32, np.dtype(np.int64): KIND_I64,
         np.dtype(np.uint64): KIND_U64, np.dtype(np.float64): KIND_F64}
_KIND_DTYPE = {v: k for k, v in _KIND.items()}
_BITS = {4: np.uint32, 8: np.uint64}


def _typed_pair(A, B):
    """Key kind of A and B (same dtype), and both as unsigned bit views."""
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    if A.dtype != B.dtype or A.dtype not in _KIND:
        raise TypeError("keys must both be one of %s, got %s and %s"
                        % (sorted(str(d) for d in _KIND), A.dtype, B.dtype))
    bits = _BITS[A.dtype.itemsize]
    return _KIND[A.dtype], A.view(bits), B.view(bits)


def _payloads(Av, Bv):
    """Payload arrays of one 4- or 8-byte dtype, as unsigned bit views."""
    Av, Bv = np.ascontiguousarray(Av), np.ascontiguousarray(Bv)
    if Av.dtype != Bv.dtype or Av.dtype.itemsize not in _BITS:
        raise TypeError("payloads must share one 4- or 8-byte dtype")
    bits = _BITS[Av.dtype.itemsize]
    return Av.dtype, Av.view(bits), Bv.view(bits)


def _ptr(x: np.ndarray):
    return ctypes.c_void_p(x.ctypes.data)


class Oracle:
    """The oracle routines of one compiled copy of ``oracle.c``."""

    def __init__(self, lib_path: str = LIB):
        lib = ctypes.CDLL(lib_path)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_merge_i32.argtypes = [p, i64, p, i64, p]
        lib.oracle_merge_i32.restype = None
        lib.oracle_merge_kv.argtypes = [p, p, i64, p, p, i64, p, p]
        lib.oracle_merge_kv.restype = None
        lib.oracle_co_rank_all.argtypes = [p, i64, p, i64, p]
        lib.oracle_co_rank_all.restype = None
        lib.oracle_merge_keys.argtypes = [ctypes.c_int, p, i64, p, i64, p]
        lib.oracle_merge_keys.restype = None
        lib.oracle_merge_pairs.argtypes = [ctypes.c_int, ctypes.c_int, p, p, i64, p, p, i64,
                                           p, p]
        lib.oracle_merge_pairs.restype = None
        lib.oracle_key_le.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64]
        lib.oracle_key_le.restype = ctypes.c_int
        lib.oracle_merge_batched.argtypes = [ctypes.c_int, ctypes.c_int, p, p, p, p, p, p, i64,
                                             p, p]
        lib.oracle_merge_batched.restype = None
        lib.oracle_sort.argtypes = [ctypes.c_int, ctypes.c_int, p, p, i64, p, p, p, p]
        lib.oracle_sort.restype = None
        lib.oracle_merge_runs.argtypes = [ctypes.c_int, ctypes.c_int, p, p, i64, i64,
                                          ctypes.c_int, p, p]
        lib.oracle_merge_runs.restype = None
        self._lib = lib
        self.path = lib_path

    def merge_i32(self, A, B) -> np.ndarray:
        """Stable merge of sorted int32 ``A`` and ``B``; equal keys: A first."""
        A, B = _i32(A), _i32(B)
        C = np.empty(A.size + B.size, dtype=np.int32)
        self._lib.oracle_merge_i32(_ptr(A), A.size, _ptr(B), B.size, _ptr(C))
        return C

    def merge_kv(self, A_keys, A_vals, B_keys, B_vals):
        """Stable merge of (int32 key, uint32 payload) pairs by key; A first on ties."""
        Ak, Bk = _i32(A_keys), _i32(B_keys)
        Av, Bv = _u32(A_vals), _u32(B_vals)
        if Ak.size != Av.size or Bk.size != Bv.size:
            raise ValueError("key and payload lengths differ")
        Ck = np.empty(Ak.size + Bk.size, dtype=np.int32)
        Cv = np.empty(Ak.size + Bk.size, dtype=np.uint32)
        self._lib.oracle_merge_kv(_ptr(Ak), _ptr(Av), Ak.size, _ptr(Bk),
                                  _ptr(Bv), Bk.size, _ptr(Ck), _ptr(Cv))
        return Ck, Cv

    def merge_keys(self, A, B, descending: bool = False) -> np.ndarray:
        """Stable merge of sorted keys (int32, uint32, float32, int64, uint64
        or float64) in that type's order (floats: IEEE 754 totalOrder),
        descending if asked; A first on ties.  Returns an array of the keys'
        dtype holding the input bits."""
        kind, A, B = _typed_pair(A, B)
        order = kind | (ORDER_DESCENDING if descending else 0)
        C = np.empty(A.size + B.size, dtype=A.dtype)
        self._lib.oracle_merge_keys(order, _ptr(A), A.size, _ptr(B), B.size, _ptr(C))
        return C.view(_KIND_DTYPE[kind])

    def merge_pairs(self, A_keys, A_vals, B_keys, B_vals, descending: bool = False):
        """merge_keys for (key, payload) pairs; payloads of any one 4- or
        8-byte dtype move with their keys and are returned in that dtype."""
        kind, Ak, Bk = _typed_pair(A_keys, B_keys)
        vdt, Av, Bv = _payloads(A_vals, B_vals)
        if Ak.size != Av.size or Bk.size != Bv.size:
            raise ValueError("key and payload lengths differ")
        order = kind | (ORDER_DESCENDING if descending else 0)
        Ck = np.empty(Ak.size + Bk.size, dtype=Ak.dtype)
        Cv = np.empty(Ak.size + Bk.size, dtype=Av.dtype)
        self._lib.oracle_merge_pairs(order, Av.dtype.itemsize, _ptr(Ak), _ptr(Av), Ak.size,
                                     _ptr(Bk), _ptr(Bv), Bk.size, _ptr(Ck), _ptr(Cv))
        return Ck.view(_KIND_DTYPE[kind]), Cv.view(vdt)

    def merge_batched(self, A, a_off, B, b_off, A_vals=None, B_vals=None,
                      descending: bool = False):
        """Independent stable merges: merge p of A[a_off[p]:a_off[p+1]] and
        B[b_off[p]:b_off[p+1]] lands at C[a_off[p]+b_off[p] ...].  Returns C
        (and the payloads when A_vals / B_vals are given)."""
        kind, A, B = _typed_pair(A, B)
        a_off = np.ascontiguousarray(a_off, dtype=np.int64)
        b_off = np.ascontiguousarray(b_off, dtype=np.int64)
        if a_off.size != b_off.size or a_off.size < 1:
            raise ValueError("offset arrays differ in length or are empty")
        if a_off[0] != 0 or b_off[0] != 0 or a_off[-1] != A.size or b_off[-1] != B.size \
                or np.any(np.diff(a_off) < 0) or np.any(np.diff(b_off) < 0):
            raise ValueError("offsets must run nondecreasing from 0 to the array sizes")
        order = kind | (ORDER_DESCENDING if descending else 0)
        C = np.empty(A.size + B.size, dtype=A.dtype)
        if A_vals is None:
            self._lib.oracle_merge_batched(order, 0, _ptr(A), None, _ptr(a_off), _ptr(B), None,
                                           _ptr(b_off), a_off.size - 1, _ptr(C), None)
            return C.view(_KIND_DTYPE[kind])
        vdt, Av, Bv = _payloads(A_vals, B_vals)
        if Av.size != A.size or Bv.size != B.size:
            raise ValueError("key and payload lengths differ")
        Cv = np.empty(A.size + B.size, dtype=Av.dtype)
        self._lib.oracle_merge_batched(order, Av.dtype.itemsize, _ptr(A), _ptr(Av), _ptr(a_off),
                                       _ptr(B), _ptr(Bv), _ptr(b_off), a_off.size - 1, _ptr(C),
                                       _ptr(Cv))
        return C.view(_KIND_DTYPE[kind]), Cv.view(vdt)

    def sort(self, keys, vals=None, descending: bool = False):
        """Stable sort by key in the key type's order (descending if asked);
        returns the sorted keys, and the payloads moved with them."""
        kind, K, _ = _typed_pair(keys, keys)
        order = kind | (ORDER_DESCENDING if descending else 0)
        out = np.empty_like(K)
        tmp = np.empty_like(K)
        if vals is None:
            self._lib.oracle_sort(order, 0, _ptr(K), None, K.size, _ptr(out), None, _ptr(tmp),
                                  None)
            return out.view(_KIND_DTYPE[kind])
        vdt, V, _ = _payloads(vals, vals)
        if V.size != K.size:
            raise ValueError("key and payload lengths differ")
        out_v, tmp_v = np.empty_like(V), np.empty_like(V)
        self._lib.oracle_sort(order, V.dtype.itemsize, _ptr(K), _ptr(V), K.size, _ptr(out),
                              _ptr(out_v), _ptr(tmp), _ptr(tmp_v))
        return out.view(_KIND_DTYPE[kind]), out_v.view(vdt)

    def merge_runs(self, keys, run, ways, vals=None, descending: bool = False):
        """One k-way merge-sort pass: every group of ``ways`` consecutive
        sorted runs of ``run`` elements becomes one sorted run (ties keep the
        input order).  Returns the keys, and the payloads moved with them."""
        kind, K, _ = _typed_pair(keys, keys)
        if not (1 <= ways <= 64) or run < 1:
            raise ValueError("ways must be 1..64 and run >= 1")
        order = kind | (ORDER_DESCENDING if descending else 0)
        out = np.empty_like(K)
        if vals is None:
            self._lib.oracle_merge_runs(order, 0, _ptr(K), None, K.size, int(run), int(ways),
                                        _ptr(out), None)
            return out.view(_KIND_DTYPE[kind])
        vdt, V, _ = _payloads(vals, vals)
        if V.size != K.size:
            raise ValueError("key and payload lengths differ")
        out_v = np.empty_like(V)
        self._lib.oracle_merge_runs(order, V.dtype.itemsize, _ptr(K), _ptr(V), K.size, int(run),
                                    int(ways), _ptr(out), _ptr(out_v))
        return out.view(_KIND_DTYPE[kind]), out_v.view(vdt)

    def key_le(self, dtype, x, y, descending: bool = False) -> bool:
        """The order relation itself: does key x come before key y, or tie?"""
        dt = np.dtype(dtype)
        kind = _KIND[dt]
        bits = _BITS[dt.itemsize]
        xb = int(np.array([x], dtype=dt).view(bits)[0])
        yb = int(np.array([y], dtype=dt).view(bits)[0])
        order = kind | (ORDER_DESCENDING if descending else 0)
        return bool(self._lib.oracle_key_le(order, xb, yb))

    def co_rank_all(self, A, B) -> np.ndarray:
        """int64 array I of length m+n+1: I[k] = number of A elements among the
        first k merged outputs (the co-rank of k); the B count is k - I[k]."""
        A, B = _i32(A), _i32(B)
        I = np.empty(A.size + B.size + 1, dtype=np.int64)
        self._lib.oracle_co_rank_all(_ptr(A), A.size, _ptr(B), B.size, _ptr(I))
        return I

    def co_rank(self, k: int, A, B) -> int:
        """Co-rank of one output rank k (0 <= k <= m+n)."""
        A, B = _i32(A), _i32(B)
        if not 0 <= k <= A.size + B.size:
            raise ValueError("k out of range")
        return int(self.co_rank_all(A, B)[k])


_default = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build(force=False)
        _default = Oracle(LIB)
    return _default


def merge_i32(A, B):
    return default().merge_i32(A, B)


def merge_kv(A_keys, A_vals, B_keys, B_vals):
    return default().merge_kv(A_keys, A_vals, B_keys, B_vals)


def merge_keys(A, B, descending=False):
    return default().merge_keys(A, B, descending)


def merge_pairs(A_keys, A_vals, B_keys, B_vals, descending=False):
    return default().merge_pairs(A_keys, A_vals, B_keys, B_vals, descending)


def key_le(dtype, x, y, descending=False):
    return default().key_le(dtype, x, y, descending)


def merge_batched(A, a_off, B, b_off, A_vals=None, B_vals=None, descending=False):
    return default().merge_batched(A, a_off, B, b_off, A_vals, B_vals, descending)


def merge_runs(keys, run, ways, vals=None, descending=False):
    return default().merge_runs(keys, run, ways, vals, descending)


def sort(keys, vals=None, descending=False):
    return default().sort(keys, vals, descending)


def co_rank_all(A, B):
    return default().co_rank_all(A, B)


def co_rank(k, A, B):
    return default().co_rank(k, A, B)
