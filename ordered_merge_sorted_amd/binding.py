"""Python binding of libomerge.so: argument marshalling only.

Every function checks its tensors (dtype, device, layout), allocates outputs
with torch when none are given, and calls the C ABI declared in
include/omerge.h on the tensors' device and the current torch stream (or the
stream given).  All work runs in the library's HIP kernels; nothing here
computes.  If the library is missing or fails to load, every call raises
OmergeError: there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

from .build import LIB

OK, INVALID_ARG, OVERFLOW, HIP_ERROR, SCRATCH_LIMIT = 0, 1, 2, 3, 4


class OmergeError(RuntimeError):
    """A libomerge call failed, or the library could not be loaded."""


_lib = None


def library_path() -> str:
    return LIB


def load_library() -> ctypes.CDLL:
    """Load libomerge.so (once).  Raises OmergeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise OmergeError(
            "libomerge.so is not built at %s; build it with "
            "`python -m ordered_merge_sorted_amd.build`" % LIB)
    try:
        lib = ctypes.CDLL(LIB)
    except OSError as e:
        raise OmergeError("cannot load %s: %s" % (LIB, e)) from e
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "merge_i32": (i32, [p, i64, p, i64, p, p]),
        "merge_i32_no_alloc": (i32, [p, i64, p, i64, p, p]),
        "merge_kv": (i32, [p, p, i64, p, p, i64, p, p, p]),
        "omerge_merge_keys": (i32, [p, i64, p, i64, p, i32, p]),
        "omerge_merge_pairs": (i32, [p, p, i64, p, p, i64, p, p, i32, i32, p]),
        "omerge_merge_batched": (i32, [p, p, p, i64, p, p, p, i64, i64, p, p, i32, i32, p]),
        "omerge_sort": (i32, [p, p, p, p, i64, i32, i32, p]),
        "omerge_merge_runs4": (i32, [p, p, i64, i64, i32, p]),
        "omerge_co_rank": (i32, [p, i64, p, i64, p, i64, p, p]),
        "omerge_segment_length": (i64, [i64, i64, i32]),
        "omerge_partition_count": (i64, [i64, i64]),
        "omerge_partition": (i32, [p, i64, p, i64, i64, p, p]),
        "omerge_merge_segments_i32": (i32, [p, i64, p, i64, p, i64, p, p]),
        "omerge_merge_segments_kv": (i32, [p, p, i64, p, p, i64, p, i64, p, p, p]),
        "omerge_stream_copy": (i32, [p, i64, p, p]),
        "omerge_merge_i32_direct": (i32, [p, i64, p, i64, p, i64, i32, p]),
        "omerge_status_string": (ctypes.c_char_p, [i32]),
        "omerge_last_hip_error": (i32, []),
        "omerge_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _raise_on(rc: int, what: str) -> None:
    if rc == OK:
        return
    lib = load_library()
    msg = lib.omerge_status_string(rc).decode()
    if rc == HIP_ERROR:
        msg += " (hipError_t %d)" % lib.omerge_last_hip_error()
    raise OmergeError("%s failed: %s" % (what, msg))


_PAYLOAD_DTYPES = (torch.int32, getattr(torch, "uint32", torch.int32))


def _vec(t: torch.Tensor, name: str, dtypes, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU, got %s" % (name, t.device))
    if device is not None and t.get_device() != device.index:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dim() != 1:
        raise ValueError("%s must be 1-D" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t: torch.Tensor) -> int:
    """Device address of t's data (0 when empty), for a void* argument."""
    return t.data_ptr() if t.numel() else 0


# The handle of a device's current stream and the current device's index,
# read without building Stream or device-guard objects (a few microseconds
# per call that small merges feel); torch's public calls where this torch
# lacks these functions.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device, stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _current_raw_stream is not None:
        index = device.index if device.index is not None else torch.cuda.current_device()
        return _current_raw_stream(index)
    return torch.cuda.current_stream(device).cuda_stream


def _on(device):
    """Makes `device` (a torch.device, an index or a name) current for a
    library call: nothing to do when it already is, torch's device guard
    otherwise."""
    if not isinstance(device, torch.device):
        device = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
    if device.index is None or torch.cuda.current_device() == device.index:
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _out(out, n: int, dtype, device, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty(n, dtype=dtype, device=device)
    _vec(out, name, (dtype,), device)
    if out.numel() != n:
        raise ValueError("%s must have %d elements, got %d" % (name, n, out.numel()))
    return out


def merge_i32(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Stable merge of sorted int32 tensors a and b (equal keys: a first)."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    out = _out(out, a.numel() + b.numel(), torch.int32, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.merge_i32(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(out),
                           _stream(a.device, stream))
    _raise_on(rc, "merge_i32")
    return out


def merge_i32_no_alloc(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """merge_i32 through the entry point that allocates no device memory (its
    scratch is a static array of the library; m + n <= 2^32).  `out` must be
    given: this call allocates nothing, here either."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    if out is None:
        raise ValueError("merge_i32_no_alloc needs an output tensor")
    out = _out(out, a.numel() + b.numel(), torch.int32, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.merge_i32_no_alloc(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(out),
                                    _stream(a.device, stream))
    _raise_on(rc, "merge_i32_no_alloc")
    return out


def merge_kv(a_keys: torch.Tensor, a_vals: torch.Tensor, b_keys: torch.Tensor,
             b_vals: torch.Tensor, out_keys: Optional[torch.Tensor] = None,
             out_vals: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable merge of (int32 key, 32-bit payload) pairs by key; payloads are
    never compared and move with their keys (a's first on equal keys)."""
    dev = a_keys.device if isinstance(a_keys, torch.Tensor) else None
    _vec(a_keys, "a_keys", (torch.int32,))
    _vec(b_keys, "b_keys", (torch.int32,), dev)
    _vec(a_vals, "a_vals", _PAYLOAD_DTYPES, dev)
    _vec(b_vals, "b_vals", (a_vals.dtype,), dev)
    if a_vals.numel() != a_keys.numel() or b_vals.numel() != b_keys.numel():
        raise ValueError("key and payload lengths differ")
    t = a_keys.numel() + b_keys.numel()
    out_keys = _out(out_keys, t, torch.int32, dev, "out_keys")
    out_vals = _out(out_vals, t, a_vals.dtype, dev, "out_vals")
    lib = load_library()
    with _on(dev):
        rc = lib.merge_kv(_ptr(a_keys), _ptr(a_vals), a_keys.numel(), _ptr(b_keys),
                          _ptr(b_vals), b_keys.numel(), _ptr(out_keys), _ptr(out_vals),
                          _stream(dev, stream))
    _raise_on(rc, "merge_kv")
    return out_keys, out_vals


# Key order codes of include/omerge.h (omerge_key_kind | OMERGE_DESCENDING).
KEY_I32, KEY_U32, KEY_F32, KEY_I64, KEY_U64, KEY_F64 = 0, 1, 2, 3, 4, 5
DESCENDING = 8
_KEY_KIND = {torch.int32: KEY_I32, torch.float32: KEY_F32,
             torch.int64: KEY_I64, torch.float64: KEY_F64}
for _name, _kind in (("uint32", KEY_U32), ("uint64", KEY_U64)):
    if hasattr(torch, _name):
        _KEY_KIND[getattr(torch, _name)] = _kind
# Payloads: any 4- or 8-byte dtype; they are moved as bits, never compared.
_ANY_PAYLOAD = tuple(d for d in (torch.int32, torch.float32, torch.int64, torch.float64,
                                 getattr(torch, "uint32", None), getattr(torch, "uint64", None))
                     if d is not None)


def order_code(dtype: torch.dtype, descending: bool = False) -> int:
    """The C ABI order code for keys of `dtype` (int32, uint32, float32,
    int64, uint64 or float64)."""
    if dtype not in _KEY_KIND:
        raise TypeError("keys must have dtype int32, uint32, float32, int64, uint64 or "
                        "float64, got %s" % dtype)
    return _KEY_KIND[dtype] | (DESCENDING if descending else 0)


def merge(a: torch.Tensor, b: torch.Tensor, descending: bool = False,
          out: Optional[torch.Tensor] = None,
          stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Stable merge of sorted key tensors (equal keys: a first).

    Integer keys compare as integers of their type; float32 and float64 keys
    compare in IEEE 754 totalOrder (-NaN < -inf < ... < -0.0 < +0.0 < ... <
    +inf < +NaN).  With
    descending=True, a and b are sorted descending and so is the result.
    Output keys are the input keys' exact bit patterns."""
    _vec(a, "a", tuple(_KEY_KIND))
    _vec(b, "b", (a.dtype,), a.device)
    order = order_code(a.dtype, descending)
    out = _out(out, a.numel() + b.numel(), a.dtype, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.omerge_merge_keys(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(out), order,
                                   _stream(a.device, stream))
    _raise_on(rc, "omerge_merge_keys")
    return out


def merge_pairs(a_keys: torch.Tensor, a_vals: torch.Tensor, b_keys: torch.Tensor,
                b_vals: torch.Tensor, descending: bool = False,
                out_keys: Optional[torch.Tensor] = None,
                out_vals: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """merge() for (key, payload) pairs, payloads of any 4- or 8-byte dtype:
    they move with their keys and are never compared (a's first on equal
    keys)."""
    dev = a_keys.device if isinstance(a_keys, torch.Tensor) else None
    _vec(a_keys, "a_keys", tuple(_KEY_KIND))
    _vec(b_keys, "b_keys", (a_keys.dtype,), dev)
    _vec(a_vals, "a_vals", _ANY_PAYLOAD, dev)
    _vec(b_vals, "b_vals", (a_vals.dtype,), dev)
    if a_vals.numel() != a_keys.numel() or b_vals.numel() != b_keys.numel():
        raise ValueError("key and payload lengths differ")
    order = order_code(a_keys.dtype, descending)
    t = a_keys.numel() + b_keys.numel()
    out_keys = _out(out_keys, t, a_keys.dtype, dev, "out_keys")
    out_vals = _out(out_vals, t, a_vals.dtype, dev, "out_vals")
    lib = load_library()
    with _on(dev):
        rc = lib.omerge_merge_pairs(_ptr(a_keys), _ptr(a_vals), a_keys.numel(), _ptr(b_keys),
                                    _ptr(b_vals), b_keys.numel(), _ptr(out_keys),
                                    _ptr(out_vals), order, a_vals.element_size(),
                                    _stream(dev, stream))
    _raise_on(rc, "omerge_merge_pairs")
    return out_keys, out_vals


def merge_batched(a: torch.Tensor, a_offsets: torch.Tensor, b: torch.Tensor,
                  b_offsets: torch.Tensor, a_vals: Optional[torch.Tensor] = None,
                  b_vals: Optional[torch.Tensor] = None, descending: bool = False,
                  out: Optional[torch.Tensor] = None, out_vals: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None):
    """Independent stable merges in one call: merge p takes
    a[a_offsets[p]:a_offsets[p+1]] and b[b_offsets[p]:b_offsets[p+1]] (each
    sorted in the keys' order) and its output lands at
    out[a_offsets[p]+b_offsets[p] ...].  Offsets are int64 device tensors of
    num_merges+1 entries, from 0 to the sizes of a and b, nondecreasing (not
    checked: they live on the device).  With payloads, returns (keys,
    payloads)."""
    _vec(a, "a", tuple(_KEY_KIND))
    dev = a.device
    _vec(b, "b", (a.dtype,), dev)
    _vec(a_offsets, "a_offsets", (torch.int64,), dev)
    _vec(b_offsets, "b_offsets", (torch.int64,), dev)
    if a_offsets.numel() != b_offsets.numel() or a_offsets.numel() < 1:
        raise ValueError("a_offsets and b_offsets must have the same, nonzero length")
    kv = a_vals is not None or b_vals is not None
    if kv:
        _vec(a_vals, "a_vals", _ANY_PAYLOAD, dev)
        _vec(b_vals, "b_vals", (a_vals.dtype,), dev)
        if a_vals.numel() != a.numel() or b_vals.numel() != b.numel():
            raise ValueError("key and payload lengths differ")
    order = order_code(a.dtype, descending)
    t = a.numel() + b.numel()
    out = _out(out, t, a.dtype, dev, "out")
    if kv:
        out_vals = _out(out_vals, t, a_vals.dtype, dev, "out_vals")
    lib = load_library()
    with _on(dev):
        rc = lib.omerge_merge_batched(
            _ptr(a), _ptr(a_vals) if kv else None, _ptr(a_offsets), a.numel(), _ptr(b),
            _ptr(b_vals) if kv else None, _ptr(b_offsets), b.numel(), a_offsets.numel() - 1,
            _ptr(out), _ptr(out_vals) if kv else None, order,
            a_vals.element_size() if kv else 0, _stream(dev, stream))
    _raise_on(rc, "omerge_merge_batched")
    return (out, out_vals) if kv else out


def sort(keys: torch.Tensor, vals: Optional[torch.Tensor] = None, descending: bool = False,
         out: Optional[torch.Tensor] = None, out_vals: Optional[torch.Tensor] = None,
         stream: Optional[torch.cuda.Stream] = None):
    """Stable merge sort of a key tensor (and payloads moved with the keys):
    equal keys keep their input order.  out / out_vals may be keys / vals
    themselves (in place).  With payloads, returns (keys, payloads)."""
    _vec(keys, "keys", tuple(_KEY_KIND))
    dev = keys.device
    kv = vals is not None
    if kv:
        _vec(vals, "vals", _ANY_PAYLOAD, dev)
        if vals.numel() != keys.numel():
            raise ValueError("key and payload lengths differ")
    order = order_code(keys.dtype, descending)
    out = _out(out, keys.numel(), keys.dtype, dev, "out")
    if kv:
        out_vals = _out(out_vals, keys.numel(), vals.dtype, dev, "out_vals")
    lib = load_library()
    with _on(dev):
        rc = lib.omerge_sort(_ptr(keys), _ptr(vals) if kv else None, _ptr(out),
                             _ptr(out_vals) if kv else None, keys.numel(), order,
                             vals.element_size() if kv else 0, _stream(dev, stream))
    _raise_on(rc, "omerge_sort")
    return (out, out_vals) if kv else out


def merge_runs4(keys: torch.Tensor, run: int, descending: bool = False,
                out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One 4-way merge-sort pass: keys holds sorted runs of `run` keys; each
    group of four consecutive runs becomes one sorted run, equal keys in
    input order (the earlier run first).  Keys alone; out must not overlap
    keys."""
    _vec(keys, "keys", tuple(_KEY_KIND))
    if run < 1:
        raise ValueError("run must be at least 1")
    dev = keys.device
    order = order_code(keys.dtype, descending)
    out = _out(out, keys.numel(), keys.dtype, dev, "out")
    lib = load_library()
    with _on(dev):
        rc = lib.omerge_merge_runs4(_ptr(keys), _ptr(out), keys.numel(), int(run), order,
                                    _stream(dev, stream))
    _raise_on(rc, "omerge_merge_runs4")
    return out


def co_rank(a: torch.Tensor, b: torch.Tensor, k: torch.Tensor,
            out: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Device co-rank i(k) for each int64 output rank in k (clamped to [0, m+n])."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    _vec(k, "k", (torch.int64,), a.device)
    out = _out(out, k.numel(), torch.int64, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.omerge_co_rank(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(k), k.numel(),
                                _ptr(out), _stream(a.device, stream))
    _raise_on(rc, "omerge_co_rank")
    return out


def segment_length(m: int, n: int, kv: bool = False, device=None) -> int:
    """Outputs per workgroup that merge_i32 / merge_kv use for these sizes."""
    lib = load_library()
    with _on(device if device is not None else torch.cuda.current_device()):
        s = lib.omerge_segment_length(int(m), int(n), int(bool(kv)))
    if s <= 0:
        raise OmergeError("omerge_segment_length failed for m=%d n=%d" % (m, n))
    return int(s)


def partition_count(total: int, seg_len: int) -> int:
    c = load_library().omerge_partition_count(int(total), int(seg_len))
    if c < 0:
        raise OmergeError("bad sizes for a partition: total=%d seg_len=%d" % (total, seg_len))
    return int(c)


def partition(a: torch.Tensor, b: torch.Tensor, seg_len: int,
              out: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """int64 co-ranks of the segment boundaries k_s = min(s*seg_len, m+n)."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    count = partition_count(a.numel() + b.numel(), seg_len)
    out = _out(out, count, torch.int64, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.omerge_partition(_ptr(a), a.numel(), _ptr(b), b.numel(), int(seg_len),
                                  _ptr(out), _stream(a.device, stream))
    _raise_on(rc, "omerge_partition")
    return out


def merge_segments_i32(a: torch.Tensor, b: torch.Tensor, part: torch.Tensor, seg_len: int,
                       out: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The segment merge kernel alone, given partition(a, b, seg_len)."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    _vec(part, "part", (torch.int64,), a.device)
    if part.numel() != partition_count(a.numel() + b.numel(), seg_len):
        raise ValueError("part has the wrong length for seg_len")
    out = _out(out, a.numel() + b.numel(), torch.int32, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.omerge_merge_segments_i32(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(part),
                                           int(seg_len), _ptr(out), _stream(a.device, stream))
    _raise_on(rc, "omerge_merge_segments_i32")
    return out


def merge_segments_kv(a_keys, a_vals, b_keys, b_vals, part, seg_len, out_keys=None,
                      out_vals=None, stream=None):
    """The key+payload segment merge kernel alone, given a partition."""
    dev = a_keys.device if isinstance(a_keys, torch.Tensor) else None
    _vec(a_keys, "a_keys", (torch.int32,))
    _vec(b_keys, "b_keys", (torch.int32,), dev)
    _vec(a_vals, "a_vals", _PAYLOAD_DTYPES, dev)
    _vec(b_vals, "b_vals", (a_vals.dtype,), dev)
    _vec(part, "part", (torch.int64,), dev)
    if a_vals.numel() != a_keys.numel() or b_vals.numel() != b_keys.numel():
        raise ValueError("key and payload lengths differ")
    t = a_keys.numel() + b_keys.numel()
    if part.numel() != partition_count(t, seg_len):
        raise ValueError("part has the wrong length for seg_len")
    out_keys = _out(out_keys, t, torch.int32, dev, "out_keys")
    out_vals = _out(out_vals, t, a_vals.dtype, dev, "out_vals")
    lib = load_library()
    with _on(dev):
        rc = lib.omerge_merge_segments_kv(
            _ptr(a_keys), _ptr(a_vals), a_keys.numel(), _ptr(b_keys), _ptr(b_vals),
            b_keys.numel(), _ptr(part), int(seg_len), _ptr(out_keys), _ptr(out_vals),
            _stream(dev, stream))
    _raise_on(rc, "omerge_merge_segments_kv")
    return out_keys, out_vals


def stream_copy(src: torch.Tensor, out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Measurement reference: copy an int32 tensor with the library's
    16-byte streaming copy kernel (the bytes a merge of as many outputs moves)."""
    _vec(src, "src", (torch.int32,))
    out = _out(out, src.numel(), torch.int32, src.device, "out")
    lib = load_library()
    with _on(src.device):
        rc = lib.omerge_stream_copy(_ptr(src), src.numel(), _ptr(out), _stream(src.device, stream))
    _raise_on(rc, "omerge_stream_copy")
    return out


def merge_i32_direct(a: torch.Tensor, b: torch.Tensor, per_thread: int = 16,
                     two_searches: bool = False, out: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The global-memory merge kernels (no LDS), for ablation against
    merge_i32: one lane per slice of per_thread outputs; two co-rank searches
    per slice (basic kernel) or one search then a walk (co-rank kernel)."""
    _vec(a, "a", (torch.int32,))
    _vec(b, "b", (torch.int32,), a.device)
    out = _out(out, a.numel() + b.numel(), torch.int32, a.device, "out")
    lib = load_library()
    with _on(a.device):
        rc = lib.omerge_merge_i32_direct(_ptr(a), a.numel(), _ptr(b), b.numel(), _ptr(out),
                                         int(per_thread), int(bool(two_searches)),
                                         _stream(a.device, stream))
    _raise_on(rc, "omerge_merge_i32_direct")
    return out
