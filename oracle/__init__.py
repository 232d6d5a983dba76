"""CPU oracle of the uzip v1 bitstream -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does; the two implementations share no code and meet only
through the bytes they produce.

The arithmetic lives in ``uzip_oracle.c`` (plain single-threaded C, one step
of the method per function, each citing the page passage it follows).  This
module only marshals numpy arrays to it through ctypes.  Every function here
is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uzip_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 1
FP32 = 2
FP16 = 3
FP8_E4M3 = 4
FP8_E5M2 = 5
DTYPES = (BF16, FP32, FP16, FP8_E4M3, FP8_E5M2)
_ELEM = {BF16: np.uint16, FP32: np.uint32, FP16: np.uint16, FP8_E4M3: np.uint8, FP8_E5M2: np.uint8}
# bits of the raw (sign+mantissa) field and of the coded exponent field
_RAW_BITS = {BF16: 8, FP32: 24, FP16: 11, FP8_E4M3: 4, FP8_E5M2: 3}
_SYM_BITS = {BF16: 8, FP32: 8, FP16: 5, FP8_E4M3: 4, FP8_E5M2: 5}
OK, INVALID, CAPACITY, CORRUPT = 0, 1, 2, 3

LANES = 32
M = 4096
L = 65536


def build(force: bool = False) -> str:
    """Compile the oracle with gcc -O2 (no hand vectorisation).

    UZIP_ORACLE_LIB may name another build of this same source (used to run
    the pins against deliberately broken copies when checking the tests)."""
    if os.environ.get("UZIP_ORACLE_LIB"):
        return os.environ["UZIP_ORACLE_LIB"]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        _lib.orc_chunk_elems.restype = u64
        _lib.orc_chunk_elems.argtypes = [i32, u64]
        _lib.orc_split.restype = None
        _lib.orc_split.argtypes = [i32, vp, u64, vp, vp]
        _lib.orc_merge.restype = None
        _lib.orc_merge.argtypes = [i32, vp, vp, u64, vp]
        _lib.orc_histogram.restype = None
        _lib.orc_histogram.argtypes = [vp, u64, vp]
        _lib.orc_normalize.restype = i32
        _lib.orc_normalize.argtypes = [vp, ctypes.c_uint32, vp]
        _lib.orc_cumulative.restype = None
        _lib.orc_cumulative.argtypes = [vp, vp]
        _lib.orc_rans_encode.restype = u64
        _lib.orc_rans_encode.argtypes = [vp, u64, i32, vp, vp, vp, vp]
        _lib.orc_rans_decode.restype = i32
        _lib.orc_rans_decode.argtypes = [vp, vp, u64, u64, i32, vp, vp, vp]
        _lib.orc_max_compressed_size.restype = u64
        _lib.orc_max_compressed_size.argtypes = [i32, u64, u64]
        _lib.orc_compress.restype = i32
        _lib.orc_compress.argtypes = [i32, vp, u64, u64, vp, u64, vp]
        _lib.orc_decompress.restype = i32
        _lib.orc_decompress.argtypes = [vp, u64, i32, u64, vp]
        _lib.orc_compress_sampled.restype = i32
        _lib.orc_compress_sampled.argtypes = [i32, vp, u64, u64, vp, u64, vp]
        _lib.orc_normalize_sampled.restype = i32
        _lib.orc_normalize_sampled.argtypes = [vp, ctypes.c_uint32, vp]
        _lib.orc_log2_q16.restype = ctypes.c_uint32
        _lib.orc_log2_q16.argtypes = [ctypes.c_uint32]
        _lib.orc_plan_call.restype = i32
        _lib.orc_plan_call.argtypes = [i32, vp, u64, u64, vp, vp]
        _lib.orc_entropy_bound.restype = ctypes.c_double
        _lib.orc_entropy_bound.argtypes = [i32, vp, u64, u64]
        _lib.orc_compress_arbitrated.restype = i32
        _lib.orc_compress_arbitrated.argtypes = [i32, vp, u64, u64, vp, vp, vp, u64, vp]
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(dtype: int, values) -> np.ndarray:
    """Bit patterns as a contiguous uint8/16/32 array (the dtype's width)."""
    a = np.ascontiguousarray(values)
    want = _ELEM[dtype]
    if a.dtype.itemsize != np.dtype(want).itemsize:
        raise ValueError("expected %d-byte elements, got %s" % (np.dtype(want).itemsize, a.dtype))
    return a.view(want).reshape(-1)


def raw_bits(dtype: int) -> int:
    """Bits of a value's raw field (sign and mantissa)."""
    return _RAW_BITS[dtype]


def sym_bits(dtype: int) -> int:
    """Bits of a value's coded symbol (its exponent field)."""
    return _SYM_BITS[dtype]


def packed_bytes(n: int, bits: int) -> int:
    """Bytes that n fields of `bits` bits take packed back to back."""
    return (n * bits + 7) // 8


def chunk_elems(dtype: int, chunk_bytes: int = 0) -> int:
    return int(lib().orc_chunk_elems(dtype, chunk_bytes))


def split(dtype: int, values):
    """The exponent field of each value (one byte each, n) and the packed raw
    fields (sign and mantissa, raw_bits(dtype) bits each, value order, least
    significant bit first)."""
    v = _bits(dtype, values)
    n = v.size
    e = np.empty(n, np.uint8)
    sm = np.empty(max(packed_bytes(n, raw_bits(dtype)), 1), np.uint8)
    lib().orc_split(dtype, _p(v), n, _p(e), _p(sm))
    return e, sm[: packed_bytes(n, raw_bits(dtype))]


def merge(dtype: int, e, sm) -> np.ndarray:
    e = np.ascontiguousarray(e, np.uint8)
    sm = np.ascontiguousarray(sm, np.uint8)
    n = e.size
    out = np.empty(n, _ELEM[dtype])
    if sm.size == 0:
        sm = np.zeros(1, np.uint8)
    lib().orc_merge(dtype, _p(e), _p(sm), n, _p(out))
    return out


def histogram(e) -> np.ndarray:
    e = np.ascontiguousarray(e, np.uint8)
    c = np.empty(256, np.uint32)
    lib().orc_histogram(_p(e), e.size, _p(c))
    return c


def normalize(counts):
    """(f[256], nsym) for a histogram whose total is n = sum(counts)."""
    c = np.ascontiguousarray(counts, np.uint32)
    assert c.size == 256
    f = np.empty(256, np.uint32)
    nsym = lib().orc_normalize(_p(c), int(c.sum()), _p(f))
    return f, int(nsym)


def cumulative(f) -> np.ndarray:
    f = np.ascontiguousarray(f, np.uint32)
    c0 = np.empty(256, np.uint32)
    lib().orc_cumulative(_p(f), _p(c0))
    return c0


def rans_encode(sym, f, c0, lanes: int = LANES):
    """Interleaved rANS over `lanes` lanes with an explicit table.

    Returns (states[lanes] uint32, words uint16 in decoder order)."""
    s = np.ascontiguousarray(sym, np.uint8)
    f = np.ascontiguousarray(f, np.uint32)
    c0 = np.ascontiguousarray(c0, np.uint32)
    states = np.empty(lanes, np.uint32)
    words = np.empty(max(s.size, 1), np.uint16)
    nw = lib().orc_rans_encode(_p(s), s.size, lanes, _p(f), _p(c0), _p(states), _p(words))
    return states, words[:nw].copy()


def rans_decode(states, words, n: int, f, c0, lanes: int = LANES):
    """Returns (status, symbols[n])."""
    st = np.ascontiguousarray(states, np.uint32)
    w = np.ascontiguousarray(words, np.uint16)
    if w.size == 0:
        w = np.zeros(1, np.uint16)
        nw = 0
    else:
        nw = w.size
    f = np.ascontiguousarray(f, np.uint32)
    c0 = np.ascontiguousarray(c0, np.uint32)
    out = np.zeros(max(n, 1), np.uint8)
    status = lib().orc_rans_decode(_p(st), _p(w), nw, n, lanes, _p(f), _p(c0), _p(out))
    return int(status), out[:n]


def max_compressed_size(dtype: int, n: int, chunk_bytes: int = 0) -> int:
    return int(lib().orc_max_compressed_size(dtype, n, chunk_bytes))


def entropy_bound(dtype: int, values, chunk_bytes: int = 0) -> float:
    """Bytes an ideal per-chunk coder of the coded symbols would reach: the raw
    bytes plus, per chunk, n_i times the empirical entropy of its symbols / 8."""
    v = _bits(dtype, values)
    r = float(lib().orc_entropy_bound(dtype, _p(v) if v.size else None, v.size, chunk_bytes))
    if r < 0:
        raise ValueError("invalid chunk_bytes")
    return r


def compress(dtype: int, values, chunk_bytes: int = 0) -> np.ndarray:
    """The whole compressed buffer as a uint8 array (exact size)."""
    v = _bits(dtype, values)
    cap = max_compressed_size(dtype, v.size, chunk_bytes)
    if cap == 0:
        raise ValueError("invalid chunk_bytes")
    out = np.empty(cap, np.uint8)
    size = ctypes.c_uint64(0)
    st = lib().orc_compress(dtype, _p(v), v.size, chunk_bytes, _p(out), cap, ctypes.byref(size))
    if st != OK:
        raise ValueError("oracle compress failed with status %d" % st)
    return out[: size.value].copy()


def decompress(buf, dtype: int, n: int):
    """Returns (status, bit patterns of the dtype's width, length n)."""
    b = np.ascontiguousarray(buf, np.uint8)
    if b.size == 0:
        b = np.zeros(1, np.uint8)
        nbytes = 0
    else:
        nbytes = b.size
    out = np.zeros(max(n, 1), _ELEM[dtype])
    st = lib().orc_decompress(_p(b), nbytes, dtype, n, _p(out))
    return int(st), out[:n]


# ---- per-call arbitration (NCCLZ Sec. IV-C, Eq. (1)-(2), Algorithm 1) -------
class Policy(ctypes.Structure):
    """Cost-model inputs: effective link bandwidth, encode and decode rates
    (bytes per microsecond), the exposed fractions of the codec time (per
    mille), the fixed cost of a coded transfer (ns), the small-call threshold
    (bytes) and the minimum predicted gain (per mille of the payload)."""
    _fields_ = [("link_bytes_per_us", ctypes.c_uint64), ("encode_bytes_per_us", ctypes.c_uint64),
                ("decode_bytes_per_us", ctypes.c_uint64), ("fixed_ns", ctypes.c_uint64),
                ("small_bytes", ctypes.c_uint64), ("exposed_encode_permil", ctypes.c_uint32),
                ("exposed_decode_permil", ctypes.c_uint32), ("min_gain_permil", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class Plan(ctypes.Structure):
    """decision 0 coded, 1 RAW by the cost model, 2 RAW as a small call."""
    _fields_ = [("decision", ctypes.c_uint32), ("sample_values", ctypes.c_uint32),
                ("predicted_bytes", ctypes.c_uint64), ("raw_ns", ctypes.c_uint64), ("coded_ns", ctypes.c_uint64)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


def log2_q16(x: int) -> int:
    """floor(2^16 log2 x) by the squaring method (x >= 1)."""
    return int(lib().orc_log2_q16(x))


def plan_call(dtype: int, values, policy: Policy, chunk_bytes: int = 0) -> dict:
    v = _bits(dtype, values)
    plan = Plan()
    st = lib().orc_plan_call(dtype, _p(v) if v.size else None, v.size, chunk_bytes, ctypes.byref(policy),
                             ctypes.byref(plan))
    if st != OK:
        raise ValueError("oracle plan failed with status %d" % st)
    return plan.as_dict()


def compress_arbitrated(dtype: int, values, policy: Policy, chunk_bytes: int = 0):
    """(compressed buffer, plan) of an arbitrated call."""
    v = _bits(dtype, values)
    cap = max_compressed_size(dtype, v.size, chunk_bytes)
    if cap == 0:
        raise ValueError("invalid chunk_bytes")
    out = np.empty(cap, np.uint8)
    size = ctypes.c_uint64(0)
    plan = Plan()
    st = lib().orc_compress_arbitrated(dtype, _p(v) if v.size else None, v.size, chunk_bytes, ctypes.byref(policy),
                                       ctypes.byref(plan), _p(out), cap, ctypes.byref(size))
    if st != OK:
        raise ValueError("oracle arbitrated compress failed with status %d" % st)
    return out[: size.value].copy(), plan.as_dict()


# ---- sampled tables (UCCL-Zip: each block's table from a sample) ------------
def normalize_sampled(counts, S: int):
    """(nsym, f[256]): the sampled symbols' frequencies summing to 4095 (ESC holds slot 4095)."""
    c = np.ascontiguousarray(counts, np.uint32)
    f = np.zeros(256, np.uint32)
    nsym = lib().orc_normalize_sampled(_p(c), S, _p(f))
    return int(nsym), f


def compress_sampled(dtype: int, values, chunk_bytes: int = 0) -> np.ndarray:
    """A frame with sampled tables (header flag bit 0), exact size."""
    v = _bits(dtype, values)
    cap = max_compressed_size(dtype, v.size, chunk_bytes)
    if cap == 0:
        raise ValueError("invalid chunk_bytes")
    out = np.empty(cap, np.uint8)
    size = ctypes.c_uint64(0)
    st = lib().orc_compress_sampled(dtype, _p(v) if v.size else None, v.size, chunk_bytes, _p(out), cap,
                                    ctypes.byref(size))
    if st != OK:
        raise ValueError("oracle sampled compress failed with status %d" % st)
    return out[: size.value].copy()
