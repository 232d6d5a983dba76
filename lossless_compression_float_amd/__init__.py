"""Python binding of the uzip C ABI (include/uzip.h): lossless bf16/fp32 (and
fp16/fp8) tensor compression on MI355X (gfx950).

The functions named ``uzip_*`` are the C entry points with the same names and
arguments (plain integers and device pointers), marshalled through ctypes.
Every step of the codec runs in the HIP kernels of ``libuzip.so``; this module
only allocates outputs and workspaces through torch (device memory and the
current stream are all torch is used for) and passes pointers.

``compress(t)`` / ``decompress(buf, dtype, n)`` and their batched forms are
convenience wrappers over those calls.  There is no CPU fallback: loading
fails loudly when the library is missing.
"""
from __future__ import annotations

import array
import ctypes
import os

import torch  # loads the HIP runtime the library links against

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libuzip.so")

UZIP_BF16 = 1
UZIP_FP32 = 2
UZIP_FP16 = 3
UZIP_FP8_E4M3 = 4
UZIP_FP8_E5M2 = 5
UZIP_OK = 0
UZIP_ERR_INVALID_ARGUMENT = 1
UZIP_ERR_CAPACITY = 2
UZIP_ERR_CORRUPT_INPUT = 3
UZIP_ERR_DEVICE = 4
UZIP_ERR_UNSUPPORTED = 5
UZIP_ERR_SCRATCH_LIMIT = 6
UZIP_NOALLOC_SCRATCH_BYTES = 64 << 20

UZIP_PLAN_CODED = 0
UZIP_PLAN_RAW = 1
UZIP_PLAN_RAW_SMALL = 2
UZIP_PLAN_RAW_REALIZED = 3


class uzip_policy(ctypes.Structure):
    """The per-call arbitration's cost-model inputs (uzip.h: uzip_policy)."""
    _fields_ = [("link_bytes_per_us", ctypes.c_uint64), ("encode_bytes_per_us", ctypes.c_uint64),
                ("decode_bytes_per_us", ctypes.c_uint64), ("fixed_ns", ctypes.c_uint64),
                ("small_bytes", ctypes.c_uint64), ("exposed_encode_permil", ctypes.c_uint32),
                ("exposed_decode_permil", ctypes.c_uint32), ("min_gain_permil", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


PLAN_FIELDS = ("decision", "sample_values", "predicted_bytes", "raw_ns", "coded_ns")
PLAN_BYTES = 32

EXPORTED = (
    "uzip_max_compressed_size",
    "uzip_workspace_size",
    "uzip_compress",
    "uzip_decompress",
    "uzip_workspace_size_batched",
    "uzip_compress_batched",
    "uzip_decompress_batched",
    "uzip_compress_arbitrated",
    "uzip_compress_batched_arbitrated",
    "uzip_compress_sampled",
    "uzip_compress_batched_sampled",
    "uzip_compress_noalloc",
    "uzip_compress_batched_timed",
    "uzip_decompress_batched_timed",
    "uzip_status_string",
)

_lib = None


class UzipError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, uzip_status_string(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libuzip.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libuzip.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        sz, i32, u64p, vp = ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
        L.uzip_max_compressed_size.restype = sz
        L.uzip_max_compressed_size.argtypes = [i32, sz, sz]
        L.uzip_workspace_size.restype = sz
        L.uzip_workspace_size.argtypes = [i32, sz, sz]
        L.uzip_compress.restype = i32
        L.uzip_compress.argtypes = [i32, vp, sz, sz, vp, sz, u64p, vp, sz, vp]
        L.uzip_compress_sampled.restype = i32
        L.uzip_compress_sampled.argtypes = [i32, vp, sz, sz, vp, sz, u64p, vp, sz, vp]
        L.uzip_decompress.restype = i32
        L.uzip_decompress.argtypes = [vp, sz, i32, sz, vp, vp, vp, sz, vp]
        L.uzip_workspace_size_batched.restype = sz
        L.uzip_workspace_size_batched.argtypes = [i32, sz, vp, sz]
        L.uzip_compress_batched.restype = i32
        L.uzip_compress_batched.argtypes = [i32, sz, vp, vp, sz, vp, vp, u64p, vp, sz, vp]
        L.uzip_compress_batched_sampled.restype = i32
        L.uzip_compress_batched_sampled.argtypes = [i32, sz, vp, vp, sz, vp, vp, u64p, vp, sz, vp]
        L.uzip_decompress_batched.restype = i32
        L.uzip_decompress_batched.argtypes = [i32, sz, vp, vp, vp, vp, vp, vp, sz, vp]
        L.uzip_compress_arbitrated.restype = i32
        L.uzip_compress_arbitrated.argtypes = [i32, vp, sz, sz, ctypes.POINTER(uzip_policy), vp, sz, u64p, vp, vp,
                                               sz, vp]
        L.uzip_compress_batched_arbitrated.restype = i32
        L.uzip_compress_batched_arbitrated.argtypes = [i32, sz, vp, vp, sz, ctypes.POINTER(uzip_policy), vp, vp,
                                                       u64p, vp, vp, sz, vp]
        L.uzip_compress_noalloc.restype = i32
        L.uzip_compress_noalloc.argtypes = [i32, vp, sz, sz, vp, sz, u64p, vp]
        L.uzip_compress_batched_timed.restype = i32
        L.uzip_compress_batched_timed.argtypes = [i32, sz, vp, vp, sz, ctypes.c_uint32, ctypes.POINTER(uzip_policy),
                                                  vp, vp, u64p, vp, vp, sz, vp, vp, vp]
        L.uzip_decompress_batched_timed.restype = i32
        L.uzip_decompress_batched_timed.argtypes = [i32, sz, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.uzip_status_string.restype = ctypes.c_char_p
        L.uzip_status_string.argtypes = [i32]
        _lib = L
    return _lib


# ---- the C entry points, same names and arguments --------------------------
def uzip_max_compressed_size(dtype: int, num_elements: int, chunk_bytes: int = 0) -> int:
    return int(lib().uzip_max_compressed_size(dtype, num_elements, chunk_bytes))


def uzip_workspace_size(dtype: int, num_elements: int, chunk_bytes: int = 0) -> int:
    return int(lib().uzip_workspace_size(dtype, num_elements, chunk_bytes))


def uzip_compress(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size, d_workspace,
                  workspace_bytes, stream) -> int:
    return int(lib().uzip_compress(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size,
                                   d_workspace, workspace_bytes, stream))


def uzip_compress_sampled(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size, d_workspace,
                          workspace_bytes, stream) -> int:
    return int(lib().uzip_compress_sampled(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size,
                                           d_workspace, workspace_bytes, stream))


def uzip_compress_noalloc(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size, stream) -> int:
    return int(lib().uzip_compress_noalloc(dtype, d_in, num_elements, chunk_bytes, d_out, out_capacity, d_out_size,
                                           stream))


def uzip_decompress(d_in, in_bytes, dtype, num_elements, d_out, d_status, d_workspace, workspace_bytes,
                    stream) -> int:
    return int(lib().uzip_decompress(d_in, in_bytes, dtype, num_elements, d_out, d_status, d_workspace,
                                     workspace_bytes, stream))


class _HostArray:
    """A contiguous host array of 64-bit unsigned values (size_t or pointer)
    for the C ABI's h_* arguments; `ptr` stays valid while the object lives."""

    def __init__(self, vals):
        self.buf = array.array("Q", vals)
        self.ptr = self.buf.buffer_info()[0] if len(self.buf) else None


def _sizes(vals):
    return _HostArray(vals)


def _ptrs(vals):
    return _HostArray(vals)


def uzip_workspace_size_batched(dtype: int, num_elements, chunk_bytes: int = 0) -> int:
    arr = _sizes(num_elements)
    return int(lib().uzip_workspace_size_batched(dtype, len(num_elements), arr.ptr, chunk_bytes))


def uzip_compress_batched(dtype, h_in, h_num_elements, chunk_bytes, h_out, h_out_capacity, d_out_sizes, d_workspace,
                          workspace_bytes, stream) -> int:
    a_in, a_n, a_out, a_cap = _ptrs(h_in), _sizes(h_num_elements), _ptrs(h_out), _sizes(h_out_capacity)
    return int(lib().uzip_compress_batched(dtype, len(h_in), a_in.ptr, a_n.ptr, chunk_bytes, a_out.ptr, a_cap.ptr,
                                           d_out_sizes, d_workspace, workspace_bytes, stream))


def uzip_compress_batched_sampled(dtype, h_in, h_num_elements, chunk_bytes, h_out, h_out_capacity, d_out_sizes,
                                  d_workspace, workspace_bytes, stream) -> int:
    a_in, a_n, a_out, a_cap = _ptrs(h_in), _sizes(h_num_elements), _ptrs(h_out), _sizes(h_out_capacity)
    return int(lib().uzip_compress_batched_sampled(dtype, len(h_in), a_in.ptr, a_n.ptr, chunk_bytes, a_out.ptr,
                                                   a_cap.ptr, d_out_sizes, d_workspace, workspace_bytes, stream))


def uzip_decompress_batched(dtype, h_in, h_in_bytes, h_num_elements, h_out, d_status, d_workspace, workspace_bytes,
                            stream) -> int:
    a_in, a_b, a_n, a_out = _ptrs(h_in), _sizes(h_in_bytes), _sizes(h_num_elements), _ptrs(h_out)
    return int(lib().uzip_decompress_batched(dtype, len(h_in), a_in.ptr, a_b.ptr, a_n.ptr, a_out.ptr, d_status,
                                             d_workspace, workspace_bytes, stream))


def uzip_compress_arbitrated(dtype, d_in, num_elements, chunk_bytes, policy, d_out, out_capacity, d_out_size,
                             d_plan, d_workspace, workspace_bytes, stream) -> int:
    pol = ctypes.byref(policy) if policy is not None else None
    return int(lib().uzip_compress_arbitrated(dtype, d_in, num_elements, chunk_bytes, pol, d_out, out_capacity,
                                              d_out_size, d_plan, d_workspace, workspace_bytes, stream))


def uzip_compress_batched_arbitrated(dtype, h_in, h_num_elements, chunk_bytes, policy, h_out, h_out_capacity,
                                     d_out_sizes, d_plans, d_workspace, workspace_bytes, stream) -> int:
    a_in, a_n, a_out, a_cap = _ptrs(h_in), _sizes(h_num_elements), _ptrs(h_out), _sizes(h_out_capacity)
    pol = ctypes.byref(policy) if policy is not None else None
    return int(lib().uzip_compress_batched_arbitrated(dtype, len(h_in), a_in.ptr, a_n.ptr, chunk_bytes, pol,
                                                      a_out.ptr, a_cap.ptr, d_out_sizes, d_plans, d_workspace,
                                                      workspace_bytes, stream))


def uzip_compress_batched_timed(dtype, h_in, h_num_elements, chunk_bytes, sampled, policy, h_out, h_out_capacity,
                                d_out_sizes, d_plans, d_workspace, workspace_bytes, stream, main_start,
                                main_stop) -> int:
    a_in, a_n, a_out, a_cap = _ptrs(h_in), _sizes(h_num_elements), _ptrs(h_out), _sizes(h_out_capacity)
    pol = ctypes.byref(policy) if policy is not None else None
    return int(lib().uzip_compress_batched_timed(dtype, len(h_in), a_in.ptr, a_n.ptr, chunk_bytes, sampled, pol,
                                                 a_out.ptr, a_cap.ptr, d_out_sizes, d_plans, d_workspace,
                                                 workspace_bytes, stream, main_start, main_stop))


def uzip_decompress_batched_timed(dtype, h_in, h_in_bytes, h_num_elements, h_out, d_status, d_workspace,
                                  workspace_bytes, stream, main_start, main_stop) -> int:
    a_in, a_b, a_n, a_out = _ptrs(h_in), _sizes(h_in_bytes), _sizes(h_num_elements), _ptrs(h_out)
    return int(lib().uzip_decompress_batched_timed(dtype, len(h_in), a_in.ptr, a_b.ptr, a_n.ptr, a_out.ptr, d_status,
                                                   d_workspace, workspace_bytes, stream, main_start, main_stop))


def uzip_status_string(status: int) -> str:
    return lib().uzip_status_string(status).decode()


# ---- torch-level convenience wrappers ---------------------------------------
_CODES = {torch.bfloat16: UZIP_BF16, torch.float32: UZIP_FP32, torch.float16: UZIP_FP16,
          torch.float8_e4m3fn: UZIP_FP8_E4M3, torch.float8_e5m2: UZIP_FP8_E5M2}


def dtype_code(t: torch.dtype) -> int:
    if t in _CODES:
        return _CODES[t]
    raise TypeError("uzip compresses bfloat16, float16, float32, float8_e4m3fn or float8_e5m2 tensors, not %s" % t)


def torch_dtype(code: int) -> torch.dtype:
    return {v: k for k, v in _CODES.items()}[code]


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _keep_for(stream, *tensors):
    """Tensors allocated here on the current stream but used by kernels on
    another `stream`: tell torch's caching allocator so (record_stream), or
    it could hand their memory to new work on the current stream while those
    kernels still read or write it.  Nothing to do when `stream` is None or
    is the current stream."""
    if stream is None:
        return
    if stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(stream)
        else:
            for u in t:
                u.record_stream(stream)


def _check(st: int, what: str):
    if st != UZIP_OK:
        raise UzipError(st, what)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def compress(t: torch.Tensor, chunk_bytes: int = 0, out: torch.Tensor | None = None,
             ws: torch.Tensor | None = None, out_size: torch.Tensor | None = None, stream=None,
             sampled: bool = False):
    """Compress a contiguous bf16/fp32/fp16/fp8 device tensor.  Returns (buffer, size)
    where `buffer` has capacity uzip_max_compressed_size and `size` is a
    one-element int64 device tensor holding the exact compressed size.
    sampled=True builds each chunk's table from a sample (uzip_compress_sampled)."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("compress needs a contiguous device tensor")
    code = dtype_code(t.dtype)
    n = t.numel()
    cap = uzip_max_compressed_size(code, n, chunk_bytes)
    if cap == 0:
        raise ValueError("invalid chunk_bytes %d, or %d values beyond the limits of one call" % (chunk_bytes, n))
    if out is None:
        out = torch.empty(cap, dtype=torch.uint8, device=t.device)
    if out_size is None:
        out_size = torch.empty(1, dtype=torch.int64, device=t.device)
    wsz = uzip_workspace_size(code, n, chunk_bytes)
    if ws is None:
        ws = workspace(wsz, t.device)
    fn = uzip_compress_sampled if sampled else uzip_compress
    st = fn(code, t.data_ptr() if n else None, n, chunk_bytes, out.data_ptr(), out.numel(),
            out_size.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, fn.__name__)
    _keep_for(stream, out, out_size, ws)
    return out, out_size


def decompress(buf: torch.Tensor, dtype: torch.dtype, n: int, in_bytes: int | None = None,
               out: torch.Tensor | None = None, status: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, stream=None):
    """Decompress into a new (or given) tensor of n values.  Returns
    (values, status) where status is a one-element int32 device tensor
    (0 = valid, 3 = corrupt input)."""
    code = dtype_code(dtype)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=buf.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=buf.device)
    if ws is None:
        ws = workspace(uzip_workspace_size(code, 0, 0), buf.device)
    nb = buf.numel() if in_bytes is None else in_bytes
    st = uzip_decompress(buf.data_ptr() if nb else None, nb, code, n, out.data_ptr() if n else None,
                         status.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, "uzip_decompress")
    _keep_for(stream, out, status, ws)
    return out, status


def compress_batched(tensors, chunk_bytes: int = 0, outs=None, ws=None, out_sizes=None, stream=None,
                     sampled: bool = False):
    """Compress a list of same-dtype contiguous device tensors in one call.
    Returns (buffers, sizes[int64 tensor of len(tensors)]).  sampled=True:
    uzip_compress_batched_sampled."""
    code = dtype_code(tensors[0].dtype)
    dev = tensors[0].device
    ns = [t.numel() for t in tensors]
    if outs is None:
        outs = [torch.empty(uzip_max_compressed_size(code, n, chunk_bytes), dtype=torch.uint8, device=dev) for n in ns]
    if out_sizes is None:
        out_sizes = torch.empty(len(tensors), dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(uzip_workspace_size_batched(code, ns, chunk_bytes), dev)
    fn = uzip_compress_batched_sampled if sampled else uzip_compress_batched
    st = fn(code, [t.data_ptr() if t.numel() else 0 for t in tensors], ns, chunk_bytes,
            [o.data_ptr() for o in outs], [o.numel() for o in outs], out_sizes.data_ptr(),
            ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, fn.__name__)
    _keep_for(stream, outs, out_sizes, ws)
    return outs, out_sizes


def decompress_batched(bufs, dtype: torch.dtype, ns, in_bytes=None, outs=None, status=None, ws=None, stream=None):
    code = dtype_code(dtype)
    dev = bufs[0].device
    if outs is None:
        outs = [torch.empty(n, dtype=dtype, device=dev) for n in ns]
    if status is None:
        status = torch.empty(len(bufs), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(uzip_workspace_size_batched(code, list(ns), 0), dev)
    nbs = [b.numel() for b in bufs] if in_bytes is None else list(in_bytes)
    st = uzip_decompress_batched(code, [b.data_ptr() for b in bufs], nbs, list(ns),
                                 [o.data_ptr() if o.numel() else 0 for o in outs], status.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream(stream))
    _check(st, "uzip_decompress_batched")
    _keep_for(stream, outs, status, ws)
    return outs, status


def policy(**fields) -> uzip_policy:
    """A uzip_policy from keyword fields (unset fields are 0)."""
    return uzip_policy(**fields)


def plans_as_dicts(plans: torch.Tensor) -> list:
    """Device plan records (int64 tensor of 4 words per buffer) as dicts."""
    w = plans.view(-1, 4).cpu().tolist()
    return [{"decision": r[0] & 0xFFFFFFFF, "sample_values": (r[0] >> 32) & 0xFFFFFFFF, "predicted_bytes": r[1],
             "raw_ns": r[2], "coded_ns": r[3]} for r in w]


def compress_arbitrated(t: torch.Tensor, pol: uzip_policy, chunk_bytes: int = 0, out=None, ws=None, out_size=None,
                        plan=None, stream=None):
    """Arbitrated compress of one tensor.  Returns (buffer, size, plan) where
    plan is an int64 device tensor of 4 words (see plans_as_dicts)."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("compress needs a contiguous device tensor")
    code = dtype_code(t.dtype)
    n = t.numel()
    cap = uzip_max_compressed_size(code, n, chunk_bytes)
    if cap == 0:
        raise ValueError("invalid chunk_bytes %d, or %d values beyond the limits of one call" % (chunk_bytes, n))
    if out is None:
        out = torch.empty(cap, dtype=torch.uint8, device=t.device)
    if out_size is None:
        out_size = torch.empty(1, dtype=torch.int64, device=t.device)
    if plan is None:
        plan = torch.empty(4, dtype=torch.int64, device=t.device)
    if ws is None:
        ws = workspace(uzip_workspace_size(code, n, chunk_bytes), t.device)
    st = uzip_compress_arbitrated(code, t.data_ptr() if n else None, n, chunk_bytes, pol, out.data_ptr(), out.numel(),
                                  out_size.data_ptr(), plan.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, "uzip_compress_arbitrated")
    _keep_for(stream, out, out_size, plan, ws)
    return out, out_size, plan


def compress_batched_arbitrated(tensors, pol: uzip_policy, chunk_bytes: int = 0, outs=None, ws=None, out_sizes=None,
                                plans=None, stream=None):
    """Arbitrated compress of a list of tensors.  Returns (buffers, sizes, plans[int64, 4 words per buffer])."""
    code = dtype_code(tensors[0].dtype)
    dev = tensors[0].device
    ns = [t.numel() for t in tensors]
    if outs is None:
        outs = [torch.empty(uzip_max_compressed_size(code, n, chunk_bytes), dtype=torch.uint8, device=dev) for n in ns]
    if out_sizes is None:
        out_sizes = torch.empty(len(tensors), dtype=torch.int64, device=dev)
    if plans is None:
        plans = torch.empty(4 * len(tensors), dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(uzip_workspace_size_batched(code, ns, chunk_bytes), dev)
    st = uzip_compress_batched_arbitrated(code, [t.data_ptr() if t.numel() else 0 for t in tensors], ns, chunk_bytes,
                                          pol, [o.data_ptr() for o in outs], [o.numel() for o in outs],
                                          out_sizes.data_ptr(), plans.data_ptr(), ws.data_ptr(), ws.numel(),
                                          _stream(stream))
    _check(st, "uzip_compress_batched_arbitrated")
    _keep_for(stream, outs, out_sizes, plans, ws)
    return outs, out_sizes, plans
