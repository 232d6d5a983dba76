"""The C ABI without a GPU: the library loads, exports every entry point that
include/uzip.h declares, its host-only size functions agree with the layout
the oracle writes, and argument errors are returned before anything is
launched (no call here reaches the device)."""
import os
import re
import subprocess

import numpy as np
import pytest

import lossless_compression_float_amd as uz
import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uzip.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uzip_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(uz.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.check_output(["nm", "-D", "--defined-only", uz.LIB_PATH], text=True)
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(uz.lib(), name)


def test_library_has_gfx950_code_object():
    # the offload bundle of our own build names its target triple
    assert b"amdgcn-amd-amdhsa--gfx950" in open(uz.LIB_PATH, "rb").read()


@pytest.mark.parametrize("dtype", [uz.UZIP_BF16, uz.UZIP_FP32, uz.UZIP_FP16, uz.UZIP_FP8_E4M3, uz.UZIP_FP8_E5M2])
@pytest.mark.parametrize("chunk_bytes", [0, 4096, 65536, 262144])
def test_max_compressed_size_matches_oracle(dtype, chunk_bytes):
    for n in [0, 1, 31, 32, 33, 1000, 32767, 32768, 32769, 65536 * 3 + 17, 268_435_456, 8_030_257_152]:
        assert uz.uzip_max_compressed_size(dtype, n, chunk_bytes) == orc.max_compressed_size(dtype, n, chunk_bytes)


def test_size_functions_reject_invalid_arguments():
    assert uz.uzip_max_compressed_size(0, 100, 0) == 0 and uz.uzip_max_compressed_size(6, 100, 0) == 0
    assert uz.uzip_max_compressed_size(uz.UZIP_BF16, 100, 100) == 0
    assert uz.uzip_max_compressed_size(uz.UZIP_BF16, 100, (1 << 21) + 64) == 0
    assert uz.uzip_max_compressed_size(uz.UZIP_FP8_E4M3, 100, 1 << 20) > 0  # 2^20 values per chunk at most
    assert uz.uzip_max_compressed_size(uz.UZIP_FP8_E4M3, 100, (1 << 20) + 32) == 0
    assert uz.uzip_workspace_size(uz.UZIP_FP32, 100, 8) == 0
    assert uz.uzip_workspace_size(uz.UZIP_BF16, 0, 0) > 0
    assert uz.uzip_workspace_size_batched(uz.UZIP_BF16, [], 0) == 0


def test_workspace_grows_with_chunks():
    a = uz.uzip_workspace_size(uz.UZIP_BF16, 1 << 20, 0)
    b = uz.uzip_workspace_size(uz.UZIP_BF16, 1 << 22, 0)
    assert b > a >= 32 * (32768 + 16)
    assert uz.uzip_workspace_size_batched(uz.UZIP_BF16, [1 << 20, 1 << 22], 0) >= a + b - 4096


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("fn", [uz.uzip_compress, uz.uzip_compress_sampled])
def test_compress_argument_errors_return_synchronously(fn):
    n = 1000
    cap = uz.uzip_max_compressed_size(uz.UZIP_BF16, n)
    ws = uz.uzip_workspace_size(uz.UZIP_BF16, n)
    call = lambda **kw: fn(**{**dict(dtype=uz.UZIP_BF16, d_in=FAKE, num_elements=n, chunk_bytes=0,
                                     d_out=FAKE, out_capacity=cap, d_out_size=FAKE,
                                     d_workspace=FAKE, workspace_bytes=ws - 1, stream=None), **kw})
    assert call(dtype=7) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(chunk_bytes=100) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_in=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_in=FAKE + 8) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_out=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_out_size=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(out_capacity=cap - 1) == uz.UZIP_ERR_CAPACITY
    assert call() == uz.UZIP_ERR_INVALID_ARGUMENT  # workspace one byte short
    assert call(d_workspace=None, workspace_bytes=ws) == uz.UZIP_ERR_INVALID_ARGUMENT


def test_decompress_argument_errors_return_synchronously():
    ws = uz.uzip_workspace_size(uz.UZIP_BF16, 0)
    call = lambda **kw: uz.uzip_decompress(**{**dict(d_in=FAKE, in_bytes=1000, dtype=uz.UZIP_BF16, num_elements=10,
                                                       d_out=FAKE, d_status=FAKE, d_workspace=FAKE,
                                                       workspace_bytes=ws - 1, stream=None), **kw})
    assert call(dtype=0) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_in=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_out=FAKE + 4) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_status=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call() == uz.UZIP_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("fn", [uz.uzip_compress_batched, uz.uzip_compress_batched_sampled])
def test_batched_argument_errors_return_synchronously(fn):
    ns = [100, 0, 5000]
    caps = [uz.uzip_max_compressed_size(uz.UZIP_BF16, n) for n in ns]
    ws = uz.uzip_workspace_size_batched(uz.UZIP_BF16, ns)
    base = dict(dtype=uz.UZIP_BF16, h_in=[FAKE, 0, FAKE], h_num_elements=ns, chunk_bytes=0, h_out=[FAKE] * 3,
                h_out_capacity=caps, d_out_sizes=FAKE, d_workspace=FAKE, workspace_bytes=ws - 1, stream=None)
    call = lambda **kw: fn(**{**base, **kw})
    assert call(h_in=[0, 0, FAKE]) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(h_out_capacity=[caps[0], caps[1], caps[2] - 16]) == uz.UZIP_ERR_CAPACITY
    assert call() == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_out_sizes=FAKE + 4) == uz.UZIP_ERR_INVALID_ARGUMENT


PAIR_LIMIT = (1 << 25) - 8  # chunk pairs of one compress call (k_compact's grid: 1024 threads per 8 pairs)


def test_counts_beyond_the_call_limits_are_rejected_on_the_host():
    """A buffer of 2^44 values or more, or more chunk pairs in one call than
    the launch grids can cover, is an argument error: the size functions
    return 0 and the compress calls return at once, also for counts whose
    byte sizes would not fit 64 bits (a size computed with wrap-around could
    otherwise pass the capacity and workspace checks)."""
    bf, ce = uz.UZIP_BF16, 32768
    n_max = 2 * ce * PAIR_LIMIT  # the largest bf16 buffer at the default chunk
    assert uz.uzip_max_compressed_size(bf, n_max, 0) == orc.max_compressed_size(bf, n_max, 0)
    assert uz.uzip_workspace_size(bf, n_max, 0) > 0
    assert uz.uzip_max_compressed_size(bf, n_max + 1, 0) == 0 and uz.uzip_workspace_size(bf, n_max + 1, 0) == 0
    # at 2^20-value chunks the value limit comes first
    assert uz.uzip_max_compressed_size(bf, (1 << 44) - 1, 1 << 21) > 0
    for n in [1 << 44, 1 << 63, (1 << 64) - 1]:
        for dt in [bf, uz.UZIP_FP32, uz.UZIP_FP8_E4M3]:
            assert uz.uzip_max_compressed_size(dt, n, 0) == 0 and uz.uzip_workspace_size(dt, n, 0) == 0
    assert uz.uzip_workspace_size_batched(bf, [2 * ce * (PAIR_LIMIT - 1), 2 * ce], 0) > 0
    assert uz.uzip_workspace_size_batched(bf, [2 * ce * (PAIR_LIMIT - 1), 2 * ce + 1], 0) == 0
    assert uz.uzip_workspace_size_batched(bf, [100, 1 << 44], 0) == 0
    huge = (1 << 64) - 1
    for n in [n_max + 1, 1 << 44, 1 << 63, huge]:
        for fn in (uz.uzip_compress, uz.uzip_compress_sampled):
            assert fn(bf, FAKE, n, 0, FAKE, huge, FAKE, FAKE, huge, None) == uz.UZIP_ERR_INVALID_ARGUMENT, (fn, n)
        # (returned before the scratch's device address is looked up)
        assert uz.uzip_compress_noalloc(bf, FAKE, n, 0, FAKE, huge, FAKE, None) == uz.UZIP_ERR_INVALID_ARGUMENT
        assert uz.uzip_compress_arbitrated(bf, FAKE, n, 0, _policy(), FAKE, huge, FAKE, FAKE, FAKE, huge,
                                           None) == uz.UZIP_ERR_INVALID_ARGUMENT
    for ns in ([100, 1 << 44], [2 * ce * (PAIR_LIMIT - 1), 2 * ce + 1], [huge, 5]):
        kw = dict(h_in=[FAKE] * len(ns), h_num_elements=ns, chunk_bytes=0, h_out=[FAKE] * len(ns),
                  h_out_capacity=[huge] * len(ns), d_out_sizes=FAKE, d_workspace=FAKE, workspace_bytes=huge,
                  stream=None)
        assert uz.uzip_compress_batched(bf, **kw) == uz.UZIP_ERR_INVALID_ARGUMENT, ns
        assert uz.uzip_compress_batched_sampled(bf, **kw) == uz.UZIP_ERR_INVALID_ARGUMENT, ns
        assert uz.uzip_compress_batched_arbitrated(bf, policy=_policy(), d_plans=FAKE,
                                                   **kw) == uz.UZIP_ERR_INVALID_ARGUMENT, ns


def test_arbitrated_batch_of_too_many_buffers_is_rejected_before_its_arrays_are_read():
    """k_plan runs a 256-thread workgroup per buffer: an arbitrated batched call
    takes at most 2^24 - 1 buffers.  The count is checked before the host
    arrays (here one entry long) are read."""
    import ctypes
    one = uz._sizes([100])
    pol = _policy()
    st = uz.lib().uzip_compress_batched_arbitrated(uz.UZIP_BF16, 1 << 24, one.ptr, one.ptr, 0, ctypes.byref(pol),
                                                   one.ptr, one.ptr, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == uz.UZIP_ERR_INVALID_ARGUMENT


def test_status_strings():
    for s in range(6):
        assert uz.uzip_status_string(s)
    assert "corrupt" in uz.uzip_status_string(uz.UZIP_ERR_CORRUPT_INPUT)


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "lossless_compression_float_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def _policy(**kw):
    base = dict(link_bytes_per_us=25000, encode_bytes_per_us=10**6, decode_bytes_per_us=10**6)
    base.update(kw)
    return uz.policy(**base)


def test_arbitration_structs_match_the_header():
    import ctypes
    assert ctypes.sizeof(uz.uzip_policy) == 56 and uz.PLAN_BYTES == 32
    assert ctypes.sizeof(uz.uzip_policy) == ctypes.sizeof(orc.Policy)
    assert ctypes.sizeof(orc.Plan) == uz.PLAN_BYTES


def test_arbitrated_argument_errors_return_synchronously():
    n = 1000
    cap = uz.uzip_max_compressed_size(uz.UZIP_BF16, n)
    ws = uz.uzip_workspace_size(uz.UZIP_BF16, n)
    call = lambda **kw: uz.uzip_compress_arbitrated(**{**dict(dtype=uz.UZIP_BF16, d_in=FAKE, num_elements=n,
                                                              chunk_bytes=0, policy=_policy(), d_out=FAKE,
                                                              out_capacity=cap, d_out_size=FAKE, d_plan=FAKE,
                                                              d_workspace=FAKE, workspace_bytes=ws - 1,
                                                              stream=None), **kw})
    assert call(policy=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    for bad in [dict(link_bytes_per_us=0), dict(encode_bytes_per_us=0), dict(decode_bytes_per_us=0),
                dict(exposed_encode_permil=1001), dict(exposed_decode_permil=1001), dict(min_gain_permil=1001),
                dict(reserved=7)]:
        assert call(policy=_policy(**bad)) == uz.UZIP_ERR_INVALID_ARGUMENT, bad
    assert call(d_plan=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(d_plan=FAKE + 4) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(num_elements=1 << 44, out_capacity=1 << 62) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert call(out_capacity=cap - 1, workspace_bytes=ws) == uz.UZIP_ERR_CAPACITY
    assert call() == uz.UZIP_ERR_INVALID_ARGUMENT  # workspace one byte short
    ns = [100, 0]
    bcall = lambda **kw: uz.uzip_compress_batched_arbitrated(**{**dict(
        dtype=uz.UZIP_BF16, h_in=[FAKE, 0], h_num_elements=ns, chunk_bytes=0, policy=_policy(), h_out=[FAKE, FAKE],
        h_out_capacity=[uz.uzip_max_compressed_size(uz.UZIP_BF16, k) for k in ns], d_out_sizes=FAKE, d_plans=FAKE,
        d_workspace=FAKE, workspace_bytes=0, stream=None), **kw})
    assert bcall(policy=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert bcall(policy=_policy(min_gain_permil=2000)) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert bcall(d_plans=None) == uz.UZIP_ERR_INVALID_ARGUMENT
    assert bcall() == uz.UZIP_ERR_INVALID_ARGUMENT  # no workspace


def test_outputs_allocated_for_another_stream_are_recorded_on_it(monkeypatch):
    """Tensors the wrappers allocate on the current stream but hand to kernels
    on another stream are recorded on that stream (record_stream), so torch's
    caching allocator cannot reuse their memory before those kernels finish;
    nothing is recorded when the stream is the current one or None."""
    import torch

    class FakeStream:
        device = "cuda:0"

    class FakeTensor(torch.Tensor):
        pass

    current, side = FakeStream(), FakeStream()
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: current)
    seen = []

    class T:
        def __init__(self, name):
            self.name = name

        def record_stream(self, s):
            seen.append((self.name, s))

    monkeypatch.setattr(torch, "Tensor", T)
    uz._keep_for(None, T("a"))
    uz._keep_for(current, T("b"))
    assert seen == []
    uz._keep_for(side, T("out"), [T("o1"), T("o2")], T("ws"))
    assert seen == [("out", side), ("o1", side), ("o2", side), ("ws", side)]
