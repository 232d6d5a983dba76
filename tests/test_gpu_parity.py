"""GPU parity: the HIP path, called through the C ABI, against the oracle.

Tolerance 0 everywhere: the compressed bytes must equal the oracle's byte for
byte, and decompression must restore every bit pattern (NaN payloads,
infinities, denormals, signed zeros included).  These cases are small enough
to compare whole buffers; the benchmark's full-size workloads are in
test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads
from uzip_testlib import corruptions, parse_buffer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


_VIEW = {np.uint8: torch.uint8, np.uint16: torch.int16, np.uint32: torch.int32}
_ORC = {torch.bfloat16: orc.BF16, torch.float32: orc.FP32, torch.float16: orc.FP16,
        torch.float8_e4m3fn: orc.FP8_E4M3, torch.float8_e5m2: orc.FP8_E5M2}


def _default_dtype(bits: np.ndarray) -> torch.dtype:
    return {np.uint16: torch.bfloat16, np.uint32: torch.float32}[bits.dtype.type]


def _bits_tensor(bits: np.ndarray, tdtype: torch.dtype = None) -> torch.Tensor:
    tdtype = tdtype or _default_dtype(bits)
    raw = torch.from_numpy(bits.view(np.int16 if bits.dtype == np.uint16 else
                                     np.int32 if bits.dtype == np.uint32 else np.uint8).copy())
    return raw.view(tdtype).to(DEV)


def _code(bits, tdtype: torch.dtype = None):
    return _ORC[tdtype or _default_dtype(bits)]


def _int_view(t: torch.Tensor) -> torch.Tensor:
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def gpu_compress(t: torch.Tensor, chunk_bytes: int = 0) -> np.ndarray:
    buf, size = uz.compress(t, chunk_bytes)
    torch.cuda.synchronize()
    n = int(size.item())
    assert n <= buf.numel()
    return buf[:n].cpu().numpy()


def gpu_decompress(buf: np.ndarray, dtype: torch.dtype, n: int, in_bytes=None):
    b = torch.from_numpy(buf.copy()).to(DEV) if buf.size else torch.empty(16, dtype=torch.uint8, device=DEV)
    out, st = uz.decompress(b, dtype, n, in_bytes=buf.size if in_bytes is None else in_bytes)
    torch.cuda.synchronize()
    return out, int(st.item())


def check_parity(bits: np.ndarray, chunk_bytes: int = 0, tdtype: torch.dtype = None):
    """GPU bytes == oracle bytes, and both decode to the input on the GPU.
    `bits` is uint16 (bf16 unless `tdtype` says float16), uint32 (fp32) or
    uint8 (one of the float8 formats, named by `tdtype`)."""
    t = _bits_tensor(bits, tdtype)
    got = gpu_compress(t, chunk_bytes)
    want = orc.compress(_code(bits, tdtype), bits, chunk_bytes)
    if not np.array_equal(got, want):
        hint = "sizes %d vs %d" % (got.size, want.size)
        if got.size == want.size:
            hint += ", first difference at byte %d" % int(np.nonzero(got != want)[0][0])
        pytest.fail("compressed bytes differ from the oracle: " + hint)
    out, st = gpu_decompress(got, t.dtype, bits.size)
    assert st == 0
    assert torch.equal(_int_view(out), _int_view(t))
    return got


def test_pr1_bytes_identical_and_roundtrip():
    bits = workloads.bits_numpy(workloads.pr1())
    got = check_parity(bits)
    hdr, idx, recs = parse_buffer(got)
    assert hdr["C"] == 32 and all(r["mode"] == 0 for r in recs)


@pytest.mark.parametrize("n", [1, 7, 31, 32, 33, 100, 1000, 32767, 32768, 32768 + 5, 65536 * 2 + 31, 300_001])
def test_bf16_ragged_sizes(n):
    bits = workloads.bits_numpy(workloads.gradient_bucket(n, seed=n, special_frac=0.01))
    check_parity(bits)


@pytest.mark.parametrize("n", [1, 3, 33, 1000, 65535, 65536, 65536 * 2 + 7, 400_003])
def test_fp32_ragged_sizes(n):
    bits = workloads.bits_numpy(workloads.fp32_gradients(n, seed=n))
    check_parity(bits)


@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
def test_empty_buffer(dtype):
    bits = np.zeros(0, dtype)
    got = gpu_compress(_bits_tensor(np.zeros(1, dtype))[:0])
    assert np.array_equal(got, orc.compress(_code(bits), bits))
    out, st = gpu_decompress(got, torch.bfloat16 if dtype == np.uint16 else torch.float32, 0)
    assert st == 0 and out.numel() == 0


def test_every_bf16_bit_pattern():
    check_parity(np.arange(65536, dtype=np.uint32).astype(np.uint16))


def test_fp32_special_classes_and_all_exponents():
    rng = np.random.default_rng(2)
    exps = np.repeat(np.arange(256, dtype=np.uint32), 300)
    v = (rng.integers(0, 2, exps.size, dtype=np.uint32) << 31) | (exps << 23) | rng.integers(0, 1 << 23, exps.size,
                                                                                               dtype=np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001, 1, 0x807FFFFF],
                       np.uint32)
    check_parity(np.concatenate([special, v, special]))


@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
def test_random_bits_go_raw(dtype):
    n = 3 * (32768 if dtype == np.uint16 else 65536) + 777
    bits = np.random.default_rng(3).integers(0, np.iinfo(dtype).max, n, dtype=np.uint64).astype(dtype)
    got = check_parity(bits)
    assert got.size == orc.max_compressed_size(_code(bits), n)


@pytest.mark.parametrize("n", [160, 161, 176, 177, 1000, 40000])
def test_single_exponent_chunks(n):
    check_parity(np.full(n, (130 << 7) | 3, np.uint16))


def test_all_256_exponents_in_one_chunk():
    rng = np.random.default_rng(1)
    e = np.concatenate([np.arange(256), rng.integers(0, 256, 30000)]).astype(np.uint16)
    check_parity(((rng.integers(0, 2, e.size) << 15) | (e << 7) | rng.integers(0, 128, e.size)).astype(np.uint16))


def test_one_dominant_exponent_plus_rare_singletons():
    rng = np.random.default_rng(4)
    e = np.full(32768, 120, np.uint16)
    e[rng.choice(32768, 255, replace=False)] = np.arange(256)[np.arange(256) != 120]
    check_parity(((e << 7) | rng.integers(0, 256, e.size).astype(np.uint16) & 0x807F).astype(np.uint16))


@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
@pytest.mark.parametrize("tail", [8, 16])
def test_burst_of_rare_exponents(dtype, tail):
    """One exponent for most of each chunk, then a run of the 255 others drawn
    uniformly: the others get f = 1 or 2, so that run costs 11-12 bits per
    value, more than 21 renormalisation words per step for a half-wave.  A
    lane of the decoder then takes new words twice within three steps, which
    the steady data of the other tests never does (the decoder's refill path
    for that case)."""
    rng = np.random.default_rng(11 + tail)
    ce = 32768 if dtype == np.uint16 else 65536
    n = 3 * ce + 1000
    e = np.full(n, 127, dtype=np.uint32)
    others = np.array([s for s in range(256) if s != 127], dtype=np.uint32)
    for c0 in range(0, n, ce):
        m = min(ce, n - c0)
        k = m // tail
        e[c0 + m - k: c0 + m] = rng.choice(others, k)
    if dtype == np.uint16:
        bits = (e << 7) | (rng.integers(0, 2, n, dtype=np.uint32) << 15) | rng.integers(0, 128, n, dtype=np.uint32)
    else:
        bits = (e << 23) | (rng.integers(0, 2, n, dtype=np.uint32) << 31) | rng.integers(0, 1 << 23, n, dtype=np.uint32)
    bits = bits.astype(dtype)
    _, _, recs = parse_buffer(orc.compress(_code(bits), bits))
    assert all(r["mode"] == 0 for r in recs)  # every chunk is coded
    check_parity(bits)


@pytest.mark.parametrize("dtype,chunk_bytes", [(np.uint16, 64), (np.uint16, 2048), (np.uint16, 131072),
                                               (np.uint16, 1 << 21), (np.uint32, 128), (np.uint32, 65536),
                                               (np.uint32, 1 << 22)])
def test_chunk_sizes(dtype, chunk_bytes):
    n = 1_200_001
    if dtype == np.uint16:
        bits = workloads.bits_numpy(workloads.gradient_bucket(n, seed=5, special_frac=1e-3))
    else:
        bits = workloads.bits_numpy(workloads.fp32_gradients(n, seed=5))
    check_parity(bits, chunk_bytes)


def test_decodes_oracle_buffers():
    bits = workloads.bits_numpy(workloads.gradient_bucket(500_000, seed=8, special_frac=1e-3))
    buf = orc.compress(orc.BF16, bits)
    out, st = gpu_decompress(buf, torch.bfloat16, bits.size)
    assert st == 0
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), bits)


def test_corrupt_buffers_are_reported():
    bits = workloads.bits_numpy(workloads.pr1())[:100_000]
    buf = orc.compress(orc.BF16, bits)
    out, st = gpu_decompress(buf, torch.bfloat16, bits.size)
    assert st == 0
    for name, bad in corruptions(buf):
        _, st = gpu_decompress(bad, torch.bfloat16, bits.size)
        assert st == uz.UZIP_ERR_CORRUPT_INPUT, name
    _, st = gpu_decompress(buf, torch.float32, bits.size // 2)
    assert st == uz.UZIP_ERR_CORRUPT_INPUT
    _, st = gpu_decompress(buf, torch.bfloat16, bits.size, in_bytes=40)
    assert st == uz.UZIP_ERR_CORRUPT_INPUT


def test_batched_matches_single_and_oracle():
    sizes = [0, 1, 5000, 32768, 100_000, 0, 33, 70_000]
    tensors = [workloads.gradient_bucket(n, seed=10 + i, special_frac=1e-3) if n else
               torch.empty(0, dtype=torch.bfloat16) for i, n in enumerate(sizes)]
    dev = [t.to(DEV) for t in tensors]
    outs, out_sizes = uz.compress_batched(dev)
    torch.cuda.synchronize()
    got_sizes = out_sizes.cpu().tolist()
    for t, o, s in zip(tensors, outs, got_sizes):
        bits = workloads.bits_numpy(t)
        assert np.array_equal(o[:s].cpu().numpy(), orc.compress(orc.BF16, bits))
    vals, status = uz.decompress_batched([o[:s] for o, s in zip(outs, got_sizes)], torch.bfloat16, sizes)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * len(sizes)
    for t, v in zip(dev, vals):
        assert torch.equal(t.view(torch.int16), v.view(torch.int16))


def test_batched_fp32_and_corrupt_member():
    sizes = [70_000, 131_072, 3]
    tensors = [workloads.fp32_gradients(n, seed=20 + i).to(DEV) for i, n in enumerate(sizes)]
    outs, out_sizes = uz.compress_batched(tensors)
    torch.cuda.synchronize()
    got = [o[:s] for o, s in zip(outs, out_sizes.cpu().tolist())]
    for t, g in zip(tensors, got):
        assert np.array_equal(g.cpu().numpy(), orc.compress(orc.FP32, workloads.bits_numpy(t)))
    bad = got[1].clone()
    bad[0] ^= 1  # magic
    vals, status = uz.decompress_batched([got[0], bad, got[2]], torch.float32, sizes)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, uz.UZIP_ERR_CORRUPT_INPUT, 0]
    assert torch.equal(vals[0].view(torch.int32), tensors[0].view(torch.int32))
    assert torch.equal(vals[2].view(torch.int32), tensors[2].view(torch.int32))


@pytest.mark.parametrize("chunk_bytes", [64, 256])
def test_batched_buffers_spanning_many_offset_tiles(chunk_bytes):
    # small chunks give buffers of hundreds to thousands of records, so the
    # record offsets of each buffer span many 64-pair tiles of the scan
    sizes = [10_000, 0, 50_001, 8_192, 300_000, 65]
    tensors = [workloads.gradient_bucket(n, seed=30 + i, special_frac=1e-3).to(DEV) if n else
               torch.empty(0, dtype=torch.bfloat16, device=DEV) for i, n in enumerate(sizes)]
    outs, out_sizes = uz.compress_batched(tensors, chunk_bytes=chunk_bytes)
    torch.cuda.synchronize()
    got = [o[:s] for o, s in zip(outs, out_sizes.cpu().tolist())]
    for t, g in zip(tensors, got):
        want = orc.compress(orc.BF16, workloads.bits_numpy(t), chunk_bytes)
        assert np.array_equal(g.cpu().numpy(), want)
    vals, status = uz.decompress_batched(got, torch.bfloat16, sizes)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * len(sizes)
    for t, v in zip(tensors, vals):
        assert torch.equal(t.view(torch.int16), v.view(torch.int16))


def test_header_flags():
    """Flag bit 0 (tables from samples, record mode 2) is a frame the decoder
    reads like the oracle; any other flag is corrupt."""
    bits = workloads.bits_numpy(workloads.gradient_bucket(100_000, seed=13, special_frac=1e-3))
    sampled = orc.compress_sampled(orc.BF16, bits)
    assert orc.decompress(sampled, orc.BF16, bits.size)[0] == orc.OK
    out, st = gpu_decompress(sampled, torch.bfloat16, bits.size)
    assert st == 0 and np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), bits)
    full = orc.compress(orc.BF16, bits)
    bad = full.copy()
    bad[10] = 2
    _, st = gpu_decompress(bad, torch.bfloat16, bits.size)
    assert st == uz.UZIP_ERR_CORRUPT_INPUT
    out, st = gpu_decompress(full, torch.bfloat16, bits.size)
    assert st == 0 and np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), bits)


def test_calls_on_a_side_stream():
    """Compress and decompress enqueued on a non-current stream, with the
    outputs and workspaces the wrappers allocate (recorded on that stream),
    while the current stream allocates and writes other memory meanwhile."""
    bits = workloads.bits_numpy(workloads.gradient_bucket(300_001, seed=21, special_frac=1e-3))
    t = _bits_tensor(bits)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    buf, size = uz.compress(t, stream=side)
    junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device=DEV) for _ in range(8)]  # reuse pressure
    side.synchronize()
    got = buf[:int(size.item())].cpu().numpy()
    assert np.array_equal(got, orc.compress(orc.BF16, bits))
    out, st = uz.decompress(buf[:got.size], torch.bfloat16, bits.size, stream=side)
    junk += [torch.full((1 << 20,), 9, dtype=torch.uint8, device=DEV) for _ in range(8)]
    side.synchronize()
    assert int(st.item()) == 0 and torch.equal(_int_view(out), _int_view(t))
    outs, sizes = uz.compress_batched([t, t[:1000]], stream=side)
    side.synchronize()
    assert np.array_equal(outs[1][:int(sizes[1].item())].cpu().numpy(), orc.compress(orc.BF16, bits[:1000]))
    del junk
