"""GPU parity for the float16 and float8 payloads (the UCCL-Zip review page,
Fig. 13, measures these types beside bf16 and fp32): the coded symbol is the
byte holding the exponent (fp16: the high byte, the low byte raw; fp8: the
whole byte, nothing raw).  Tolerance 0, as for bf16 and fp32."""
import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads
from test_gpu_parity import DEV, check_parity, gpu_compress, gpu_decompress, _int_view
from uzip_testlib import corruptions, parse_buffer

pytestmark = pytest.mark.gpu
FP8 = [torch.float8_e4m3fn, torch.float8_e5m2]


def _fp16(n, seed=5):
    return workloads.bits_numpy(workloads.fp16_activations(n, seed=seed))


def _fp8(n, fmt, seed=6):
    return workloads.bits_numpy(workloads.fp8_weights(n, seed=seed, fmt=fmt))


@pytest.mark.parametrize("n", [1, 7, 33, 1000, 32767, 32768, 32768 + 5, 32768 + 20_001, 65536 * 2 + 31, 300_001])
def test_fp16_ragged_sizes(n):
    check_parity(_fp16(n), tdtype=torch.float16)


@pytest.mark.parametrize("fmt", FP8)
@pytest.mark.parametrize("n", [1, 3, 33, 1000, 65535, 65536, 65536 + 3, 65536 + 20_007, 65536 * 3 + 40_001, 500_001])
def test_fp8_ragged_sizes(fmt, n):
    check_parity(_fp8(n, fmt), tdtype=fmt)


@pytest.mark.parametrize("tdtype", [torch.float16] + FP8)
def test_empty_buffer(tdtype):
    e = np.zeros(0, np.uint16 if tdtype == torch.float16 else np.uint8)
    got = gpu_compress(torch.empty(0, dtype=tdtype, device=DEV))
    assert np.array_equal(got, orc.compress(orc.FP16 if tdtype == torch.float16 else
                                            orc.FP8_E4M3 if tdtype == FP8[0] else orc.FP8_E5M2, e))
    out, st = gpu_decompress(got, tdtype, 0)
    assert st == 0 and out.numel() == 0


def test_every_fp16_bit_pattern():
    rng = np.random.default_rng(3)
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    check_parity(np.concatenate([v, rng.permutation(v), v[::-1]]), tdtype=torch.float16)


@pytest.mark.parametrize("fmt", FP8)
def test_every_fp8_bit_pattern(fmt):
    rng = np.random.default_rng(4)
    v = np.arange(256, dtype=np.uint16).astype(np.uint8)
    check_parity(np.concatenate([np.tile(v, 300), rng.permutation(np.tile(v, 700))]), tdtype=fmt)


@pytest.mark.parametrize("tdtype", [torch.float16] + FP8)
@pytest.mark.parametrize("n", [200_000, 200_003, 70_001, 47])
def test_random_bits_go_raw(tdtype, n):
    # RAW records rebuilt by whole groups of 32 values, the ragged last group
    # value by value (sizes with and without one)
    dt = np.uint16 if tdtype == torch.float16 else np.uint8
    bits = np.random.default_rng(5).integers(0, np.iinfo(dt).max + 1, n).astype(dt)
    got = check_parity(bits, tdtype=tdtype)
    _, _, recs = parse_buffer(got)
    assert all(r["mode"] == 1 for r in recs)


@pytest.mark.parametrize("fmt", FP8)
@pytest.mark.parametrize("n", [160, 161, 1000, 65536 + 4000])
def test_fp8_single_symbol_chunks(fmt, n):
    check_parity(np.full(n, 0x38, np.uint8), tdtype=fmt)


@pytest.mark.parametrize("tail", [8, 16])
def test_fp8_burst_of_rare_symbols(tail):
    """The dominant byte for most of each chunk, then a run of the 255 others:
    a lane of the decoder takes new words twice within three steps."""
    rng = np.random.default_rng(21 + tail)
    ce, n = 65536, 3 * 65536 + 3000
    e = np.full(n, 0x40, np.uint8)
    others = np.array([s for s in range(256) if s != 0x40], np.uint8)
    for c0 in range(0, n, ce):
        m = min(ce, n - c0)
        e[c0 + m - m // tail: c0 + m] = rng.choice(others, m // tail)
    _, _, recs = parse_buffer(orc.compress(orc.FP8_E4M3, e))
    assert all(r["mode"] == 0 for r in recs)
    check_parity(e, tdtype=torch.float8_e4m3fn)


def test_fp16_burst_of_rare_symbols():
    rng = np.random.default_rng(31)
    ce, n = 32768, 3 * 32768 + 3000
    hi = np.full(n, 0x3C, np.uint16)
    others = np.array([s for s in range(256) if s != 0x3C], np.uint16)
    for c0 in range(0, n, ce):
        m = min(ce, n - c0)
        hi[c0 + m - m // 8: c0 + m] = rng.choice(others, m // 8)
    check_parity((hi << 8) | rng.integers(0, 256, n).astype(np.uint16), tdtype=torch.float16)


@pytest.mark.parametrize("tdtype,chunk_bytes", [(torch.float16, 64), (torch.float16, 2048), (torch.float16, 262144),
                                                (torch.float16, 1 << 21), (torch.float8_e4m3fn, 64),
                                                (torch.float8_e4m3fn, 4096), (torch.float8_e4m3fn, 262144),
                                                (torch.float8_e4m3fn, 1 << 20), (torch.float8_e5m2, 1 << 20)])
def test_chunk_sizes(tdtype, chunk_bytes):
    n = 1_200_001
    bits = _fp16(n, seed=9) if tdtype == torch.float16 else _fp8(n, tdtype, seed=9)
    check_parity(bits, chunk_bytes, tdtype=tdtype)


@pytest.mark.parametrize("tdtype", [torch.float16] + FP8)
def test_decodes_oracle_buffers_and_reports_corruption(tdtype):
    code = {torch.float16: orc.FP16, FP8[0]: orc.FP8_E4M3, FP8[1]: orc.FP8_E5M2}[tdtype]
    n = 150_000
    bits = _fp16(n, seed=12) if tdtype == torch.float16 else _fp8(n, tdtype, seed=12)
    buf = orc.compress(code, bits)
    out, st = gpu_decompress(buf, tdtype, n)
    assert st == 0
    assert np.array_equal(_int_view(out).cpu().numpy().view(bits.dtype), bits)
    for name, bad in corruptions(buf):
        _, st = gpu_decompress(bad, tdtype, n)
        assert st == uz.UZIP_ERR_CORRUPT_INPUT, name
    _, st = gpu_decompress(buf, torch.float16 if tdtype != torch.float16 else torch.bfloat16, n)
    assert st == uz.UZIP_ERR_CORRUPT_INPUT  # dtype differs from the header's


@pytest.mark.parametrize("tdtype", [torch.float16] + FP8)
def test_batched_matches_oracle(tdtype):
    code = {torch.float16: orc.FP16, FP8[0]: orc.FP8_E4M3, FP8[1]: orc.FP8_E5M2}[tdtype]
    sizes = [0, 1, 5000, 65536, 100_000, 0, 33, 170_000]
    tensors = []
    for i, n in enumerate(sizes):
        if n == 0:
            tensors.append(torch.empty(0, dtype=tdtype, device=DEV))
        elif tdtype == torch.float16:
            tensors.append(workloads.fp16_activations(n, seed=40 + i).to(DEV))
        else:
            tensors.append(workloads.fp8_weights(n, seed=40 + i, fmt=tdtype).to(DEV))
    outs, out_sizes = uz.compress_batched(tensors)
    torch.cuda.synchronize()
    got = [o[:s] for o, s in zip(outs, out_sizes.cpu().tolist())]
    for t, g in zip(tensors, got):
        assert np.array_equal(g.cpu().numpy(), orc.compress(code, workloads.bits_numpy(t)))
    vals, status = uz.decompress_batched(got, tdtype, sizes)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * len(sizes)
    for t, v in zip(tensors, vals):
        assert torch.equal(_int_view(t), _int_view(v))
