"""Seeded sweep of random corruptions: the GPU decoder's verdict equals the oracle's.

Frames of both kinds (full tables and sampled tables, several value types) are
made by the oracle; each corrupted copy flips one byte, chosen at random in the
header, the record index, the sign+mantissa region or the records.  For every
copy the GPU decoder (one batched call over all copies) must report corrupt
exactly when the oracle does (NCCLZ Algorithm 2: validate, then decode), and
when both accept it the GPU's values must equal the oracle's bit for bit (a
flipped sign+mantissa byte is a valid frame of other values).
"""
import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
COPIES = 96


def _frames():
    rng = np.random.default_rng(7)
    bucket = workloads.bits_numpy(workloads.gradient_bucket(70_001, seed=11, special_frac=1e-3))
    fp32 = rng.normal(0, 1e-3, 40_000).astype(np.float32).view(np.uint32)
    fp16 = workloads.bits_numpy(torch.from_numpy(rng.normal(0, 1.0, 90_000)).to(torch.float16))
    fp8 = workloads.bits_numpy(torch.from_numpy(rng.normal(0, 0.02, 100_000)).to(torch.float8_e5m2))
    return [
        ("bf16 full", orc.BF16, torch.bfloat16, bucket, orc.compress(orc.BF16, bucket)),
        ("bf16 sampled", orc.BF16, torch.bfloat16, bucket, orc.compress_sampled(orc.BF16, bucket)),
        ("fp32 sampled", orc.FP32, torch.float32, fp32, orc.compress_sampled(orc.FP32, fp32, 32768)),
        ("fp16 sampled", orc.FP16, torch.float16, fp16, orc.compress_sampled(orc.FP16, fp16)),
        ("fp8 full", orc.FP8_E5M2, torch.float8_e5m2, fp8, orc.compress(orc.FP8_E5M2, fp8)),
    ]


def _corrupt(buf: np.ndarray, rng) -> np.ndarray:
    hdr = np.frombuffer(buf[:64].tobytes(), dtype=np.uint64)
    sm_off, exp_off = int(hdr[4]), int(hdr[5])
    region = rng.integers(0, 4)
    lo, hi = [(0, 64), (64, sm_off), (sm_off, exp_off), (exp_off, buf.size)][region]
    if hi <= lo:
        lo, hi = exp_off, buf.size
    b = buf.copy()
    k = int(rng.integers(lo, hi))
    b[k] ^= np.uint8(1 << int(rng.integers(0, 8)))
    return b


@pytest.mark.parametrize("which", range(5))
def test_random_corruptions_match_the_oracle_verdict(which):
    name, code, tdtype, bits, frame = _frames()[which]
    rng = np.random.default_rng(100 + which)
    copies = [_corrupt(frame, rng) for _ in range(COPIES)]
    want = [orc.decompress(c, code, bits.size) for c in copies]
    bufs = [torch.from_numpy(c).to(DEV) for c in copies]
    vals, status = uz.decompress_batched(bufs, tdtype, [bits.size] * COPIES)
    torch.cuda.synchronize()
    st = status.cpu().tolist()
    iv = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[vals[0].element_size()]
    accepted = 0
    for i, ((ost, oval), gst, gval) in enumerate(zip(want, st, vals)):
        assert (gst == 0) == (ost == orc.OK), "%s copy %d: GPU status %d, oracle %d" % (name, i, gst, ost)
        if ost == orc.OK:
            accepted += 1
            got = gval.view(iv).cpu().numpy().view(oval.dtype)
            assert np.array_equal(got, oval), "%s copy %d: values differ" % (name, i)
    # the sweep reaches both verdicts
    assert 0 < accepted < COPIES, name


def test_coded_records_not_smaller_than_raw_get_the_oracle_verdict():
    """Frames with valid rANS streams whose coded record is longer than the
    chunk's RAW record (table {120: 4095, 121: 1}, 49,344 bytes against
    32,784), exactly its size, or 16 bytes smaller: the GPU decoder gives each
    the oracle's verdict (corrupt, corrupt, valid), decoded in one batched
    call.  These are ordinary rejected decodes."""
    from uzip_testlib import coded_frame, long_record_frame, parse_buffer
    frames = [long_record_frame(orc.rans_encode)]
    sized = {}
    for k in range(21700, 21900):
        sym = np.full(32768, 120, np.uint8)
        sym[:k] = 121
        fr = coded_frame(sym, {120: 4095, 121: 1}, orc.rans_encode)
        size = parse_buffer(fr[0])[2][0]["bytes"]
        if size in (32784, 32768) and size not in sized:
            sized[size] = fr
        if len(sized) == 2:
            break
    frames += [sized[32784], sized[32768]]
    want = [orc.decompress(f, orc.BF16, v.size) for f, v in frames]
    assert [w[0] for w in want] == [orc.CORRUPT, orc.CORRUPT, orc.OK]
    bufs = [torch.from_numpy(f).to(DEV) for f, _ in frames]
    vals, status = uz.decompress_batched(bufs, torch.bfloat16, [v.size for _, v in frames])
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [3, 3, 0]
    assert np.array_equal(vals[2].view(torch.int16).cpu().numpy().view(np.uint16), frames[2][1])
    # and each alone, through the single-buffer call
    for (f, v), (ost, _) in zip(frames, want):
        out, st = uz.decompress(torch.from_numpy(f).to(DEV), torch.bfloat16, v.size)
        torch.cuda.synchronize()
        assert (int(st.item()) == 0) == (ost == orc.OK)


def test_symbols_beyond_the_exponent_range_get_the_oracle_verdict():
    """fp16 frames naming a symbol no 5-bit exponent holds (in the table, or
    as an escape byte): corrupt on the GPU as in the oracle; the unmodified
    frames decode."""
    from test_oracle_pins import _fp16_escape_out_of_range_frame, _fp16_moved_symbol_frame
    for make in (_fp16_moved_symbol_frame, _fp16_escape_out_of_range_frame):
        vals, good, bad = make()
        for frame, want in ((good, 0), (bad, 3)):
            assert (orc.decompress(frame, orc.FP16, vals.size)[0] == orc.OK) == (want == 0)
            out, st = uz.decompress(torch.from_numpy(frame).to(DEV), torch.float16, vals.size)
            torch.cuda.synchronize()
            assert int(st.item()) == want, make.__name__
            if want == 0:
                assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), vals)
