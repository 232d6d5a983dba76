"""One buffer larger than 4 GiB, compressed and decompressed by the GPU.

The kernels address each chunk pair through buffer resources with 32-bit
offsets on 64-bit bases; a frame offset computed in 32 bits would show only
past 4 GiB.  Single buffers just over 4 GiB of input with a ragged last
chunk: bf16 near-Gaussian values (a coded frame; full and sampled tables),
bf16 uniform random bits (every record RAW, so the frame itself exceeds
4 GiB) and fp32 gradients (256 KiB chunks, three raw bytes per value).
The chunks on either side of byte 2^32 of the input, the first and the last
are compared with the oracle's frame of the same values alone (a chunk's
record and its sign+mantissa bytes depend on the chunk's values only: the
per-chunk framing of NCCLZ Sec. IV-D2), the header and index are checked
against the layout, and the whole frame must round-trip bit for bit.
"""
import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_BF16 = (1 << 31) + 3 * 32768 + 12345
N_FP32 = (1 << 30) + 3 * 65536 + 777


def _u64(buf: torch.Tensor, off: int, count: int = 1) -> np.ndarray:
    return buf[off:off + 8 * count].cpu().numpy().view(np.uint64)


def _check(t: torch.Tensor, sampled: bool = False):
    n, eb = t.numel(), t.element_size()
    code, r, ce = (orc.BF16, 1, 32768) if eb == 2 else (orc.FP32, 3, 65536)
    iv, nv = (torch.int16, np.uint16) if eb == 2 else (torch.int32, np.uint32)
    assert n * eb > 1 << 32
    buf, size = uz.compress(t, sampled=sampled)
    torch.cuda.synchronize()
    total = int(size.item())
    hdr = buf[:64].cpu().numpy()
    h64 = hdr.view(np.uint64)
    assert hdr[:4].tobytes() == b"UZP1"
    chunks = (n + ce - 1) // ce
    assert int(h64[2]) == n and int(h64[3]) == chunks and int(h64[6]) == total
    sm_off, exp_off = int(h64[4]), int(h64[5])
    assert sm_off == 64 + ((8 * (chunks + 1) + 15) // 16) * 16 and exp_off >= sm_off + n * r
    assert int(_u64(buf, 64 + 8 * chunks)[0]) == total - exp_off
    mid = (1 << 32) // (eb * ce)  # the chunk that starts at input byte 2^32
    for c in sorted({0, mid - 1, mid, mid + 1, chunks - 1}):
        lo, hi = (int(v) for v in _u64(buf, 64 + 8 * c, 2))
        vals = t[c * ce:min(n, (c + 1) * ce)].view(iv).cpu().numpy().view(nv)
        want = orc.compress_sampled(code, vals, ce * eb) if sampled else orc.compress(code, vals, ce * eb)
        w64 = want[:64].view(np.uint64)
        w_sm, w_exp, w_total = int(w64[4]), int(w64[5]), int(w64[6])
        got_rec = buf[exp_off + lo:exp_off + hi].cpu().numpy()
        assert np.array_equal(got_rec, want[w_exp:w_total]), "record of chunk %d differs from the oracle's" % c
        got_sm = buf[sm_off + c * ce * r:sm_off + (c * ce + vals.size) * r].cpu().numpy()
        assert np.array_equal(got_sm, want[w_sm:w_sm + vals.size * r]), "sign+mantissa bytes of chunk %d differ" % c
    out, st = uz.decompress(buf[:total], t.dtype, n)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(out.view(iv), t.view(iv))
    del buf, out
    return total


@pytest.mark.parametrize("sampled", [False, True])
def test_coded_bf16_buffer_over_4gib(sampled):
    t = workloads.gradient_bucket(N_BF16, device=DEV, seed=21)
    total = _check(t, sampled)
    assert total < 0.7 * 2 * N_BF16  # coded: about 0.66 of the input
    del t
    torch.cuda.empty_cache()


def test_raw_bf16_frame_over_4gib():
    g = torch.Generator(device=DEV)
    g.manual_seed(22)
    t = torch.randint(-32768, 32768, (N_BF16,), generator=g, device=DEV, dtype=torch.int32).to(torch.int16)
    total = _check(t.view(torch.bfloat16))
    assert total > 1 << 32  # every record RAW: the frame itself passes 4 GiB
    del t
    torch.cuda.empty_cache()


def test_fp32_buffer_over_4gib():
    t = workloads.fp32_gradients(N_FP32, device=DEV, seed=23)
    total = _check(t)
    assert total < 0.9 * 4 * N_FP32
    del t
    torch.cuda.empty_cache()


def test_batched_call_with_a_buffer_over_4gib():
    """The same buffer between two small ones in one batched call: every frame
    equals its single-buffer frame (itself checked above against the oracle
    around byte 2^32), and the batch decodes bit for bit."""
    big = workloads.gradient_bucket(N_BF16, device=DEV, seed=21)
    small = [workloads.gradient_bucket(n, device=DEV, seed=s) for n, s in ((40_000, 24), (1, 25))]
    ts = [small[0], big, small[1]]
    bufs, sizes = uz.compress_batched(ts)
    torch.cuda.synchronize()
    sz = sizes.cpu().tolist()
    for t, b, s in zip(ts, bufs, sz):
        one, one_size = uz.compress(t)
        torch.cuda.synchronize()
        assert int(one_size.item()) == s
        assert torch.equal(one[:s], b[:s])
        del one
    outs, status = uz.decompress_batched([b[:s] for b, s in zip(bufs, sz)], torch.bfloat16, [t.numel() for t in ts])
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 0, 0]
    for t, o in zip(ts, outs):
        assert torch.equal(t.view(torch.int16), o.view(torch.int16))
    del big, bufs, outs
    torch.cuda.empty_cache()
