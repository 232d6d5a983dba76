"""Streams, host threads and graph capture.

The library never synchronises the caller's stream, keeps no state shared
between calls beyond each host thread's pinned descriptor staging, and its
calls with caller-provided memory launch kernels only, so they can be
captured into a graph.  These tests run: two host threads, each on its own
stream, making batched round trips at once (every output equal to the
single-threaded reference); and compress + decompress (with a caller
workspace, and the allocation-free compress) captured into a HIP graph and
replayed several times with eager work between the replays (every replay
equal to the eager result, which is itself equal to the oracle's frame).
"""
import threading

import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_two_threads_on_two_streams_batched_round_trips():
    batches = [[workloads.gradient_bucket(n, device=DEV, seed=s) for n, s in sizes]
               for sizes in (((1_000_003, 41), (65_536, 42), (7, 43), (300_000, 44)),
                             ((2_000_000, 45), (123_457, 46), (32_768, 47)))]
    refs = []
    for ts in batches:
        bufs, sizes = uz.compress_batched(ts)
        torch.cuda.synchronize()
        sz = sizes.cpu().tolist()
        refs.append([b[:s].clone() for b, s in zip(bufs, sz)])
    # (the references equal the oracle's frames)
    for ts, rf in zip(batches, refs):
        for t, r in zip(ts, rf):
            bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(r.cpu().numpy(), orc.compress(orc.BF16, bits))
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(12):
                    bufs, sizes = uz.compress_batched(batches[i], stream=s)
                    sz = sizes.cpu().tolist()  # (waits for the stream's work)
                    outs, status = uz.decompress_batched([b[:n] for b, n in zip(bufs, sz)], torch.bfloat16,
                                                         [t.numel() for t in batches[i]], stream=s)
                    s.synchronize()
                    assert status.cpu().tolist() == [0] * len(batches[i])
                    for b, n, r, t, o in zip(bufs, sz, refs[i], batches[i], outs):
                        assert n == r.numel() and torch.equal(b[:n], r)
                        assert torch.equal(o.view(torch.int16), t.view(torch.int16))
        except Exception as e:  # reported by the main thread
            errors.append("thread %d: %r" % (i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors


def test_graph_capture_replays_equal_the_eager_calls():
    t = workloads.gradient_bucket(300_001, device=DEV, seed=31)
    code, n = orc.BF16, t.numel()
    cap = uz.uzip_max_compressed_size(code, n, 0)
    out = torch.empty(cap, dtype=torch.uint8, device=DEV)
    out2 = torch.empty(cap, dtype=torch.uint8, device=DEV)
    size = torch.empty(1, dtype=torch.int64, device=DEV)
    size2 = torch.empty(1, dtype=torch.int64, device=DEV)
    ws = torch.empty(uz.uzip_workspace_size(code, n, 0), dtype=torch.uint8, device=DEV)
    back = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)

    def calls(stream):
        assert uz.uzip_compress(code, t.data_ptr(), n, 0, out.data_ptr(), cap, size.data_ptr(), ws.data_ptr(),
                                ws.numel(), stream) == uz.UZIP_OK
        # the frame is self-describing: decode reads its size from the header
        assert uz.uzip_decompress(out.data_ptr(), cap, code, n, back.data_ptr(), status.data_ptr(), ws.data_ptr(),
                                  ws.numel(), stream) == uz.UZIP_OK
        assert uz.uzip_compress_noalloc(code, t.data_ptr(), n, 0, out2.data_ptr(), cap, size2.data_ptr(),
                                        stream) == uz.UZIP_OK

    # eager reference, equal to the oracle's frame
    calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref_size = int(size.item())
    ref = out[:ref_size].clone()
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ref.cpu().numpy(), orc.compress(orc.BF16, bits))
    assert int(size2.item()) == ref_size and torch.equal(out2[:ref_size], ref)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        # eager work between the replays overwrites every output
        out.fill_(0xAB)
        out2.fill_(0xCD)
        back.zero_()
        status.fill_(-1)
        size.fill_(-1)
        size2.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(size.item()) == ref_size and torch.equal(out[:ref_size], ref), "replay %d: frame" % rep
        assert int(status.item()) == 0 and torch.equal(back.view(torch.int16), t.view(torch.int16)), "replay %d" % rep
        assert int(size2.item()) == ref_size and torch.equal(out2[:ref_size], ref), "replay %d: noalloc frame" % rep
    del g
