"""uzip_compress_noalloc, the compress for callers that cannot allocate
device memory: called through the C ABI, its output equals uzip_compress's
(with a caller workspace) byte for byte, on consecutive calls that share the
device's scratch (the second with a smaller input, then another type), and
the round trip is bit-exact.  Inputs whose workspace exceeds the scratch are
rejected at once, nothing written."""
import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _with_workspace(t, code, cb=0):
    """uzip_compress through the C ABI, caller-allocated workspace."""
    n = t.numel()
    cap = uz.uzip_max_compressed_size(code, n, cb)
    out = torch.empty(cap, dtype=torch.uint8, device=DEV)
    size = torch.empty(1, dtype=torch.int64, device=DEV)
    ws = torch.empty(uz.uzip_workspace_size(code, n, cb), dtype=torch.uint8, device=DEV)
    st = uz.uzip_compress(code, t.data_ptr(), n, cb, out.data_ptr(), cap, size.data_ptr(), ws.data_ptr(), ws.numel(),
                          _stream())
    assert st == uz.UZIP_OK
    torch.cuda.synchronize()
    return out[:int(size.item())].cpu().numpy()


def _outputs(t, code, cb=0):
    cap = uz.uzip_max_compressed_size(code, t.numel(), cb)
    return torch.empty(cap, dtype=torch.uint8, device=DEV), torch.full((1,), -1, dtype=torch.int64, device=DEV)


def test_noalloc_equals_uzip_compress_on_consecutive_calls():
    big = workloads.gradient_bucket(3_000_001, device=DEV, seed=31, special_frac=1e-3)  # 92 chunks
    small = workloads.pr1(DEV)[:100_003].contiguous()                                    # 4 chunks
    f32 = workloads.fp32_gradients(1_000_003, device=DEV, seed=32)                        # 16 chunks of 256 KiB
    cases = [(big, uz.UZIP_BF16, 0), (small, uz.UZIP_BF16, 0), (f32, uz.UZIP_FP32, 0), (small, uz.UZIP_BF16, 4096)]
    # every output buffer exists before the first call: the calls themselves allocate nothing
    outs = [_outputs(t, code, cb) for t, code, cb in cases]
    got = []
    for (t, code, cb), (out, size) in zip(cases, outs):
        st = uz.uzip_compress_noalloc(code, t.data_ptr(), t.numel(), cb, out.data_ptr(), out.numel(), size.data_ptr(),
                                      _stream())
        assert st == uz.UZIP_OK
        torch.cuda.synchronize()  # one call at a time: calls share the device's scratch
        got.append(out[:int(size.item())].cpu().numpy())
    for (t, code, cb), g in zip(cases, got):
        assert np.array_equal(g, _with_workspace(t, code, cb))
    assert np.array_equal(got[1], orc.compress(orc.BF16, workloads.bits_numpy(small)))
    for (t, code, cb), g in zip(cases, got):
        back, st = uz.decompress(torch.from_numpy(g).to(DEV), t.dtype, t.numel())
        torch.cuda.synchronize()
        iv = {2: torch.int16, 4: torch.int32}[t.element_size()]
        assert int(st.item()) == 0 and torch.equal(back.view(iv), t.view(iv))


def test_noalloc_back_to_back_on_one_stream():
    """Two calls enqueued without a host wait between them (the second with a
    smaller input): stream order keeps them apart, each output is right."""
    a = workloads.gradient_bucket(2_000_000, device=DEV, seed=33, special_frac=1e-3)
    b = workloads.gradient_bucket(70_001, device=DEV, seed=34, special_frac=1e-3)
    (oa, sa), (ob, sb) = _outputs(a, uz.UZIP_BF16), _outputs(b, uz.UZIP_BF16)
    for t, o, s in ((a, oa, sa), (b, ob, sb)):
        assert uz.uzip_compress_noalloc(uz.UZIP_BF16, t.data_ptr(), t.numel(), 0, o.data_ptr(), o.numel(),
                                        s.data_ptr(), _stream()) == uz.UZIP_OK
    torch.cuda.synchronize()
    assert np.array_equal(oa[:int(sa.item())].cpu().numpy(), _with_workspace(a, uz.UZIP_BF16))
    assert np.array_equal(ob[:int(sb.item())].cpu().numpy(), _with_workspace(b, uz.UZIP_BF16))


def test_noalloc_limit():
    """At the default 64 KiB chunks the scratch holds 2046 chunks: 67,043,328
    bf16 values are accepted, one more value is rejected synchronously."""
    n_max = 2046 * 32768
    assert uz.uzip_workspace_size(uz.UZIP_BF16, n_max) <= uz.UZIP_NOALLOC_SCRATCH_BYTES
    assert uz.uzip_workspace_size(uz.UZIP_BF16, n_max + 1) > uz.UZIP_NOALLOC_SCRATCH_BYTES
    t = workloads.gradient_bucket(n_max + 1, device=DEV, seed=35)
    out, size = _outputs(t, uz.UZIP_BF16)
    st = uz.uzip_compress_noalloc(uz.UZIP_BF16, t.data_ptr(), n_max + 1, 0, out.data_ptr(), out.numel(),
                                  size.data_ptr(), _stream())
    assert st == uz.UZIP_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert int(size.item()) == -1  # nothing was launched
    tm = t[:n_max]
    st = uz.uzip_compress_noalloc(uz.UZIP_BF16, tm.data_ptr(), n_max, 0, out.data_ptr(), out.numel(), size.data_ptr(),
                                  _stream())
    assert st == uz.UZIP_OK
    torch.cuda.synchronize()
    assert np.array_equal(out[:int(size.item())].cpu().numpy(), _with_workspace(tm, uz.UZIP_BF16))
