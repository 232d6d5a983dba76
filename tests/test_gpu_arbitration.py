"""GPU parity of the per-call arbitration (NCCLZ Sec. IV-C, Eq. (1) and (2),
Algorithm 1): the plan the device computes equals the oracle's field by
field, and the frame it commits (coded, or every record RAW) equals the
oracle's byte for byte and decodes to the input.  Tolerance 0."""
import json
import os

import numpy as np
import pytest
import torch

import lossless_compression_float_amd as uz
import oracle as orc
import workloads
from test_gpu_parity import DEV, _bits_tensor, _int_view, gpu_decompress
from uzip_testlib import parse_buffer

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ORC_CODE = {torch.bfloat16: orc.BF16, torch.float32: orc.FP32, torch.float16: orc.FP16,
            torch.float8_e4m3fn: orc.FP8_E4M3, torch.float8_e5m2: orc.FP8_E5M2}
NP_ELEM = {torch.bfloat16: np.uint16, torch.float16: np.uint16, torch.float32: np.uint32,
           torch.float8_e4m3fn: np.uint8, torch.float8_e5m2: np.uint8}

FIELDS = dict(link_bytes_per_us=50_000, encode_bytes_per_us=1_300_000, decode_bytes_per_us=1_600_000,
              fixed_ns=2_000, small_bytes=0, exposed_encode_permil=1000, exposed_decode_permil=1000,
              min_gain_permil=20, reserved=0)


def both_policies(**kw):
    f = dict(FIELDS, **kw)
    return uz.policy(**f), orc.Policy(**f)


def check_arbitrated(bits: np.ndarray, tdtype: torch.dtype, chunk_bytes: int = 0, **kw):
    gp, op = both_policies(**kw)
    t = _bits_tensor(bits, tdtype)
    buf, size, plan = uz.compress_arbitrated(t, gp, chunk_bytes)
    torch.cuda.synchronize()
    got = buf[:int(size.item())].cpu().numpy()
    want, want_plan = orc.compress_arbitrated(ORC_CODE[tdtype], bits, op, chunk_bytes)
    assert uz.plans_as_dicts(plan)[0] == want_plan
    assert np.array_equal(got, want), "frame differs from the oracle (sizes %d vs %d)" % (got.size, want.size)
    out, st = gpu_decompress(got, tdtype, bits.size)
    assert st == 0 and torch.equal(_int_view(out), _int_view(t))
    return want_plan, got


def _workload(tdtype, n, seed):
    if tdtype == torch.bfloat16:
        return workloads.bits_numpy(workloads.gradient_bucket(n, seed=seed, special_frac=1e-3))
    if tdtype == torch.float32:
        return workloads.bits_numpy(workloads.fp32_gradients(n, seed=seed))
    if tdtype == torch.float16:
        return workloads.bits_numpy(workloads.fp16_activations(n, seed=seed))
    return workloads.bits_numpy(workloads.fp8_weights(n, seed=seed, fmt=tdtype))


def test_worked_example_w3_on_the_gpu():
    g = json.load(open(os.path.join(GOLDEN, "arbitration_w3.json")))
    rng = np.random.default_rng(0)
    for case in g["cases"]:
        e = np.concatenate([np.full(c, int(s), np.uint16) for s, c in case["exponents"].items()])
        e = rng.permutation(e)
        bits = ((e << 7) | rng.integers(0, 256, e.size).astype(np.uint16) & 0x807F).astype(np.uint16)
        if "fill" in case:  # values past the sample, which the plan sees only through N
            bits = np.concatenate([bits, np.full(case["n"] - bits.size, case["fill"], np.uint16)])
        pol = uz.policy(**case["policy"])
        _, _, plan = uz.compress_arbitrated(_bits_tensor(bits, torch.bfloat16), pol)
        torch.cuda.synchronize()
        assert uz.plans_as_dicts(plan)[0] == case["plan"], case["what"]


@pytest.mark.parametrize("tdtype", list(ORC_CODE))
@pytest.mark.parametrize("link", [5_000, 50_000, 5_000_000])
def test_plan_and_frame_match_the_oracle(tdtype, link):
    bits = _workload(tdtype, 300_001, seed=3)
    plan, _ = check_arbitrated(bits, tdtype, link_bytes_per_us=link)
    # a slow link makes coding pay; a link far faster than the codec does not
    if link == 5_000:
        assert plan["decision"] == uz.UZIP_PLAN_CODED
    if link == 5_000_000:
        assert plan["decision"] == uz.UZIP_PLAN_RAW


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float32, torch.float16, torch.float8_e4m3fn,
                                    torch.float8_e5m2])
@pytest.mark.parametrize("n", [250_000, 100_003, 45])
def test_raw_plan_writes_every_record_raw(tdtype, n):
    # (the narrow types' RAW frames pack whole groups of 32 values and the
    # ragged last group separately: sizes with and without such a group)
    bits = _workload(tdtype, n, seed=4)
    plan, got = check_arbitrated(bits, tdtype, link_bytes_per_us=10**9)
    assert plan["decision"] == uz.UZIP_PLAN_RAW
    _, _, recs = parse_buffer(got)
    assert all(r["mode"] == 1 for r in recs)
    assert got.size == orc.max_compressed_size(ORC_CODE[tdtype], bits.size)


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float8_e5m2])
@pytest.mark.parametrize("n", [1, 33, 1000, 32767, 32768, 32769, 65535, 65536, 65537, 100_003])
def test_sample_boundaries(tdtype, n):
    # around the sample size (32768 bf16 values, 65536 fp8 values) and the chunk size
    bits = _workload(tdtype, n, seed=n % 97)
    check_arbitrated(bits, tdtype, link_bytes_per_us=5_000, fixed_ns=0)


def test_small_path_and_empty_call():
    bits = _workload(torch.bfloat16, 5000, seed=5)
    plan, got = check_arbitrated(bits, torch.bfloat16, small_bytes=10_000)
    assert plan["decision"] == uz.UZIP_PLAN_RAW_SMALL
    plan, got = check_arbitrated(np.zeros(0, np.uint16), torch.bfloat16)
    assert plan["decision"] == uz.UZIP_PLAN_RAW_SMALL and got.size == 80


def test_random_bits_are_never_coded():
    bits = np.random.default_rng(6).integers(0, 1 << 16, 200_000).astype(np.uint16)
    plan, _ = check_arbitrated(bits, torch.bfloat16, link_bytes_per_us=1, fixed_ns=0)
    assert plan["decision"] == uz.UZIP_PLAN_RAW  # no predicted gain: not admitted


@pytest.mark.parametrize("tdtype,chunk_bytes", [(torch.bfloat16, 0), (torch.bfloat16, 4096), (torch.float32, 0),
                                                (torch.float16, 0), (torch.float8_e4m3fn, 0), (torch.float8_e5m2, 8192)])
def test_batched_mixed_decisions(tdtype, chunk_bytes):
    """Small buffers take the fast path, random bits go RAW by the model, the
    rest is coded; every buffer equals its own oracle call."""
    rng = np.random.default_rng(7)
    elem = NP_ELEM[tdtype]
    eb = np.dtype(elem).itemsize
    rand = rng.integers(0, 1 << (8 * eb), 160_000 // eb, dtype=np.uint64).astype(elem)
    bits = [_workload(tdtype, 200_000 // eb, seed=1), np.zeros(0, elem), _workload(tdtype, 600 // eb, seed=2),
            rand, _workload(tdtype, 131_074 // eb, seed=3), _workload(tdtype, 4_000 // eb, seed=4)]
    kw = dict(link_bytes_per_us=5_000, small_bytes=4_096)
    gp, op = both_policies(**kw)
    ts = [_bits_tensor(b, tdtype) if b.size else torch.empty(0, dtype=tdtype, device=DEV) for b in bits]
    outs, sizes, plans = uz.compress_batched_arbitrated(ts, gp, chunk_bytes)
    torch.cuda.synchronize()
    got_plans = uz.plans_as_dicts(plans)
    decisions = []
    for b, o, s, p in zip(bits, outs, sizes.cpu().tolist(), got_plans):
        want, want_plan = orc.compress_arbitrated(ORC_CODE[tdtype], b, op, chunk_bytes)
        assert p == want_plan
        assert np.array_equal(o[:s].cpu().numpy(), want)
        decisions.append(p["decision"])
    assert decisions == [0, 2, 2, 1, 0, 2]
    vals, status = uz.decompress_batched([o[:s] for o, s in zip(outs, sizes.cpu().tolist())], tdtype,
                                         [b.size for b in bits])
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * len(bits)
    for t, v in zip(ts, vals):
        assert torch.equal(_int_view(t), _int_view(v))


def test_plain_compress_is_unchanged_by_a_previous_raw_plan():
    # the plan lives in caller memory; a plain call after an arbitrated one codes as before
    bits = _workload(torch.bfloat16, 120_000, seed=8)
    t = _bits_tensor(bits, torch.bfloat16)
    ws = uz.workspace(uz.uzip_workspace_size(uz.UZIP_BF16, bits.size), DEV)
    gp, _ = both_policies(link_bytes_per_us=10**9)
    uz.compress_arbitrated(t, gp, ws=ws)
    buf, size = uz.compress(t, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(buf[:int(size.item())].cpu().numpy(), orc.compress(orc.BF16, bits))


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float32, torch.float8_e5m2])
def test_corrupt_raw_frames_are_reported(tdtype):
    """The decoder's RAW-record path validates as the coded one does: every
    corruption of an all-RAW frame is reported, and the clean frame decodes."""
    from uzip_testlib import raw_corruptions
    bits = _workload(tdtype, 150_000, seed=9)
    _, op = both_policies(link_bytes_per_us=10**9)
    buf, plan = orc.compress_arbitrated(ORC_CODE[tdtype], bits, op)
    assert plan["decision"] == uz.UZIP_PLAN_RAW
    out, st = gpu_decompress(buf, tdtype, bits.size)
    assert st == 0 and np.array_equal(_int_view(out).cpu().numpy().view(bits.dtype), bits)
    n_bad = 0
    for name, bad in raw_corruptions(buf):
        want = orc.decompress(bad, ORC_CODE[tdtype], bits.size)[0]
        _, st = gpu_decompress(bad, tdtype, bits.size)
        assert st == (uz.UZIP_ERR_CORRUPT_INPUT if want == orc.CORRUPT else 0), name
        n_bad += want == orc.CORRUPT
    assert n_bad == 13  # every one of them is a corruption the oracle reports


def _prefix_compressible(n=8 * 32768, seed=5):
    """bf16: a near-Gaussian first 64 KiB chunk (the sample), random bits after it."""
    head = workloads.bits_numpy(workloads.pr1())[:32768]
    tail = np.random.default_rng(seed).integers(0, 1 << 16, n - 32768, dtype=np.uint32).astype(np.uint16)
    return np.concatenate([head, tail])


def test_realised_gain_check_on_the_gpu():
    """A prefix that over-predicts: the plan codes, the realised frame fails
    the gain check, and the device commits the all-RAW frame (decision 3),
    as the oracle does; at the exact boundary (g* = floor((P_raw - R) 1000 / B))
    the coded frame stays."""
    bits = _prefix_compressible()
    B = 2 * bits.size
    R = orc.compress(orc.BF16, bits).size
    g_star = (orc.max_compressed_size(orc.BF16, bits.size) - R) * 1000 // B
    plan, got = check_arbitrated(bits, torch.bfloat16, link_bytes_per_us=1000, fixed_ns=0,
                                 min_gain_permil=g_star + 1)
    assert plan["decision"] == uz.UZIP_PLAN_RAW_REALIZED
    assert all(r["mode"] == 1 for r in parse_buffer(got)[2])
    plan, got = check_arbitrated(bits, torch.bfloat16, link_bytes_per_us=1000, fixed_ns=0, min_gain_permil=g_star)
    assert plan["decision"] == uz.UZIP_PLAN_CODED and got.size == R


def test_realised_check_in_a_batch():
    """One batched call in which every decision occurs: coded and kept, coded
    then rejected once realised, RAW by the model, and the small path; each
    buffer equals its own oracle call."""
    good = workloads.bits_numpy(workloads.pr1())[:5 * 32768]
    bad = _prefix_compressible(6 * 32768, seed=6)
    rand = np.random.default_rng(8).integers(0, 1 << 16, 70_000, dtype=np.uint32).astype(np.uint16)
    small = good[:1000].copy()
    bits = [good, bad, rand, small, bad[:32768 + 5000].copy()]
    kw = dict(link_bytes_per_us=1000, fixed_ns=0, small_bytes=4096, min_gain_permil=150)
    gp, op = both_policies(**kw)
    ts = [_bits_tensor(b, torch.bfloat16) for b in bits]
    outs, sizes, plans = uz.compress_batched_arbitrated(ts, gp)
    torch.cuda.synchronize()
    got_plans = uz.plans_as_dicts(plans)
    for b, o, s, p in zip(bits, outs, sizes.cpu().tolist(), got_plans):
        want, want_plan = orc.compress_arbitrated(orc.BF16, b, op)
        assert p == want_plan
        assert np.array_equal(o[:s].cpu().numpy(), want)
    assert [p["decision"] for p in got_plans] == [0, 3, 1, 2, 0]
    vals, status = uz.decompress_batched([o[:s] for o, s in zip(outs, sizes.cpu().tolist())], torch.bfloat16,
                                         [b.size for b in bits])
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * len(bits)
    for t, v in zip(ts, vals):
        assert torch.equal(_int_view(t), _int_view(v))
