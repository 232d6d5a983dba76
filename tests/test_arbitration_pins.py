"""Pins of the oracle's per-call arbitration (NCCLZ Sec. IV-C, Eq. (1) and (2),
Algorithm 1): hand-derived plans, the integer logarithm against the
mathematics, the boundary cases of the rule, and the frames each decision
commits.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from uzip_testlib import parse_buffer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def policy(**kw):
    base = dict(link_bytes_per_us=25000, encode_bytes_per_us=1_000_000, decode_bytes_per_us=1_000_000, fixed_ns=0,
                small_bytes=0, exposed_encode_permil=1000, exposed_decode_permil=1000, min_gain_permil=0, reserved=0)
    base.update(kw)
    return orc.Policy(**base)


def bf16_with_exponents(counts: dict, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    e = np.concatenate([np.full(c, int(s), np.uint16) for s, c in counts.items()])
    e = rng.permutation(e)
    return ((e << 7) | (rng.integers(0, 2, e.size).astype(np.uint16) << 15) |
            rng.integers(0, 128, e.size).astype(np.uint16)).astype(np.uint16)


def test_log2_q16_against_the_logarithm():
    xs = np.arange(1, 1 << 17)
    L = np.array([orc.log2_q16(int(x)) for x in xs], dtype=np.int64)
    d = np.log2(xs.astype(np.float64)) * 65536 - L
    assert d.min() >= 0 and d.max() < 1.001  # rounded down, at most one unit off
    assert np.all(np.diff(L) >= 0)
    for k in range(17):
        assert orc.log2_q16(1 << k) == k << 16  # exact at powers of two
    assert orc.log2_q16(3) == math.floor(65536 * math.log2(3))


def test_worked_example_w3():
    g = json.load(open(os.path.join(GOLDEN, "arbitration_w3.json")))
    for i, case in enumerate(g["cases"]):
        bits = bf16_with_exponents(case["exponents"], seed=i)
        if "fill" in case:  # values past the sample, which the plan sees only through N
            bits = np.concatenate([bits, np.full(case["n"] - bits.size, case["fill"], np.uint16)])
        assert bits.size == case["n"]
        plan = orc.plan_call(orc.BF16, bits, orc.Policy(**case["policy"]))
        assert plan == case["plan"], case["what"]


def test_frames_each_decision_commits():
    bits = bf16_with_exponents({"124": 8192, "125": 8192, "126": 8192, "127": 8192}, seed=7)
    coded, plan = orc.compress_arbitrated(orc.BF16, bits, policy())
    assert plan["decision"] == 0 and np.array_equal(coded, orc.compress(orc.BF16, bits))
    raw, plan = orc.compress_arbitrated(orc.BF16, bits, policy(fixed_ns=5000))
    assert plan["decision"] == 1
    assert raw.size == orc.max_compressed_size(orc.BF16, bits.size)
    hdr, _, recs = parse_buffer(raw)
    assert all(r["mode"] == 1 for r in recs)
    st, back = orc.decompress(raw, orc.BF16, bits.size)
    assert st == orc.OK and np.array_equal(back, bits)
    # both frames carry the same sign+mantissa region; only the index and the
    # records differ
    assert np.array_equal(raw[hdr["sm_off"]:hdr["exp_off"]], coded[hdr["sm_off"]:hdr["exp_off"]])
    assert np.array_equal(raw[:16], coded[:16])


@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32, orc.FP16, orc.FP8_E4M3, orc.FP8_E5M2])
def test_sample_is_the_bounded_prefix(dtype):
    eb = np.dtype(orc._ELEM[dtype]).itemsize
    n = 200_000
    bits = np.random.default_rng(dtype).integers(0, 1 << (8 * eb), n, dtype=np.uint64).astype(orc._ELEM[dtype])
    plan = orc.plan_call(dtype, bits, policy())
    assert plan["sample_values"] == 65536 // eb
    # values after the sample do not move the plan's sample statistics: the
    # predicted size depends on them only through n
    other = bits.copy()
    other[65536 // eb:] = 0
    p2 = orc.plan_call(dtype, other, policy())
    assert p2["predicted_bytes"] == plan["predicted_bytes"]
    # random bits: no gain predicted, RAW
    assert plan["decision"] == 1


def test_boundaries_of_the_rule():
    bits = bf16_with_exponents({"124": 8192, "125": 8192, "126": 8192, "127": 8192}, seed=3)
    B = 2 * bits.size
    # small-call fast path: at the threshold RAW, one byte below it sampled
    assert orc.plan_call(orc.BF16, bits, policy(small_bytes=B))["decision"] == 2
    assert orc.plan_call(orc.BF16, bits, policy(small_bytes=B - 1))["decision"] == 0
    # an empty call is always the small path
    assert orc.plan_call(orc.BF16, np.zeros(0, np.uint16), policy())["decision"] == 2
    # ties go RAW: pick the fixed cost that makes coded_ns == raw_ns
    p = orc.plan_call(orc.BF16, bits, policy())
    gap = p["raw_ns"] - p["coded_ns"]
    assert orc.plan_call(orc.BF16, bits, policy(fixed_ns=gap))["decision"] == 1
    assert orc.plan_call(orc.BF16, bits, policy(fixed_ns=gap - 1))["decision"] == 0
    # a fast link makes RAW cheaper than any codec time; a slow one favours coding
    assert orc.plan_call(orc.BF16, bits, policy(link_bytes_per_us=10**9))["decision"] == 1
    assert orc.plan_call(orc.BF16, bits, policy(link_bytes_per_us=1, fixed_ns=10**6))["decision"] == 0
    # the codec's exposed fractions scale its cost linearly
    p0 = orc.plan_call(orc.BF16, bits, policy(exposed_encode_permil=0, exposed_decode_permil=0))
    assert p0["coded_ns"] == p["coded_ns"] - 2 * math.ceil(1000 * B / 1_000_000)
    # a minimum gain of the whole payload can never be met
    assert orc.plan_call(orc.BF16, bits, policy(min_gain_permil=1000))["decision"] == 1


@pytest.mark.parametrize("bad", [dict(link_bytes_per_us=0), dict(encode_bytes_per_us=0), dict(decode_bytes_per_us=0),
                                 dict(exposed_encode_permil=1001), dict(exposed_decode_permil=1001),
                                 dict(min_gain_permil=1001), dict(reserved=1)])
def test_invalid_policies_are_rejected(bad):
    with pytest.raises(ValueError):
        orc.plan_call(orc.BF16, np.zeros(100, np.uint16), policy(**bad))


def test_prediction_tracks_the_coded_size_on_iid_data():
    # PR1 is i.i.d., so a 64 KiB prefix is representative: the prediction
    # lies within 1% of the frame the codec writes
    bits = workloads.bits_numpy(workloads.pr1())
    plan = orc.plan_call(orc.BF16, bits, policy())
    actual = orc.compress(orc.BF16, bits).size
    assert abs(plan["predicted_bytes"] / actual - 1) < 0.01
    assert plan["decision"] == 0


@pytest.mark.parametrize("dtype", [orc.FP16, orc.FP8_E4M3])
def test_prediction_other_dtypes(dtype):
    if dtype == orc.FP16:
        bits = workloads.bits_numpy(workloads.fp16_activations(1 << 20))
    else:
        bits = workloads.bits_numpy(workloads.fp8_weights(1 << 21, fmt=torch.float8_e4m3fn))
    plan = orc.plan_call(dtype, bits, policy())
    actual = orc.compress(dtype, bits).size
    assert abs(plan["predicted_bytes"] / actual - 1) < 0.02


@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32, orc.FP16, orc.FP8_E4M3])
def test_oracle_reports_every_raw_record_corruption(dtype):
    from uzip_testlib import raw_corruptions
    eb = np.dtype(orc._ELEM[dtype]).itemsize
    bits = np.random.default_rng(dtype).integers(0, 1 << (8 * eb), 100_000, dtype=np.uint64).astype(orc._ELEM[dtype])
    buf, plan = orc.compress_arbitrated(dtype, bits, policy(link_bytes_per_us=10**9))
    assert plan["decision"] == 1
    assert orc.decompress(buf, dtype, bits.size)[0] == orc.OK
    for name, bad in raw_corruptions(buf):
        assert orc.decompress(bad, dtype, bits.size)[0] == orc.CORRUPT, name


def _prefix_compressible(seed=5):
    """bf16, 8 chunks of 64 KiB: the first chunk (exactly the 64 KiB sample)
    near-Gaussian, the other seven random bit patterns.  The sample predicts
    a frame about two thirds of the payload; the realised frame codes one
    chunk and stores seven RAW."""
    rng = np.random.default_rng(seed)
    head = workloads.bits_numpy(workloads.pr1())[:32768]
    tail = rng.integers(0, 1 << 16, 7 * 32768, dtype=np.uint32).astype(np.uint16)
    return np.concatenate([head, tail])


def test_realised_gain_check_commits_raw():
    """NCCLZ Algorithm 1 accepts a materialised coded frame only if its
    realised size passes the gain check; otherwise the RAW frame is committed
    (decision 3).  The rule's boundary is found from the sizes alone: the
    realised size R of the coded frame (what uzip_compress writes), the RAW
    frame P_raw and B = 2N; the largest minimum gain that R meets is
    g* = floor((P_raw - R) * 1000 / B)."""
    bits = _prefix_compressible()
    B = 2 * bits.size
    P_raw = orc.max_compressed_size(orc.BF16, bits.size)
    coded = orc.compress(orc.BF16, bits)
    R = coded.size
    assert R < P_raw
    g_star = (P_raw - R) * 1000 // B
    slow = dict(link_bytes_per_us=1000)  # coding pays on a slow link
    plan = orc.plan_call(orc.BF16, bits, policy(**slow, min_gain_permil=g_star + 1))
    # the prefix over-predicts: coding is admitted and chosen...
    assert plan["decision"] == 0
    assert (P_raw - plan["predicted_bytes"]) * 1000 >= (g_star + 1) * B
    # ...and at g* + 1 the realised frame fails the check: the RAW frame is committed
    buf, plan = orc.compress_arbitrated(orc.BF16, bits, policy(**slow, min_gain_permil=g_star + 1))
    assert plan["decision"] == 3
    assert buf.size == P_raw
    assert all(r["mode"] == 1 for r in parse_buffer(buf)[2])
    st, back = orc.decompress(buf, orc.BF16, bits.size)
    assert st == orc.OK and np.array_equal(back, bits)
    raw_plan, p1 = orc.compress_arbitrated(orc.BF16, bits, policy(link_bytes_per_us=10**9))
    assert p1["decision"] == 1 and np.array_equal(buf, raw_plan)
    # at g* it passes: the coded frame is committed
    buf, plan = orc.compress_arbitrated(orc.BF16, bits, policy(**slow, min_gain_permil=g_star))
    assert plan["decision"] == 0 and np.array_equal(buf, coded)
    # the plan's other fields are those of the prediction, unchanged by the check
    p_pred = orc.plan_call(orc.BF16, bits, policy(**slow, min_gain_permil=g_star + 1))
    _, p_real = orc.compress_arbitrated(orc.BF16, bits, policy(**slow, min_gain_permil=g_star + 1))
    assert {k: v for k, v in p_real.items() if k != "decision"} == {k: v for k, v in p_pred.items() if k != "decision"}


def test_realised_check_on_iid_data_keeps_the_coded_frame():
    """On i.i.d. data the prediction is close (within 1%), so a coded plan
    admitted with a margin is also accepted once realised."""
    bits = workloads.bits_numpy(workloads.pr1())
    buf, plan = orc.compress_arbitrated(orc.BF16, bits, policy(min_gain_permil=300))
    assert plan["decision"] == 0 and np.array_equal(buf, orc.compress(orc.BF16, bits))


def test_realised_gain_boundary_is_inclusive():
    """A realised gain exactly at the minimum passes, as the admission rule
    does (gain * 1000 >= min_gain * B).  80,000 bf16 values: the first 32,768
    are PR1's first chunk (its coded record is 22,240 bytes below its RAW
    record), the rest random bits stored RAW, so P_raw - R = 22,240 and
    22,240 * 1000 = 139 * B exactly (B = 160,000)."""
    head = workloads.bits_numpy(workloads.pr1())[:32768]
    tail = np.random.default_rng(1).integers(0, 1 << 16, 80000 - 32768, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([head, tail])
    B = 2 * bits.size
    coded = orc.compress(orc.BF16, bits)
    assert orc.max_compressed_size(orc.BF16, bits.size) - coded.size == 22240 and 22240 * 1000 == 139 * B
    buf, plan = orc.compress_arbitrated(orc.BF16, bits, policy(link_bytes_per_us=1000, min_gain_permil=139))
    assert plan["decision"] == 0 and np.array_equal(buf, coded)
    _, plan = orc.compress_arbitrated(orc.BF16, bits, policy(link_bytes_per_us=1000, min_gain_permil=140))
    assert plan["decision"] == 3
