"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test pins one oracle function to something other than the oracle
itself: a hand-derived trace (tests/golden, each with its derivation), a
closed form, a library routine, brute force over tiny inputs, or an
invariant of the method.  A plausible mistake in the oracle (a dropped term,
a wrong sign or index, swapped lanes, a wrong word order, an off-by-one in
the layout) fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from uzip_testlib import coded_frame, corruptions as _corruptions, long_record_frame, parse_buffer

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def _table(d):
    f = np.zeros(256, np.uint32)
    c0 = np.zeros(256, np.uint32)
    for k, (fs, cs) in d.items():
        f[int(k)] = fs
        c0[int(k)] = cs
    return f, c0


def entropy_bits(counts):
    c = np.asarray(counts, np.float64)
    c = c[c > 0]
    n = c.sum()
    return float(-(c * np.log2(c / n)).sum())


# --------------------------------------------------------------------------
# P1: field split -- a bijection, and it agrees with the float semantics
# --------------------------------------------------------------------------
def test_split_bf16_exhaustive_bijection():
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e, sm = orc.split(orc.BF16, v)
    assert np.array_equal(orc.merge(orc.BF16, e, sm), v)
    assert np.unique(e.astype(np.uint32) * 256 + sm).size == 65536


def _expected_fields(x, mant_bits, bias, emax):
    """(exponent field, sign, mantissa field) from the float value itself."""
    sign = np.signbit(x).astype(np.uint64)
    ax = np.abs(x)
    e = np.zeros(x.shape, np.uint64)
    mant = np.zeros(x.shape, np.uint64)
    finite = np.isfinite(x)
    tiny = 2.0 ** (1 - bias)
    normal = finite & (ax >= tiny)
    m, ex = np.frexp(ax[normal])  # ax = m * 2^ex, m in [0.5, 1)
    e[normal] = (ex - 1 + bias).astype(np.uint64)
    mant[normal] = ((2 * m - 1) * 2.0 ** mant_bits).astype(np.uint64)
    sub = finite & (ax < tiny)
    mant[sub] = (ax[sub] / 2.0 ** (1 - bias - mant_bits)).astype(np.uint64)
    e[~finite] = emax
    return e, sign, mant, np.isnan(x)


def test_split_bf16_matches_float_semantics():
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # bf16 is the top half of fp32
    e_exp, sign, mant, isnan = _expected_fields(x, 7, 127, 255)
    e, sm = orc.split(orc.BF16, v)
    assert np.array_equal(e.astype(np.uint64), e_exp)
    assert np.array_equal((sm >> 7).astype(np.uint64), sign)
    ok = ~isnan
    assert np.array_equal((sm[ok] & 0x7F).astype(np.uint64), mant[ok])
    assert np.all((sm[isnan] & 0x7F) != 0)  # NaN keeps a nonzero payload


def test_split_fp32_all_exponents_and_special_classes():
    rng = np.random.default_rng(11)
    exps = np.repeat(np.arange(256, dtype=np.uint32), 64)
    mants = rng.integers(0, 1 << 23, exps.size, dtype=np.uint32)
    mants[::64] = 0
    mants[1::64] = (1 << 23) - 1
    mants[2::64] = 1
    signs = rng.integers(0, 2, exps.size, dtype=np.uint32)
    v = (signs << 31) | (exps << 23) | mants
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001,
                        0x00000001, 0x807FFFFF, 0x00400000, 0x3F800000], np.uint32)
    v = np.concatenate([v, special])
    e, sm = orc.split(orc.FP32, v)
    assert np.array_equal(orc.merge(orc.FP32, e, sm), v)
    x = v.view(np.float32).astype(np.float64)
    e_exp, sign, mant, isnan = _expected_fields(x, 23, 127, 255)
    assert np.array_equal(e.astype(np.uint64), e_exp)
    s24 = sm[0::3].astype(np.uint64) | (sm[1::3].astype(np.uint64) << 8) | (sm[2::3].astype(np.uint64) << 16)
    assert np.array_equal(s24 >> 23, sign)
    ok = ~isnan
    assert np.array_equal((s24 & 0x7FFFFF)[ok], mant[ok])


# --------------------------------------------------------------------------
# P2: histogram == numpy.bincount
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_histogram_is_bincount(seed):
    rng = np.random.default_rng(seed)
    e = rng.geometric(0.3, 50_000).clip(0, 255).astype(np.uint8) if seed else rng.integers(0, 256, 50_000).astype(
        np.uint8)
    assert np.array_equal(orc.histogram(e), np.bincount(e, minlength=256).astype(np.uint32))


# --------------------------------------------------------------------------
# P3: normalisation to 4096
# --------------------------------------------------------------------------
def test_normalize_hand_trace_t2():
    g = _gold("normalize_t2.json")
    counts = np.zeros(256, np.uint32)
    for k, v in g["counts"].items():
        counts[int(k)] = v
    f, nsym = orc.normalize(counts)
    assert nsym == 4
    for k, v in g["f"].items():
        assert f[int(k)] == v
    c0 = orc.cumulative(f)
    for k, v in g["c0"].items():
        assert c0[int(k)] == v


@pytest.mark.parametrize("n", [1, 5, 4096, 32768, 1 << 20])
def test_normalize_single_symbol_takes_whole_table(n):
    for s in (0, 1, 127, 200, 255):
        c = np.zeros(256, np.uint32)
        c[s] = n
        f, nsym = orc.normalize(c)
        assert nsym == 1 and f[s] == 4096 and f.sum() == 4096


@pytest.mark.parametrize("k", range(0, 9))
def test_normalize_equiprobable_power_of_two(k):
    syms = np.random.default_rng(k).choice(256, 1 << k, replace=False)
    for per in (1, 3, 1000):
        c = np.zeros(256, np.uint32)
        c[syms] = per
        f, nsym = orc.normalize(c)
        assert nsym == 1 << k
        assert np.all(f[syms] == 4096 >> k) and f.sum() == 4096


def _hamilton(counts):
    """Largest-remainder apportionment in exact rationals: reserve one slot
    per present symbol, give each floor(quota) of the rest, then the leftover
    slots to the largest fractional parts (lower symbol on ties)."""
    present = [s for s in range(len(counts)) if counts[s] > 0]
    n = sum(counts)
    R = 4096 - len(present)
    quota = {s: Fraction(counts[s] * R, n) for s in present}
    f = {s: 1 + math.floor(quota[s]) for s in present}
    left = R - sum(math.floor(q) for q in quota.values())
    order = sorted(present, key=lambda s: (-(quota[s] - math.floor(quota[s])), s))
    for s in order[:left]:
        f[s] += 1
    return f


def test_normalize_all_tiny_histograms_match_rational_hamilton():
    syms = [0, 7, 128, 255]
    checked = 0
    for n in range(1, 9):
        for comp in itertools.product(range(n + 1), repeat=4):
            if sum(comp) != n:
                continue
            c = np.zeros(256, np.uint32)
            for s, v in zip(syms, comp):
                c[s] = v
            f, _ = orc.normalize(c)
            want = _hamilton([int(x) for x in c])
            assert {s: int(f[s]) for s in range(256) if f[s]} == want
            checked += 1
    assert checked == 494


def test_normalize_random_histograms_invariants_and_quota_property():
    rng = np.random.default_rng(5)
    for trial in range(300):
        nsym = int(rng.integers(1, 257))
        syms = rng.choice(256, nsym, replace=False)
        n = int(rng.integers(nsym, 1 << 20))
        if trial % 3 == 0:  # adversarial: one dominant symbol, the rest singletons
            cnt = np.ones(nsym, np.int64)
            cnt[0] = n - (nsym - 1)
        else:
            cnt = rng.multinomial(n - nsym, rng.dirichlet(np.full(nsym, 0.3))) + 1
        c = np.zeros(256, np.uint32)
        c[syms] = cnt
        f, k = orc.normalize(c)
        assert k == nsym
        assert int(f.sum()) == 4096
        assert np.array_equal(f > 0, c > 0)
        R = 4096 - nsym
        quota = c[syms].astype(np.float64) * R / n
        # Hamilton's quota property: every share is floor or ceil of the quota
        assert np.all(np.abs(f[syms].astype(np.float64) - 1 - quota) < 1.0)
        if trial % 50 == 0:
            want = _hamilton([int(x) for x in c])
            assert {s: int(f[s]) for s in range(256) if f[s]} == want


# --------------------------------------------------------------------------
# P4: rANS core -- hand traces, closed forms, brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["rans_k1_trace.json", "interleave_k2_trace.json", "renorm_boundary_t5.json"])
def test_rans_hand_traces(name):
    g = _gold(name)
    f, c0 = _table(g["table"])
    sym = np.array(g["symbols"], np.uint8)
    states, words = orc.rans_encode(sym, f, c0, lanes=g["lanes"])
    assert states.tolist() == g["final_states"]
    assert words.tolist() == g["words"]
    st, back = orc.rans_decode(states, words, sym.size, f, c0, lanes=g["lanes"])
    assert st == orc.OK and np.array_equal(back, sym)


def test_rans_t2_encode_no_words():
    g = _gold("normalize_t2.json")
    f = np.zeros(256, np.uint32)
    for k, v in g["f"].items():
        f[int(k)] = v
    c0 = orc.cumulative(f)
    states, words = orc.rans_encode(np.array(g["symbols"], np.uint8), f, c0, lanes=1)
    assert states.tolist() == g["final_states"] and words.tolist() == g["words"]


def test_rans_one_symbol_per_lane_t3():
    # four symbols with f = 1024: lane j ends at (65536/1024)*4096 + c0 = 262144 + 1024 j
    f = np.zeros(256, np.uint32)
    sy = [10, 20, 30, 40]
    f[sy] = 1024
    c0 = orc.cumulative(f)
    states, words = orc.rans_encode(np.array(sy, np.uint8), f, c0, lanes=32)
    assert words.size == 0
    assert states[:4].tolist() == [262144, 263168, 264192, 265216]
    assert np.all(states[4:] == 65536)


def test_rans_single_symbol_is_identity_on_state():
    # f = 4096: x -> (x/4096)*4096 + x mod 4096 = x, never renormalises
    f = np.zeros(256, np.uint32)
    f[77] = 4096
    c0 = orc.cumulative(f)
    states, words = orc.rans_encode(np.full(5000, 77, np.uint8), f, c0)
    assert words.size == 0 and np.all(states == 65536)


def _roundtrip_seq(seq, lanes):
    sym = np.array(seq, np.uint8)
    f, _ = orc.normalize(np.bincount(sym, minlength=256).astype(np.uint32))
    c0 = orc.cumulative(f)
    states, words = orc.rans_encode(sym, f, c0, lanes=lanes)
    st, back = orc.rans_decode(states, words, sym.size, f, c0, lanes=lanes)
    assert st == orc.OK, seq
    assert np.array_equal(back, sym), seq
    assert np.all(states >= 65536)


def test_rans_bruteforce_all_short_sequences_over_four_symbols():
    alphabet = [3, 100, 101, 250]
    for length in range(1, 7):
        for seq in itertools.product(alphabet, repeat=length):
            _roundtrip_seq(seq, 1)
            _roundtrip_seq(seq, 32)


def test_rans_bruteforce_all_pairs_over_256_symbols():
    for a in range(256):
        for b in range(0, 256, 3 if a % 2 else 1):
            _roundtrip_seq((a, b), 1)


def test_every_single_exponent_chunk_roundtrips_with_zero_words():
    for s in range(256):
        v = np.full(1000, (s << 7) | 0x15, np.uint16)
        buf = orc.compress(orc.BF16, v)
        _, _, recs = parse_buffer(buf)
        assert recs[0]["mode"] == 0 and recs[0]["n_words"] == 0 and recs[0]["f"] == {s: 4096}
        assert recs[0]["states"] == [65536] * 32
        st, back = orc.decompress(buf, orc.BF16, v.size)
        assert st == orc.OK and np.array_equal(back, v)


# --------------------------------------------------------------------------
# P5: coded size against the entropy
# --------------------------------------------------------------------------
def _check_entropy_invariants(dtype, bits, gaussian):
    buf = orc.compress(dtype, bits)
    hdr, idx, recs = parse_buffer(buf)
    e, _ = orc.split(dtype, bits)
    ce = hdr["chunk_elems"]
    for i, rec in enumerate(recs):
        chunk = e[i * ce:(i + 1) * ce]
        cnt = np.bincount(chunk, minlength=256)
        if rec["mode"] != 0 or chunk.size < 4096:
            continue
        f = rec["f"]
        cross = -sum(cnt[s] * math.log2(f[s] / 4096.0) for s in f)
        assert 16 * rec["n_words"] <= cross + 0.01 * chunk.size, (i, rec["n_words"], cross)
        if gaussian:
            # words + final states within 2048 bits of N_i * H(empirical)
            assert 16 * rec["n_words"] + 32 * 32 <= entropy_bits(cnt) + 2048, i


def test_entropy_invariant_pr1():
    _check_entropy_invariants(orc.BF16, workloads.bits_numpy(workloads.pr1()), True)


def test_entropy_invariant_gradient_bucket_small():
    t = workloads.gradient_bucket(1 << 21, device="cpu", seed=1, special_frac=1e-3)
    _check_entropy_invariants(orc.BF16, workloads.bits_numpy(t), True)


def test_entropy_invariant_fp32_small():
    t = workloads.fp32_gradients(65536 * 6 + 1000, device="cpu", seed=3)
    _check_entropy_invariants(orc.FP32, workloads.bits_numpy(t), True)


def entropy_bound_bytes(dtype, bits, chunk_elems):
    e, _ = orc.split(dtype, bits)
    w = orc.raw_bits(dtype)
    total = 0.0
    for i in range(0, e.size, chunk_elems):
        c = e[i:i + chunk_elems]
        total += w * c.size / 8.0 + entropy_bits(np.bincount(c, minlength=256)) / 8.0
    return total


def test_pr1_ratio_within_one_percent_of_entropy_bound():
    bits = workloads.bits_numpy(workloads.pr1())
    buf = orc.compress(orc.BF16, bits)
    bound = entropy_bound_bytes(orc.BF16, bits, 32768)
    orig = bits.size * 2
    assert 0.655 < bound / orig < 0.663  # H ~ 2.54 bits per exponent
    assert buf.size <= 1.01 * bound


def test_page_anchor_uniform_bf16_ratio_near_64_percent():
    # UCCL-Zip P2P evaluation (text after Fig. 8): bf16 uniform in [-1, 1)
    # reaches about a 64% compressed/original size; loose band, the coder,
    # chunking and headers there differ.
    x = np.random.default_rng(9).uniform(-1, 1, 1 << 20).astype(np.float32)
    bits = workloads.bits_numpy(__import__("torch").from_numpy(x).to(__import__("torch").bfloat16))
    buf = orc.compress(orc.BF16, bits)
    assert 0.60 < buf.size / (2 * bits.size) < 0.66


# --------------------------------------------------------------------------
# P6: layout
# --------------------------------------------------------------------------
def test_format_worked_example_w1():
    g = _gold("format_w1.json")
    buf = orc.compress(g["dtype"], np.array(g["values"], np.uint16))
    assert buf.tobytes().hex() == "".join(g["hex_lines"])
    st, back = orc.decompress(buf, g["dtype"], 4)
    assert st == orc.OK and back.tolist() == g["values"]


@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32])
def test_empty_input_is_header_and_one_index_entry(dtype):
    buf = orc.compress(dtype, np.zeros(0, np.uint16 if dtype == orc.BF16 else np.uint32))
    assert buf.size == 80
    hdr, idx, recs = parse_buffer(buf)
    assert hdr["n"] == 0 and hdr["C"] == 0 and hdr["sm_off"] == 80 and hdr["exp_off"] == 80 and hdr["total"] == 80
    assert idx == [0] and recs == []
    assert orc.max_compressed_size(dtype, 0) == 80
    st, back = orc.decompress(buf, dtype, 0)
    assert st == orc.OK and back.size == 0


@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32])
def test_random_bits_go_raw_and_hit_the_exact_bound(dtype):
    n = 3 * (32768 if dtype == orc.BF16 else 65536) + 777
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << (16 if dtype == orc.BF16 else 32), n, dtype=np.uint64)
    bits = bits.astype(np.uint16 if dtype == orc.BF16 else np.uint32)
    buf = orc.compress(dtype, bits)
    _, _, recs = parse_buffer(buf)
    assert all(r["mode"] == 1 for r in recs)
    assert buf.size == orc.max_compressed_size(dtype, n)
    st, back = orc.decompress(buf, dtype, n)
    assert st == orc.OK and np.array_equal(back, bits)


def test_layout_offsets_and_zero_padding():
    bits = workloads.bits_numpy(workloads.gradient_bucket(100_003, seed=7, special_frac=1e-3))
    buf = orc.compress(orc.BF16, bits, chunk_bytes=2048)
    hdr, idx, recs = parse_buffer(buf)
    ce = 1024
    C = (bits.size + ce - 1) // ce
    assert hdr["C"] == C and hdr["chunk_elems"] == ce
    sm_off = (64 + 8 * (C + 1) + 15) // 16 * 16
    exp_off = (sm_off + bits.size + 15) // 16 * 16
    assert hdr["sm_off"] == sm_off and hdr["exp_off"] == exp_off and hdr["total"] == buf.size
    assert idx[0] == 0 and idx[-1] == buf.size - exp_off
    assert all(b - a == r["bytes"] and (a % 16 == 0) for a, b, r in zip(idx, idx[1:], recs))
    assert not buf[64 + 8 * (C + 1):sm_off].any() and not buf[sm_off + bits.size:exp_off].any()
    e, sm = orc.split(orc.BF16, bits)
    assert np.array_equal(buf[sm_off:sm_off + bits.size], sm)
    for i, r in enumerate(recs):
        raw = r["raw"]
        if r["mode"] == 1:
            n_i = r["n_values"]
            assert np.array_equal(np.frombuffer(raw[16:16 + n_i], np.uint8), e[i * ce:i * ce + n_i])
            assert not any(raw[16 + n_i:])
        else:
            end = (48 + 2 * r["nsym"] + 3) // 4 * 4 + 128 + 2 * r["n_words"]
            assert not any(raw[end:]) and not any(raw[48 + 2 * r["nsym"]:(48 + 2 * r["nsym"] + 3) // 4 * 4])


@pytest.mark.parametrize("n,mode", [(160, 1), (161, 1), (170, 1), (176, 1), (177, 0), (1000, 0)])
def test_mode_choice_tie_goes_raw(n, mode):
    # one exponent: the RANS record is align16(16 + 32 + 2*1 -> 52, + 128) =
    # 192 bytes; RAW is align16(16 + n).  n in 161..176 ties at 192 -> RAW.
    bits = np.full(n, (130 << 7) | 3, np.uint16)
    _, _, recs = parse_buffer(orc.compress(orc.BF16, bits))
    assert recs[0]["mode"] == mode
    assert recs[0]["bytes"] == (192 if mode == 0 else (16 + n + 15) // 16 * 16)


def test_mode_choice_small_chunks_go_raw():
    # a 64-value chunk cannot pay for 176+ bytes of table and states
    bits = workloads.bits_numpy(workloads.pr1())[:64]
    _, _, recs = parse_buffer(orc.compress(orc.BF16, bits))
    assert recs[0]["mode"] == 1 and recs[0]["bytes"] == 80


# --------------------------------------------------------------------------
# round trips over the edge cases the method has
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000, 32768 + 5, 65536 * 2 + 31])
def test_roundtrip_ragged_sizes(dtype, n):
    if dtype == orc.BF16:
        bits = workloads.bits_numpy(workloads.gradient_bucket(n, seed=n, special_frac=0.01))
    else:
        bits = workloads.bits_numpy(workloads.fp32_gradients(n, seed=n))
    buf = orc.compress(dtype, bits)
    assert buf.size <= orc.max_compressed_size(dtype, n)
    st, back = orc.decompress(buf, dtype, n)
    assert st == orc.OK and np.array_equal(back, bits)


def test_roundtrip_all_256_exponents_in_one_chunk():
    rng = np.random.default_rng(1)
    e = np.concatenate([np.arange(256), rng.integers(0, 256, 30000)]).astype(np.uint16)
    bits = ((rng.integers(0, 2, e.size) << 15) | (e << 7) | rng.integers(0, 128, e.size)).astype(np.uint16)
    buf = orc.compress(orc.BF16, bits)
    _, _, recs = parse_buffer(buf)
    st, back = orc.decompress(buf, orc.BF16, bits.size)
    assert st == orc.OK and np.array_equal(back, bits)


def test_invalid_chunk_sizes_rejected():
    assert orc.chunk_elems(orc.BF16, 65536) == 32768
    assert orc.chunk_elems(orc.FP32, 0) == 65536
    assert orc.chunk_elems(orc.BF16, 100) == 0  # not a multiple of 32 values
    assert orc.chunk_elems(orc.BF16, (1 << 21) + 64) == 0  # more than 2^20 values


# --------------------------------------------------------------------------
# P7: corruption is reported, never decoded into garbage
# --------------------------------------------------------------------------
def test_corruption_detected():
    bits = workloads.bits_numpy(workloads.pr1())[:100_000]
    buf = orc.compress(orc.BF16, bits)
    seen = 0
    for name, bad in _corruptions(buf):
        st, _ = orc.decompress(bad, orc.BF16, bits.size)
        assert st == orc.CORRUPT, name
        seen += 1
    assert seen == 24
    st, _ = orc.decompress(buf, orc.FP32, bits.size // 2)
    assert st == orc.CORRUPT
    st, _ = orc.decompress(buf[:40], orc.BF16, bits.size)
    assert st == orc.CORRUPT


def test_coded_record_longer_than_raw_is_rejected():
    """A coded record exists only because it is strictly smaller than the
    chunk's RAW record (the RAW rule of NCCLZ Sec. IV-C); a frame whose coded
    record is longer (non-canonical table {120: 4095, 121: 1} over 32,768
    values of exponent 121: 24,576 words, 49,344 bytes against 32,784 RAW) is
    corrupt, although its rANS stream itself decodes."""
    buf, values = long_record_frame(orc.rans_encode)
    hdr, idx, recs = parse_buffer(buf)
    rec = recs[0]
    assert rec["mode"] == 0 and rec["n_words"] == 24576 and rec["bytes"] == 49344
    assert rec["bytes"] > (16 + 32768 + 15) // 16 * 16 == 32784
    # the stream alone is valid: it decodes to the chunk's exponents
    f = np.zeros(256, np.uint32)
    f[120], f[121] = 4095, 1
    c0 = orc.cumulative(f)
    words_at = (16 + 32 + 2 * 2 + 3) // 4 * 4 + 128
    words = np.frombuffer(rec["raw"][words_at:words_at + 2 * 24576], "<u2")
    st, sym = orc.rans_decode(np.array(rec["states"], np.uint32), words, 32768, f, c0)
    assert st == orc.OK and np.all(sym == 121)
    # ...but the frame is rejected for the record length alone
    st, _ = orc.decompress(buf, orc.BF16, values.size)
    assert st == orc.CORRUPT
    # and the canonical frame of the same values is a RANS record of 0 words
    good = orc.compress(orc.BF16, values)
    st, back = orc.decompress(good, orc.BF16, values.size)
    assert st == orc.OK and np.array_equal(back, values)
    assert parse_buffer(good)[2][0]["n_words"] == 0


def _raw_sized_records():
    """Two valid one-chunk frames (32,768 bf16 values, table {120: 4095, 121: 1},
    the first k values of exponent 121 and the rest 120): one whose coded
    record is exactly the RAW record's 32,784 bytes, one 16 bytes smaller."""
    out = {}
    for k in range(21700, 21900):
        sym = np.full(32768, 120, np.uint8)
        sym[:k] = 121
        buf, values = coded_frame(sym, {120: 4095, 121: 1}, orc.rans_encode)
        size = parse_buffer(buf)[2][0]["bytes"]
        if size in (32784, 32768) and size not in out:
            out[size] = (buf, values)
        if len(out) == 2:
            return out
    raise AssertionError("no k gives both record sizes")


def test_coded_record_bound_is_strict():
    """The bound is strict, as the mode rule is: a chunk is coded only when
    that is strictly smaller than RAW.  A coded record of exactly the RAW size
    (a valid stream) is rejected; one 16 bytes smaller is accepted."""
    recs = _raw_sized_records()
    buf, values = recs[32784]
    st, _ = orc.decompress(buf, orc.BF16, values.size)
    assert st == orc.CORRUPT
    buf, values = recs[32768]
    st, back = orc.decompress(buf, orc.BF16, values.size)
    assert st == orc.OK and np.array_equal(back, values)


# ---- fp16 and fp8 payloads (UCCL-Zip Fig. 13 types): the coded symbol is the
# exponent field alone, the sign and mantissa bits are packed raw (Figure 2) -----
def _unpack_fields(packed, n, w):
    """n fields of w bits from a byte string packed least significant bit
    first (numpy's little-endian bit order), as integers."""
    bits = np.unpackbits(np.asarray(packed, np.uint8), bitorder="little")[: n * w].reshape(n, w).astype(np.int64)
    return (bits << np.arange(w)).sum(axis=1)


def _float_fields(x, bias, mbits, emax_field):
    """Exponent field and mantissa field of finite values from their float
    semantics alone: a normal |x| = 2^(e - bias) (1 + m / 2^mbits), a
    subnormal |x| = 2^(1 - bias) m / 2^mbits (e = 0)."""
    ax = np.abs(x.astype(np.float64))
    f, k = np.frexp(ax)                      # ax = f 2^k, f in [0.5, 1)
    e = np.where(ax >= 2.0 ** (1 - bias), k - 1 + bias, 0)
    scale = np.where(e > 0, np.exp2((e - bias).astype(np.float64)), 2.0 ** (1 - bias))
    m = np.where(e > 0, (ax / scale - 1.0) * 2 ** mbits, ax / scale * 2 ** mbits)
    assert np.all(e <= emax_field) and np.all(m == np.round(m))
    return e.astype(np.int64), np.round(m).astype(np.int64)


@pytest.mark.parametrize("dtype,tdtype,bias,mbits,w", [
    (orc.FP16, torch.float16, 15, 10, 11), (orc.FP8_E4M3, torch.float8_e4m3fn, 7, 3, 4),
    (orc.FP8_E5M2, torch.float8_e5m2, 15, 2, 3)])
def test_split_narrow_types_exhaustive(dtype, tdtype, bias, mbits, w):
    """Every bit pattern of fp16, e4m3fn and e5m2: the symbol is the exponent
    field and the raw field holds the sign above the mantissa, both as the
    float semantics give them for finite values; NaN and Inf take the largest
    exponent field; the raw fields are packed at w bits each; merge inverts."""
    eb = 2 if dtype == orc.FP16 else 1
    v = np.arange(1 << (8 * eb), dtype=np.uint32).astype(orc._ELEM[dtype])
    e, sm = orc.split(dtype, v)
    assert orc.raw_bits(dtype) == w and orc.sym_bits(dtype) == 8 * eb - w
    assert sm.size == (v.size * w + 7) // 8
    raw = _unpack_fields(sm, v.size, w)
    x = torch.from_numpy(v.view(np.int16 if eb == 2 else np.uint8).copy()).view(tdtype).float().numpy()
    # the top bit of the raw field is the sign (NaN signs included)
    assert np.array_equal(raw >> (w - 1), (v >> (8 * eb - 1)).astype(np.int64))
    fin = np.isfinite(x)
    ef, mf = _float_fields(x[fin], bias, mbits, (1 << (8 * eb - 1 - mbits)) - 1)
    assert np.array_equal(e[fin].astype(np.int64), ef)
    assert np.array_equal(raw[fin] & ((1 << mbits) - 1), mf)
    assert np.array_equal((raw[fin] >> mbits).astype(bool), np.signbit(x[fin]))
    assert np.all(e[~fin] == (1 << (8 * eb - 1 - mbits)) - 1)  # NaN / Inf: the all-ones exponent
    assert np.array_equal(orc.merge(dtype, e, sm), v)


@pytest.mark.parametrize("name,n", [("format_w5_fp16.json", 4), ("format_w6_e4m3.json", 5), ("format_w7_e5m2.json", 3)])
def test_format_worked_examples_narrow_types(name, n):
    g = _gold(name)
    vals = np.array(g["values"], orc._ELEM[g["dtype"]])
    buf = orc.compress(g["dtype"], vals)
    assert buf.tobytes().hex() == "".join(g["hex_lines"])
    st, back = orc.decompress(buf, g["dtype"], n)
    assert st == orc.OK and back.tolist() == g["values"]


@pytest.mark.parametrize("dtype,ce,w,sb", [(orc.FP16, 32768, 11, 5), (orc.FP8_E4M3, 65536, 4, 4),
                                          (orc.FP8_E5M2, 65536, 3, 5), (orc.BF16, 32768, 8, 8),
                                          (orc.FP32, 65536, 24, 8)])
def test_header_raw_bits_and_packed_regions(dtype, ce, w, sb):
    """Header byte 9 holds the raw bits per value; the raw region is the
    packed raw fields; an incompressible chunk's RAW record holds its symbols
    packed at the exponent width, so the all-RAW frame is the input's bits
    rearranged plus framing."""
    n = 2 * ce + 77
    bits = np.random.default_rng(dtype).integers(0, 1 << (8 * orc._ELEM[dtype]().itemsize), n).astype(orc._ELEM[dtype])
    buf = orc.compress(dtype, bits)
    hdr, idx, recs = parse_buffer(buf)
    assert hdr["dtype"] == dtype and hdr["r"] == w and hdr["chunk_elems"] == ce and hdr["C"] == 3
    assert hdr["sm_off"] == (64 + 8 * 4 + 15) // 16 * 16
    assert hdr["exp_off"] == (hdr["sm_off"] + (w * n + 7) // 8 + 15) // 16 * 16
    assert orc.chunk_elems(dtype) == ce
    e, sm = orc.split(dtype, bits)
    assert np.array_equal(buf[hdr["sm_off"]:hdr["sm_off"] + sm.size], sm)
    if dtype in (orc.FP8_E4M3, orc.FP8_E5M2, orc.FP16):
        # uniformly random bits: the exponent field is near-uniform, a RANS
        # record cannot beat the packed RAW record by its table and states
        sizes = [(ce * sb + 7) // 8, (ce * sb + 7) // 8, (77 * sb + 7) // 8]
        for i, rec in enumerate(recs):
            if rec["mode"] != 1:
                continue
            body = np.frombuffer(rec["raw"][16:16 + sizes[i]], np.uint8)
            assert np.array_equal(_unpack_fields(body, recs[i]["n_values"], sb), e[i * ce:i * ce + rec["n_values"]])
    assert orc.max_compressed_size(dtype, n) == hdr["exp_off"] + sum(
        (16 + (k * sb + 7) // 8 + 15) // 16 * 16 for k in (ce, ce, 77))


@pytest.mark.parametrize("dtype", [orc.FP16, orc.FP8_E4M3, orc.FP8_E5M2])
@pytest.mark.parametrize("n", [0, 1, 31, 33, 1000, 65536 + 17])
def test_new_dtypes_roundtrip_ragged(dtype, n):
    rng = np.random.default_rng(n + 7 * dtype)
    if dtype == orc.FP16:
        bits = workloads.bits_numpy(workloads.fp16_activations(max(n, 1))[:n])
    else:
        fmt = torch.float8_e4m3fn if dtype == orc.FP8_E4M3 else torch.float8_e5m2
        bits = workloads.bits_numpy(workloads.fp8_weights(max(n, 1), fmt=fmt)[:n])
    bits = bits.copy()
    if n > 10:
        bits[rng.choice(n, 5, replace=False)] = rng.integers(0, 256, 5).astype(bits.dtype)  # any bit pattern
    buf = orc.compress(dtype, bits)
    st, back = orc.decompress(buf, dtype, n)
    assert st == orc.OK and np.array_equal(back, bits)
    assert buf.size <= orc.max_compressed_size(dtype, n)


@pytest.mark.parametrize("dtype", [orc.FP16, orc.FP8_E4M3, orc.FP8_E5M2])
def test_new_dtypes_entropy_invariants(dtype):
    if dtype == orc.FP16:
        t = workloads.fp16_activations(32768 * 4 + 100)
    else:
        t = workloads.fp8_weights(65536 * 3 + 100, fmt=torch.float8_e4m3fn if dtype == orc.FP8_E4M3 else torch.float8_e5m2)
    _check_entropy_invariants(dtype, workloads.bits_numpy(t), True)


@pytest.mark.parametrize("dtype", [orc.FP16, orc.FP8_E4M3, orc.FP8_E5M2])
def test_new_dtypes_within_one_percent_of_entropy_bound(dtype):
    # the coded symbol is the 4- or 5-bit exponent field: a chunk's table holds
    # at most 32 symbols, so the default chunk is within 1% (0.4-0.5% measured)
    if dtype == orc.FP16:
        bits = workloads.bits_numpy(workloads.fp16_activations(1 << 20))
    else:
        fmt = torch.float8_e4m3fn if dtype == orc.FP8_E4M3 else torch.float8_e5m2
        bits = workloads.bits_numpy(workloads.fp8_weights(1 << 21, fmt=fmt))
    cases = [(0, 1.01), (262144 if dtype != orc.FP16 else 131072, 1.01)]
    for chunk_bytes, tol in cases:
        buf = orc.compress(dtype, bits, chunk_bytes)
        bound = entropy_bound_bytes(dtype, bits, orc.chunk_elems(dtype, chunk_bytes))
        assert buf.size <= tol * bound, (chunk_bytes, buf.size / bound)


# --------------------------------------------------------------------------
# the entropy bound the compressed sizes are measured against
# --------------------------------------------------------------------------
def test_entropy_bound_closed_forms():
    """Per chunk: raw bytes + n_i H_i / 8.  A constant chunk has H = 0; a chunk
    of 2^k equally frequent exponents has H = k bits exactly; the histogram is
    per chunk (two constant chunks of different exponents have H = 0 each,
    where one histogram over both would give 1 bit)."""
    ce = 32768
    const = np.full(ce, 0x3F80, np.uint16)  # exponent 127
    assert orc.entropy_bound(orc.BF16, const) == ce
    for k in (1, 2, 3, 5, 8):
        e = np.arange(ce) % (1 << k)
        v = ((e + (0 if k == 8 else 100)) << 7).astype(np.uint16)
        assert orc.entropy_bound(orc.BF16, v) == pytest.approx(ce + ce * k / 8, abs=1e-6)
    two = np.concatenate([np.full(ce, 100 << 7, np.uint16), np.full(ce, 101 << 7, np.uint16)])
    assert orc.entropy_bound(orc.BF16, two) == 2 * ce
    # fp32: three raw bytes per value; a 256 KiB chunk of two exponents, half each
    f = np.where(np.arange(65536) % 2 == 0, 1.5, 3.0).astype(np.float32).view(np.uint32)
    assert orc.entropy_bound(orc.FP32, f) == pytest.approx(3 * 65536 + 65536 / 8, abs=1e-6)
    # a ragged last chunk is its own chunk
    tail = np.concatenate([np.full(ce, 100 << 7, np.uint16), (np.arange(64) % 4 + 100 << 7).astype(np.uint16)])
    assert orc.entropy_bound(orc.BF16, tail) == pytest.approx(ce + 64 + 64 * 2 / 8, abs=1e-6)


def test_entropy_bound_pr1_matches_the_independent_numpy_figure():
    """PR1 (1,048,576 bf16 values N(0, 0.02^2), seed 0): 0.6590 of the input,
    the figure computed independently with numpy when the workloads were
    specified."""
    b = workloads.bits_numpy(workloads.pr1())
    assert orc.entropy_bound(orc.BF16, b) / (2 * b.size) == pytest.approx(0.6590, abs=5e-5)


def _fp16_moved_symbol_frame():
    """A valid fp16 frame whose first coded record has its largest table
    symbol s moved to s + 32 in the bitmap (the frequency list stays in
    ascending order, the stream stays decodable): it names a symbol that no
    5-bit exponent field holds."""
    bits = workloads.bits_numpy(workloads.fp16_activations(40000))
    buf = orc.compress(orc.FP16, bits)
    hdr, idx, recs = parse_buffer(buf)
    ri = next(i for i, r in enumerate(recs) if r["mode"] == 0)
    s = max(recs[ri]["f"])
    assert s + 32 < 256
    bad = buf.copy()
    base = hdr["exp_off"] + idx[ri] + 16
    bad[base + s // 8] &= ~np.uint8(1 << (s % 8))
    bad[base + (s + 32) // 8] |= np.uint8(1 << ((s + 32) % 8))
    return bits, buf, bad


def _fp16_escape_out_of_range_frame():
    """A sampled-table fp16 frame of one chunk: every value 1.0 (exponent 15)
    except value 600, outside the eight sampled runs, whose exponent 20 is
    escaped; then the escape byte is changed to 52 (no 5-bit exponent)."""
    v = np.full(32768, 0x3C00, np.uint16)
    v[600] = (20 << 10) | 0x155
    buf = orc.compress_sampled(orc.FP16, v)
    hdr, idx, recs = parse_buffer(buf)
    rec = recs[0]
    assert rec["mode"] == 2
    raw = rec["raw"]
    tab_end = (48 + 2 * rec["nsym"] + 3) // 4 * 4
    assert int.from_bytes(raw[tab_end:tab_end + 4], "little") == 1  # one escape
    esc_at = tab_end + 4 + 128 + 2 * rec["n_words"]
    assert raw[esc_at] == 20
    bad = buf.copy()
    bad[hdr["exp_off"] + idx[0] + esc_at] = 52
    return v, buf, bad


def test_symbols_beyond_the_exponent_range_are_rejected():
    """A coded symbol is an exponent field value, below 2^SB (32 for fp16):
    a table or an escape naming a larger one is corrupt, although the rest of
    the record is consistent."""
    bits, good, bad = _fp16_moved_symbol_frame()
    assert orc.decompress(good, orc.FP16, bits.size)[0] == orc.OK
    assert orc.decompress(bad, orc.FP16, bits.size)[0] == orc.CORRUPT
    v, good, bad = _fp16_escape_out_of_range_frame()
    st, back = orc.decompress(good, orc.FP16, v.size)
    assert st == orc.OK and np.array_equal(back, v)
    assert orc.decompress(bad, orc.FP16, v.size)[0] == orc.CORRUPT
