"""Pins of the oracle's sampled-table frames (UCCL-Zip Sec. 3, Figure 5 text:
each block builds its table from a sample of its data).  The codec's reading:
a chunk's table comes from eight evenly spaced runs of its values (an eighth
of the chunk); a symbol the sample missed is coded as the escape symbol ESC,
which holds the last slot (f = 1, c0 = 4095), and its byte goes to the
record's escape list in value order; such frames set flag bit 0 of the
header and use record mode 2.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from test_oracle_pins import entropy_bound_bytes
from uzip_testlib import parse_buffer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mode2(rec):
    """Fields of a mode-2 record read back byte by byte."""
    r = rec["raw"]
    nsym = rec["nsym"]
    bitmap = r[16:48]
    syms = [s for s in range(256) if (bitmap[s >> 3] >> (s & 7)) & 1]
    f = [int.from_bytes(r[48 + 2 * k:50 + 2 * k], "little") for k in range(nsym)]
    tab_end = (48 + 2 * nsym + 3) // 4 * 4
    n_esc = int.from_bytes(r[tab_end:tab_end + 4], "little")
    states = [int.from_bytes(r[tab_end + 4 + 4 * j:tab_end + 8 + 4 * j], "little") for j in range(32)]
    words_at = tab_end + 4 + 128
    esc = list(r[words_at + 2 * rec["n_words"]:words_at + 2 * rec["n_words"] + n_esc])
    return dict(syms=syms, f=f, n_esc=n_esc, states=states, esc=esc, tab_end=tab_end)


def test_normalize_sampled_closed_forms():
    c = np.zeros(256, np.uint32)
    c[100] = 7
    assert orc.normalize_sampled(c, 7)[1][100] == 4095  # one symbol: all but ESC's slot
    c[:] = 0
    c[10] = c[20] = 5  # R = 4093, quotas 2046.5: one leftover slot, lower symbol first
    nsym, f = orc.normalize_sampled(c, 10)
    assert nsym == 2 and f[10] == 2048 and f[20] == 2047
    c[:] = 0
    c[[1, 2, 3, 4]] = 1  # R = 4091, quotas 1022.75: three leftover slots to symbols 1, 2, 3
    nsym, f = orc.normalize_sampled(c, 4)
    assert list(f[1:5]) == [1024, 1024, 1024, 1023]


def _hamilton_sampled(counts):
    """Independent largest-remainder apportionment with exact fractions over
    the sampled symbols plus ESC (count 0, last), one reserved slot each."""
    counts = [int(c) for c in counts]
    present = [s for s in range(256) if counts[s] > 0]
    S = sum(counts[s] for s in present)
    R = 4096 - len(present) - 1
    quota = {s: Fraction(counts[s] * R, S) for s in present}
    f = {s: 1 + (quota[s].numerator // quota[s].denominator) for s in present}
    left = R - sum(f[s] - 1 for s in present)
    order = sorted(present, key=lambda s: (-(quota[s] - (f[s] - 1)), s))
    for s in order[:left]:
        f[s] += 1
    return f


def test_normalize_sampled_against_exact_fractions():
    rng = np.random.default_rng(0)
    for trial in range(300):
        k = int(rng.integers(1, 40))
        syms = rng.choice(256, k, replace=False)
        c = np.zeros(256, np.uint32)
        c[syms] = rng.integers(1, 5000, k)
        nsym, f = orc.normalize_sampled(c, int(c.sum()))
        want = _hamilton_sampled(c)
        assert nsym == k and int(f.sum()) == 4095
        assert all(int(f[s]) == want[s] for s in want) and all(f[s] == 0 for s in range(256) if s not in want)


def test_worked_example_w4():
    g = json.load(open(os.path.join(GOLDEN, "sampled_w4.json")))
    e = np.full(g["n"], g["default_exponent"], np.uint16)
    for i, x in g["exponents"].items():
        e[int(i)] = x
    bits = (e << 7).astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, bits, g["chunk_bytes"])
    hdr, idx, recs = parse_buffer(buf)
    assert int.from_bytes(bytes(buf[10:12]), "little") == 1
    assert hdr["chunk_elems"] == 256 and hdr["sm_off"] == 80 and hdr["exp_off"] == 336 and hdr["total"] == g["total"]
    assert buf.size == g["total"] and idx == [0, g["rec_bytes"]] and not buf[80:336].any()
    rec = recs[0]
    assert rec["mode"] == 2 and rec["nsym"] == 1 and rec["n_words"] == 0 and rec["bytes"] == g["rec_bytes"]
    m = _mode2(rec)
    assert m["syms"] == [127] and m["f"] == [4095] and m["tab_end"] == 52 and m["esc"] == g["escapes"]
    want = [g["states"].get(str(j), g["states"]["default"]) for j in range(32)]
    assert m["states"] == want
    assert not any(rec["raw"][186:])  # zero padding
    st, back = orc.decompress(buf, orc.BF16, g["n"])
    assert st == orc.OK and np.array_equal(back, bits)


def test_sample_is_eight_spread_runs():
    # exponent = the value's index mod 256 over a chunk of 32768: the sample's
    # histogram is numpy's over the values whose index mod 4096 is below 512
    n = 32768
    e = (np.arange(n) % 256).astype(np.uint16)
    bits = (e << 7).astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, bits)
    _, _, recs = parse_buffer(buf)
    if recs[0]["mode"] == 2:
        m = _mode2(recs[0])
        sel = (np.arange(n) % 4096) < 512
        assert m["syms"] == sorted(set(np.unique(e[sel]).tolist()))
    # a chunk whose second half uses exponents its first half never does still
    # samples them: no escapes
    e = np.where(np.arange(n) < n // 2, 120 + (np.arange(n) % 4), 124 + (np.arange(n) % 4)).astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, ((e << 7) | (np.arange(n) & 0x7F)).astype(np.uint16))
    _, _, recs = parse_buffer(buf)
    assert recs[0]["mode"] == 2 and _mode2(recs[0])["n_esc"] == 0


def test_escapes_in_value_order_and_round_trip():
    rng = np.random.default_rng(3)
    n = 32768
    e = np.full(n, 127, np.uint16)
    period, run = 4096, 512
    unsampled = np.nonzero((np.arange(n) % period) >= run)[0]
    pos = np.sort(rng.choice(unsampled, 40, replace=False))
    e[pos] = rng.choice([90, 91, 200, 201], 40)
    bits = ((e << 7) | rng.integers(0, 2, n).astype(np.uint16) << 15 | rng.integers(0, 128, n).astype(np.uint16))
    bits = bits.astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, bits)
    _, _, recs = parse_buffer(buf)
    m = _mode2(recs[0])
    assert recs[0]["mode"] == 2 and m["syms"] == [127] and m["esc"] == e[pos].tolist()
    st, back = orc.decompress(buf, orc.BF16, n)
    assert st == orc.OK and np.array_equal(back, bits)


@pytest.mark.parametrize("dtype", [orc.BF16, orc.FP32, orc.FP16, orc.FP8_E4M3, orc.FP8_E5M2])
@pytest.mark.parametrize("n,chunk_bytes", [(0, 0), (1, 0), (33, 0), (1000, 0), (70001, 0), (5000, 64 * 4),
                                           (20011, 96 * 4), (131072 + 77, 0)])
def test_round_trips(dtype, n, chunk_bytes):
    eb = np.dtype(orc._ELEM[dtype]).itemsize
    chunk_bytes = chunk_bytes // 4 * eb if chunk_bytes else 0
    if dtype == orc.FP16:
        bits = workloads.bits_numpy(workloads.fp16_activations(max(n, 1))[:n])
    elif dtype in (orc.FP8_E4M3, orc.FP8_E5M2):
        fmt = torch.float8_e4m3fn if dtype == orc.FP8_E4M3 else torch.float8_e5m2
        bits = workloads.bits_numpy(workloads.fp8_weights(max(n, 1), fmt=fmt)[:n])
    elif dtype == orc.FP32:
        bits = workloads.bits_numpy(workloads.fp32_gradients(max(n, 1), seed=4)[:n])
    else:
        bits = workloads.bits_numpy(workloads.gradient_bucket(max(n, 1), seed=4, special_frac=1e-3)[:n])
    bits = bits.copy()
    buf = orc.compress_sampled(dtype, bits, chunk_bytes)
    assert buf.size <= orc.max_compressed_size(dtype, n, chunk_bytes)
    st, back = orc.decompress(buf, dtype, n)
    assert st == orc.OK and np.array_equal(back, bits)
    if n:
        assert int.from_bytes(bytes(buf[10:12]), "little") == 1
        _, _, recs = parse_buffer(buf)
        assert all(r["mode"] in (1, 2) for r in recs)


def test_special_cases():
    # random bits: every chunk RAW; one symbol everywhere: no escapes, no words
    for bits in [np.random.default_rng(1).integers(0, 1 << 16, 100_000).astype(np.uint16),
                 np.full(70_000, 0x3F80, np.uint16)]:
        buf = orc.compress_sampled(orc.BF16, bits)
        st, back = orc.decompress(buf, orc.BF16, bits.size)
        assert st == orc.OK and np.array_equal(back, bits)
    _, _, recs = parse_buffer(orc.compress_sampled(orc.BF16, np.full(70_000, 0x3F80, np.uint16)))
    assert [r["mode"] for r in recs] == [2, 2, 2]
    # all 256 fp8 values in every sample run: nsym 256, ESC never used
    v = np.tile(np.arange(256, dtype=np.uint16).astype(np.uint8), 512)
    buf = orc.compress_sampled(orc.FP8_E4M3, v)
    st, back = orc.decompress(buf, orc.FP8_E4M3, v.size)
    assert st == orc.OK and np.array_equal(back, v)


@pytest.mark.parametrize("name", ["grad", "pr1", "fp32", "fp16", "e4m3"])
def test_ratio_cost_of_sampling_is_small(name):
    if name == "grad":
        code, bits, ce = orc.BF16, workloads.bits_numpy(workloads.gradient_bucket(1 << 21, seed=1)), 32768
    elif name == "pr1":
        code, bits, ce = orc.BF16, workloads.bits_numpy(workloads.pr1()), 32768
    elif name == "fp32":
        code, bits, ce = orc.FP32, workloads.bits_numpy(workloads.fp32_gradients(1 << 20, seed=3)), 65536
    elif name == "fp16":
        code, bits, ce = orc.FP16, workloads.bits_numpy(workloads.fp16_activations(1 << 20)), 32768
    else:
        code, bits, ce = orc.FP8_E4M3, workloads.bits_numpy(workloads.fp8_weights(1 << 21, fmt=torch.float8_e4m3fn)), 65536
    full, samp = orc.compress(code, bits), orc.compress_sampled(code, bits)
    assert samp.size <= 1.002 * full.size
    if code in (orc.BF16, orc.FP32):
        assert samp.size <= 1.01 * entropy_bound_bytes(code, bits, ce)


def _patch(buf, off, val, width):
    b = buf.copy()
    b[off:off + width] = np.frombuffer(int(val).to_bytes(width, "little"), np.uint8)
    return b


def test_corruptions_of_sampled_frames():
    g = json.load(open(os.path.join(GOLDEN, "sampled_w4.json")))
    e = np.full(g["n"], 127, np.uint16)
    e[113], e[229] = 126, 130
    bits = (e << 7).astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, bits, g["chunk_bytes"])
    base = 336
    bad = {
        "flags_2": _patch(buf, 10, 2, 2),
        "flags_0": _patch(buf, 10, 0, 2),  # a mode-2 record in a full-histogram frame
        "mode_0": _patch(buf, base, 0, 1),
        "n_esc_up": _patch(buf, base + 52, 3, 4),
        "n_esc_down": _patch(buf, base + 52, 1, 4),
        "escape_is_sampled": _patch(buf, base + 184, 127, 1),
        "freq_sum": _patch(buf, base + 48, 4096, 2),
        "state": _patch(buf, base + 56 + 4 * 5, 268898759, 4),
    }
    for name, b in bad.items():
        assert orc.decompress(b, orc.BF16, g["n"])[0] == orc.CORRUPT, name
    # and a full-histogram frame with the flag set
    assert orc.decompress(_patch(orc.compress(orc.BF16, bits), 10, 1, 2), orc.BF16, g["n"])[0] == orc.CORRUPT


def test_sample_run_boundaries():
    # bf16, 64 KiB chunk: runs [4096 k, 4096 k + 512); index 511 is sampled,
    # 512 is not, 4095 is not, 4096 is
    n = 32768
    e = np.full(n, 127, np.uint16)
    e[511], e[512], e[4095], e[4096] = 51, 50, 53, 52
    bits = ((e << 7) | (np.arange(n) & 0x7F)).astype(np.uint16)
    buf = orc.compress_sampled(orc.BF16, bits)
    _, _, recs = parse_buffer(buf)
    m = _mode2(recs[0])
    assert recs[0]["mode"] == 2 and m["syms"] == [51, 52, 127] and m["esc"] == [50, 53]
    st, back = orc.decompress(buf, orc.BF16, n)
    assert st == orc.OK and np.array_equal(back, bits)
