"""Helpers shared by the oracle pins and the GPU parity tests: reading a v1
buffer back byte by byte, and the list of corruptions a decoder must report.
Nothing here computes the codec; it only reads and patches bytes."""
import numpy as np


def parse_buffer(buf):
    b = bytes(buf)
    hdr = dict(
        magic=int.from_bytes(b[0:4], "little"), version=int.from_bytes(b[4:6], "little"), dtype=b[6],
        prob_bits=b[7], lanes=b[8], r=b[9], chunk_elems=int.from_bytes(b[12:16], "little"),
        n=int.from_bytes(b[16:24], "little"), C=int.from_bytes(b[24:32], "little"),
        sm_off=int.from_bytes(b[32:40], "little"), exp_off=int.from_bytes(b[40:48], "little"),
        total=int.from_bytes(b[48:56], "little"))
    C = hdr["C"]
    idx = [int.from_bytes(b[64 + 8 * i:72 + 8 * i], "little") for i in range(C + 1)]
    recs = []
    for i in range(C):
        r = b[hdr["exp_off"] + idx[i]:hdr["exp_off"] + idx[i + 1]]
        mode, nsym = r[0], int.from_bytes(r[2:4], "little")
        n_words = int.from_bytes(r[4:8], "little")
        n_values = int.from_bytes(r[8:12], "little")
        rec = dict(mode=mode, nsym=nsym, n_words=n_words, n_values=n_values, bytes=len(r), raw=r)
        if mode == 0:
            bitmap = r[16:48]
            syms = [s for s in range(256) if (bitmap[s >> 3] >> (s & 7)) & 1]
            f = {s: int.from_bytes(r[48 + 2 * k:50 + 2 * k], "little") for k, s in enumerate(syms)}
            tab_end = (48 + 2 * nsym + 3) // 4 * 4
            states = [int.from_bytes(r[tab_end + 4 * j:tab_end + 4 * j + 4], "little") for j in range(32)]
            rec.update(f=f, states=states)
        recs.append(rec)
    return hdr, idx, recs


def corruptions(buf):
    hdr, idx, recs = parse_buffer(buf)
    exp_off = hdr["exp_off"]
    ri = next(i for i, r in enumerate(recs) if r["mode"] == 0)
    base = exp_off + idx[ri]
    rec = recs[ri]
    tab_end = (48 + 2 * rec["nsym"] + 3) // 4 * 4

    def patch(off, val, width):
        b = buf.copy()
        b[off:off + width] = np.frombuffer(int(val).to_bytes(width, "little"), np.uint8)
        return b

    yield "truncated", buf[:-16]
    yield "magic", patch(0, 0x31505A56, 4)
    yield "version", patch(4, 2, 2)
    yield "dtype", patch(6, 2, 1)
    yield "prob_bits", patch(7, 11, 1)
    yield "flags", patch(10, 2, 2)
    yield "count", patch(16, hdr["n"] + 1, 8)
    yield "chunk_elems", patch(12, 1000, 4)
    yield "sm_off", patch(32, hdr["sm_off"] + 16, 8)
    yield "total", patch(48, buf.size + 16, 8)
    yield "index_first", patch(64, 16, 8)
    yield "index_unaligned", patch(64 + 8 * (ri + 1), idx[ri + 1] + 2, 8)
    yield "index_decreasing", patch(64 + 8 * (ri + 1), idx[ri] - 16 if idx[ri] >= 16 else 0, 8)
    yield "rec_mode", patch(base, 2, 1)
    yield "rec_n_values", patch(base + 8, rec["n_values"] - 1, 4)
    yield "rec_bytes", patch(base + 12, rec["bytes"] + 16, 4)
    yield "rec_n_words_up", patch(base + 4, rec["n_words"] + 1, 4)
    yield "rec_n_words_down", patch(base + 4, rec["n_words"] - 8, 4)
    yield "nsym", patch(base + 2, rec["nsym"] + 1, 2)
    yield "freq_sum", patch(base + 48, rec["f"][min(rec["f"])] + 1, 2)
    yield "freq_zero", patch(base + 48, 0, 2)
    yield "state_low", patch(base + tab_end, 65535, 4)
    yield "state_value", patch(base + tab_end + 4, rec["states"][1] ^ 0x40, 4)
    yield "word", patch(base + tab_end + 128 + 2 * (rec["n_words"] // 2), 0x1234, 2)




def raw_corruptions(buf):
    """Corruptions of a buffer whose records are RAW: the header ones, and the
    record fields a RAW record must hold exactly (mode, nsym 0, n_words 0,
    n_values, rec_bytes = align16(16 + n_values))."""
    hdr, idx, recs = parse_buffer(buf)
    ri = next(i for i, r in enumerate(recs) if r["mode"] == 1)
    base = hdr["exp_off"] + idx[ri]
    rec = recs[ri]

    def patch(off, val, width):
        b = buf.copy()
        b[off:off + width] = np.frombuffer(int(val).to_bytes(width, "little"), np.uint8)
        return b

    yield "truncated", buf[:-16]
    yield "magic", patch(0, 0x31505A56, 4)
    yield "dtype", patch(6, 6, 1)
    yield "flags", patch(10, 2, 2)
    yield "count", patch(16, hdr["n"] + 1, 8)
    yield "total", patch(48, buf.size + 16, 8)
    yield "index_unaligned", patch(64 + 8 * (ri + 1), idx[ri + 1] + 2, 8)
    yield "raw_mode", patch(base, 2, 1)
    yield "raw_nsym", patch(base + 2, 1, 2)
    yield "raw_n_words", patch(base + 4, 1, 4)
    yield "raw_n_values", patch(base + 8, rec["n_values"] - 1, 4)
    yield "raw_bytes", patch(base + 12, rec["bytes"] - 16, 4)
    yield "raw_as_rans", patch(base, 0, 1)



def coded_frame(sym, ftab, rans_encode):
    """A bf16 frame of one chunk holding len(sym) <= 32,768 values whose
    exponents are `sym` (sign+mantissa 0), its record coded (mode 0) with the
    explicit table `ftab` ({symbol: frequency}, summing to 4096) whether or
    not that is canonical.  The states and words come from `rans_encode` (the
    oracle's coder), so the stream decodes.  Returns (frame, values)."""
    sym = np.ascontiguousarray(sym, np.uint8)
    n, ce = sym.size, 32768
    f = np.zeros(256, np.uint32)
    for k, v in ftab.items():
        f[k] = v
    c0 = np.concatenate([[0], np.cumsum(f)[:-1]]).astype(np.uint32)
    states, words = rans_encode(sym, f, c0)
    syms = sorted(ftab)
    nsym = len(syms)
    tab_end = (16 + 32 + 2 * nsym + 3) // 4 * 4
    words_at = tab_end + 4 * 32
    rec_bytes = (words_at + 2 * words.size + 15) // 16 * 16
    rec = np.zeros(rec_bytes, np.uint8)

    def put_to(a, off, val, width):
        a[off:off + width] = np.frombuffer(int(val).to_bytes(width, "little"), np.uint8)

    put_to(rec, 2, nsym, 2)
    put_to(rec, 4, words.size, 4)
    put_to(rec, 8, n, 4)
    put_to(rec, 12, rec_bytes, 4)
    for k, s_ in enumerate(syms):
        rec[16 + s_ // 8] |= 1 << (s_ % 8)
        put_to(rec, 48 + 2 * k, ftab[s_], 2)
    rec[tab_end:words_at] = states.astype("<u4").view(np.uint8)
    rec[words_at:words_at + 2 * words.size] = words.astype("<u2").view(np.uint8)
    C = 1
    sm_off = (64 + 8 * (C + 1) + 15) // 16 * 16
    exp_off = (sm_off + n + 15) // 16 * 16
    total = exp_off + rec_bytes
    buf = np.zeros(total, np.uint8)
    put_to(buf, 0, 0x31505A55, 4)
    put_to(buf, 4, 1, 2)
    buf[6], buf[7], buf[8], buf[9] = 1, 12, 32, 8
    put_to(buf, 12, ce, 4)
    put_to(buf, 16, n, 8)
    put_to(buf, 24, C, 8)
    put_to(buf, 32, sm_off, 8)
    put_to(buf, 40, exp_off, 8)
    put_to(buf, 48, total, 8)
    put_to(buf, 72, rec_bytes, 8)
    buf[exp_off:] = rec
    values = (sym.astype(np.uint16) << 7).astype(np.uint16)
    return buf, values


def long_record_frame(rans_encode):
    """One full 64 KiB bf16 chunk (32,768 values, all exponent 121) coded with
    the valid but non-canonical table {120: 4095, 121: 1}: every value costs
    ~12 bits, so the record (24,576 words, 49,344 bytes) is longer than the
    chunk's RAW record (32,784 bytes); only the record-length rule can reject
    the frame."""
    return coded_frame(np.full(32768, 121, np.uint8), {120: 4095, 121: 1}, rans_encode)
