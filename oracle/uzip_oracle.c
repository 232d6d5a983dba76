/*
 * uzip_oracle.c -- plain, slow, single-threaded CPU oracle of the uzip v1
 * bitstream (lossless bf16/fp32, and fp16/fp8, compression by exponent /
 * sign+mantissa split and 32-lane interleaved rANS of the exponent stream),
 * and of the per-call RAW arbitration.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP implementation; the two meet only through the byte
 * strings they produce.
 *
 * What the method is, and where each step comes from:
 *  - UCCL-Zip: Lossless Compression Supercharged GPU Communication
 *    (arXiv 2604.17172; review page on pith.science), Figure 2 and its body
 *    text: the floating-point ANS pipeline separates every value's exponent
 *    field from its sign and fraction bits and entropy-codes only the
 *    exponents; the sign and fraction are left as they are.
 *  - same page, Figure 5(b): each thread block builds its own local frequency
 *    table, so there is no global table and no cross-block synchronisation.
 *    Here: one table per fixed-size chunk, counted over the whole chunk.
 *  - NCCLZ: Compression-Enabled GPU Collectives with Decoupled Quantization
 *    and Entropy Coding (arXiv 2605.12396), Sec. IV-D2 "batch framing":
 *    every coded unit is a self-describing header + payload (codec id, raw
 *    size, payload size, codec parameters); Sec. IV-C / Algorithm 1: a RAW
 *    frame is committed when coding does not pay; Algorithm 2: the receiver
 *    validates the header before decoding.
 *  - UCCL-Zip review page, Figure 13: the payload types bfloat16, float16,
 *    float32, float8_e4m3fn and float8_e5m2.  For every type the coded symbol
 *    is the exponent field alone (Figure 2's split) and the sign and mantissa
 *    bits are stored raw, bit-packed (orc_split).
 *  - NCCLZ Sec. IV-C, Eq. (1) and (2), Algorithm 1: the runtime arbitration
 *    between coding and RAW from a bounded sample and a link/codec time
 *    model (orc_plan_call, orc_compress_arbitrated).
 *  - The pages give no formulas for the coder.  The textbook methods used
 *    where they are silent: J. Duda, "Asymmetric numeral systems" (arXiv
 *    1311.2540) for rANS with a 2^12 table, 32-bit state and 16-bit
 *    renormalisation; F. Giesen, "Interleaved entropy coders" (arXiv
 *    1402.3392) for the 32 interleaved lanes; largest-remainder (Hamilton)
 *    apportionment for the frequency table.
 *
 * Parity pins: every exported function is pinned by the -m "not gpu" tests
 * (hand-derived traces, closed forms, brute force, invariants, library
 * routines); none is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC -o liboracle.so uzip_oracle.c -lm
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- format constants of bitstream v1 --------------------------------- */
#define ORC_PROB_BITS 12
#define ORC_M 4096u            /* 2^PROB_BITS: total of the frequency table */
#define ORC_LANES 32           /* interleaved rANS lanes per chunk */
#define ORC_L 65536u           /* lower end of the normalised state interval */
#define ORC_MAGIC 0x31505A55u  /* "UZP1" little-endian */
#define ORC_VERSION 1
#define ORC_HDR_BYTES 64
#define ORC_REC_HDR 16
#define ORC_MAX_CHUNK_ELEMS (1u << 20)

#define ORC_DT_BF16 1
#define ORC_DT_FP32 2
#define ORC_DT_FP16 3
#define ORC_DT_FP8_E4M3 4
#define ORC_DT_FP8_E5M2 5

enum { ORC_OK = 0, ORC_INVALID = 1, ORC_CAPACITY = 2, ORC_CORRUPT = 3 };

static uint64_t orc_align16(uint64_t v) { return (v + 15u) & ~(uint64_t)15u; }
static uint64_t orc_align4(uint64_t v) { return (v + 3u) & ~(uint64_t)3u; }

/* little-endian stores / loads, byte by byte */
static void put16(uint8_t *p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t *p, uint32_t v) {
    for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k));
}
static void put64(uint8_t *p, uint64_t v) {
    for (int k = 0; k < 8; ++k) p[k] = (uint8_t)(v >> (8 * k));
}
static uint32_t get16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get32(const uint8_t *p) {
    uint32_t v = 0;
    for (int k = 0; k < 4; ++k) v |= (uint32_t)p[k] << (8 * k);
    return v;
}
static uint64_t get64(const uint8_t *p) {
    uint64_t v = 0;
    for (int k = 0; k < 8; ++k) v |= (uint64_t)p[k] << (8 * k);
    return v;
}

/* Bits of a value's sign+mantissa field (stored raw) and of its exponent
 * field (the coded symbol): bf16 1+7 and 8, fp32 1+23 and 8, fp16 1+10 and
 * 5, fp8 e4m3fn 1+3 and 4, fp8 e5m2 1+2 and 5. */
static int orc_raw_bits(int dtype) {
    switch (dtype) {
    case ORC_DT_BF16: return 8;
    case ORC_DT_FP32: return 24;
    case ORC_DT_FP16: return 11;
    case ORC_DT_FP8_E4M3: return 4;
    case ORC_DT_FP8_E5M2: return 3;
    default: return 0;
    }
}
static int orc_sym_bits(int dtype) {
    switch (dtype) {
    case ORC_DT_FP16: case ORC_DT_FP8_E5M2: return 5;
    case ORC_DT_FP8_E4M3: return 4;
    default: return 8;
    }
}

/* Bytes that n fields of w bits take when packed (see orc_put_bits). */
static uint64_t orc_packed_bytes(uint64_t n, int w) { return (n * (uint64_t)w + 7) / 8; }

/* Packing of w-bit fields, value order, least significant bit first: field i
 * occupies bits w*i .. w*i + w - 1 of the byte string, where bit k is bit
 * (k mod 8) of byte k / 8.  Eight-bit fields are plain bytes, 24-bit fields
 * three bytes little-endian.  dst must be zeroed beforehand. */
static void orc_put_bits(uint8_t *dst, uint64_t i, int w, uint32_t v) {
    for (int b = 0; b < w; ++b) {
        uint64_t k = i * (uint64_t)w + (uint64_t)b;
        if ((v >> b) & 1u) dst[k >> 3] |= (uint8_t)(1u << (k & 7));
    }
}
static uint32_t orc_get_bits(const uint8_t *src, uint64_t i, int w) {
    uint32_t v = 0;
    for (int b = 0; b < w; ++b) {
        uint64_t k = i * (uint64_t)w + (uint64_t)b;
        v |= (uint32_t)((src[k >> 3] >> (k & 7)) & 1u) << b;
    }
    return v;
}
static int orc_elem_bytes(int dtype) {
    switch (dtype) {
    case ORC_DT_BF16: case ORC_DT_FP16: return 2;
    case ORC_DT_FP32: return 4;
    case ORC_DT_FP8_E4M3: case ORC_DT_FP8_E5M2: return 1;
    default: return 0;
    }
}

/* chunk_bytes 0 selects the per-dtype default (256 KiB fp32, 64 KiB others).
 * Returns chunk_elems, or 0 when the chunk size is invalid. */
uint64_t orc_chunk_elems(int dtype, uint64_t chunk_bytes) {
    int eb = orc_elem_bytes(dtype);
    if (eb == 0) return 0;
    if (chunk_bytes == 0) chunk_bytes = dtype == ORC_DT_FP32 ? 262144u : 65536u;
    if (chunk_bytes % (uint64_t)(32 * eb) != 0) return 0;
    uint64_t ce = chunk_bytes / (uint64_t)eb;
    if (ce == 0 || ce > ORC_MAX_CHUNK_ELEMS) return 0;
    return ce;
}

/* ---- step 1: field split (UCCL-Zip Fig. 2) ------------------------------
 * Every value is split into its exponent field e (the coded symbol) and the
 * rest, sign and mantissa, which is stored raw: the sign becomes the top bit
 * of the raw field, above the mantissa bits.  The pages split every type
 * this way (only the exponent field is compressed):
 *   bf16 v:      e = bits 14..7  (8 bits), raw = sign << 7  | bits 6..0
 *   fp32 v:      e = bits 30..23 (8 bits), raw = sign << 23 | bits 22..0
 *   fp16 v:      e = bits 14..10 (5 bits), raw = sign << 10 | bits 9..0
 *   e4m3fn v:    e = bits 6..3   (4 bits), raw = sign << 3  | bits 2..0
 *   e5m2 v:      e = bits 6..2   (5 bits), raw = sign << 2  | bits 1..0
 * The raw fields are packed back to back in value order (orc_put_bits): one
 * byte per value for bf16, three bytes little-endian for fp32, 11, 4 and 3
 * bits for fp16 and the fp8 types.  e_out receives one byte per value (the
 * field's value); sm_out receives orc_packed_bytes(n, raw bits) bytes.
 * NaN payloads, infinities, subnormals and signed zeros pass through
 * unchanged: the split is a bijection of the bit pattern. */
static void orc_fields(int dtype, uint32_t v, uint32_t *e, uint32_t *raw) {
    switch (dtype) {
    case ORC_DT_BF16: *e = (v >> 7) & 0xFFu; *raw = ((v >> 15) << 7) | (v & 0x7Fu); break;
    case ORC_DT_FP32: *e = (v >> 23) & 0xFFu; *raw = ((v >> 31) << 23) | (v & 0x7FFFFFu); break;
    case ORC_DT_FP16: *e = (v >> 10) & 0x1Fu; *raw = ((v >> 15) << 10) | (v & 0x3FFu); break;
    case ORC_DT_FP8_E4M3: *e = (v >> 3) & 0xFu; *raw = ((v >> 7) << 3) | (v & 0x7u); break;
    default: *e = (v >> 2) & 0x1Fu; *raw = ((v >> 7) << 2) | (v & 0x3u); break; /* e5m2 */
    }
}
static uint32_t orc_join(int dtype, uint32_t e, uint32_t raw) {
    switch (dtype) {
    case ORC_DT_BF16: return ((raw >> 7) << 15) | (e << 7) | (raw & 0x7Fu);
    case ORC_DT_FP32: return ((raw >> 23) << 31) | (e << 23) | (raw & 0x7FFFFFu);
    case ORC_DT_FP16: return ((raw >> 10) << 15) | (e << 10) | (raw & 0x3FFu);
    case ORC_DT_FP8_E4M3: return ((raw >> 3) << 7) | (e << 3) | (raw & 0x7u);
    default: return ((raw >> 2) << 7) | (e << 2) | (raw & 0x3u);
    }
}
static uint32_t orc_load(int dtype, const void *in, uint64_t i) {
    switch (orc_elem_bytes(dtype)) {
    case 1: return ((const uint8_t *)in)[i];
    case 2: return ((const uint16_t *)in)[i];
    default: return ((const uint32_t *)in)[i];
    }
}
static void orc_store(int dtype, void *out, uint64_t i, uint32_t v) {
    switch (orc_elem_bytes(dtype)) {
    case 1: ((uint8_t *)out)[i] = (uint8_t)v; break;
    case 2: ((uint16_t *)out)[i] = (uint16_t)v; break;
    default: ((uint32_t *)out)[i] = v; break;
    }
}

void orc_split(int dtype, const void *in, uint64_t n, uint8_t *e_out, uint8_t *sm_out) {
    int w = orc_raw_bits(dtype);
    memset(sm_out, 0, (size_t)orc_packed_bytes(n, w));
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t e, raw;
        orc_fields(dtype, orc_load(dtype, in, i), &e, &raw);
        e_out[i] = (uint8_t)e;
        orc_put_bits(sm_out, i, w, raw);
    }
}

/* inverse of orc_split */
void orc_merge(int dtype, const uint8_t *e, const uint8_t *sm, uint64_t n, void *out) {
    int w = orc_raw_bits(dtype);
    for (uint64_t i = 0; i < n; ++i) orc_store(dtype, out, i, orc_join(dtype, e[i], orc_get_bits(sm, i, w)));
}

/* ---- step 2: histogram of the chunk's exponents (UCCL-Zip Fig. 5(b)) ----
 * A full count over every exponent of the chunk; no sampling. */
void orc_histogram(const uint8_t *e, uint64_t n, uint32_t counts[256]) {
    for (int s = 0; s < 256; ++s) counts[s] = 0;
    for (uint64_t i = 0; i < n; ++i) counts[e[i]] += 1;
}

/* ---- step 3: normalise the counts to a table summing to M = 4096 --------
 * Reserve one slot for each present symbol, share the remaining
 * R = M - nsym slots in proportion to the counts (floor of the quota), and
 * hand the d leftover slots to the symbols with the largest remainders,
 * lower symbol first on equal remainders (Hamilton / largest remainder).
 * n must equal the sum of the counts and be >= 1.  Returns nsym. */
int orc_normalize(const uint32_t counts[256], uint32_t n, uint32_t f[256]) {
    int nsym = 0;
    for (int s = 0; s < 256; ++s) {
        f[s] = 0;
        if (counts[s] > 0) nsym += 1;
    }
    if (nsym == 0) return 0;
    uint64_t R = ORC_M - (uint64_t)nsym;
    uint64_t rem[256];
    uint64_t given = 0;
    for (int s = 0; s < 256; ++s) {
        if (counts[s] == 0) continue;
        uint64_t q = (uint64_t)counts[s] * R;
        f[s] = 1u + (uint32_t)(q / n);
        rem[s] = q % n;
        given += q / n;
    }
    uint64_t d = R - given;
    /* hand out d extra slots, one at a time, each to the present symbol with
     * the largest remainder not yet served (lowest symbol on ties) */
    int served[256];
    for (int s = 0; s < 256; ++s) served[s] = 0;
    for (uint64_t k = 0; k < d; ++k) {
        int best = -1;
        for (int s = 0; s < 256; ++s) {
            if (counts[s] == 0 || served[s]) continue;
            if (best < 0 || rem[s] > rem[best]) best = s;
        }
        served[best] = 1;
        f[best] += 1;
    }
    return nsym;
}

/* cumulative frequencies in ascending symbol order */
void orc_cumulative(const uint32_t f[256], uint32_t c0[256]) {
    uint32_t acc = 0;
    for (int s = 0; s < 256; ++s) {
        c0[s] = acc;
        acc += f[s];
    }
}

/* ---- sampled tables (UCCL-Zip Sec. 3, Figure 5 text: each block builds its
 * table from a sample of its data) ------------------------------------------
 * The table of a chunk is normalised from the counts of a sample spread over
 * the chunk: value i belongs to it when i mod (chunk_elems / 8) is below
 * max(1, chunk_elems / 64), i.e. eight evenly spaced runs of contiguous values,
 * an eighth of a full chunk (so a chunk whose scale drifts, row by row, is
 * sampled throughout).  A symbol the sample did not see has
 * no slot of its own; it is coded as the escape symbol ESC, which always holds
 * exactly one slot, the last one (c0 = 4095), and its byte goes to the
 * record's escape list in value order.  The sampled symbols share the other
 * 4095 slots by the rule of orc_normalize: one reserved slot each, the rest
 * by the floor of each quota of R = 4096 - nsym - 1, and the leftover slots to
 * the largest remainders, lower symbol first.  (The same rule over nsym + 1
 * symbols with ESC last and counted 0 gives ESC exactly its reserved slot: the
 * leftover count is the sum of the fractional quotas, below the number of
 * symbols whose quota has one.)  Returns nsym, the sampled symbols. */
int orc_normalize_sampled(const uint32_t counts[256], uint32_t S, uint32_t f[256]) {
    int nsym = 0;
    for (int s = 0; s < 256; ++s) {
        f[s] = 0;
        if (counts[s] > 0) nsym += 1;
    }
    if (nsym == 0) return 0;
    uint64_t R = ORC_M - (uint64_t)nsym - 1;
    uint64_t rem[256];
    uint64_t given = 0;
    for (int s = 0; s < 256; ++s) {
        if (counts[s] == 0) continue;
        uint64_t q = (uint64_t)counts[s] * R;
        f[s] = 1u + (uint32_t)(q / S);
        rem[s] = q % S;
        given += q / S;
    }
    uint64_t d = R - given;
    int served[256];
    for (int s = 0; s < 256; ++s) served[s] = 0;
    for (uint64_t k = 0; k < d; ++k) {
        int best = -1;
        for (int s = 0; s < 256; ++s) {
            if (counts[s] == 0 || served[s]) continue;
            if (best < 0 || rem[s] > rem[best]) best = s;
        }
        served[best] = 1;
        f[best] += 1;
    }
    return nsym;
}

/* ---- step 4: interleaved rANS encode (Duda; Giesen) ----------------------
 * Value i belongs to lane i mod K and step i / K.  Every lane starts at
 * x = L.  Steps run from the last one down to 0.  For each lane with a value
 * at that step: if x >= f[s] * 2^20 the low 16 bits of x are emitted and x is
 * shifted down by 16; then x = (x / f) * M + (x mod f) + c0[s].
 * Words are returned in the order the decoder consumes them: step 0's words
 * (lanes ascending), then step 1's, and so on.  The encoder meets the groups
 * in the opposite order, so it fills its buffer from the end, one step group
 * at a time, lanes ascending inside the group.
 * words must hold n entries (at most one word per value).  Returns n_words. */
uint64_t orc_rans_encode(const uint8_t *sym, uint64_t n, int K, const uint32_t f[256], const uint32_t c0[256],
                         uint32_t *states, uint16_t *words) {
    for (int j = 0; j < K; ++j) states[j] = ORC_L;
    if (n == 0) return 0;
    uint64_t T = (n + (uint64_t)K - 1) / (uint64_t)K;
    uint16_t *group = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)K);
    uint64_t end = n; /* words so far occupy words[end .. n) */
    for (uint64_t t = T; t-- > 0;) {
        int cnt = 0;
        for (int j = 0; j < K; ++j) {
            uint64_t i = t * (uint64_t)K + (uint64_t)j;
            if (i >= n) continue;
            uint32_t s = sym[i];
            uint64_t x = states[j];
            uint64_t fs = f[s];
            if (x >= (fs << 20)) {
                group[cnt++] = (uint16_t)(x & 0xFFFFu);
                x >>= 16;
            }
            x = (x / fs) * ORC_M + (x % fs) + c0[s];
            states[j] = (uint32_t)x;
        }
        end -= (uint64_t)cnt;
        for (int k = 0; k < cnt; ++k) words[end + (uint64_t)k] = group[k];
    }
    free(group);
    uint64_t n_words = n - end;
    memmove(words, words + end, sizeof(uint16_t) * (size_t)n_words);
    return n_words;
}

/* ---- inverse: interleaved rANS decode ------------------------------------
 * For step t = 0, 1, ... and lanes ascending: slot = x mod M; s is the symbol
 * with c0[s] <= slot < c0[s] + f[s]; x = f[s] * (x >> 12) + slot - c0[s];
 * if x < L the next word is shifted in.  Returns ORC_OK, or ORC_CORRUPT when
 * the word stream runs out, a slot maps to no symbol, or the end state is not
 * L on every lane with every word consumed. */
int orc_rans_decode(const uint32_t *states_in, const uint16_t *words, uint64_t n_words, uint64_t n, int K,
                    const uint32_t f[256], const uint32_t c0[256], uint8_t *sym_out) {
    uint32_t *x = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)K);
    int16_t slot_sym[ORC_M];
    for (uint32_t k = 0; k < ORC_M; ++k) slot_sym[k] = -1;
    for (int s = 0; s < 256; ++s)
        for (uint32_t k = 0; k < f[s]; ++k)
            if (c0[s] + k < ORC_M) slot_sym[c0[s] + k] = (int16_t)s;
    for (int j = 0; j < K; ++j) x[j] = states_in[j];
    uint64_t pos = 0;
    int status = ORC_OK;
    uint64_t T = n == 0 ? 0 : (n + (uint64_t)K - 1) / (uint64_t)K;
    for (uint64_t t = 0; t < T && status == ORC_OK; ++t) {
        for (int j = 0; j < K; ++j) {
            uint64_t i = t * (uint64_t)K + (uint64_t)j;
            if (i >= n) continue;
            uint32_t slot = x[j] & (ORC_M - 1u);
            int s = slot_sym[slot];
            if (s < 0) { status = ORC_CORRUPT; break; }
            uint32_t nx = f[s] * (x[j] >> ORC_PROB_BITS) + slot - c0[s];
            if (nx < ORC_L) {
                if (pos >= n_words) { status = ORC_CORRUPT; break; }
                nx = (nx << 16) | words[pos++];
            }
            x[j] = nx;
            sym_out[i] = (uint8_t)s;
        }
    }
    if (status == ORC_OK) {
        for (int j = 0; j < K; ++j)
            if (x[j] != ORC_L) status = ORC_CORRUPT;
        if (pos != n_words) status = ORC_CORRUPT;
    }
    free(x);
    return status;
}

/* ---- buffer layout ------------------------------------------------------
 * [0,64) header | [64, 64+8(C+1)) u64 rec_off[C+1] | pad | raw region at
 * sm_off = align16(64+8(C+1)): the raw fields of all N values packed in value
 * order, ceil(raw_bits * N / 8) bytes | pad | records from
 * exp_off = align16(sm_off + ceil(raw_bits * N / 8)).
 * total = exp_off + rec_off[C]. */
static void orc_layout(int dtype, uint64_t n, uint64_t ce, uint64_t *C, uint64_t *sm_off, uint64_t *exp_off) {
    uint64_t c = (n + ce - 1) / ce;
    *C = c;
    *sm_off = orc_align16(ORC_HDR_BYTES + 8 * (c + 1));
    *exp_off = orc_align16(*sm_off + orc_packed_bytes(n, orc_raw_bits(dtype)));
}

/* Size of a chunk's RAW record: the 16-byte record header and the chunk's
 * symbols packed at the type's exponent width, padded to 16 bytes. */
static uint64_t orc_raw_record_bytes(int dtype, uint64_t ni) {
    return orc_align16(ORC_REC_HDR + orc_packed_bytes(ni, orc_sym_bits(dtype)));
}

uint64_t orc_max_compressed_size(int dtype, uint64_t n, uint64_t chunk_bytes) {
    uint64_t ce = orc_chunk_elems(dtype, chunk_bytes);
    if (ce == 0) return 0;
    uint64_t C, sm_off, exp_off;
    orc_layout(dtype, n, ce, &C, &sm_off, &exp_off);
    uint64_t total = exp_off;
    for (uint64_t i = 0; i < C; ++i) {
        uint64_t ni = (i + 1 < C) ? ce : n - i * ce;
        total += orc_raw_record_bytes(dtype, ni);
    }
    return total;
}

/* The entropy bound of a buffer in bytes: for every chunk, its raw
 * sign+mantissa bits / 8 plus n_i H_i / 8, where H_i is the empirical entropy
 * (bits per value) of the chunk's coded symbols, -sum_s (c_s / n_i)
 * log2(c_s / n_i) over the chunk's histogram.  It is the size an ideal coder
 * of each chunk's symbols with the chunk's own table would reach, with no
 * table, state or framing bytes; the compressed size is measured against it.
 * Computed in binary64. */
double orc_entropy_bound(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes) {
    uint64_t ce = orc_chunk_elems(dtype, chunk_bytes);
    if (ce == 0) return -1.0;
    int w = orc_raw_bits(dtype);
    uint8_t *e = (uint8_t *)malloc((size_t)(n ? n : 1));
    uint8_t *sm = (uint8_t *)malloc((size_t)(orc_packed_bytes(n, w) + 1));
    orc_split(dtype, in, n, e, sm);
    free(sm);
    double total = (double)w * (double)n / 8.0;
    for (uint64_t c0 = 0; c0 < n; c0 += ce) {
        uint64_t ni = n - c0 < ce ? n - c0 : ce;
        uint32_t counts[256];
        orc_histogram(e + c0, ni, counts);
        double bits = 0.0;
        for (int s = 0; s < 256; ++s) {
            if (counts[s] == 0) continue;
            double p = (double)counts[s] / (double)ni;
            bits -= (double)counts[s] * log2(p);
        }
        total += bits / 8.0;
    }
    free(e);
    return total;
}

/* The body of a RAW record: the chunk's symbols packed at sb bits. */
static void orc_raw_body(const uint8_t *e, uint64_t ni, int sb, uint8_t *body) {
    for (uint64_t i = 0; i < ni; ++i) orc_put_bits(body, i, sb, e[i]);
}

/* Encode one chunk's record (steps 2-4 plus the RANS/RAW choice) into rec,
 * which must hold orc_raw_record_bytes bytes.  sb: the symbols' width.
 * Returns the record size. */
static uint64_t orc_encode_record(const uint8_t *e, uint64_t ni, int sb, uint8_t *rec, int force_raw) {
    uint32_t counts[256], f[256], c0[256], states[ORC_LANES];
    orc_histogram(e, ni, counts);
    int nsym = orc_normalize(counts, (uint32_t)ni, f);
    orc_cumulative(f, c0);
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(ni ? ni : 1));
    uint64_t n_words = orc_rans_encode(e, ni, ORC_LANES, f, c0, states, words);
    uint64_t tab_end = orc_align4(ORC_REC_HDR + 32 + 2 * (uint64_t)nsym);
    uint64_t words_at = tab_end + 4 * ORC_LANES;
    uint64_t rans_bytes = orc_align16(words_at + 2 * n_words);
    uint64_t raw_bytes = orc_align16(ORC_REC_HDR + orc_packed_bytes(ni, sb));
    uint64_t rec_bytes;
    if (!force_raw && rans_bytes < raw_bytes) {
        rec_bytes = rans_bytes;
        memset(rec, 0, (size_t)rec_bytes);
        rec[0] = 0; /* mode RANS */
        put16(rec + 2, (uint32_t)nsym);
        put32(rec + 4, (uint32_t)n_words);
        put32(rec + 8, (uint32_t)ni);
        put32(rec + 12, (uint32_t)rec_bytes);
        int k = 0;
        for (int s = 0; s < 256; ++s) {
            if (f[s] == 0) continue;
            rec[16 + (s >> 3)] |= (uint8_t)(1u << (s & 7));
            put16(rec + 48 + 2 * k, f[s]);
            k += 1;
        }
        for (int j = 0; j < ORC_LANES; ++j) put32(rec + tab_end + 4 * (uint64_t)j, states[j]);
        for (uint64_t w = 0; w < n_words; ++w) put16(rec + words_at + 2 * w, words[w]);
    } else {
        rec_bytes = raw_bytes;
        memset(rec, 0, (size_t)rec_bytes);
        rec[0] = 1; /* mode RAW */
        put32(rec + 8, (uint32_t)ni);
        put32(rec + 12, (uint32_t)rec_bytes);
        orc_raw_body(e, ni, sb, rec + ORC_REC_HDR);
    }
    free(words);
    return rec_bytes;
}

/* One chunk's record in a sampled-table frame: mode 2 (coded with a table
 * from the chunk's sample and an escape list) when strictly smaller than the
 * RAW record, else RAW.  Layout of mode 2: the 16-byte header (mode 2, nsym,
 * n_words, n_values, rec_bytes), the bitmap of the sampled symbols, their
 * frequencies (ascending symbol), zero padding to 4 bytes, u32 n_esc, the 32
 * final states, the words, the n_esc escaped bytes in value order, zero
 * padding to 16 bytes.  The coder works on ranks: rank r < nsym is the r-th
 * sampled symbol, rank nsym is ESC (f = 1, c0 = 4095). */
/* counts of the chunk's sample (see above); returns its size S >= 1 for ni >= 1 */
uint64_t orc_sample_counts(const uint8_t *e, uint64_t ni, uint64_t ce, uint32_t counts[256]) {
    uint64_t period = ce / 8, run = ce / 64 > 0 ? ce / 64 : 1, S = 0;
    for (int s = 0; s < 256; ++s) counts[s] = 0;
    for (uint64_t i = 0; i < ni; ++i) {
        if (i % period < run) {
            counts[e[i]] += 1;
            S += 1;
        }
    }
    return S;
}

static uint64_t orc_encode_record_sampled(const uint8_t *e, uint64_t ni, uint64_t ce, int sb, uint8_t *rec) {
    uint32_t counts[256], f[256], c0[256], states[ORC_LANES];
    uint64_t S = orc_sample_counts(e, ni, ce, counts);
    int nsym = orc_normalize_sampled(counts, (uint32_t)S, f);
    orc_cumulative(f, c0);
    /* rank tables: the sampled symbols in ascending order, then ESC */
    uint32_t fr[256], cr[256];
    int rank[256];
    int r = 0;
    for (int s = 0; s < 256; ++s) {
        rank[s] = -1;
        if (f[s] == 0) continue;
        rank[s] = r;
        fr[r] = f[s];
        cr[r] = c0[s];
        r += 1;
    }
    for (int k = r; k < 256; ++k) fr[k] = cr[k] = 0;
    if (nsym < 256) {
        fr[nsym] = 1;
        cr[nsym] = ORC_M - 1;
    }
    uint8_t *m = (uint8_t *)malloc((size_t)(ni ? ni : 1));
    uint8_t *esc = (uint8_t *)malloc((size_t)(ni ? ni : 1));
    uint64_t n_esc = 0;
    for (uint64_t i = 0; i < ni; ++i) {
        if (rank[e[i]] >= 0) {
            m[i] = (uint8_t)rank[e[i]];
        } else {  /* unseen by the sample (so nsym < 256) */
            m[i] = (uint8_t)nsym;
            esc[n_esc++] = e[i];
        }
    }
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(ni ? ni : 1));
    uint64_t n_words = orc_rans_encode(m, ni, ORC_LANES, fr, cr, states, words);
    uint64_t tab_end = orc_align4(ORC_REC_HDR + 32 + 2 * (uint64_t)nsym);
    uint64_t states_at = tab_end + 4, words_at = states_at + 4 * ORC_LANES;
    uint64_t esc_at = words_at + 2 * n_words;
    uint64_t coded_bytes = orc_align16(esc_at + n_esc);
    uint64_t raw_bytes = orc_align16(ORC_REC_HDR + orc_packed_bytes(ni, sb));
    uint64_t rec_bytes;
    if (coded_bytes < raw_bytes) {
        rec_bytes = coded_bytes;
        memset(rec, 0, (size_t)rec_bytes);
        rec[0] = 2; /* mode: coded with a sampled table */
        put16(rec + 2, (uint32_t)nsym);
        put32(rec + 4, (uint32_t)n_words);
        put32(rec + 8, (uint32_t)ni);
        put32(rec + 12, (uint32_t)rec_bytes);
        int k = 0;
        for (int s = 0; s < 256; ++s) {
            if (f[s] == 0) continue;
            rec[16 + (s >> 3)] |= (uint8_t)(1u << (s & 7));
            put16(rec + 48 + 2 * k, f[s]);
            k += 1;
        }
        put32(rec + tab_end, (uint32_t)n_esc);
        for (int j = 0; j < ORC_LANES; ++j) put32(rec + states_at + 4 * (uint64_t)j, states[j]);
        for (uint64_t w = 0; w < n_words; ++w) put16(rec + words_at + 2 * w, words[w]);
        memcpy(rec + esc_at, esc, (size_t)n_esc);
    } else {
        rec_bytes = raw_bytes;
        memset(rec, 0, (size_t)rec_bytes);
        rec[0] = 1;
        put32(rec + 8, (uint32_t)ni);
        put32(rec + 12, (uint32_t)rec_bytes);
        orc_raw_body(e, ni, sb, rec + ORC_REC_HDR);
    }
    free(m);
    free(esc);
    free(words);
    return rec_bytes;
}

/* Whole-buffer compression.  out must hold cap >= orc_max_compressed_size
 * bytes.  *out_size receives the exact compressed size.  force_raw stores
 * every record RAW (the frame a RAW plan commits). */
static int orc_compress_frame(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes, uint8_t *out, uint64_t cap,
                              uint64_t *out_size, int force_raw, int sampled) {
    uint64_t ce = orc_chunk_elems(dtype, chunk_bytes);
    if (ce == 0) return ORC_INVALID;
    if (cap < orc_max_compressed_size(dtype, n, chunk_bytes)) return ORC_CAPACITY;
    int w = orc_raw_bits(dtype), sb = orc_sym_bits(dtype);
    uint64_t C, sm_off, exp_off;
    orc_layout(dtype, n, ce, &C, &sm_off, &exp_off);
    uint8_t *e = (uint8_t *)malloc((size_t)(n ? n : 1));
    const uint64_t sm_bytes = orc_packed_bytes(n, w);
    uint8_t *sm = (uint8_t *)malloc((size_t)(sm_bytes > 0 ? sm_bytes : 1));
    orc_split(dtype, in, n, e, sm);
    memset(out, 0, (size_t)exp_off);
    memcpy(out + sm_off, sm, (size_t)sm_bytes);
    uint64_t off = 0;
    put64(out + ORC_HDR_BYTES, 0);
    for (uint64_t i = 0; i < C; ++i) {
        uint64_t ni = (i + 1 < C) ? ce : n - i * ce;
        off += sampled && !force_raw ? orc_encode_record_sampled(e + i * ce, ni, ce, sb, out + exp_off + off)
                                     : orc_encode_record(e + i * ce, ni, sb, out + exp_off + off, force_raw);
        put64(out + ORC_HDR_BYTES + 8 * (i + 1), off);
    }
    uint64_t total = exp_off + off;
    put32(out + 0, ORC_MAGIC);
    put16(out + 4, ORC_VERSION);
    out[6] = (uint8_t)dtype;
    out[7] = ORC_PROB_BITS;
    out[8] = ORC_LANES;
    out[9] = (uint8_t)w; /* raw bits per value */
    put16(out + 10, sampled ? 1u : 0u); /* flags: bit 0 = sampled tables */
    put32(out + 12, (uint32_t)ce);
    put64(out + 16, n);
    put64(out + 24, C);
    put64(out + 32, sm_off);
    put64(out + 40, exp_off);
    put64(out + 48, total);
    put64(out + 56, 0);
    free(e);
    free(sm);
    *out_size = total;
    return ORC_OK;
}

int orc_compress(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes, uint8_t *out, uint64_t cap,
                 uint64_t *out_size) {
    return orc_compress_frame(dtype, in, n, chunk_bytes, out, cap, out_size, 0, 0);
}

/* Whole-buffer compression with sampled tables (header flag bit 0). */
int orc_compress_sampled(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes, uint8_t *out, uint64_t cap,
                         uint64_t *out_size) {
    return orc_compress_frame(dtype, in, n, chunk_bytes, out, cap, out_size, 0, 1);
}

/* ---- per-call arbitration: code the call, or send it RAW ------------------
 * NCCLZ Sec. IV-C ("runtime entropy-coding arbitration", Eq. (1) and (2),
 * Algorithm 1): a call that is small goes RAW at once; otherwise a bounded
 * sample taken from the start of the payload predicts the coded size P, and
 * the time of each choice is modelled as
 *     T = alpha + P / beta_eff + lambda_enc * E + lambda_dec * D
 * (RAW: P = its frame size, no codec cost, no alpha).  Coding is admitted
 * only if the predicted frame is smaller than the RAW frame by at least the
 * minimum gain; the smaller T wins, RAW on ties.  Every quantity is an
 * integer, so that the decision is one fixed function of the input.
 * Readings where the pages leave the step open: the sample is the first
 * min(N, 65536 / bytes-per-value) values (at most 64 KiB, the pages' sample
 * bound); the coded-size prediction is the sample's empirical entropy per
 * value times N, plus each chunk's fixed record part and half a padding unit;
 * logarithms are 2^16 log2 x in integers, by the squaring method.
 * Algorithm 1 accepts a materialised coded frame only if it passes the same
 * checks on its realised size (capacity and gain); otherwise it commits the
 * RAW frame.  Capacity always holds here (a coded frame is never larger than
 * the RAW frame, whose size is the output's capacity); the gain check is the
 * admission rule with the realised size R in place of P:
 * R < P_raw and (P_raw - R) * 1000 >= min_gain * B.  A coded plan that fails
 * it becomes decision 3 and writes the all-RAW frame. */
typedef struct {
    uint64_t link_bytes_per_us;   /* beta_eff, > 0 */
    uint64_t encode_bytes_per_us; /* E = B / encode rate, rate > 0 */
    uint64_t decode_bytes_per_us; /* D = B / decode rate, rate > 0 */
    uint64_t fixed_ns;            /* alpha of a coded transfer */
    uint64_t small_bytes;         /* calls with B <= this go RAW unsampled */
    uint32_t exposed_encode_permil;
    uint32_t exposed_decode_permil;
    uint32_t min_gain_permil;
    uint32_t reserved;
} orc_policy;

typedef struct {
    uint32_t decision; /* 0 coded, 1 RAW by the cost model, 2 RAW as a small call,
                          3 RAW because the realised coded frame failed the gain check */
    uint32_t sample_values;
    uint64_t predicted_bytes;
    uint64_t raw_ns;
    uint64_t coded_ns;
} orc_plan;

#define ORC_SAMPLE_BYTES 65536u

/* 2^16 * log2(x) for x >= 1, rounded down, digit by digit: with
 * x = 2^y * z, z in [1, 2), each squaring of z doubles log2(z), and its
 * integer part is the next binary digit.  z is kept in fixed point with 31
 * fraction bits, truncated after every squaring, so the result is exact at
 * powers of two and at most one unit (plus the truncation, < 1e-5 unit)
 * below 2^16 log2(x) elsewhere. */
uint32_t orc_log2_q16(uint32_t x) {
    uint32_t y = 0;
    while ((x >> y) > 1u) y += 1;
    uint64_t z = (uint64_t)x << (31 - y);
    uint32_t frac = 0;
    for (int i = 0; i < 16; ++i) {
        z = (z * z) >> 31;
        frac <<= 1;
        if (z >= ((uint64_t)1 << 32)) {
            z >>= 1;
            frac |= 1u;
        }
    }
    return (y << 16) | frac;
}

static uint64_t orc_ceil_div(uint64_t a, uint64_t b) { return a / b + (a % b != 0); }

int orc_plan_call(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes, const orc_policy *pol, orc_plan *plan) {
    uint64_t ce = orc_chunk_elems(dtype, chunk_bytes);
    if (ce == 0 || pol->link_bytes_per_us == 0 || pol->encode_bytes_per_us == 0 || pol->decode_bytes_per_us == 0 ||
        pol->exposed_encode_permil > 1000 || pol->exposed_decode_permil > 1000 || pol->min_gain_permil > 1000 ||
        pol->reserved != 0)
        return ORC_INVALID;
    memset(plan, 0, sizeof(*plan));
    uint64_t eb = (uint64_t)orc_elem_bytes(dtype);
    uint64_t B = n * eb;
    /* Algorithm 1's fast path: a small call is committed RAW at once */
    if (B <= pol->small_bytes) {
        plan->decision = 2;
        return ORC_OK;
    }
    /* the bounded sample and its statistics */
    uint64_t S = n < ORC_SAMPLE_BYTES / eb ? n : ORC_SAMPLE_BYTES / eb;
    uint8_t *e = (uint8_t *)malloc((size_t)S);
    uint8_t *sm = (uint8_t *)malloc((size_t)(orc_packed_bytes(S, orc_raw_bits(dtype)) + 1));
    orc_split(dtype, in, S, e, sm);
    uint32_t counts[256];
    orc_histogram(e, S, counts);
    free(e);
    free(sm);
    uint64_t hs = 0; /* sample entropy in bits, times 2^16 */
    uint32_t nsym = 0;
    for (int s = 0; s < 256; ++s) {
        if (counts[s] == 0) continue;
        nsym += 1;
        hs += (uint64_t)counts[s] * (orc_log2_q16((uint32_t)S) - orc_log2_q16(counts[s]));
    }
    uint64_t h = hs / S; /* bits per value, times 2^16 */
    /* the predicted coded frame: header, index and raw bytes as laid out,
     * the coded symbols at the sample's entropy, each record's fixed part */
    uint64_t C, sm_off, exp_off;
    orc_layout(dtype, n, ce, &C, &sm_off, &exp_off);
    uint64_t rec_fixed = orc_align4(ORC_REC_HDR + 32 + 2 * (uint64_t)nsym) + 4 * ORC_LANES + 8;
    uint64_t P = exp_off + orc_ceil_div(n * h, (uint64_t)1 << 19) + C * rec_fixed;
    uint64_t P_raw = orc_max_compressed_size(dtype, n, chunk_bytes);
    /* Eq. (1) for RAW and for coding, in nanoseconds */
    uint64_t t_raw = orc_ceil_div(P_raw * 1000, pol->link_bytes_per_us);
    uint64_t t_code = pol->fixed_ns + orc_ceil_div(P * 1000, pol->link_bytes_per_us) +
                      orc_ceil_div((uint64_t)pol->exposed_encode_permil * B, pol->encode_bytes_per_us) +
                      orc_ceil_div((uint64_t)pol->exposed_decode_permil * B, pol->decode_bytes_per_us);
    /* admission (predicted gain at least the minimum), then Eq. (2) */
    int admitted = P < P_raw && (P_raw - P) * 1000 >= (uint64_t)pol->min_gain_permil * B;
    plan->decision = (admitted && t_code < t_raw) ? 0u : 1u;
    plan->sample_values = (uint32_t)S;
    plan->predicted_bytes = P;
    plan->raw_ns = t_raw;
    plan->coded_ns = t_code;
    return ORC_OK;
}

/* Plan the call, write the frame the plan chose, and check a coded frame's
 * realised gain (Algorithm 1's acceptance of the materialised plan): one that
 * fails it is replaced by the RAW frame. */
int orc_compress_arbitrated(int dtype, const void *in, uint64_t n, uint64_t chunk_bytes, const orc_policy *pol,
                            orc_plan *plan, uint8_t *out, uint64_t cap, uint64_t *out_size) {
    int st = orc_plan_call(dtype, in, n, chunk_bytes, pol, plan);
    if (st != ORC_OK) return st;
    st = orc_compress_frame(dtype, in, n, chunk_bytes, out, cap, out_size, plan->decision != 0, 0);
    if (st != ORC_OK || plan->decision != 0) return st;
    uint64_t B = n * (uint64_t)orc_elem_bytes(dtype);
    uint64_t P_raw = orc_max_compressed_size(dtype, n, chunk_bytes);
    uint64_t R = *out_size;
    int accepted = R < P_raw && (P_raw - R) * 1000 >= (uint64_t)pol->min_gain_permil * B;
    if (accepted) return ORC_OK;
    plan->decision = 3;
    return orc_compress_frame(dtype, in, n, chunk_bytes, out, cap, out_size, 1, 0);
}

/* Decode one record into the chunk's exponents.  rec holds rec_len bytes
 * (already known to lie inside the buffer).  Checks V6-V9. */
static int orc_decode_record_sampled(const uint8_t *rec, uint64_t rec_len, uint64_t ni, uint32_t nsym,
                                     uint64_t n_words, int sb, uint8_t *e);

/* A table names only symbols the type's exponent field can hold (below 2^sb:
 * 32 for fp16 and e5m2, 16 for e4m3fn, all 256 for bf16 and fp32). */
static int orc_bitmap_in_range(const uint8_t *bitmap, int sb) {
    for (int s = 1 << sb; s < 256; ++s)
        if ((bitmap[s >> 3] >> (s & 7)) & 1u) return 0;
    return 1;
}

static int orc_decode_record(const uint8_t *rec, uint64_t rec_len, uint64_t ni, int sb, uint8_t *e, int sampled) {
    if (rec_len < ORC_REC_HDR) return ORC_CORRUPT;
    uint32_t mode = rec[0];
    uint32_t nsym = get16(rec + 2);
    uint64_t n_words = get32(rec + 4);
    uint64_t n_values = get32(rec + 8);
    uint64_t rec_bytes = get32(rec + 12);
    if (mode > 2 || n_values != ni || rec_bytes != rec_len) return ORC_CORRUPT;
    if (mode == 1) {
        if (nsym != 0 || n_words != 0 || rec_len != orc_align16(ORC_REC_HDR + orc_packed_bytes(ni, sb)))
            return ORC_CORRUPT;
        for (uint64_t i = 0; i < ni; ++i) e[i] = (uint8_t)orc_get_bits(rec + ORC_REC_HDR, i, sb);
        return ORC_OK;
    }
    /* a frame uses one kind of coded record: mode 0 (full histograms) or mode 2 (sampled) */
    if ((mode == 2) != (sampled != 0)) return ORC_CORRUPT;
    /* a coded record exists only because it is strictly smaller than the
     * chunk's RAW record (the RAW rule, NCCLZ Sec. IV-C); one that is not is
     * rejected, so no record is ever longer than its RAW record and the
     * all-RAW size bounds every valid frame */
    if (rec_len >= orc_align16(ORC_REC_HDR + orc_packed_bytes(ni, sb))) return ORC_CORRUPT;
    if (mode == 2) return orc_decode_record_sampled(rec, rec_len, ni, nsym, n_words, sb, e);
    /* RANS: bitmap, frequencies, states, words */
    if (rec_len < ORC_REC_HDR + 32) return ORC_CORRUPT;
    uint32_t pop = 0;
    for (int s = 0; s < 256; ++s) pop += (rec[16 + (s >> 3)] >> (s & 7)) & 1u;
    if (pop != nsym || nsym < 1 || nsym > 256 || !orc_bitmap_in_range(rec + 16, sb)) return ORC_CORRUPT;
    uint64_t tab_end = orc_align4(ORC_REC_HDR + 32 + 2 * (uint64_t)nsym);
    uint64_t words_at = tab_end + 4 * ORC_LANES;
    if (rec_len != orc_align16(words_at + 2 * n_words)) return ORC_CORRUPT;
    uint32_t f[256], c0[256], states[ORC_LANES];
    uint32_t sum = 0;
    int k = 0;
    for (int s = 0; s < 256; ++s) {
        f[s] = 0;
        if ((rec[16 + (s >> 3)] >> (s & 7)) & 1u) {
            f[s] = get16(rec + 48 + 2 * k);
            k += 1;
            if (f[s] == 0) return ORC_CORRUPT;
            sum += f[s];
        }
    }
    if (sum != ORC_M) return ORC_CORRUPT;
    orc_cumulative(f, c0);
    for (int j = 0; j < ORC_LANES; ++j) {
        states[j] = get32(rec + tab_end + 4 * (uint64_t)j);
        if (states[j] < ORC_L) return ORC_CORRUPT;
    }
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n_words ? n_words : 1));
    for (uint64_t w = 0; w < n_words; ++w) words[w] = (uint16_t)get16(rec + words_at + 2 * w);
    int st = orc_rans_decode(states, words, n_words, ni, ORC_LANES, f, c0, e);
    free(words);
    return st;
}

/* Whole-buffer decompression with validation V1-V9.  The caller states the
 * dtype and element count, as a receiver does.  Returns ORC_OK, or
 * ORC_CORRUPT for any inconsistency; never reads outside in[0, in_bytes). */
/* Mode 2: the sampled table, ESC in the last slot, the escape list in value
 * order.  Checks: bitmap and nsym agree (1..256), no symbol beyond the
 * exponent field's range, every frequency >= 1 and they sum to 4095, n_esc
 * and the words fit the record exactly, the rANS stream ends as in
 * orc_rans_decode, every escape of the list is used, and no escaped byte is a
 * sampled symbol (such a value would have been coded directly) or beyond the
 * exponent field's range. */
static int orc_decode_record_sampled(const uint8_t *rec, uint64_t rec_len, uint64_t ni, uint32_t nsym,
                                     uint64_t n_words, int sb, uint8_t *e) {
    if (rec_len < ORC_REC_HDR + 32) return ORC_CORRUPT;
    uint32_t pop = 0;
    for (int s = 0; s < 256; ++s) pop += (rec[16 + (s >> 3)] >> (s & 7)) & 1u;
    if (pop != nsym || nsym < 1 || nsym > 256 || !orc_bitmap_in_range(rec + 16, sb)) return ORC_CORRUPT;
    uint64_t tab_end = orc_align4(ORC_REC_HDR + 32 + 2 * (uint64_t)nsym);
    uint64_t states_at = tab_end + 4, words_at = states_at + 4 * ORC_LANES;
    if (rec_len < words_at) return ORC_CORRUPT;
    uint64_t n_esc = get32(rec + tab_end);
    if (n_esc > ni || rec_len != orc_align16(words_at + 2 * n_words + n_esc)) return ORC_CORRUPT;
    uint32_t fr[256], cr[256], states[ORC_LANES];
    uint8_t sym_of_rank[256];
    int present[256];
    uint32_t acc = 0;
    int k = 0;
    for (int s = 0; s < 256; ++s) {
        present[s] = (rec[16 + (s >> 3)] >> (s & 7)) & 1u;
        if (!present[s]) continue;
        uint32_t fs = get16(rec + 48 + 2 * k);
        if (fs == 0) return ORC_CORRUPT;
        fr[k] = fs;
        cr[k] = acc;
        sym_of_rank[k] = (uint8_t)s;
        acc += fs;
        k += 1;
    }
    if (acc != ORC_M - 1) return ORC_CORRUPT;
    for (int j = k; j < 256; ++j) fr[j] = cr[j] = 0;
    if (nsym < 256) {
        fr[nsym] = 1;
        cr[nsym] = ORC_M - 1;
    }
    for (int j = 0; j < ORC_LANES; ++j) {
        states[j] = get32(rec + states_at + 4 * (uint64_t)j);
        if (states[j] < ORC_L) return ORC_CORRUPT;
    }
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n_words ? n_words : 1));
    for (uint64_t w = 0; w < n_words; ++w) words[w] = (uint16_t)get16(rec + words_at + 2 * w);
    uint8_t *ranks = (uint8_t *)malloc((size_t)(ni ? ni : 1));
    int st = orc_rans_decode(states, words, n_words, ni, ORC_LANES, fr, cr, ranks);
    free(words);
    const uint8_t *esc = rec + words_at + 2 * n_words;
    uint64_t used = 0;
    for (uint64_t i = 0; i < ni && st == ORC_OK; ++i) {
        if (ranks[i] < nsym) {
            e[i] = sym_of_rank[ranks[i]];
        } else {  /* ESC (only reachable when nsym < 256) */
            if (used >= n_esc || present[esc[used]] || esc[used] >= (1u << sb)) st = ORC_CORRUPT;
            else e[i] = esc[used++];
        }
    }
    if (st == ORC_OK && used != n_esc) st = ORC_CORRUPT;
    free(ranks);
    return st;
}

int orc_decompress(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n, void *out) {
    int w = orc_raw_bits(dtype), sb = orc_sym_bits(dtype);
    if (orc_elem_bytes(dtype) == 0) return ORC_INVALID;
    if (in_bytes < ORC_HDR_BYTES) return ORC_CORRUPT;
    /* V1: magic, version and the fixed coder parameters */
    if (get32(in) != ORC_MAGIC || get16(in + 4) != ORC_VERSION) return ORC_CORRUPT;
    if (in[7] != ORC_PROB_BITS || in[8] != ORC_LANES || in[9] != (uint8_t)w) return ORC_CORRUPT;
    /* flags: bit 0 = sampled tables; no other bit is defined */
    uint32_t flags = get16(in + 10);
    if (flags > 1) return ORC_CORRUPT;
    /* V2: dtype and element count as the caller states them */
    if (in[6] != (uint8_t)dtype || get64(in + 16) != n) return ORC_CORRUPT;
    /* V3: chunk size and chunk count */
    uint64_t ce = get32(in + 12);
    if (ce == 0 || ce % 32 != 0 || ce > ORC_MAX_CHUNK_ELEMS) return ORC_CORRUPT;
    uint64_t C, sm_off, exp_off;
    orc_layout(dtype, n, ce, &C, &sm_off, &exp_off);
    if (get64(in + 24) != C) return ORC_CORRUPT;
    /* V4: region offsets and total size */
    uint64_t total = get64(in + 48);
    if (get64(in + 32) != sm_off || get64(in + 40) != exp_off) return ORC_CORRUPT;
    if (total > in_bytes || total < exp_off) return ORC_CORRUPT;
    /* V5: the record index */
    if (get64(in + ORC_HDR_BYTES) != 0) return ORC_CORRUPT;
    if (get64(in + ORC_HDR_BYTES + 8 * C) != total - exp_off) return ORC_CORRUPT;
    for (uint64_t i = 0; i < C; ++i) {
        uint64_t a = get64(in + ORC_HDR_BYTES + 8 * i), b = get64(in + ORC_HDR_BYTES + 8 * (i + 1));
        if (b < a || (a & 15u) != 0 || (b & 15u) != 0) return ORC_CORRUPT;
    }
    uint8_t *e = (uint8_t *)malloc((size_t)(n ? n : 1));
    int st = ORC_OK;
    for (uint64_t i = 0; i < C && st == ORC_OK; ++i) {
        uint64_t ni = (i + 1 < C) ? ce : n - i * ce;
        uint64_t a = get64(in + ORC_HDR_BYTES + 8 * i), b = get64(in + ORC_HDR_BYTES + 8 * (i + 1));
        st = orc_decode_record(in + exp_off + a, b - a, ni, sb, e + i * ce, (int)(flags & 1u));
    }
    if (st == ORC_OK) orc_merge(dtype, e, in + sm_off, n, out);
    free(e);
    return st;
}
