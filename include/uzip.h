/*
 * uzip.h -- C ABI of the MI355X (gfx950) lossless bf16/fp32 (and fp16/fp8)
 * tensor codec.
 *
 * What it computes.  A tensor is shrunk losslessly before a send and restored
 * bit for bit after the receive, with the communication API left unchanged
 * (UCCL-Zip: Lossless Compression Supercharged GPU Communication, abstract).
 * Each value's exponent field is split from its sign and mantissa bits and
 * only the exponents are entropy-coded (same page, Figure 2 and its text);
 * every chunk of the tensor builds its own frequency table, so chunks need no
 * global coordination (Figure 5(b)).  The exponent coder is 32-lane
 * interleaved rANS with a 2^12 table; sign+mantissa bytes are stored raw.
 * The output is one self-describing buffer, header + payload, in the manner of
 * NCCLZ's batch framing (NCCLZ: Compression-Enabled GPU Collectives with
 * Decoupled Quantization and Entropy Coding, Sec. IV-D2), a chunk is stored
 * RAW whenever coding it would not make it smaller (Sec. IV-C, Algorithm 1),
 * and the receiver validates the header before decoding (Algorithm 2).
 *
 * Buffer layout (bitstream v1, little-endian, 16-byte aligned sections):
 *   [0, 64)            header: magic "UZP1", version 1, dtype, prob_bits 12,
 *                      lanes 32, raw bytes per value r, u16 flags,
 *                      chunk_elems, N, C, sm_off, exp_off, total_bytes
 *                      (flags: 0, or bit 0 = chunk tables taken from samples
 *                      with an escape list, record mode 2, written by the
 *                      *_sampled calls; the decoder reads both kinds)
 *   [64, 64+8(C+1))    u64 record offsets (exclusive prefix sum of sizes)
 *   [sm_off, +r*N)     sign+mantissa bytes of every value, in value order
 *                      (bf16: 1 byte; fp32: 3 bytes little-endian; fp16: the
 *                      low byte; fp8: none)
 *   [exp_off, total)   one record per chunk: a 16-byte record header, then
 *                      either the rANS table, 32 final states and 16-bit words
 *                      (mode RANS; mode 2 adds the escape count before the
 *                      states and the escaped exponent bytes after the words)
 *                      or the chunk's raw exponent bytes (RAW).
 *
 * Memory and ownership.  Every pointer named d_* is device memory of the
 * current HIP device; every h_* pointer is host memory.  The caller owns all
 * buffers.  Device input/output/workspace pointers must be 16-byte aligned
 * (a null input is allowed when its element count is 0).  The library
 * allocates no device memory: work memory comes from the caller's workspace,
 * whose size the *_workspace_size functions give.  Host arrays need only live
 * for the duration of the call: a batched call over more than one buffer
 * copies its per-buffer descriptors through a small pinned host staging area
 * that the library keeps per calling thread and device (eight buffers of at
 * least 64 KiB, allocated on that thread's first such call, grown when a call
 * needs more, and kept until the process ends, also after the thread exits),
 * so the call never waits for work already queued on the stream.  Calls enqueue work on `stream` and return without synchronising
 * it; results (d_out_size, d_status, output bytes) are valid once the
 * stream's work has completed.  Calls on different streams are independent
 * when their workspaces differ.  The library keeps no other state between
 * calls.
 *
 * Errors.  Argument errors are found on the host and returned at once, with
 * nothing launched: UZIP_ERR_INVALID_ARGUMENT (bad dtype, null or misaligned
 * pointer, chunk_bytes not a multiple of 32 values or above 2^20 values,
 * workspace too small, or a compress call beyond its limits: a buffer of 2^44
 * values or more, more than 33,554,424 (2^25 - 8) chunk pairs in one call,
 * which keeps every launch grid within one grid dimension (at the default
 * chunk sizes about 2.2 * 10^12 values), or an arbitrated batched call of
 * more than 2^24 - 1 buffers), UZIP_ERR_CAPACITY (output capacity below
 * uzip_max_compressed_size).  Corrupt compressed input is found on the device
 * and reported per buffer in d_status (0 = valid, else
 * UZIP_ERR_CORRUPT_INPUT); the library never falls back to copying bytes it
 * could not validate, and never writes outside [d_out, d_out + N*sizeof(T)).
 * UZIP_ERR_DEVICE reports a failed HIP launch or copy.
 */
#ifndef UZIP_H
#define UZIP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value types (UCCL-Zip, Fig. 13: bfloat16, float16, float32, float8_e4m3fn
 * and float8_e5m2 payloads).  The coded symbol of a value is the byte of its
 * exponent field: bf16 bits 14..7 and fp32 bits 30..23 (the exponent; the
 * sign and mantissa are stored raw, 1 and 3 bytes per value); fp16 bits 15..8
 * (sign, the 5 exponent bits and the top 2 mantissa bits; the low mantissa
 * byte is raw); fp8 the whole byte (nothing raw).  Neither fp16 nor fp8 has a
 * byte-aligned field of exponent bits alone. */
typedef enum { UZIP_BF16 = 1, UZIP_FP32 = 2, UZIP_FP16 = 3, UZIP_FP8_E4M3 = 4, UZIP_FP8_E5M2 = 5 } uzip_dtype;

typedef enum {
    UZIP_OK = 0,
    UZIP_ERR_INVALID_ARGUMENT = 1,
    UZIP_ERR_CAPACITY = 2,
    UZIP_ERR_CORRUPT_INPUT = 3,
    UZIP_ERR_DEVICE = 4,
    UZIP_ERR_UNSUPPORTED = 5, /* reserved: no call of this version returns it */
    UZIP_ERR_SCRATCH_LIMIT = 6 /* uzip_compress_noalloc: the input needs more than its scratch */
} uzip_status;

/* Exact upper bound of the compressed size of num_elements values: the size
 * of the self-describing frame (NCCLZ Sec. IV-D2, batch framing: header,
 * record index, raw region, records) when every chunk is stored RAW, the
 * frame a RAW decision commits (Sec. IV-C, Algorithm 1).  It is exact because
 * a chunk is coded only when that is strictly smaller, and a frame holding a
 * longer coded record is rejected as corrupt.  chunk_bytes is the
 * uncompressed chunk size (0 = default: 256 KiB for fp32, 64 KiB for the
 * others).  Pure host function; returns 0 for an invalid dtype or chunk size,
 * or a count beyond the compress limits above. */
size_t uzip_max_compressed_size(uzip_dtype dtype, size_t num_elements, size_t chunk_bytes);

/* Workspace bytes that uzip_compress or uzip_decompress needs for one buffer
 * of num_elements values (the larger of the two): the per-chunk record slots
 * and sizes in which each chunk's record (its local table, UCCL-Zip
 * Figure 5(b), and its rANS words) is built before the offset scan places it
 * in the frame (NCCLZ Sec. IV-D2), plus the scan's look-back words.  Pure
 * host function; 0 for invalid arguments. */
size_t uzip_workspace_size(uzip_dtype dtype, size_t num_elements, size_t chunk_bytes);

/* Compress num_elements values of `dtype` at d_in (bit patterns, any values
 * including NaN/Inf/denormals) into d_out (out_capacity bytes, at least
 * uzip_max_compressed_size).  The exact compressed size is written to the
 * device word *d_out_size.  Passages: UCCL-Zip Fig. 2 (exponent split),
 * Fig. 5(b) (per-chunk local tables); NCCLZ Sec. IV-D2 (self-describing
 * frame), Sec. IV-C (RAW when coding does not pay). */
uzip_status uzip_compress(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                          void *d_out, size_t out_capacity, uint64_t *d_out_size,
                          void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- compress without allocating --------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): uzip_compress
 * without the workspace argument.  Its work memory is a static device array of
 * UZIP_NOALLOC_SCRATCH_BYTES (64 MiB) that every device loading the library
 * holds until the process ends; the call allocates nothing (no hipMalloc or
 * hipFree, no allocating library routine).  Inputs whose workspace
 * (uzip_workspace_size) exceeds the scratch are rejected at once with
 * UZIP_ERR_SCRATCH_LIMIT, nothing launched: at the default chunk sizes up to
 * 2046 chunks, 67,043,328 values of any type.  Output bytes, size, ownership
 * and other errors are those of uzip_compress.  All calls on one device share
 * that device's scratch, which keeps the last call's contents: calls that
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller; sequential calls on one stream are safe. */
#define UZIP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
uzip_status uzip_compress_noalloc(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                  void *d_out, size_t out_capacity, uint64_t *d_out_size, hipStream_t stream);

/* Decompress the buffer at d_in (in_bytes bytes available) holding
 * num_elements values of `dtype`, as the receiver expects them, into d_out
 * (num_elements * sizeof(T) bytes).  The buffer is validated on the device
 * (header, record index, every record, and the rANS end state of every lane)
 * and *d_status receives 0 or UZIP_ERR_CORRUPT_INPUT.  Frames of both kinds
 * (full tables, or sampled tables: header flag bit 0) are read; the kind
 * comes from the frame.  Passage: NCCLZ Algorithm 2 (parse and validate the
 * header, then decode). */
uzip_status uzip_decompress(const void *d_in, size_t in_bytes, uzip_dtype dtype, size_t num_elements,
                            void *d_out, uint32_t *d_status,
                            void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace for one batched call over num_buffers buffers whose element
 * counts are h_num_elements[0..num_buffers) (the larger of the compress and
 * decompress needs): that of uzip_workspace_size over all the chunks, plus
 * one descriptor per buffer.  Pure host function; 0 for invalid arguments. */
size_t uzip_workspace_size_batched(uzip_dtype dtype, size_t num_buffers, const size_t *h_num_elements,
                                   size_t chunk_bytes);

/* Compress num_buffers independent buffers in one set of launches.  Buffer b
 * reads h_in[b] (h_num_elements[b] values) and writes its own self-describing
 * buffer to h_out[b] (capacity h_out_capacity[b]); its size goes to
 * d_out_sizes[b].  The result for each buffer is byte-identical to a
 * uzip_compress call on that buffer alone.  Same passages as uzip_compress;
 * the batching serves many small messages (UCCL-Zip Fig. 11, KV transfer)
 * and whole weight sets (Fig. 10, RL weight sync). */
uzip_status uzip_compress_batched(uzip_dtype dtype, size_t num_buffers,
                                  const void *const *h_in, const size_t *h_num_elements, size_t chunk_bytes,
                                  void *const *h_out, const size_t *h_out_capacity, uint64_t *d_out_sizes,
                                  void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- sampled tables: one read of the input --------------------------------
 * UCCL-Zip (Sec. 3, the text on Figure 5) lets each block build its table
 * from a sample of its own data.  These calls take each chunk's table from
 * eight evenly spaced runs of max(1, chunk_elems / 64) values, one every
 * chunk_elems / 8 (an eighth of a full chunk).  The sampled symbols share
 * 4095 table slots (one each, the rest by largest remainder of the sample's
 * counts); the table's last slot is an escape symbol, and a value whose
 * exponent the sample missed is coded as the escape, its exponent byte
 * appended to the record's escape list in value order (record mode 2, header
 * flag bit 0).  The encoder then splits, stores the sign+mantissa bytes and
 * codes in one backward pass over the input, instead of a counting pass and
 * a coding pass.  Arguments, sizes (uzip_max_compressed_size,
 * uzip_workspace_size*), ownership and errors are those of uzip_compress and
 * uzip_compress_batched; a chunk is still stored RAW when coding does not
 * make it smaller.  uzip_decompress and uzip_decompress_batched read these
 * frames (and batches mixing both kinds). */
uzip_status uzip_compress_sampled(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                  void *d_out, size_t out_capacity, uint64_t *d_out_size,
                                  void *d_workspace, size_t workspace_bytes, hipStream_t stream);
uzip_status uzip_compress_batched_sampled(uzip_dtype dtype, size_t num_buffers,
                                          const void *const *h_in, const size_t *h_num_elements, size_t chunk_bytes,
                                          void *const *h_out, const size_t *h_out_capacity, uint64_t *d_out_sizes,
                                          void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* Decompress num_buffers buffers in one set of launches; d_status[b] receives
 * buffer b's validation result.  Same passage as uzip_decompress. */
uzip_status uzip_decompress_batched(uzip_dtype dtype, size_t num_buffers,
                                    const void *const *h_in, const size_t *h_in_bytes,
                                    const size_t *h_num_elements, void *const *h_out, uint32_t *d_status,
                                    void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- per-call arbitration: code the call, or send it RAW ----------------
 * NCCLZ Sec. IV-C (runtime entropy-coding arbitration, Eq. (1) and (2),
 * Algorithm 1).  A call whose payload B = num_elements * sizeof(T) is at most
 * small_bytes is stored RAW without looking at it.  Otherwise the first
 * min(num_elements, 65536 / sizeof(T)) values (at most 64 KiB) are sampled:
 * their coded-symbol histogram gives the empirical entropy h (bits per value,
 * in units of 2^-16, logarithms as integers by the squaring method), and the
 * coded frame is predicted as
 *   P = exp_off + ceil(N h / 2^19) + C (align4(48 + 2 nsym) + 136)
 * (the layout's fixed part, the symbols at the sample's entropy, and each
 * record's fixed part plus half a padding unit; nsym = symbols present in the
 * sample).  With P_raw = uzip_max_compressed_size (the all-RAW frame), the
 * times of Eq. (1) in nanoseconds are
 *   raw_ns   = ceil(P_raw * 1000 / link_bytes_per_us)
 *   coded_ns = fixed_ns + ceil(P * 1000 / link_bytes_per_us)
 *              + ceil(exposed_encode_permil * B / encode_bytes_per_us)
 *              + ceil(exposed_decode_permil * B / decode_bytes_per_us).
 * Coding is admitted when P < P_raw and (P_raw - P) * 1000 >=
 * min_gain_permil * B; it is chosen when admitted and coded_ns < raw_ns
 * (Eq. (2); ties go RAW).  A RAW plan writes the all-RAW frame (every record
 * RAW, size P_raw); a coded plan writes exactly what uzip_compress writes,
 * unless that frame's realised size fails the same gain rule, in which case
 * the all-RAW frame is written instead (UZIP_PLAN_RAW_REALIZED).
 * Either frame decodes with uzip_decompress.  Every step is integer
 * arithmetic, so the plan is one fixed function of the input and the policy.
 * Rates are bytes per microsecond (= MB/s); all must be > 0; the per-mille
 * fields are at most 1000; reserved must be 0; num_elements < 2^44. */
typedef struct uzip_policy {
    uint64_t link_bytes_per_us;   /* effective link bandwidth (beta_eff) */
    uint64_t encode_bytes_per_us; /* compress rate of uncompressed bytes */
    uint64_t decode_bytes_per_us; /* decompress rate of uncompressed bytes */
    uint64_t fixed_ns;            /* fixed cost a coded transfer adds (alpha) */
    uint64_t small_bytes;         /* payloads of at most this size go RAW unsampled */
    uint32_t exposed_encode_permil; /* share of the encode time not hidden by overlap */
    uint32_t exposed_decode_permil; /* share of the decode time not hidden by overlap */
    uint32_t min_gain_permil;     /* least predicted saving, per mille of B */
    uint32_t reserved;
} uzip_policy;

/* What a call decided (device-written, 32 bytes per buffer).  A coded plan
 * is checked once its frame is written (Algorithm 1 accepts a materialised
 * plan only if its realised output passes the gain check): when the realised
 * size R fails R < P_raw and (P_raw - R) * 1000 >= min_gain_permil * B, the
 * all-RAW frame replaces it and the decision becomes UZIP_PLAN_RAW_REALIZED
 * (the other plan fields keep the prediction). */
typedef enum {
    UZIP_PLAN_CODED = 0,
    UZIP_PLAN_RAW = 1,
    UZIP_PLAN_RAW_SMALL = 2,
    UZIP_PLAN_RAW_REALIZED = 3
} uzip_plan_decision;
typedef struct uzip_plan {
    uint32_t decision;        /* uzip_plan_decision */
    uint32_t sample_values;   /* values sampled (0 on the small path) */
    uint64_t predicted_bytes; /* P (0 on the small path) */
    uint64_t raw_ns;          /* 0 on the small path */
    uint64_t coded_ns;        /* 0 on the small path */
} uzip_plan;

/* uzip_compress with the arbitration above.  *policy is read on the host
 * before the call returns; d_plan (device, 8-byte aligned, caller-owned)
 * receives the plan, which the encoder reads on the device, so the call stays
 * asynchronous.  Same workspace as uzip_compress.  Errors as uzip_compress,
 * plus UZIP_ERR_INVALID_ARGUMENT for a null d_plan or an invalid policy. */
uzip_status uzip_compress_arbitrated(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                     const uzip_policy *policy, void *d_out, size_t out_capacity,
                                     uint64_t *d_out_size, uzip_plan *d_plan,
                                     void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* The batched form: one plan per buffer (d_plans[b]), each buffer's frame
 * byte-identical to uzip_compress_arbitrated on that buffer alone. */
uzip_status uzip_compress_batched_arbitrated(uzip_dtype dtype, size_t num_buffers,
                                             const void *const *h_in, const size_t *h_num_elements,
                                             size_t chunk_bytes, const uzip_policy *policy,
                                             void *const *h_out, const size_t *h_out_capacity,
                                             uint64_t *d_out_sizes, uzip_plan *d_plans,
                                             void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- instrumented forms (benchmarks) --------------------------------------
 * The batched compress and decompress with two caller events recorded on
 * `stream` around the main coding kernel: main_start right before the kernel
 * that splits, counts, normalises and rANS-encodes (compress) or the rANS
 * decoders (decompress), main_stop right after it, so that the caller can
 * time that kernel alone with hipEventElapsedTime.  Both events or neither
 * (nulls: no events); they belong to the caller (hipEventCreate) and are
 * used during this call only.  sampled (0 or 1) selects the
 * uzip_compress_batched_sampled form, a non-null policy (with d_plans) the
 * arbitrated one (not both).  Otherwise arguments, results and errors are
 * those of uzip_compress_batched / uzip_decompress_batched; a call over one
 * buffer writes exactly what the single-buffer call writes. */
uzip_status uzip_compress_batched_timed(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                        const size_t *h_num_elements, size_t chunk_bytes, uint32_t sampled,
                                        const uzip_policy *policy, void *const *h_out, const size_t *h_out_capacity,
                                        uint64_t *d_out_sizes, uzip_plan *d_plans, void *d_workspace,
                                        size_t workspace_bytes, hipStream_t stream, hipEvent_t main_start,
                                        hipEvent_t main_stop);
uzip_status uzip_decompress_batched_timed(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                          const size_t *h_in_bytes, const size_t *h_num_elements,
                                          void *const *h_out, uint32_t *d_status, void *d_workspace,
                                          size_t workspace_bytes, hipStream_t stream, hipEvent_t main_start,
                                          hipEvent_t main_stop);

/* Static English name of a status code. */
const char *uzip_status_string(uzip_status s);

#ifdef __cplusplus
}
#endif

#endif /* UZIP_H */
