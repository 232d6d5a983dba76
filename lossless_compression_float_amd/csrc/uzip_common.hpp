// uzip_common.hpp -- layout arithmetic and descriptors shared by the host
// orchestration and the gfx950 kernels of the codec.
//
// Bitstream v1 constants: a 2^12 frequency table, 32 interleaved rANS lanes
// per chunk, 32-bit states renormalised by 16-bit words with lower bound
// 2^16 (rANS after J. Duda, arXiv 1311.2540; lane interleaving after
// F. Giesen, arXiv 1402.3392).  The exponent/sign+mantissa split is the
// floating-point ANS pipeline of UCCL-Zip (Figure 2); the per-chunk tables are
// its localized per-block tables (Figure 5(b)); the header + payload framing
// and the RAW fallback follow NCCLZ Sec. IV-D2 and Sec. IV-C.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace uzip {

constexpr uint32_t kProbBits = 12;
constexpr uint32_t kTableSize = 1u << kProbBits;  // M = 4096
constexpr uint32_t kLanes = 32;                   // rANS lanes per chunk
constexpr uint32_t kStateLow = 1u << 16;          // L
constexpr uint32_t kMagic = 0x31505A55u;          // "UZP1"
constexpr uint32_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 64;
constexpr uint32_t kRecHeaderBytes = 16;
constexpr uint32_t kMaxChunkElems = 1u << 20;
constexpr uint32_t kPairTile = 64;  // chunk pairs per tile of the record-offset scan

__host__ __device__ inline uint64_t align16(uint64_t v) { return (v + 15u) & ~uint64_t(15); }
__host__ __device__ inline uint64_t align4(uint64_t v) { return (v + 3u) & ~uint64_t(3); }

// Every value splits into its exponent field (the coded symbol) and its sign
// and mantissa bits (stored raw, the sign on top).  Bits of the raw field:
// bf16 8, fp32 24, fp16 11, fp8 e4m3fn 4, fp8 e5m2 3; bits of the symbol:
// 8, 8, 5, 4, 5; bytes per value 2, 4, 2, 1, 1.
__host__ __device__ inline uint32_t raw_bits(int dtype) {
    return dtype == 1 ? 8u : dtype == 2 ? 24u : dtype == 3 ? 11u : dtype == 4 ? 4u : 3u;
}
__host__ __device__ inline uint32_t sym_bits(int dtype) { return dtype == 3 || dtype == 5 ? 5u : dtype == 4 ? 4u : 8u; }
__host__ __device__ inline uint32_t elem_bytes(int dtype) { return dtype == 2 ? 4u : (dtype == 1 || dtype == 3) ? 2u : 1u; }

// bytes of n fields of w bits packed back to back (value order, least
// significant bit first): the raw region, and the body of a RAW record
__host__ __device__ inline uint64_t packed_bytes(uint64_t n, uint32_t w) { return (n * w + 7) / 8; }

// record bytes of a chunk stored RAW: 16-byte record header + the symbols
// packed at sb bits, padded to 16 bytes
__host__ __device__ inline uint64_t raw_record_bytes(uint64_t n_values, uint32_t sb) {
    return align16(kRecHeaderBytes + packed_bytes(n_values, sb));
}

// offset of the 32 final states inside a RANS record (after header, 32-byte
// presence bitmap and nsym u16 frequencies, padded to 4 bytes)
__host__ __device__ inline uint64_t states_offset(uint32_t nsym) { return align4(kRecHeaderBytes + 32 + 2ull * nsym); }
__host__ __device__ inline uint64_t words_offset(uint32_t nsym) { return states_offset(nsym) + 4ull * kLanes; }

// A record coded with a table from the chunk's sample (record mode 2, frames
// with header flag bit 0): after the frequencies and their padding comes the
// u32 count of escaped values, then the 32 states, the words, and the escaped
// exponent bytes in value order.  The escape symbol holds the table's last
// slot (f = 1, c0 = 4095); the sampled symbols share the other 4095.
constexpr uint32_t kEscSlot = kTableSize - 1;
__host__ __device__ inline uint64_t esc_count_offset(uint32_t nsym) { return align4(kRecHeaderBytes + 32 + 2ull * nsym); }
__host__ __device__ inline uint64_t states_offset_sampled(uint32_t nsym) { return esc_count_offset(nsym) + 4; }
__host__ __device__ inline uint64_t words_offset_sampled(uint32_t nsym) { return states_offset_sampled(nsym) + 4ull * kLanes; }

struct Layout {
    uint64_t chunks;   // C
    uint64_t sm_off;   // start of the sign+mantissa region
    uint64_t exp_off;  // start of the records
};

__host__ __device__ inline Layout layout_of(int dtype, uint64_t n, uint64_t chunk_elems) {
    Layout l;
    l.chunks = (n + chunk_elems - 1) / chunk_elems;
    l.sm_off = align16(kHeaderBytes + 8 * (l.chunks + 1));
    l.exp_off = align16(l.sm_off + packed_bytes(n, raw_bits(dtype)));
    return l;
}

// One buffer of a compress call (uploaded to the workspace for batched calls,
// passed by value for single calls).
struct alignas(16) EncDesc {
    const uint8_t *in;      // values
    uint8_t *out;           // compressed buffer
    uint64_t *out_size;     // device word receiving the compressed size
    uint64_t n;             // values
    uint64_t chunk_first;   // global index of the buffer's first chunk
    uint64_t sm_off;
    uint64_t exp_off;
    uint64_t chunks;
    uint64_t pair_first;    // global index of the buffer's first chunk pair
    uint64_t tile_first;    // global index of the buffer's first tile of kPairTile chunk pairs
};

// One buffer of a decompress call as the caller states it.
struct alignas(16) DecDesc {
    const uint8_t *in;  // compressed buffer
    uint8_t *out;       // values
    uint64_t in_bytes;  // bytes readable at `in`
    uint64_t n;         // values the caller expects
};

// What validation of a buffer's header established (device-written).
struct alignas(16) DecInfo {
    uint64_t chunks;       // C (0 when the header is corrupt)
    uint64_t chunk_elems;
    uint64_t sm_off;
    uint64_t exp_off;
    uint64_t total;
    uint64_t flags;        // header flags (bit 0: sampled tables, record mode 2)
    uint64_t pad[2];
};

}  // namespace uzip
