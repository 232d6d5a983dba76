// uzip_kernels.hip -- gfx950 kernels of the lossless bf16/fp32 codec.
//
// Compression of one chunk (UCCL-Zip, Figure 2: split the exponent field
// from the sign and fraction bits and entropy-code only the exponents;
// Figure 5(b): every block builds its own local table, so there is no global
// pass and no cross-block synchronisation):
//   k_encode     one half-wave (32 lanes) per chunk, two chunks per wave:
//                pass 1 streams the chunk forward with 128-bit loads, writes
//                the sign+mantissa bytes straight to their final place in the
//                output and counts the exponents in LDS sub-histograms; the
//                half-wave then normalises the counts to a 2^12 table and runs
//                the 32-lane rANS encoder backward over the chunk (re-reading
//                the input, which the cache still holds), placing each step's
//                renormalisation words by wave ballot + lane rank.  The record
//                is built in a workspace slot (words filled from its end).
//                With tables from each chunk's sample (k_encode<DT, true>;
//                UCCL-Zip Sec. 3, the text on Figure 5) there is no counting
//                pass: the sample fixes the table and one backward pass
//                splits, stores the sign+mantissa bytes and codes, unseen
//                exponents going to the record's escape list.
//   k_compact    one wave per record, workgroups in ticket order: the record
//                offsets (an exclusive scan of the record sizes: tile sums
//                plus a decoupled look-back over tiles), the records copied
//                to their final place, the index entries, and for a buffer's
//                last record the header and the compressed size (NCCLZ
//                Sec. IV-D2: self-describing frames).
//   k_prepare    zeroes the look-back words; writes the buffers of empty inputs.
// Decompression (NCCLZ Algorithm 2: validate the header, then decode):
//   k_dec_validate  one thread per buffer checks the buffer header.
//   k_dec_scan      (batched calls) pair offsets, and which frame kinds occur.
//   k_decode        one half-wave per chunk: validates the record, builds the
//                   slot->symbol table in LDS, runs the rANS decoder forward
//                   and merges each exponent with its sign+mantissa bytes;
//                   k_decode<DT, true> reads sampled-table frames (escapes).
//                   Both variants are launched; each leaves at once unless
//                   the call holds a valid frame of its kind.
//
// Nothing here is a dense contraction: all arithmetic is 32-bit integer and
// bit manipulation on the vector ALU (plus one exact binary64 multiply per
// encoded symbol), and the kernels are bounded by HBM bandwidth, VALU issue
// and the serial per-lane rANS chain, not by the matrix cores.
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "uzip_common.hpp"
#include "uzip_kernels.hpp"

namespace uzip {

// ---------------------------------------------------------------------------
// Global memory is accessed through address-space-1 pointers.  The buffers
// arrive as generic pointers inside descriptors, and generic (flat) accesses
// also count against the LDS wait counter, so every LDS wait in a step loop
// would also wait for the prefetched global loads.
// ---------------------------------------------------------------------------
#define UZ_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
struct GAccess {
    __device__ static T load(const void *p) { return *(const UZ_GLOBAL T *)p; }
    __device__ static void store(void *p, T v) { *(UZ_GLOBAL T *)p = v; }
};
template <>
struct GAccess<uint4> {
    __device__ static uint4 load(const void *p) {
        const u32x4 v = *(const UZ_GLOBAL u32x4 *)p;
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    __device__ static void store(void *p, uint4 v) { *(UZ_GLOBAL u32x4 *)p = u32x4{v.x, v.y, v.z, v.w}; }
};
template <>
struct GAccess<uint2> {
    __device__ static uint2 load(const void *p) {
        const u32x2 v = *(const UZ_GLOBAL u32x2 *)p;
        return make_uint2(v.x, v.y);
    }
    __device__ static void store(void *p, uint2 v) { *(UZ_GLOBAL u32x2 *)p = u32x2{v.x, v.y}; }
};
template <typename T>
__device__ inline T gload(const void *p) {
    return GAccess<T>::load(p);
}
template <typename T>
__device__ inline void gstore(void *p, T v) {
    GAccess<T>::store(p, v);
}

// Raw buffer resources.  A resource carries a wave-uniform base address and
// a byte size; lanes pass 32-bit offsets, and the hardware range check turns
// loads at or past the size into zeros and drops such stores.  The coding
// kernels give each wave a resource per region of its chunk pair, so ragged
// tails, idle half-waves and corrupt offsets never touch memory outside that
// region, without per-step clamping or branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw 32-bit buffer access on the gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every resource's size

__device__ inline uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (uint64_t(hi) << 32) | lo;
}
__device__ inline uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = uniform_u64(reinterpret_cast<uint64_t>(base));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(b), (short)0, (int)uniform_u32(bytes),
                                            (int)kRsrcWord3);
}
__device__ inline uint32_t bld8(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0); }
__device__ inline uint32_t bld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0); }
__device__ inline uint32_t bld32(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0); }
__device__ inline uint4 bld128(rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void bst16(rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, 0);
}
__device__ inline void bst8(rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, (int)off, 0, 0);
}
__device__ inline void bst32(rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
// Loops that issue loads in asm and wait for them explicitly start with this:
// scalar registers of a buffer resource written by a vector instruction need
// five wait states before a memory instruction reads them, which the compiler
// does not insert before asm.
__device__ inline void asm_vmem_fence() { asm volatile("s_nop 4"); }

// Lane masks.  lanes_lt(a, b) is the 64-bit mask of lanes with a < b (one
// compare, no 0/1 materialisation).  vsel(mask, a, b) picks b in the lanes
// set in a wave-uniform mask and a elsewhere: a single v_cndmask_b32 reading
// the mask from scalar registers.  The mask must be written by the scalar
// unit (e.g. a compare result and-ed with another mask), not straight by a
// vector compare: a vector read of scalar registers that a vector instruction
// just wrote needs wait states, which the compiler does not insert for asm.
__device__ inline uint64_t lanes_lt(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 36 /* ULT */); }
__device__ inline uint64_t lanes_eq(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 32 /* EQ */); }
__device__ inline uint32_t vsel(uint64_t mask, uint32_t if0, uint32_t if1) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if0), "v"(if1), "s"(mask));
    return r;
}
// mask of the first min(k, 32) lanes of half-wave h, computed on the scalar unit
__device__ inline uint64_t half_prefix_mask(uint32_t k, uint32_t h) {
    const uint32_t m = k >= 32 ? 0xFFFFFFFFu : ((1u << k) - 1u);
    return h ? uint64_t(m) << 32 : uint64_t(m);
}
constexpr uint64_t kHighHalf = 0xFFFFFFFF00000000ull;

// ---------------------------------------------------------------------------
// half-wave (32-lane segment of a wave64) collectives
// ---------------------------------------------------------------------------
__device__ inline uint32_t half_sum(uint32_t v) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 32);
    return v;
}

__device__ inline uint32_t half_excl_scan(uint32_t v, uint32_t lj) {
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        uint32_t t = __shfl_up(inc, o, 32);
        if (lj >= (uint32_t)o) inc += t;
    }
    return inc - v;
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// bits of the 32-lane mask of this lane's half
__device__ inline uint32_t half_mask(uint64_t m, uint32_t h) { return h ? uint32_t(m >> 32) : uint32_t(m); }

// Ballot of `pred` split per half-wave: number of set lanes in this lane's
// half, and how many of them sit below this lane.  lo_bits is all-ones in the
// upper half (whose lanes discount the lower half's bits) and zero below.
struct HalfBallot {
    uint32_t cnt, rank;
};
__device__ inline HalfBallot half_ballot(bool pred, uint32_t h, uint32_t lo_bits) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(pred);
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
    const uint32_t plo = __popc(mlo);
    return HalfBallot{h ? (uint32_t)__popc(mhi) : plo, below - (plo & lo_bits)};
}

__device__ inline uint32_t find_dec_buffer(const uint64_t *chunk_first, uint32_t nbuf, uint64_t g) {
    uint32_t lo = 0, hi = nbuf - 1;
    while (lo < hi) {
        uint32_t mid = (lo + hi + 1) >> 1;
        if (gload<uint64_t>(chunk_first + mid) <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ inline EncDesc load_enc_desc(const EncDesc *d) {
    static_assert(sizeof(EncDesc) == 80, "descriptor layout");
    const uint4 *q = reinterpret_cast<const uint4 *>(d);
    EncDesc r;
    uint4 *o = reinterpret_cast<uint4 *>(&r);
#pragma unroll
    for (int k = 0; k < 5; ++k) o[k] = gload<uint4>(q + k);
    return r;
}

// the buffer holding global chunk pair q: the largest b with pair_first[b] <= q
__device__ inline uint32_t find_enc_pair_buffer(const EncDesc *d, uint32_t nbuf, uint64_t q) {
    uint32_t lo = 0, hi = nbuf - 1;
    while (lo < hi) {
        uint32_t mid = (lo + hi + 1) >> 1;
        if (gload<uint64_t>(&d[mid].pair_first) <= q) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ inline DecDesc load_dec_desc(const DecDesc *d) {
    const uint4 *q = reinterpret_cast<const uint4 *>(d);
    DecDesc r;
    uint4 *o = reinterpret_cast<uint4 *>(&r);
    o[0] = gload<uint4>(q);
    o[1] = gload<uint4>(q + 1);
    return r;
}

// Value formats (kernel template parameter DT = the dtype code): 1 bf16,
// 2 fp32, 3 fp16, 4 fp8 e4m3fn, 5 fp8 e5m2.  EB bytes per value.  The coded
// symbol is the exponent field, SB bits at bit SYM; the raw field is the sign
// above the mantissa bits, RB bits, and the raw fields of all values are
// packed back to back in the raw region.  R = RB / 8 for the types whose raw
// field is whole bytes (bf16 1, fp32 3); 0 for fp16 and fp8, whose raw fields
// are bit-packed and whose RAW records pack their symbols at SB bits.
template <int DT> struct Fmt;
template <> struct Fmt<1> { static constexpr uint32_t EB = 2, R = 1, RB = 8, SB = 8, SYM = 7; };
template <> struct Fmt<2> { static constexpr uint32_t EB = 4, R = 3, RB = 24, SB = 8, SYM = 23; };
template <> struct Fmt<3> { static constexpr uint32_t EB = 2, R = 0, RB = 11, SB = 5, SYM = 10; };
template <> struct Fmt<4> { static constexpr uint32_t EB = 1, R = 0, RB = 4, SB = 4, SYM = 3; };
template <> struct Fmt<5> { static constexpr uint32_t EB = 1, R = 0, RB = 3, SB = 5, SYM = 2; };

template <int DT>
__device__ inline uint32_t exponent_of(uint32_t v) {
    return (v >> Fmt<DT>::SYM) & ((1u << Fmt<DT>::SB) - 1u);
}
// the raw field of a value: bf16 sign at bit 7 and 7 mantissa bits, fp32 sign
// at bit 23 and 23 mantissa bits, fp16 sign at bit 10 and 10 mantissa bits,
// e4m3fn sign at bit 3 and 3 mantissa bits, e5m2 sign at bit 2 and 2
template <int DT>
__device__ inline uint32_t raw_of(uint32_t v) {
    if (DT == 1) return ((v >> 8) & 0x80u) | (v & 0x7Fu);
    if (DT == 2) return ((v >> 8) & 0x800000u) | (v & 0x7FFFFFu);
    if (DT == 3) return ((v >> 5) & 0x400u) | (v & 0x3FFu);
    if (DT == 4) return ((v >> 4) & 0x8u) | (v & 0x7u);
    return ((v >> 5) & 0x4u) | (v & 0x3u);
}
// inverse of the split: a value from its symbol and its raw field
template <int DT>
__device__ inline uint32_t join_value(uint32_t sym, uint32_t raw) {
    if (DT == 1) return ((raw & 0x80u) << 8) | (sym << 7) | (raw & 0x7Fu);
    if (DT == 2) return ((raw & 0x800000u) << 8) | (sym << 23) | (raw & 0x7FFFFFu);
    if (DT == 3) return ((raw & 0x400u) << 5) | (sym << 10) | (raw & 0x3FFu);
    if (DT == 4) return ((raw & 0x8u) << 4) | (sym << 3) | (raw & 0x7u);
    return ((raw & 0x4u) << 5) | (sym << 2) | (raw & 0x3u);
}
// one value through a buffer resource (zero-extended)
template <int DT>
__device__ inline uint32_t bld_value(rsrc_t r, uint32_t off) {
    if (Fmt<DT>::EB == 1) return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
    if (Fmt<DT>::EB == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
template <int DT>
__device__ inline void bst_value(rsrc_t r, uint32_t off, uint32_t v) {
    if (Fmt<DT>::EB == 1) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, (int)off, 0, 0);
    else if (Fmt<DT>::EB == 2) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

// 32-bit word k (0..15) of a buffer header (bitstream v1; NCCLZ Sec. IV-D2
// self-describing frame: magic, version, codec parameters, sizes)
__device__ inline uint32_t header_word(uint32_t k, int dtype, uint32_t chunk_elems, uint64_t n, uint64_t chunks,
                                       uint64_t sm_off, uint64_t exp_off, uint64_t total, uint32_t flags = 0) {
    switch (k) {
        case 0: return kMagic;
        case 1: return kVersion | (uint32_t(dtype) << 16) | (kProbBits << 24);
        case 2: return kLanes | (raw_bits(dtype) << 8) | (flags << 16);
        case 3: return chunk_elems;
        case 4: return (uint32_t)n;
        case 5: return (uint32_t)(n >> 32);
        case 6: return (uint32_t)chunks;
        case 7: return (uint32_t)(chunks >> 32);
        case 8: return (uint32_t)sm_off;
        case 9: return (uint32_t)(sm_off >> 32);
        case 10: return (uint32_t)exp_off;
        case 11: return (uint32_t)(exp_off >> 32);
        case 12: return (uint32_t)total;
        case 13: return (uint32_t)(total >> 32);
        default: return 0;
    }
}

// Exclusive prefix of the record bytes of the tiles before tile t of a buffer
// (first tile tfirst), by decoupled look-back (Merrill & Garland, single-pass
// prefix scan).  A tile's leader publishes the tile's total at once, then sums
// the published totals of the tiles before it back to the nearest one whose
// inclusive prefix is already known, and publishes its own inclusive prefix;
// the other waves of the tile read the same words without publishing.  A
// look-back word holds a 2-bit state (0 nothing yet, 1 total, 2 inclusive
// prefix) over a 62-bit byte count, so one 64-bit access carries both.  The
// buffer's first tile publishes its inclusive prefix without waiting, so a
// walk never leaves its buffer, and a wave only waits for tiles whose leaders
// hold lower tickets and already run.  Lane l reads the tile at distance
// back + l; a wave waiting for a tile re-reads its window after a short pause.
// The whole wave calls this; the result is wave-uniform.
__device__ inline uint64_t tile_lookback(uint64_t *flags, uint64_t t, uint64_t tfirst, uint64_t agg, bool leader,
                                         uint32_t lane) {
    constexpr uint64_t kAggregate = 1ull << 62, kInclusive = 2ull << 62, kCount = kAggregate - 1;
    if (t == tfirst) {
        if (leader && lane == 0) __hip_atomic_store(flags + t, kInclusive | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (leader && lane == 0) __hip_atomic_store(flags + t, kAggregate | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t excl = 0;
    for (uint64_t back = 1;;) {
        const uint64_t b = back + lane;
        const uint64_t v =
            b <= t - tfirst ? __hip_atomic_load(flags + (t - b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kInclusive;
        const uint64_t incl = __builtin_amdgcn_ballot_w64((v >> 62) == 2);
        const uint64_t none = __builtin_amdgcn_ballot_w64((v >> 62) == 0);
        const uint64_t upto = incl ? ((incl & (0 - incl)) << 1) - 1 : ~0ull;  // lanes up to the nearest inclusive one
        if (none & upto) {  // a needed tile has not published yet
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += wave_sum_u64(((upto >> lane) & 1) ? (v & kCount) : 0);
        if (incl) break;
        back += 64;
    }
    if (leader && lane == 0)
        __hip_atomic_store(flags + t, kInclusive | (excl + agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return excl;
}

// Bytes [sh, sh + 16) of the 32 bytes L:H (sh = 4 DS + bs, bs in {0, 2}).
template <int DS>
__device__ inline uint4 funnel16(const uint4 &L, const uint4 &H, uint32_t bs) {
    const uint32_t w[8] = {L.x, L.y, L.z, L.w, H.x, H.y, H.z, H.w};
    return make_uint4(__builtin_amdgcn_alignbyte(w[DS + 1], w[DS], bs), __builtin_amdgcn_alignbyte(w[DS + 2], w[DS + 1], bs),
                      __builtin_amdgcn_alignbyte(w[DS + 3], w[DS + 2], bs), __builtin_amdgcn_alignbyte(w[DS + 4], w[DS + 3], bs));
}

// mask of the bytes of dword j (bytes [4j, 4j + 4) of a unit) below n, n even
__device__ inline uint32_t low_bytes_mask(uint32_t n, uint32_t j) {
    const uint32_t vb = n > 4 * j ? min(n - 4 * j, 4u) : 0u;
    return vb >= 4 ? 0xFFFFFFFFu : (1u << (8 * vb)) - 1u;
}

// Word area of a coded record: record bytes [wofs, size) get the W bytes of
// words found at byte src of the slot resource, then zeros.  The whole wave
// calls this with wave-uniform arguments; wofs is a multiple of 4, size of
// 16, W and src are even.  Up to three head dwords bring the destination to a
// 16-byte boundary; each later 16-byte unit is funnelled out of two aligned
// 16-byte loads, four units per lane in flight.
__device__ inline void copy_words(rsrc_t rslot, uint8_t *rec, uint32_t wofs, uint32_t size, uint32_t W, uint32_t src,
                                  uint32_t lane) {
    const uint32_t a = (wofs + 15u) & ~15u;
    if (lane < (a - wofs) / 4) {
        const uint32_t rel = 4 * lane, sb = src + rel;
        uint32_t v = (sb & 2u) ? __builtin_amdgcn_alignbit(bld32(rslot, sb + 2), bld32(rslot, sb - 2), 16)
                               : bld32(rslot, sb);
        v &= low_bytes_mask(W > rel ? min(W - rel, 4u) : 0u, 0);
        gstore<uint32_t>(rec + wofs + rel, v);
    }
    const uint32_t s0 = src + (a - wofs), sh = s0 & 15u, base = s0 - sh, bs = sh & 3u, ds = sh >> 2;
    const uint32_t nu = (size - a) / 16;
    for (uint32_t u0 = 0; u0 < nu; u0 += 256) {
        uint4 L[4], H[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t u = u0 + 64 * k + lane;
            const uint32_t o = u < nu ? base + 16 * u : kOutOfRange;
            L[k] = bld128(rslot, o);
            H[k] = bld128(rslot, o + 16);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t u = u0 + 64 * k + lane;
            if (u < nu) {
                uint4 v;
                switch (ds) {
                    case 0: v = funnel16<0>(L[k], H[k], bs); break;
                    case 1: v = funnel16<1>(L[k], H[k], bs); break;
                    case 2: v = funnel16<2>(L[k], H[k], bs); break;
                    default: v = funnel16<3>(L[k], H[k], bs); break;
                }
                const uint32_t rel = (a - wofs) + 16 * u;
                const uint32_t n = W > rel ? min(W - rel, 16u) : 0u;
                v.x &= low_bytes_mask(n, 0);
                v.y &= low_bytes_mask(n, 1);
                v.z &= low_bytes_mask(n, 2);
                v.w &= low_bytes_mask(n, 3);
                gstore<uint4>(rec + a + 16 * u, v);
            }
        }
    }
}

// Bits of a value's field packed at w bits: the w bits at bit position bit
// of the byte string behind r (two aligned dwords, so nothing is read more
// than 4 bytes past the dword holding the field's first bit).
__device__ inline uint32_t packed_field(rsrc_t r, uint32_t base, uint32_t bit, uint32_t w) {
    const uint32_t o = base + 4 * (bit >> 5);
    const uint32_t lo = bld32(r, o);
    const uint32_t hi = (bit & 31u) + w > 32 ? bld32(r, o + 4) : 0u;
    return __builtin_amdgcn_alignbit(hi, lo, bit & 31u) & ((1u << w) - 1u);
}

// dword k of the w-bit packing of fields f(0) .. f(n - 1) (zeros past n)
template <typename F>
__device__ inline uint32_t packed_dword(uint32_t k, uint32_t n, uint32_t w, F f) {
    uint32_t acc = 0;
    const uint32_t i0 = 32 * k / w, i1 = (32 * k + 31) / w;
    for (uint32_t i = i0; i <= i1 && i < n; ++i) {
        const int sh = (int)(i * w) - (int)(32 * k);
        const uint32_t v = f(i);
        acc |= sh >= 0 ? v << sh : v >> -sh;
    }
    return acc;
}

// Whole groups of 32 values of the bit-packed types: 32 fields of W bits,
// packed LSB-first, fill exactly W dwords, so a group's fields start on a
// dword boundary wherever the packing starts on one.  pack32 packs f into o;
// field32 is field i of such a group (i a compile-time constant in the
// unrolled loops below).
template <uint32_t W>
__device__ inline void pack32(const uint32_t (&f)[32], uint32_t (&o)[W]) {
#pragma unroll
    for (uint32_t d = 0; d < W; ++d) o[d] = 0;
#pragma unroll
    for (uint32_t i = 0; i < 32; ++i) {
        const uint32_t b = i * W, d = b >> 5, sh = b & 31u;
        o[d] |= f[i] << sh;
        if (sh + W > 32) o[d + 1] |= f[i] >> (32 - sh);
    }
}
template <uint32_t W>
__device__ inline uint32_t field32(const uint32_t (&o)[W], uint32_t i) {
    const uint32_t b = i * W, d = b >> 5, sh = b & 31u;
    const uint32_t v = sh + W > 32 ? __builtin_amdgcn_alignbit(o[d + 1], o[d], sh) : o[d] >> sh;
    return v & ((1u << W) - 1u);
}
// W consecutive dwords at a dword-aligned offset of r, in 128-bit pieces and
// one 96-, 64- or 32-bit remainder (out of range: loads read zero, stores are
// dropped, dword by dword)
template <uint32_t W>
__device__ inline void load_dwords(rsrc_t r, uint32_t off, uint32_t (&o)[W]) {
#pragma unroll
    for (uint32_t d = 0; d + 4 <= W; d += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * d), 0, 0);
        o[d] = v.x; o[d + 1] = v.y; o[d + 2] = v.z; o[d + 3] = v.w;
    }
    constexpr uint32_t d = W & ~3u;
    if constexpr (W - d == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)(off + 4 * d), 0, 0);
        o[d] = v.x; o[d + 1] = v.y; o[d + 2] = v.z;
    } else if constexpr (W - d == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 4 * d), 0, 0);
        o[d] = v.x; o[d + 1] = v.y;
    } else if constexpr (W - d == 1) {
        o[d] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4 * d), 0, 0);
    }
}
template <uint32_t W>
__device__ inline void store_dwords(rsrc_t r, uint32_t off, const uint32_t (&o)[W]) {
#pragma unroll
    for (uint32_t d = 0; d + 4 <= W; d += 4)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[d], o[d + 1], o[d + 2], o[d + 3]}, r, (int)(off + 4 * d), 0, 0);
    constexpr uint32_t d = W & ~3u;
    if constexpr (W - d == 3) {
        __builtin_amdgcn_raw_buffer_store_b96(u32x3{o[d], o[d + 1], o[d + 2]}, r, (int)(off + 4 * d), 0, 0);
    } else if constexpr (W - d == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{o[d], o[d + 1]}, r, (int)(off + 4 * d), 0, 0);
    } else if constexpr (W - d == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(o[d], r, (int)(off + 4 * d), 0, 0);
    }
}

// Body of a RAW record: bytes [16, size) get the symbols of the chunk's ni
// values (at byte in0 of the input resource), packed at SB bits (bytes for
// bf16 and fp32), then zeros.  Whole wave, wave-uniform arguments; bf16 and
// fp32 one 16-byte unit (16 exponents) per lane, the others a dword per lane.
template <int DT>
__device__ inline void raw_exponents(rsrc_t rin, uint8_t *rec, uint32_t size, uint32_t ni, uint32_t in0, uint32_t lane) {
    constexpr uint32_t EB = Fmt<DT>::EB;
    if constexpr (Fmt<DT>::R == 0) {
        const uint32_t nd = (size - kRecHeaderBytes) / 4;
        for (uint32_t k = lane; k < nd; k += 64) {
            const uint32_t w = packed_dword(k, ni, Fmt<DT>::SB, [&](uint32_t i) {
                return exponent_of<DT>(bld_value<DT>(rin, in0 + i * EB));
            });
            gstore<uint32_t>(rec + kRecHeaderBytes + 4 * k, w);
        }
        return;
    }
    const uint32_t nu = (size - kRecHeaderBytes) / 16;
    for (uint32_t u = lane; u < nu; u += 64) {
        uint32_t w[16];
        if (16 * u + 16 <= ni) {
#pragma unroll
            for (uint32_t k = 0; k < 16 * EB / 16; ++k) {
                const uint4 q = bld128(rin, in0 + (16 * u) * EB + 16 * k);
                const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (uint32_t t = 0; t < 4; ++t) {
#pragma unroll
                    for (uint32_t b = 0; b < 4 / EB; ++b)  // values per dword
                        w[(16 / EB) * k + (4 / EB) * t + b] = EB == 4 ? qq[t] : (qq[t] >> (8 * EB * b)) & ((1u << (8 * EB)) - 1u);
                }
            }
        } else {  // the chunk's end: value by value, nothing read past it
#pragma unroll
            for (uint32_t k = 0; k < 16; ++k) {
                const uint32_t e = 16 * u + k;
                const uint32_t o = e < ni ? in0 + e * EB : kOutOfRange;
                w[k] = bld_value<DT>(rin, o);
            }
        }
        uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k)
            if (16 * u + k < ni) v[k >> 2] |= exponent_of<DT>(w[k]) << (8 * (k & 3));
        gstore<uint4>(rec + kRecHeaderBytes + 16 * u, make_uint4(v[0], v[1], v[2], v[3]));
    }
}

// ---------------------------------------------------------------------------
// k_encode: split + histogram + normalise + interleaved rANS, per chunk
// ---------------------------------------------------------------------------
// LDS of one workgroup (two chunks), 10 KiB, reused between phases:
//   pass 1       4 sub-histograms per chunk (lane j counts into sub j mod 4),
//                rows padded to 264 words so the four copies of a bin sit in
//                four different banks: hot bins no longer serialise a wave
//   normalise    keys of the present symbols          words [0, 512)
//   pass 2       per-symbol coder table, 16 B/entry   words [512, 2560)
// fp8 counts 32 values per group with eight waves per CU (a chunk holds 64 Ki
// values): it takes 8 sub-histograms in rows of 260 words (eight copies of a
// bin in eight banks, 16.25 KiB in all), which its occupancy affords; the
// 2-byte types keep 10 KiB for 16 waves per CU.
template <int DT> struct EncLds {
    static constexpr uint32_t kSubHist = Fmt<DT>::EB == 1 ? 8 : 4;
    static constexpr uint32_t kSubRow = Fmt<DT>::EB == 1 ? 260 : 264;
    static constexpr uint32_t kWords = 2 * kSubHist * kSubRow > 2560 ? 2 * kSubHist * kSubRow : 2560;
};

// Exact floor(x / f) for the encoder, where x < f * 2^20 (so the quotient is
// below 2^20) and 1 <= f <= 4096: one binary64 multiply by
// r_f = (1 + 2^-44) / f.  The bias keeps the product at or above x / f
// despite both roundings, and the product exceeds x / f by less than 2^-23,
// while x / f lies at least 1/f >= 2^-12 below the next integer; truncation
// therefore gives the exact quotient.
__device__ inline double enc_reciprocal(uint32_t f) { return (1.0 + 0x1p-44) / (double)f; }
__device__ inline uint32_t enc_quotient(uint32_t x, double r) { return (uint32_t)((double)x * r); }

template <int DT, bool S>
__global__ __launch_bounds__(64) void k_encode(EncParams p) {
    constexpr uint32_t EB = Fmt<DT>::EB;      // bytes per value
    constexpr uint32_t R = Fmt<DT>::R;        // raw bytes per value
    constexpr uint32_t VPL = 16 / EB;         // values per lane per 128-bit load
    constexpr uint32_t VPI = 32 * VPL;        // values per half-wave per pass-1 step

    constexpr uint32_t kSubHist = EncLds<DT>::kSubHist, kSubRow = EncLds<DT>::kSubRow;
    __shared__ __align__(16) uint32_t lds[EncLds<DT>::kWords];

    const uint32_t lane = threadIdx.x;
    const uint32_t h = lane >> 5, lj = lane & 31;

    // ---- the pair: buffer and chunks (wave-uniform); half-wave h codes chunk c0 + h ----
    const uint64_t q = blockIdx.x;
    const uint32_t bi = p.nbuf == 1 ? 0u : uniform_u32(find_enc_pair_buffer(p.descs, p.nbuf, q));
    // a buffer that the per-call arbitration sends RAW is written by k_raw_frame
    if (p.plans != nullptr && uniform_u32(gload<uint32_t>(&p.plans[bi].decision)) != UZIP_PLAN_CODED) return;
    const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + bi);
    const uint64_t ce = p.chunk_elems;
    const uint64_t n = uniform_u64(d.n);
    const uint64_t c0 = 2 * (q - uniform_u64(d.pair_first));
    const uint64_t chunks = uniform_u64(d.chunks);
    const uint32_t nch = chunks - c0 >= 2 ? 2u : 1u;
    const uint32_t vals0 = (uint32_t)min<uint64_t>(ce, n - c0 * ce);
    const uint32_t vals1 = nch == 2 ? (uint32_t)min<uint64_t>(ce, n - (c0 + 1) * ce) : 0u;
    const uint64_t g0 = uniform_u64(d.chunk_first) + c0;  // global index of the pair's first chunk
    const bool valid = h < nch;
    const uint64_t g = g0 + (valid ? h : 0u);
    const uint32_t ni = h ? vals1 : vals0;
    const uint32_t pair_vals = vals0 + vals1;
    const rsrc_t rin = make_rsrc(d.in + c0 * ce * EB, pair_vals * EB);
    const rsrc_t rslot = make_rsrc(p.slots + g0 * p.slot_stride, (uint32_t)(nch * p.slot_stride));
    const uint32_t in0 = (h ? vals0 : 0u) * EB;  // this half's chunk inside rin
    uint8_t *sm_out = d.out + d.sm_off + (c0 * ce + (h ? vals0 : 0u)) * R;
    uint8_t *slot = p.slots + g * p.slot_stride;

    uint32_t *hist = lds + h * (kSubHist * kSubRow) + (lj & (kSubHist - 1)) * kSubRow;
    uint32_t first_it = 0;
    for (uint32_t k = lane; k < 2 * kSubHist * kSubRow; k += 64) lds[k] = 0;
    __syncthreads();

    uint32_t scnt = 0;  // sampled values of this half's chunk (S)
    if constexpr (S) {
        // ---- the chunk's sample: eight evenly spaced runs of max(1, ce/64)
        // contiguous values, one every ce/8 (an eighth of a full chunk), counted
        // into the LDS histogram; the sign+mantissa split happens in the coding
        // pass, which reads every value once ----
        const uint32_t period = (uint32_t)ce / 8, runlen = max(1u, (uint32_t)ce / 64);
        for (uint32_t r = 0; r < 8; ++r) scnt += r * period < ni ? min(runlen, ni - r * period) : 0u;
        if (runlen % VPL == 0) {
            const uint32_t rv = runlen / VPL, nvec = 8 * rv;  // 128-bit vectors per run and per sample
            for (uint32_t k0 = 0; k0 < nvec; k0 += 4 * 32) {
                uint4 qv[4];
                uint32_t i0[4];
#pragma unroll
                for (uint32_t u = 0; u < 4; ++u) {
                    const uint32_t k = k0 + 32 * u + lj;
                    i0[u] = k < nvec ? (k / rv) * period + (k % rv) * VPL : 0xFFFFFFFFu;
                    qv[u] = bld128(rin, i0[u] < ni ? in0 + i0[u] * EB : kOutOfRange);  // past the pair: zeros
                }
#pragma unroll
                for (uint32_t u = 0; u < 4; ++u) {
                    if (i0[u] >= ni) continue;
                    uint32_t w[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
                    if (i0[u] + VPL > ni) {
                        // a vector that the chunk's end cuts: value by value (the
                        // 128-bit load read the dword crossing the pair's end as zero)
                        w[0] = w[1] = w[2] = w[3] = 0;
                        for (uint32_t k = 0; i0[u] + k < ni; ++k)
                            w[k / (4 / EB)] |= bld_value<DT>(rin, in0 + (i0[u] + k) * EB) << (8 * EB * (k % (4 / EB)));
                    }
#pragma unroll
                    for (uint32_t k = 0; k < VPL; ++k) {
                        const uint32_t v = EB == 4 ? w[k] : (w[k / (4 / EB)] >> (8 * EB * (k % (4 / EB)))) & ((1u << (8 * EB)) - 1u);
                        if (i0[u] + k < ni) atomicAdd(&hist[exponent_of<DT>(v)], 1u);
                    }
                }
            }
        } else {  // runs shorter than a vector (small chunks): value by value
            for (uint32_t j = lj; j < 8 * runlen; j += 32) {
                const uint32_t i = (j / runlen) * period + j % runlen;
                if (i < ni) atomicAdd(&hist[exponent_of<DT>(bld_value<DT>(rin, in0 + i * EB))], 1u);
            }
        }
    }
    if constexpr (Fmt<DT>::R == 0) {
        // ---- fp16 and fp8: raw fields bit-packed (RB bits a value), and with
        // full tables the LDS histogram.  Lane lj takes groups gi = lj, lj + 32,
        // ... of 32 consecutive values of its half's chunk: 32 RB bits are RB
        // dwords of the raw region (dword-aligned: chunks hold multiples of 32
        // values).  It loads the group (32 EB bytes, 128-bit loads), packs the
        // 32 raw fields, counts the 32 exponents and stores the RB dwords.
        // A group that the chunk's end cuts is read value by value (a 128-bit
        // load crossing the end of the pair's range would read the dword
        // holding the last values as zero); the values past the end are zero,
        // so their bits are, and are not counted.  The resource is the pair's
        // raw region (its base wave-uniform; half 1's chunk starts vals0 RB / 8
        // bytes in), and the last group's dwords past it are dropped.
        constexpr uint32_t RB = Fmt<DT>::RB;
        const rsrc_t rraw = make_rsrc(d.out + d.sm_off + c0 * ce * RB / 8,
                                      (uint32_t)((packed_bytes(pair_vals, RB) + 3) & ~3ull));
        const uint32_t hraw = (h ? vals0 : 0u) * RB / 8;  // this half's chunk in rraw (vals0 = ce then)
        const uint32_t ngroups = (ni + 31) / 32;
        for (uint32_t gi = lj; gi < ngroups; gi += 32) {
            uint32_t w[8 * EB];
            if (32 * gi + 32 <= ni) {
#pragma unroll
                for (uint32_t u = 0; u < 2 * EB; ++u) {
                    const uint4 qv = bld128(rin, in0 + gi * 32 * EB + 16 * u);
                    w[4 * u] = qv.x; w[4 * u + 1] = qv.y; w[4 * u + 2] = qv.z; w[4 * u + 3] = qv.w;
                }
            } else {
#pragma unroll
                for (uint32_t u = 0; u < 8 * EB; ++u) w[u] = 0;
                for (uint32_t k = 0; 32 * gi + k < ni; ++k)
                    w[k * EB / 4] |= bld_value<DT>(rin, in0 + (32 * gi + k) * EB) << (8 * EB * (k % (4 / EB)));
            }
            uint32_t acc[RB];
#pragma unroll
            for (uint32_t k = 0; k < RB; ++k) acc[k] = 0;
#pragma unroll
            for (uint32_t k = 0; k < 32; ++k) {
                const uint32_t v = (w[k * EB / 4] >> (8 * EB * (k % (4 / EB)))) & ((1u << (8 * EB)) - 1u);
                if (!S && 32 * gi + k < ni) atomicAdd(&hist[exponent_of<DT>(v)], 1u);
                const uint32_t r = raw_of<DT>(v), bit = k * RB;
                acc[bit >> 5] |= r << (bit & 31);
                if ((bit & 31) + RB > 32) acc[(bit >> 5) + 1] |= r >> (32 - (bit & 31));
            }
            const uint32_t o = hraw + gi * 4 * RB;
            if (32 * gi + 32 <= ni) {
#pragma unroll
                for (uint32_t k = 0; k + 4 <= RB; k += 4)
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]}, rraw,
                                                           (int)(o + 4 * k), 0, 0);
                constexpr uint32_t k4 = RB & ~3u;
                if constexpr (RB - k4 == 3)
                    __builtin_amdgcn_raw_buffer_store_b96(u32x3{acc[k4], acc[k4 + 1], acc[k4 + 2]}, rraw, (int)(o + 4 * k4), 0, 0);
                if constexpr (RB - k4 == 2)
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{acc[k4], acc[k4 + 1]}, rraw, (int)(o + 4 * k4), 0, 0);
                if constexpr (RB - k4 == 1) bst32(rraw, o + 4 * k4, acc[k4]);
            } else {
#pragma unroll
                for (uint32_t k = 0; k < RB; ++k) bst32(rraw, o + 4 * k, acc[k]);
            }
        }
    } else if constexpr (!S) {
    // ---- pass 1: split, sign+mantissa bytes to the output, LDS histogram ----
    // Main loop: iterations in which every lane of each coding half holds a
    // full 128-bit vector, with four to eight loads in flight per lane.  A half without
    // a chunk (the buffer's odd last chunk) reads zeros past the pair, counts
    // them into the padding words of its histogram rows (a word per lane, so
    // without conflicts) and stores nothing: its sign+mantissa offsets lie
    // past the pair's output range.
    {
        // Sets of kSet vectors, software-pipelined (below): four, or eight for
        // fp32, whose few waves need more loads in flight each
        constexpr uint32_t kSet = DT == 2 ? 8u : 4u;
        // (a multiple of kSet iterations, so that no step of the loop is conditional)
        const uint32_t fullmin = min(vals0 / VPI, nch == 2 ? vals1 / VPI : 0xFFFFFFFFu) & ~(kSet - 1u);
        uint32_t *hm = valid ? hist : hist + 256 + lj / kSubHist;
        const rsrc_t rsmo = make_rsrc(d.out + d.sm_off + c0 * ce * R, pair_vals * R);
        const uint32_t smo = (h ? vals0 : 0u) * R + lj * VPL * R;  // this lane's first sign+mantissa byte
        auto split = [&](const uint4 &qv, uint32_t it) __attribute__((always_inline)) {
            const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
            const uint32_t o = smo + it * VPI * R;
            if (DT == 1) {
                uint32_t smw[2] = {0, 0};
#pragma unroll
                for (uint32_t k = 0; k < 8; ++k) {
                    const uint32_t v = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                    smw[k >> 2] |= raw_of<DT>(v) << (8 * (k & 3));
                    atomicAdd(&hm[exponent_of<DT>(v)], 1u);
                }
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{smw[0], smw[1]}, rsmo, (int)o, 0, 0);
            } else {
                uint32_t sm[4];
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k) {
                    sm[k] = ((w[k] >> 8) & 0x800000u) | (w[k] & 0x7FFFFFu);
                    atomicAdd(&hm[(w[k] >> 23) & 0xFFu], 1u);
                }
                __builtin_amdgcn_raw_buffer_store_b96(
                    u32x3{sm[0] | (sm[1] << 24), (sm[1] >> 8) | (sm[2] << 16), (sm[2] >> 16) | (sm[3] << 8)}, rsmo, (int)o,
                    0, 0);
            }
        };
        // Sets of kSet vectors (iterations kSet s .. kSet s + kSet - 1),
        // software-pipelined: the next set is loaded while a set is split.  As
        // in the coding pass, the loads are issued in asm and waited for
        // explicitly, so that the wait does not also cover the raw-byte stores:
        // between a set's loads and its wait lies only the straight-line split
        // of the set before, with exactly one store per vector.
        constexpr uint32_t kSetStores = kSet;
        auto asm_load_set = [&](uint32_t st, u32x4(&V)[kSet]) __attribute__((always_inline)) {
#pragma unroll
            for (uint32_t k = 0; k < kSet; ++k) {
                const uint32_t it = kSet * st + k;
                const uint32_t o = it < fullmin ? in0 + (it * VPI + lj * VPL) * EB : kOutOfRange;
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(V[k]) : "v"(o), "s"(rin));
            }
        };
        auto split_set = [&](uint32_t st, const u32x4(&V)[kSet]) __attribute__((always_inline)) {
#pragma unroll
            for (uint32_t k = 0; k < kSet; ++k) split(make_uint4(V[k].x, V[k].y, V[k].z, V[k].w), kSet * st + k);
        };
        // (the wait names every register of the set, so that none is read before it)
#define UZIP_WAIT_SET(N, V)                                                                                        \
    do {                                                                                                           \
        if constexpr (kSet == 8)                                                                                   \
            asm volatile("s_waitcnt vmcnt(%8)"                                                                     \
                         : "+v"(V[0]), "+v"(V[1]), "+v"(V[2]), "+v"(V[3]), "+v"(V[4 % kSet]), "+v"(V[5 % kSet]), \
                           "+v"(V[6 % kSet]), "+v"(V[7 % kSet])                                                    \
                         : "i"(N));                                                                                \
        else                                                                                                       \
            asm volatile("s_waitcnt vmcnt(%4)" : "+v"(V[0]), "+v"(V[1]), "+v"(V[2]), "+v"(V[3]) : "i"(N));       \
    } while (0)
        const uint32_t nsets = fullmin / kSet;
        if (nsets > 0) {
            u32x4 A[kSet], B[kSet];
            asm_vmem_fence();
            asm_load_set(0, A);
            UZIP_WAIT_SET(0, A);
            for (uint32_t st = 0;;) {
                asm_load_set(st + 1, B);
                split_set(st, A);
                UZIP_WAIT_SET(kSetStores, B);
                if (++st >= nsets) break;
                asm_load_set(st + 1, A);
                split_set(st, B);
                UZIP_WAIT_SET(kSetStores, A);
                if (++st >= nsets) break;
            }
        }
#undef UZIP_WAIT_SET
        first_it = fullmin;
    }
    // the rest: the longer half's remaining vectors and the ragged ends
    const uint32_t iters = (ni + VPI - 1) / VPI;
    const uint32_t iters_w = max(iters, (uint32_t)__shfl_xor(iters, 32, 64));
    for (uint32_t it = first_it; it < iters_w; ++it) {
        const uint32_t i0 = it * VPI + lj * VPL;
        if (i0 >= ni) continue;
        const bool full = i0 + VPL <= ni;
        uint32_t w[4];
        if (full) {
            const uint4 qv = bld128(rin, in0 + i0 * EB);
            w[0] = qv.x; w[1] = qv.y; w[2] = qv.z; w[3] = qv.w;
        } else {  // the chunk's ragged end: value by value, nothing read past the pair
            for (int k = 0; k < 4; ++k) w[k] = 0;
            for (uint32_t k = 0; k < VPL; ++k) {
                const uint32_t o = i0 + k < ni ? in0 + (i0 + k) * EB : kOutOfRange;
                w[k / (4 / EB)] |= bld_value<DT>(rin, o) << (8 * EB * (k % (4 / EB)));
            }
        }
        if (DT == 1) {
            uint32_t smw[2] = {0, 0};
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                const uint32_t v = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                smw[k >> 2] |= raw_of<DT>(v) << (8 * (k & 3));
                if (full || i0 + k < ni) atomicAdd(&hist[exponent_of<DT>(v)], 1u);
            }
            if (full) {
                gstore<uint2>(sm_out + i0, make_uint2(smw[0], smw[1]));
            } else {
                for (uint32_t k = 0; k < 8; ++k)
                    if (i0 + k < ni) gstore<uint8_t>(sm_out + i0 + k, (uint8_t)(smw[k >> 2] >> (8 * (k & 3))));
            }
        } else {
            uint32_t sm[4];
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t v = w[k];
                sm[k] = ((v >> 8) & 0x800000u) | (v & 0x7FFFFFu);
                if (full || i0 + k < ni) atomicAdd(&hist[(v >> 23) & 0xFFu], 1u);
            }
            if (full) {
                uint8_t *o = sm_out + 3ull * i0;
                gstore<uint32_t>(o, sm[0] | (sm[1] << 24));
                gstore<uint32_t>(o + 4, (sm[1] >> 8) | (sm[2] << 16));
                gstore<uint32_t>(o + 8, (sm[2] >> 16) | (sm[3] << 8));
            } else {
                for (uint32_t k = 0; k < 4; ++k) {
                    if (i0 + k < ni) {
                        uint8_t *o = sm_out + 3ull * (i0 + k);
                        gstore<uint8_t>(o, (uint8_t)sm[k]);
                        gstore<uint8_t>(o + 1, (uint8_t)(sm[k] >> 8));
                        gstore<uint8_t>(o + 2, (uint8_t)(sm[k] >> 16));
                    }
                }
            }
        }
    }
    }  // pass 1
    __syncthreads();

    // ---- normalise the counts to a table of 4096 (lane lj owns symbols 8lj..8lj+7) ----
    // Reserve one slot per present symbol, share R = 4096 - nsym slots by the
    // floor of each quota, give the leftover slots to the largest remainders
    // (lower symbol first on equal remainders).
    uint32_t c[8], pm = 0;
    {
        const uint32_t *hh = lds + h * (kSubHist * kSubRow);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t s = lj * 8 + k;
            c[k] = 0;
#pragma unroll
            for (uint32_t r = 0; r < kSubHist; ++r) c[k] += hh[r * kSubRow + s];
            if (c[k]) pm |= 1u << k;
        }
    }
    __syncthreads();  // the histogram area is reused below
    uint32_t *keys = lds + h * 256;
    uint4 *tab = reinterpret_cast<uint4 *>(lds + 512) + h * 256;
    const uint32_t np = __popc(pm);
    const uint32_t nsym = half_sum(np);
    const uint32_t pre = half_excl_scan(np, lj);
    // full tables share R = 4096 - nsym slots by the chunk's counts; sampled
    // ones R = 4095 - nsym by the sample's (the escape symbol keeps slot 4095)
    const uint32_t den = S ? scnt : ni;
    const uint32_t Rr = kTableSize - nsym - (S ? 1u : 0u);
    uint32_t fl[8], key[8], given = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        fl[k] = 0;
        key[k] = 0;
        if (c[k]) {
            const uint32_t qq = c[k] * Rr;  // < 2^32: c <= 2^20, R < 2^12
            fl[k] = qq / den;
            key[k] = ((qq - fl[k] * den) << 8) | (255u - (lj * 8 + k));
            given += fl[k];
        }
    }
    given = half_sum(given);
    const uint32_t left = Rr - given;
    {
        uint32_t k2 = pre;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (c[k]) keys[k2++] = key[k];
    }
    __syncthreads();
    uint32_t above[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint32_t nsym_w = max(nsym, (uint32_t)__shfl_xor(nsym, 32, 64));
    const uint32_t left_w = max(left * (ni > 0), (uint32_t)__shfl_xor(left * (ni > 0), 32, 64));
    if (left_w > 0) {
        for (uint32_t m = 0; m < nsym_w; ++m) {
            const uint32_t km = keys[m & 255];
            const bool in_list = m < nsym;
#pragma unroll
            for (int k = 0; k < 8; ++k) above[k] += (in_list && km > key[k]) ? 1u : 0u;
        }
    }
    uint32_t f[8], lsum = 0, cpre[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        f[k] = c[k] ? 1u + fl[k] + (above[k] < left ? 1u : 0u) : 0u;
        cpre[k] = lsum;
        lsum += f[k];
    }
    const uint32_t cbase = half_excl_scan(lsum, lj);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        // a symbol the sample missed is coded as the escape symbol (f = 1, c0 = 4095)
        const bool esc = S && f[k] == 0;
        const uint32_t fe = esc ? 1u : f[k], ce0 = esc ? kEscSlot : cbase + cpre[k];
        const double r = fe ? enc_reciprocal(fe) : 0.0;
        const uint64_t rb = (uint64_t)__double_as_longlong(r);
        // (16 f - 1) | (4096 - f) << 16: the emission threshold (x >= f * 2^20
        // exactly when x >> 16 > 16 f - 1) and the multiplier of the coding step
        tab[lj * 8 + k] = make_uint4((((fe << 4) - 1) & 0xFFFFu) | ((kTableSize - fe) << 16), ce0, (uint32_t)rb,
                                     (uint32_t)(rb >> 32));
    }

    // record prefix in the slot: presence bitmap, frequencies (ascending symbols), pad
    if (valid) {
        gstore<uint8_t>(slot + kRecHeaderBytes + lj, (uint8_t)pm);
        uint32_t k2 = pre;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (c[k]) gstore<uint16_t>(slot + 48 + 2 * (k2++), (uint16_t)f[k]);
        if (lj == 0 && (nsym & 1)) gstore<uint16_t>(slot + 48 + 2 * nsym, 0);
    }
    __syncthreads();

    // ---- pass 2: 32-lane interleaved rANS, steps from the last down to 0 ----
    // Words of one step are placed, lanes ascending, right before the words of
    // the following step, filling the slot from its end.  The word counts of
    // the two halves are wave-uniform scalars; a lane's store offset comes from
    // one mbcnt pair, and lanes without a word store out of range (dropped).
    // Input values are prefetched one 8-step block ahead through the pair's
    // input resource (past the pair: zeros, never coded).
    const uint32_t nsym0 = uniform_u32(__shfl((int)nsym, 0, 64)), nsym1 = uniform_u32(__shfl((int)nsym, 32, 64));
    const uint32_t raw0 = (uint32_t)raw_record_bytes(vals0, Fmt<DT>::SB), raw1 = (uint32_t)raw_record_bytes(vals1, Fmt<DT>::SB);
    const uint32_t wofs0 = (uint32_t)(S ? words_offset_sampled(nsym0) : words_offset(nsym0));
    const uint32_t wofs1 = (uint32_t)(S ? words_offset_sampled(nsym1) : words_offset(nsym1));
    // words that fit before a record reaches its RAW size; a chunk whose table
    // alone reaches it is RAW without coding
    const uint32_t wcap0 = raw0 > wofs0 ? (raw0 - wofs0) / 2 : 0u;
    const uint32_t wcap1 = nch == 2 && raw1 > wofs1 ? (raw1 - wofs1) / 2 : 0u;
    const uint32_t end0 = raw0 / 2, end1 = ((uint32_t)p.slot_stride + raw1) / 2;  // word index just past each slot's words
    uint32_t r0 = end0, r1 = end1;  // word index just past the words still to come, per half
    // sampled tables: the bytes for words and escapes before a record reaches its RAW size
    const uint32_t room0 = raw0 > wofs0 ? raw0 - wofs0 : 0u, room1 = nch == 2 && raw1 > wofs1 ? raw1 - wofs1 : 0u;
    // a half stops coding once its words (and escapes) outgrow the RAW size
    bool alive0 = S ? room0 > 0 : wcap0 > 0, alive1 = S ? room1 > 0 : wcap1 > 0;
    uint32_t nesc0 = 0, nesc1 = 0;  // escaped values so far, per half (sampled tables)
    uint32_t x = kStateLow;
    // (with sampled tables every value is visited: the pass also writes the sign+mantissa bytes)
    const uint32_t T0 = S || alive0 ? (vals0 + 31) / 32 : 0u, T1 = S || alive1 ? (vals1 + 31) / 32 : 0u;
    // sampled tables: the pair's sign+mantissa bytes (past a chunk's end: out of range, dropped)
    const rsrc_t rsm2 = make_rsrc(d.out + d.sm_off + c0 * ce * R, pair_vals * R);
    const uint32_t smo2 = ((h ? vals0 : 0u) + lj) * R;
    const uint32_t escbase = h * (uint32_t)p.slot_stride + (h ? wofs1 : wofs0);  // this half's escape area in rslot
    // Escaped exponents go to the slot's escape area, last value first (a
    // value's byte lands at the count of escapes after it); the compaction
    // writes them after the words in value order.
    auto put_escapes = [&](uint64_t escm, uint32_t ex) __attribute__((always_inline)) {
        const uint32_t elo = __builtin_popcount((uint32_t)escm), ehi = __builtin_popcount((uint32_t)(escm >> 32));
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(escm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)escm, 0u));
        const uint32_t above = (h ? ehi : elo) - (below - (h ? elo : 0u)) - 1u;
        const uint32_t pos = (h ? nesc1 : nesc0) + above;
        bst8(rslot, (escm >> lane) & 1u ? escbase + pos : kOutOfRange, ex);
        nesc0 += elo;
        nesc1 += ehi;
    };
    const uint32_t nblk = (max(T0, T1) + 7) / 8;
    const uint32_t hsel = h ? 0xFFFFFFFFu : 0u;
    uint32_t escsteps = 0;  // FAST blocks (sampled tables): bit k set when step k has an escape not yet placed
    // One step; CAREFUL steps rebuild the lane masks and check the room
    // (a ragged chunk end, or words close to the RAW size), the others use
    // the block's loop-invariant mask.
    // (FAST steps get the exponent from the block's staging area, have_ex;
    // CAREFUL steps extract it from the value v)
    auto step = [&](int32_t b, int k, uint32_t v, bool careful, uint64_t act, bool have_ex = false,
                    uint32_t ex_in = 0u) __attribute__((always_inline)) {
        const uint32_t t = (uint32_t)b * 8 + k;
        if (careful)
            act = (alive0 && vals0 > 32 * t ? half_prefix_mask(vals0 - 32 * t, 0) : 0ull) |
                  (alive1 && vals1 > 32 * t ? half_prefix_mask(vals1 - 32 * t, 1) : 0ull);
        uint32_t ex = ex_in;  // the value's exponent
        if (!have_ex) asm("v_bfe_u32 %0, %1, %2, %3" : "=v"(ex) : "v"(v), "i"(Fmt<DT>::SYM), "i"(Fmt<DT>::SB));
        const uint4 te = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(tab) + (ex << 4));
        uint64_t m = lanes_lt(te.x & 0xFFFFu, x >> 16) & act;  // x >= f * 2^20
        uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
        uint32_t clo = __builtin_popcount(lo), chi = __builtin_popcount(hi);
        uint64_t escm = 0;
        if (careful) {
            if (S) {
                escm = lanes_eq(te.y, kEscSlot) & act;
                const uint32_t elo = __builtin_popcount((uint32_t)escm), ehi = __builtin_popcount((uint32_t)(escm >> 32));
                if (alive0 && 2 * ((end0 - r0) + clo) + nesc0 + elo > room0) alive0 = false;
                if (alive1 && 2 * ((end1 - r1) + chi) + nesc1 + ehi > room1) alive1 = false;
            } else {
                if (alive0 && (end0 - r0) + clo > wcap0) alive0 = false;
                if (alive1 && (end1 - r1) + chi > wcap1) alive1 = false;
            }
            const uint64_t am = (alive0 ? 0xFFFFFFFFull : 0ull) | (alive1 ? kHighHalf : 0ull);
            m &= am;
            act &= am;
            escm &= am;
            lo = (uint32_t)m;
            hi = (uint32_t)(m >> 32);
            clo = __builtin_popcount(lo);
            chi = __builtin_popcount(hi);
        }
        // The state's chain first (select, quotient, new state), the word's
        // place and store after it, so that the next step's chain may overlap them.
        const uint32_t xold = x;
        // (the state's select reads the compare's own result, not the masked
        // copy: lanes outside act keep their state below, and a stopped half's
        // state is never used)
        const uint32_t xs = (te.x & 0xFFFFu) < (x >> 16) ? x >> 16 : x;
        const uint32_t qd = enc_quotient(xs, __hiloint2double((int)te.w, (int)te.z));
        const uint32_t xe = __umul24(qd, te.x >> 16) + (xs + te.y);  // = q * M + (xs - q * f) + c0
        // Lanes past a ragged chunk end keep their state.  Outside CAREFUL
        // steps every lane of a live half codes a value, and a stopped
        // half's state is never used (its chunk is stored RAW).
        x = careful ? vsel(act, x, xe) : xe;
        // word index: end of the slot's words - (words so far + this step's) + rank in the half
        // (r0, r1: word index just past the words still to come)
        const uint32_t e0 = r0 - clo;
        r1 -= chi;
        const uint32_t e1 = r1 - clo;
        r0 = e0;
        uint32_t hb;  // e1 - e0 in the upper half, 0 in the lower
        asm("v_and_b32 %0, %1, %2" : "=v"(hb) : "s"(e1 - e0), "v"(hsel));
        const uint32_t kk = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, e0 + hb));
        bst16(rslot, vsel(m, kOutOfRange, kk << 1), xold);
        if (S && careful) {  // (FAST blocks store their sign+mantissa bytes when the block is staged)
            if (R == 1) bst8(rsm2, smo2 + t * 32 * R, raw_of<DT>(v));
            if (R == 3) {
                const uint32_t smv = raw_of<DT>(v);
                bst16(rsm2, smo2 + t * 32 * R, smv);
                bst8(rsm2, smo2 + t * 32 * R + 2, smv >> 16);
            }
            if (escm) put_escapes(escm, ex);
        } else if (S) {
            escsteps |= lanes_eq(te.y, kEscSlot) != 0 ? 1u << k : 0u;
        }
    };
    // a block codes at most 256 values, so at most 256 words, per half: a
    // FAST block needs no per-step checks
    // (sampled tables: at most 256 escapes too, and every value of the block
    // inside its chunk: the block's sign+mantissa bytes leave in whole units)
    auto block_fast = [&](int32_t b) __attribute__((always_inline)) {
        const uint32_t tend = ((uint32_t)b + 1) * 256;
        if (S)
            return vals0 >= tend && (nch == 1 || vals1 >= tend) &&
                   (!alive0 || 2 * ((end0 - r0) + 256) + nesc0 + 256 <= room0) &&
                   (!alive1 || 2 * ((end1 - r1) + 256) + nesc1 + 256 <= room1);
        return (!alive0 || (vals0 >= tend && (end0 - r0) + 256 <= wcap0)) &&
               (!alive1 || (vals1 >= tend && (end1 - r1) + 256 <= wcap1));
    };
    // A FAST block is read as whole units, lane lj taking values 8lj .. 8lj + 7
    // of its half's 256 (one 128-bit load; fp32 two, fp8 one 64-bit), and
    // staged: the lane writes their eight exponents to the half's 256-byte
    // staging area in LDS, from which step k of lane j reads byte 32k + j
    // (value 256b + 32k + j, the value that step codes); with sampled tables
    // it also stores their sign+mantissa bytes as one unit.  (Measured against
    // one 16-bit load per value and step in the full-table encoder: 0.7% faster
    // for bf16, 1.5% fp16, 3-4.5% fp8.)
    // Runs of FAST blocks are software-pipelined: the next block's unit is
    // loaded while a block is coded, and staged after its wait.  One counter
    // tracks loads and stores in issue order, so the compiler's wait for those
    // values, placed after the block's word stores, would also wait for the
    // stores.  The loads are therefore issued in asm and waited for
    // explicitly: between the loads and their wait lies only the coding of one
    // FAST block, straight-line code with exactly eight word stores (and the
    // unit's sign+mantissa stores), so at most that many operations may remain
    // outstanding.  Every branch and loop edge comes after a wait, so no
    // register with a load in flight is ever copied (a test checks the
    // generated code for this).  Other blocks use ordinary loads.
    // With sampled tables the unit loads carry the non-temporal hint: each
    // value is read once (measured: about 2% faster than the default policy on
    // the gradient bucket; the same hint on the sign+mantissa stores, on the
    // full-table encoder's loads, which re-read what pass 1 read, or on the
    // decoder's loads was slower).
    uint8_t *stage = reinterpret_cast<uint8_t *>(lds) + h * 256;  // (the keys' words, free in this pass)
    constexpr uint32_t NU = EB == 4 ? 2 : 1;  // loads per unit (fp8: one 64-bit)
    using UnitT = typename std::conditional<EB == 1, u32x2, u32x4>::type;
    auto asm_load_unit = [&](int32_t bb, UnitT(&U)[2]) __attribute__((always_inline)) {
        const uint32_t o = bb >= 0 ? in0 + ((uint32_t)bb * 256 + 8 * lj) * EB : kOutOfRange;
        if constexpr (EB == 1 && S) {
            asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen nt" : "=v"(U[0]) : "v"(o), "s"(rin));
        } else if constexpr (EB == 1) {
            asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen" : "=v"(U[0]) : "v"(o), "s"(rin));
        } else if constexpr (S) {
#pragma unroll
            for (uint32_t u = 0; u < NU; ++u)
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3 nt" : "=v"(U[u]) : "v"(o), "s"(rin), "i"(16 * u));
        } else {
#pragma unroll
            for (uint32_t u = 0; u < NU; ++u)
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3" : "=v"(U[u]) : "v"(o), "s"(rin), "i"(16 * u));
        }
    };
    // the unit's sign+mantissa bytes (bf16, fp16: 8; fp32: 24), stored by store_sm
    constexpr uint32_t kSmStores = !S || R == 0 ? 0 : R == 1 ? 1 : 2;
    auto stage_unit = [&](const UnitT(&U)[2], uint32_t(&SM)[6]) __attribute__((always_inline)) {
        uint32_t e0, e1;  // the eight exponents, value order
        if constexpr (DT == 1 || DT == 3) {
            // low and high bytes of four values at once
            const uint32_t lo0 = __builtin_amdgcn_perm(U[0].y, U[0].x, 0x06040200u);
            const uint32_t hi0 = __builtin_amdgcn_perm(U[0].y, U[0].x, 0x07050301u);
            const uint32_t lo1 = __builtin_amdgcn_perm(U[0].w, U[0].z, 0x06040200u);
            const uint32_t hi1 = __builtin_amdgcn_perm(U[0].w, U[0].z, 0x07050301u);
            uint32_t s0 = lo0, s1 = lo1;
            e0 = hi0;
            e1 = hi1;
            if (DT == 1) {  // sign = bit 7 of the high byte, exponent = its bits 0-6 and bit 7 of the low byte
                s0 = (hi0 & 0x80808080u) | (lo0 & 0x7F7F7F7Fu);
                s1 = (hi1 & 0x80808080u) | (lo1 & 0x7F7F7F7Fu);
                e0 = ((hi0 << 1) & 0xFEFEFEFEu) | ((lo0 >> 7) & 0x01010101u);
                e1 = ((hi1 << 1) & 0xFEFEFEFEu) | ((lo1 >> 7) & 0x01010101u);
            } else {  // fp16: the exponent is bits 2-6 of the high byte
                e0 = (hi0 >> 2) & 0x1F1F1F1Fu;
                e1 = (hi1 >> 2) & 0x1F1F1F1Fu;
            }
            SM[0] = s0;
            SM[1] = s1;
        } else if constexpr (DT == 2) {
            const uint32_t w[8] = {U[0].x, U[0].y, U[0].z, U[0].w, U[1].x, U[1].y, U[1].z, U[1].w};
            uint32_t sm[8], ex[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sm[k] = ((w[k] >> 8) & 0x800000u) | (w[k] & 0x7FFFFFu);
                ex[k] = (w[k] >> 23) & 0xFFu;
            }
            e0 = ex[0] | (ex[1] << 8) | (ex[2] << 16) | (ex[3] << 24);
            e1 = ex[4] | (ex[5] << 8) | (ex[6] << 16) | (ex[7] << 24);
            SM[0] = sm[0] | (sm[1] << 24);
            SM[1] = (sm[1] >> 8) | (sm[2] << 16);
            SM[2] = (sm[2] >> 16) | (sm[3] << 8);
            SM[3] = sm[4] | (sm[5] << 24);
            SM[4] = (sm[5] >> 8) | (sm[6] << 16);
            SM[5] = (sm[6] >> 16) | (sm[7] << 8);
        } else {  // fp8: bits 3-6 (e4m3fn) or 2-6 (e5m2) of each byte
            e0 = (U[0].x >> Fmt<DT>::SYM) & (((1u << Fmt<DT>::SB) - 1u) * 0x01010101u);
            e1 = (U[0].y >> Fmt<DT>::SYM) & (((1u << Fmt<DT>::SB) - 1u) * 0x01010101u);
        }
        asm volatile("" ::: "memory");  // (after the last block's reads of the area)
        *reinterpret_cast<u32x2 *>(stage + 8 * lj) = u32x2{e0, e1};
    };
    // (issued after the next unit's loads, so that the wait for those loads
    // does not also wait for this store)
    auto store_sm = [&](int32_t bb, const uint32_t(&SM)[6]) __attribute__((always_inline)) {
        const uint32_t so = ((h ? vals0 : 0u) + (uint32_t)bb * 256 + 8 * lj) * R;  // past the pair: dropped
        if constexpr (!S) {
            (void)so;
        } else if constexpr (R == 1) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{SM[0], SM[1]}, rsm2, (int)so, 0, 0);
        } else if constexpr (R == 3) {
            __builtin_amdgcn_raw_buffer_store_b96(u32x3{SM[0], SM[1], SM[2]}, rsm2, (int)so, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b96(u32x3{SM[3], SM[4], SM[5]}, rsm2, (int)(so + 12), 0, 0);
        }
    };
    auto fast_block = [&](int32_t b) __attribute__((always_inline)) {
        const uint64_t act = (alive0 ? 0xFFFFFFFFull : 0ull) | (alive1 ? kHighHalf : 0ull);
        asm volatile("" ::: "memory");  // (after the staging writes)
        uint32_t E[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) E[k] = stage[32 * k + lj];
#pragma unroll
        for (int k = 7; k >= 0; --k) step(b, k, 0u, false, act, true, E[k]);
    };
    // escapes of a FAST block, placed after the block from the staged exponents, last first
    auto block_escapes_s = [&]() __attribute__((always_inline)) {
        const uint64_t act = (alive0 ? 0xFFFFFFFFull : 0ull) | (alive1 ? kHighHalf : 0ull);
        for (int k = 7; k >= 0; --k) {
            if (((escsteps >> k) & 1u) == 0) continue;
            const uint32_t ex = stage[32 * k + lj];
            const uint32_t cy = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(tab) + (ex << 4) + 4);
            const uint64_t escm = lanes_eq(cy, kEscSlot) & act;
            if (escm) put_escapes(escm, ex);
        }
    };
#define UZIP_WAIT_UNIT(N, U) asm volatile("s_waitcnt vmcnt(%2)" : "+v"(U[0]), "+v"(U[1]) : "i"(N))
    for (int32_t b = (int32_t)nblk - 1; b >= 0;) {
        if (!block_fast(b)) {
            const uint32_t o = in0 + ((uint32_t)b * 8 * 32 + lj) * EB;
            uint32_t V[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) V[k] = bld_value<DT>(rin, o + k * 32 * EB);
#pragma unroll
            for (int k = 7; k >= 0; --k) step(b, k, V[k], true, 0ull);
            --b;
            continue;
        }
        UnitT UA[2] = {}, UB[2] = {};
        uint32_t SM[6] = {0, 0, 0, 0, 0, 0};
        asm_vmem_fence();
        asm_load_unit(b, UA);
        UZIP_WAIT_UNIT(0, UA);
        stage_unit(UA, SM);
        for (;;) {
            asm_load_unit(b - 1, UB);
            store_sm(b, SM);
            fast_block(b);
            UZIP_WAIT_UNIT(8 + kSmStores, UB);
            if (escsteps) {
                block_escapes_s();
                escsteps = 0;
            }
            if (--b < 0 || !block_fast(b)) break;
            stage_unit(UB, SM);
            asm_load_unit(b - 1, UA);
            store_sm(b, SM);
            fast_block(b);
            UZIP_WAIT_UNIT(8 + kSmStores, UA);
            if (escsteps) {
                block_escapes_s();
                escsteps = 0;
            }
            if (--b < 0 || !block_fast(b)) break;
            stage_unit(UA, SM);
        }
    }
#undef UZIP_WAIT_UNIT

    // ---- the record's fixed part into the slot (the words are already at its
    // end); a RAW record gets its header only: k_compact takes its exponents
    // from the input ----
    const uint32_t nw = h ? end1 - r1 : end0 - r0;  // words emitted
    const uint32_t ne = h ? nesc1 : nesc0;          // values escaped (sampled tables)
    const bool alive = h ? alive1 : alive0;
    const uint32_t raw_i = h ? raw1 : raw0;
    const uint32_t rans_bytes = (uint32_t)(S ? align16(words_offset_sampled(nsym) + 2ull * nw + ne)
                                             : align16(words_offset(nsym) + 2ull * nw));
    if (valid) {
        const bool rans = alive && rans_bytes < raw_i;  // ties go RAW
        if (rans) gstore<uint32_t>(slot + (S ? states_offset_sampled(nsym) : states_offset(nsym)) + 4 * lj, x);
        if (lj == 0) {
            if (S && rans) gstore<uint32_t>(slot + esc_count_offset(nsym), ne);
            // record mode 0 (full table) or 2 (sampled table), else 1 (RAW)
            gstore<uint4>(slot, rans ? make_uint4((S ? 2u : 0u) | (nsym << 16), nw, ni, rans_bytes)
                                     : make_uint4(1u, 0u, ni, raw_i));
            gstore<uint32_t>(p.rec_sizes + g, rans ? rans_bytes : raw_i);
        }
    }
}

// ---------------------------------------------------------------------------
// k_plan: per-call arbitration (NCCLZ Sec. IV-C, Eq. (1) and (2), Algorithm 1)
// ---------------------------------------------------------------------------
// 2^16 log2(x) for x >= 1, rounded down, digit by digit (the squaring method):
// with x = 2^y z, z in [1, 2), squaring z doubles log2 z, and the integer part
// of the square is the next binary digit.  z has 31 fraction bits and is
// truncated after every squaring, so the result is exact at powers of two
// and at most one unit below 2^16 log2 x elsewhere.
__device__ inline uint32_t log2_q16(uint32_t x) {
    const uint32_t y = 31u - (uint32_t)__builtin_clz(x);
    uint64_t z = uint64_t(x) << (31u - y);
    uint32_t frac = 0;
    for (int i = 0; i < 16; ++i) {
        z = (z * z) >> 31;
        frac <<= 1;
        if (z >> 32) {
            z >>= 1;
            frac |= 1u;
        }
    }
    return (y << 16) | frac;
}

__device__ inline uint64_t ceil_div_u64(uint64_t a, uint64_t b) { return a / b + (a % b != 0); }

// One workgroup of 256 threads per buffer.  A buffer of at most small_bytes
// goes RAW unsampled.  Otherwise the workgroup counts the coded symbols of the
// buffer's first min(N, 64 KiB / value size) values in LDS, sums
// c (log2 S - log2 c) over the 256 counts (one count per thread) for the
// sample's entropy, predicts the coded frame from it, and evaluates the two
// transfer times of the cost model in integer nanoseconds: coded when the
// predicted gain is admitted and coding is strictly faster, RAW otherwise.
// k_encode reads the decision on the device.
template <int DT>
__global__ __launch_bounds__(256) void k_plan(EncParams p) {
    constexpr uint32_t EB = Fmt<DT>::EB;
    __shared__ uint32_t hist[8][257];  // 8 sub-histograms (thread t counts into t & 7), padded rows
    __shared__ uint64_t part[4];
    __shared__ uint32_t present[4];
    const uint32_t t = threadIdx.x;
    const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + blockIdx.x);
    uint8_t *out = reinterpret_cast<uint8_t *>(p.plans + blockIdx.x);
    const uzip_policy &pol = p.policy;
    const uint64_t n = d.n, B = n * EB;
    if (B <= pol.small_bytes) {  // the small-call fast path
        if (t < 4) gstore<uint2>(out + 8 * t, make_uint2(t == 0 ? UZIP_PLAN_RAW_SMALL : 0u, 0u));
        return;
    }
    const uint32_t S = (uint32_t)min<uint64_t>(n, 65536u / EB);
    for (uint32_t k = 0; k < 8; ++k) hist[k][t] = 0;
    if (t < 8) hist[t][256] = 0;
    __syncthreads();
    uint32_t *sub = hist[t & 7];
    // the sample in one round of loads: thread t takes the whole 16-byte
    // units t + 256 k (k < 16) of the at most 64 KiB; a partial last unit is
    // read value by value (a 128-bit load that crosses the end of the range
    // would read its last dword as zero)
    const rsrc_t rin = make_rsrc(d.in, S * EB);
    constexpr uint32_t VPU = 16 / EB;
    const uint32_t units = S / VPU;
    uint4 q[16];
#pragma unroll
    for (uint32_t k = 0; k < 16; ++k) q[k] = bld128(rin, t + 256 * k < units ? 16 * (t + 256 * k) : kOutOfRange);
#pragma unroll
    for (uint32_t k = 0; k < 16; ++k) {
        if (t + 256 * k >= units) continue;
        const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
        for (uint32_t j = 0; j < VPU; ++j) {
            const uint32_t v = EB == 4 ? w[j] : (w[j / (4 / EB)] >> (8 * EB * (j % (4 / EB)))) & ((1u << (8 * EB)) - 1u);
            atomicAdd(&sub[exponent_of<DT>(v)], 1u);
        }
    }
    if (t == 0)
        for (uint32_t i = units * VPU; i < S; ++i) atomicAdd(&sub[exponent_of<DT>(bld_value<DT>(rin, i * EB))], 1u);
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) c += hist[k][t];
    const uint64_t term = c ? uint64_t(c) * (log2_q16(S) - log2_q16(c)) : 0ull;
    const uint64_t wsum = wave_sum_u64(term);
    const uint32_t wpresent = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(c != 0));
    if ((t & 63) == 0) {
        part[t >> 6] = wsum;
        present[t >> 6] = wpresent;
    }
    __syncthreads();
    if (t != 0) return;
    const uint64_t hs = part[0] + part[1] + part[2] + part[3];
    const uint32_t nsym = present[0] + present[1] + present[2] + present[3];
    const uint64_t h = hs / S;  // bits per value in units of 2^-16
    const uint64_t ce = p.chunk_elems;
    const Layout l = layout_of(p.dtype, n, ce);
    const uint64_t pred = l.exp_off + ceil_div_u64(n * h, 1ull << 19) + l.chunks * (words_offset(nsym) + 8);
    const uint64_t praw = l.exp_off + (l.chunks - 1) * raw_record_bytes(ce, Fmt<DT>::SB) +
                          raw_record_bytes(n - (l.chunks - 1) * ce, Fmt<DT>::SB);
    const uint64_t t_raw = ceil_div_u64(praw * 1000, pol.link_bytes_per_us);
    const uint64_t t_code = pol.fixed_ns + ceil_div_u64(pred * 1000, pol.link_bytes_per_us) +
                            ceil_div_u64(uint64_t(pol.exposed_encode_permil) * B, pol.encode_bytes_per_us) +
                            ceil_div_u64(uint64_t(pol.exposed_decode_permil) * B, pol.decode_bytes_per_us);
    const bool admitted = pred < praw && (praw - pred) * 1000 >= uint64_t(pol.min_gain_permil) * B;
    const uint32_t decision = admitted && t_code < t_raw ? UZIP_PLAN_CODED : UZIP_PLAN_RAW;
    // the plan as uzip_plan lays it out (8-byte aligned: four 8-byte stores)
    gstore<uint2>(out, make_uint2(decision, S));
    gstore<uint2>(out + 8, make_uint2((uint32_t)pred, (uint32_t)(pred >> 32)));
    gstore<uint2>(out + 16, make_uint2((uint32_t)t_raw, (uint32_t)(t_raw >> 32)));
    gstore<uint2>(out + 24, make_uint2((uint32_t)t_code, (uint32_t)(t_code >> 32)));
}

// The frame of a buffer that its plan sends RAW, in one pass over the input:
// every record is RAW, so record c starts at c * align16(16 + chunk_elems)
// with no scan.  A workgroup (256 threads) takes a chunk at a time: each
// thread reads units of 16 values (EB 128-bit loads) and writes their raw
// bytes to the sign+mantissa region and their symbol bytes to the record
// (128-bit stores); the chunk's ragged end goes value by value, with the
// record's zero padding.  Thread 0 writes the record header and the chunk's
// index entry; the buffer's last chunk also writes the final index entry,
// the header, the zero gaps and the compressed size.  Coded buffers are left
// to k_encode and k_compact.
__device__ inline uint32_t find_enc_chunk_buffer(const EncDesc *d, uint32_t nbuf, uint64_t g) {
    uint32_t lo = 0, hi = nbuf - 1;  // the last buffer whose first chunk is <= g (empty ones own none)
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (gload<uint64_t>(&d[mid].chunk_first) <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int DT>
__global__ __launch_bounds__(256) void k_raw_frame(EncParams p) {
    constexpr uint32_t EB = Fmt<DT>::EB, R = Fmt<DT>::R;
    const uint32_t t = threadIdx.x;
    for (uint64_t g = blockIdx.x; g < p.total_chunks; g += gridDim.x) {
        const uint32_t bi = p.nbuf == 1 ? 0u : uniform_u32(find_enc_chunk_buffer(p.descs, p.nbuf, g));
        // pass 0 (before the compaction): the buffers planned RAW; pass 1
        // (after the realised-gain check): the buffers whose coded frame failed it
        const uint32_t dec = uniform_u32(gload<uint32_t>(&p.plans[bi].decision));
        if (dec == UZIP_PLAN_CODED || (dec == UZIP_PLAN_RAW_REALIZED) != (p.raw_pass != 0)) continue;
        const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + bi);
        const uint64_t ce = p.chunk_elems, n = uniform_u64(d.n), chunks = uniform_u64(d.chunks);
        const uint64_t c = g - uniform_u64(d.chunk_first);
        const uint32_t ni = (uint32_t)min<uint64_t>(ce, n - c * ce);
        const uint64_t rrb = raw_record_bytes(ce, Fmt<DT>::SB), off = c * rrb;
        uint8_t *out = d.out;
        const uint64_t exp_off = uniform_u64(d.exp_off), sm_off = uniform_u64(d.sm_off);
        const rsrc_t rin = make_rsrc(d.in + c * ce * EB, ni * EB);
        const rsrc_t rsm = make_rsrc(out + sm_off + c * ce * R, ni * R);
        const uint32_t rbytes = (uint32_t)raw_record_bytes(ni, Fmt<DT>::SB);
        const rsrc_t rrec = make_rsrc(out + exp_off + off, rbytes);
        if constexpr (R == 0) {
            // fp16 and fp8: the chunk's raw fields and its symbols, each packed.
            // A thread takes whole groups of 32 values (8 EB dwords in, RB raw
            // and SB symbol dwords out, all aligned); the dwords of the
            // chunk's ragged last group and the record's padding after the
            // groups are built one dword per thread from the values they
            // cover.  The raw region's last dword may reach into the zero gap
            // after it.
            constexpr uint32_t RB = Fmt<DT>::RB, SB = Fmt<DT>::SB;
            uint8_t *rawp = out + sm_off + c * ce * RB / 8;
            const uint32_t nd_raw = (uint32_t)((packed_bytes(ni, RB) + 3) / 4);
            const rsrc_t rraw = make_rsrc(rawp, 4 * nd_raw);
            const uint32_t ng = ni / 32;
            for (uint32_t g = t; g < ng; g += 256) {
                uint32_t w[8 * EB], fr[32], fs[32], orw[RB], osy[SB];
                load_dwords<8 * EB>(rin, 32 * EB * g, w);
#pragma unroll
                for (uint32_t i = 0; i < 32; ++i) {
                    const uint32_t v = (w[i * EB / 4] >> (8 * EB * (i % (4 / EB)))) & ((1u << (8 * EB)) - 1u);
                    fr[i] = raw_of<DT>(v);
                    fs[i] = exponent_of<DT>(v);
                }
                pack32<RB>(fr, orw);
                pack32<SB>(fs, osy);
                store_dwords<RB>(rraw, 4 * RB * g, orw);
                store_dwords<SB>(rrec, kRecHeaderBytes + 4 * SB * g, osy);
            }
            for (uint32_t k = RB * ng + t; k < nd_raw; k += 256)
                gstore<uint32_t>(rawp + 4 * k, packed_dword(k, ni, RB, [&](uint32_t i) {
                    return raw_of<DT>(bld_value<DT>(rin, i * EB));
                }));
            for (uint32_t k = SB * ng + t; k < (rbytes - kRecHeaderBytes) / 4; k += 256)
                gstore<uint32_t>(out + exp_off + off + kRecHeaderBytes + 4 * k, packed_dword(k, ni, SB, [&](uint32_t i) {
                    return exponent_of<DT>(bld_value<DT>(rin, i * EB));
                }));
        } else {
        const uint32_t nu = ni / 16;
        constexpr uint32_t U = 4;  // units per thread in flight
        for (uint32_t u0 = t; u0 < nu; u0 += 256 * U) {
            uint4 qs[U][EB];
#pragma unroll
            for (uint32_t j = 0; j < U; ++j) {
                const uint32_t u = u0 + 256 * j;
#pragma unroll
                for (uint32_t k = 0; k < EB; ++k) qs[j][k] = bld128(rin, u < nu ? 16 * EB * u + 16 * k : kOutOfRange);
            }
#pragma unroll
            for (uint32_t j = 0; j < U; ++j) {
                const uint32_t u = u0 + 256 * j;
                const uint32_t so = u < nu ? 16 * R * u : kOutOfRange, eo = u < nu ? kRecHeaderBytes + 16 * u : kOutOfRange;
                uint32_t w[4 * EB];
#pragma unroll
                for (uint32_t k = 0; k < EB; ++k) {
                    w[4 * k] = qs[j][k].x; w[4 * k + 1] = qs[j][k].y; w[4 * k + 2] = qs[j][k].z; w[4 * k + 3] = qs[j][k].w;
                }
                uint32_t ex[4] = {0, 0, 0, 0}, rw[12] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (uint32_t k = 0; k < 16; ++k) {
                    const uint32_t v = EB == 4 ? w[k] : (w[k / (4 / EB)] >> (8 * EB * (k % (4 / EB)))) & ((1u << (8 * EB)) - 1u);
                    ex[k >> 2] |= exponent_of<DT>(v) << (8 * (k & 3));
                    if (R == 1) rw[k >> 2] |= raw_of<DT>(v) << (8 * (k & 3));
                    if (R == 3) {  // 3 bytes at byte 3k of rw
                        const uint32_t b = 3 * k, sm = raw_of<DT>(v);
                        rw[b >> 2] |= sm << (8 * (b & 3));
                        if ((b & 3) > 1) rw[(b >> 2) + 1] |= sm >> (32 - 8 * (b & 3));
                    }
                }
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{ex[0], ex[1], ex[2], ex[3]}, rrec, (int)eo, 0, 0);
#pragma unroll
                for (uint32_t k = 0; k < R; ++k)
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{rw[4 * k], rw[4 * k + 1], rw[4 * k + 2], rw[4 * k + 3]}, rsm,
                                                           (int)(so + 16 * k), 0, 0);
            }
        }
        // the chunk's ragged end: the last unit of symbol bytes with its zero
        // padding, and the raw bytes value by value
        if (nu * 16 < ni && t == 0) {
            uint32_t ex[4] = {0, 0, 0, 0};
            for (uint32_t k = 0; 16 * nu + k < ni; ++k) {
                const uint32_t v = bld_value<DT>(rin, (16 * nu + k) * EB);
                ex[k >> 2] |= exponent_of<DT>(v) << (8 * (k & 3));
                const uint32_t sm = raw_of<DT>(v);
                for (uint32_t r = 0; r < R; ++r)
                    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(sm >> (8 * r)), rsm, (int)((16 * nu + k) * R + r), 0, 0);
            }
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{ex[0], ex[1], ex[2], ex[3]}, rrec, (int)(kRecHeaderBytes + 16 * nu), 0, 0);
        }
        }  // byte types
        if (t == 0) {
            gstore<uint4>(out + exp_off + off, make_uint4(1u, 0u, ni, rbytes));
            gstore<uint64_t>(out + kHeaderBytes + 8 * c, off);
        }
        if (c + 1 == chunks) {  // the buffer's last record
            const uint64_t total = exp_off + off + rbytes;
            if (t == 0) {
                gstore<uint64_t>(out + kHeaderBytes + 8 * chunks, off + rbytes);
                gstore<uint64_t>(d.out_size, total);
            }
            if (t < 16) gstore<uint32_t>(out + 4 * t, header_word(t, p.dtype, p.chunk_elems, n, chunks, sm_off, exp_off, total));
            for (uint64_t k = kHeaderBytes + 8 * (chunks + 1) + t; k < sm_off; k += 256) gstore<uint8_t>(out + k, 0);
            for (uint64_t k = sm_off + packed_bytes(n, Fmt<DT>::RB) + t; k < exp_off; k += 256) gstore<uint8_t>(out + k, 0);
        }
    }
}

// Acceptance of the realised frame (NCCLZ Algorithm 1: a materialised coded
// plan is kept only if its realised output passes the capacity and gain
// checks, else the RAW frame is committed).  One thread per buffer, after the
// compaction has written each coded buffer's size R: the coded frame stays
// when R < P_raw and (P_raw - R) * 1000 >= min_gain * B, the admission rule
// on the realised size; otherwise the plan becomes UZIP_PLAN_RAW_REALIZED and
// the second k_raw_frame pass rewrites the buffer as its all-RAW frame.
// (Capacity always holds: no record exceeds its RAW record.)
template <int DT>
__global__ __launch_bounds__(256) void k_accept(EncParams p) {
    const uint32_t bi = blockIdx.x * 256 + threadIdx.x;
    if (bi >= p.nbuf) return;
    if (gload<uint32_t>(&p.plans[bi].decision) != UZIP_PLAN_CODED) return;
    const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + bi);
    const uint64_t ce = p.chunk_elems, n = d.n, B = n * Fmt<DT>::EB;
    const Layout l = layout_of(p.dtype, n, ce);
    const uint64_t praw = l.exp_off + (l.chunks - 1) * raw_record_bytes(ce, Fmt<DT>::SB) +
                          raw_record_bytes(n - (l.chunks - 1) * ce, Fmt<DT>::SB);
    const uint64_t R = gload<uint64_t>(d.out_size);
    const bool accepted = R < praw && (praw - R) * 1000 >= uint64_t(p.policy.min_gain_permil) * B;
    if (!accepted) gstore<uint32_t>(&p.plans[bi].decision, UZIP_PLAN_RAW_REALIZED);
}

// ---------------------------------------------------------------------------
// k_compact: record offsets (exclusive scan of the record sizes) and the
// records at their final place
// ---------------------------------------------------------------------------
// A workgroup of 2 * kCompactPairs waves takes the next kCompactPairs chunk
// pairs in ticket order; wave w works on record w & 1 of pair w >> 1.  Both
// waves of a pair find the offset of the pair's records (the sizes of the
// pair's tile summed directly, plus the tile's prefix by look-back over the
// buffer's tiles, whose totals the tile's first pair publishes); then each
// wave writes its index entry and copies its record from the slot (RAW
// records are rebuilt from the input), and the buffer's last record writes
// the final index entry, the header, the zero gaps and the compressed size
// (NCCLZ Sec. IV-D2: self-describing frames).  A wave only waits for tile
// leaders in workgroups with lower tickets, or in its own workgroup, all of
// which already run.  Eight pairs per 1024-thread workgroup: fewer tickets and
// workgroup launches than four or two per workgroup (gradient bucket: the
// compaction and its launch gaps ≈10 µs shorter than with four).
constexpr uint32_t kCompactPairs = 8;

template <int DT>
__global__ __launch_bounds__(128 * kCompactPairs) void k_compact(EncParams p) {
    constexpr uint32_t EB = Fmt<DT>::EB;
    __shared__ uint32_t s_ticket;
    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint64_t q = uint64_t(uniform_u32(s_ticket)) * kCompactPairs + (w >> 1);
    const uint32_t r = w & 1;
    if (q >= p.total_pairs) return;
    const uint32_t bi = p.nbuf == 1 ? 0u : uniform_u32(find_enc_pair_buffer(p.descs, p.nbuf, q));
    // RAW-planned buffers are complete (k_raw_frame); their tiles take no part
    // in any other buffer's look-back
    if (p.plans != nullptr && uniform_u32(gload<uint32_t>(&p.plans[bi].decision)) != UZIP_PLAN_CODED) return;
    const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + bi);
    const uint64_t ce = p.chunk_elems;
    const uint64_t n = uniform_u64(d.n);
    const uint64_t c0 = 2 * (q - uniform_u64(d.pair_first));
    const uint64_t chunks = uniform_u64(d.chunks);
    const uint32_t nch = chunks - c0 >= 2 ? 2u : 1u;
    const uint64_t g0 = uniform_u64(d.chunk_first) + c0;
    const uint32_t size0 = uniform_u32(gload<uint32_t>(p.rec_sizes + g0));
    const uint32_t size1 = nch == 2 ? uniform_u32(gload<uint32_t>(p.rec_sizes + g0 + 1)) : 0u;
    // Offset of the pair's records in two levels: the sizes of the pairs of
    // its tile (lane l: pair l of the tile), summed directly, plus the tile's
    // exclusive prefix by look-back over the buffer's tiles.
    const uint64_t lp = q - uniform_u64(d.pair_first);  // pair index in the buffer
    const uint64_t lt = lp / kPairTile;
    const uint32_t pos = (uint32_t)(lp % kPairTile);
    const uint64_t pl = lt * kPairTile + lane, cf = uniform_u64(d.chunk_first);
    uint64_t ps = 0;
    if (lane < kPairTile && 2 * pl < chunks) {
        ps = gload<uint32_t>(p.rec_sizes + cf + 2 * pl);
        if (2 * pl + 1 < chunks) ps += gload<uint32_t>(p.rec_sizes + cf + 2 * pl + 1);
    }
    const uint64_t tile_total = wave_sum_u64(ps);
    const uint64_t in_tile = wave_sum_u64(lane < pos ? ps : 0);
    const uint64_t tfirst = uniform_u64(d.tile_first);
    const uint64_t rec0 = in_tile + tile_lookback(p.flags, tfirst + lt, tfirst, tile_total, pos == 0 && r == 0, lane);
    if (r >= nch) return;

    // this wave's record
    const uint32_t stride = (uint32_t)p.slot_stride;
    const uint32_t vals0 = (uint32_t)min<uint64_t>(ce, n - c0 * ce);
    const uint32_t ni = r ? (uint32_t)min<uint64_t>(ce, n - (c0 + 1) * ce) : vals0;
    const uint32_t size = r ? size1 : size0;
    const uint64_t off = r ? rec0 + size0 : rec0;
    uint8_t *out = d.out;
    const uint64_t exp_off = uniform_u64(d.exp_off);
    uint8_t *rec = out + exp_off + off;
    if (lane == 0) gstore<uint64_t>(out + kHeaderBytes + 8 * (c0 + r), off);
    const rsrc_t rslot = make_rsrc(p.slots + (g0 + r) * p.slot_stride, stride);
    const uint4 hd = bld128(rslot, 0);
    const uint32_t mode = uniform_u32(hd.x) & 0xFFu, nsym = uniform_u32(hd.x) >> 16, nw = uniform_u32(hd.y);
    if (mode == 0 || mode == 2) {
        // header, bitmap, frequencies, pad, (escape count,) states, then the
        // words; a sampled-table record ends with its escaped exponents
        const uint32_t wofs = (uint32_t)(mode == 2 ? words_offset_sampled(nsym) : words_offset(nsym));
        for (uint32_t k = lane; k < wofs / 4; k += 64) gstore<uint32_t>(rec + 4 * k, bld32(rslot, 4 * k));
        copy_words(rslot, rec, wofs, size, 2 * nw, (uint32_t)raw_record_bytes(ni, Fmt<DT>::SB) - 2 * nw, lane);
        if (mode == 2) {
            const uint32_t ne = uniform_u32(bld32(rslot, (uint32_t)esc_count_offset(nsym)));
            if (ne > 0) {
                // the escape area holds them last value first, from byte wofs of the
                // slot; the zero padding the word copy wrote there must land first
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                for (uint32_t j = lane; j < ne; j += 64)
                    gstore<uint8_t>(rec + wofs + 2 * nw + j, (uint8_t)bld8(rslot, wofs + ne - 1 - j));
            }
        }
    } else {
        const rsrc_t rin = make_rsrc(d.in + (c0 + r) * ce * EB, ni * EB);
        if (lane < 4) gstore<uint32_t>(rec + 4 * lane, bld32(rslot, 4 * lane));
        raw_exponents<DT>(rin, rec, size, ni, 0u, lane);
    }

    if (c0 + r + 1 == chunks) {  // the buffer's last record
        const uint64_t recs = off + size;
        const uint64_t total = exp_off + recs;
        if (lane == 0) {
            gstore<uint64_t>(out + kHeaderBytes + 8 * chunks, recs);
            gstore<uint64_t>(d.out_size, total);
        }
        if (lane < 16)
            gstore<uint32_t>(out + 4 * lane,
                             header_word(lane, p.dtype, p.chunk_elems, n, chunks, d.sm_off, exp_off, total, p.sampled));
        const uint64_t gap0 = kHeaderBytes + 8 * (chunks + 1);
        for (uint64_t k = gap0 + lane; k < d.sm_off; k += 64) gstore<uint8_t>(out + k, 0);
        const uint64_t gap1 = d.sm_off + packed_bytes(n, Fmt<DT>::RB);
        for (uint64_t k = gap1 + lane; k < exp_off; k += 64) gstore<uint8_t>(out + k, 0);
    }
}

// ---------------------------------------------------------------------------
// scans
// ---------------------------------------------------------------------------
// exclusive scan of n values into out[0..n] (out[n] = total) by one workgroup
// of 1024 threads; in may equal out
__device__ inline void block_scan_u64(const uint64_t *in, uint64_t *out, uint64_t n) {
    __shared__ uint64_t s[1024];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < n; base += 1024) {
        const uint64_t i = base + threadIdx.x;
        const uint64_t v = i < n ? gload<uint64_t>(in + i) : 0;
        s[threadIdx.x] = v;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const uint64_t t = (int)threadIdx.x >= o ? s[threadIdx.x - o] : 0;
            __syncthreads();
            s[threadIdx.x] += t;
            __syncthreads();
        }
        if (i < n) gstore<uint64_t>(out + i, carry + s[threadIdx.x] - v);
        carry += s[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) gstore<uint64_t>(out + n, carry);
}

// Batched decompression, after validation (one workgroup): the exclusive scan
// of the buffers' chunk-pair counts, in place, and which decoders have work
// (bit 0: a valid buffer with full tables, bit 1: one with sampled tables).
__global__ __launch_bounds__(1024) void k_dec_scan(DecParams p) {
    __shared__ uint32_t s_kinds;
    if (threadIdx.x == 0) s_kinds = 0;
    __syncthreads();
    uint32_t kinds = 0;
    for (uint32_t b = threadIdx.x; b < p.nbuf; b += 1024)
        if (gload<uint32_t>(p.status + b) == 0) kinds |= (gload<uint64_t>(&p.info[b].flags) & 1u) ? 2u : 1u;
    if (kinds) atomicOr(&s_kinds, kinds);
    __syncthreads();
    if (threadIdx.x == 0) gstore<uint32_t>(p.kinds, s_kinds);
    block_scan_u64(p.pair_first, p.pair_first, p.nbuf);
}

// Before the encoder: zero the look-back words and the ticket counter (a fill
// kernel rather than a memset, so the call stays valid inside a captured
// graph), and write the 80-byte buffer of every empty input (N = 0).
__global__ __launch_bounds__(256) void k_prepare(EncParams p) {
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < p.total_pairs) gstore<uint64_t>(p.flags + i, 0);
    if (i == 0) gstore<uint32_t>(p.ticket, 0);
    if (i < p.nbuf) {
        const EncDesc d = p.nbuf == 1 ? p.single : load_enc_desc(p.descs + i);
        if (d.n == 0) {
            for (uint32_t k = 0; k < 16; ++k)
                gstore<uint32_t>(d.out + 4 * k, header_word(k, p.dtype, p.chunk_elems, 0, 0, 80, 80, 80, p.sampled));
            gstore<uint64_t>(d.out + kHeaderBytes, 0);
            gstore<uint64_t>(d.out + kHeaderBytes + 8, 0);
            gstore<uint64_t>(d.out_size, 80);
        }
    }
}

// ---------------------------------------------------------------------------
// decompression
// ---------------------------------------------------------------------------
__global__ void k_dec_validate(DecParams p) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= p.nbuf) return;
    const DecDesc d = p.nbuf == 1 ? p.single : load_dec_desc(p.descs + b);
    bool ok = d.in_bytes >= kHeaderBytes;
    bool sampled = false;  // flag bit 0: tables from samples (record mode 2)
    DecInfo inf = {};
    if (ok) {
        const uint4 h0 = gload<uint4>(d.in), h1 = gload<uint4>(d.in + 16);
        const uint4 h2 = gload<uint4>(d.in + 32), h3 = gload<uint4>(d.in + 48);
        const uint32_t r = raw_bits(p.dtype);
        // V1 magic, version, fixed coder parameters, flags (bit 0 the only
        // one defined); V2 dtype and count
        const uint32_t flags = h0.z >> 16;
        ok = h0.x == kMagic && (h0.y & 0xFFFFu) == kVersion && ((h0.y >> 16) & 0xFFu) == (uint32_t)p.dtype &&
             (h0.y >> 24) == kProbBits && (h0.z & 0xFFu) == kLanes && ((h0.z >> 8) & 0xFFu) == r && flags <= 1;
        sampled = flags == 1;
        const uint64_t n = uint64_t(h1.x) | (uint64_t(h1.y) << 32);
        const uint64_t C = uint64_t(h1.z) | (uint64_t(h1.w) << 32);
        const uint64_t ce = h0.w;
        ok = ok && n == d.n;
        // V3 chunk size and count; V4 region offsets and total size
        ok = ok && ce >= 32 && ce % 32 == 0 && ce <= kMaxChunkElems;
        if (ok) {
            const Layout l = layout_of(p.dtype, n, ce);
            const uint64_t sm_off = uint64_t(h2.x) | (uint64_t(h2.y) << 32);
            const uint64_t exp_off = uint64_t(h2.z) | (uint64_t(h2.w) << 32);
            const uint64_t total = uint64_t(h3.x) | (uint64_t(h3.y) << 32);
            ok = C == l.chunks && sm_off == l.sm_off && exp_off == l.exp_off && total <= d.in_bytes &&
                 total >= exp_off;
            if (ok) {
                // V5 ends of the index
                const uint64_t first = gload<uint64_t>(d.in + kHeaderBytes);
                const uint64_t last = gload<uint64_t>(d.in + kHeaderBytes + 8 * C);
                ok = first == 0 && last == total - exp_off;
            }
            inf.chunks = ok ? C : 0;
            inf.chunk_elems = ce;
            inf.sm_off = sm_off;
            inf.exp_off = exp_off;
            inf.total = total;
            inf.flags = flags;
        }
    }
    if (!ok) inf.chunks = 0;
    const uint4 *iv = reinterpret_cast<const uint4 *>(&inf);
    for (int k = 0; k < 4; ++k) gstore<uint4>(reinterpret_cast<uint4 *>(p.info + b) + k, iv[k]);
    gstore<uint32_t>(p.status + b, ok ? 0u : 3u);
    const uint64_t pairs = (inf.chunks + 1) / 2;
    if (p.nbuf == 1) {
        gstore<uint64_t>(p.pair_first, 0);
        gstore<uint64_t>(p.pair_first + 1, pairs);
        gstore<uint32_t>(p.kinds, ok ? (sampled ? 2u : 1u) : 0u);
    } else {
        gstore<uint64_t>(p.pair_first + b, pairs);  // counts; scanned in place afterwards
    }
}

// LDS of one decode workgroup (two chunks), 10 KiB:
//   s_sym [2][4096] u8   slot -> rank of its symbol among the present symbols
//   s_rk  [2][256]  u32  rank -> (4096 - f) | c0 << 12 | symbol << 24
// so one step costs two dependent LDS reads; fp32 adds s_slot [2][4096] u32
// (slot -> its rank's entry, 34 KiB in all) and reads once per step.  The
// symbol sits in the entry's top byte, so that byte permutes can gather the
// symbols of several steps.  A workgroup decodes a pair of consecutive chunks
// of one buffer (half-wave h decodes chunk 2p + h), so the record,
// sign+mantissa and output regions of the pair each get one buffer resource.
// Renormalisation words come from a register window (two 16-bit words per
// lane: 64 words per half-wave) refilled from loads issued four steps ahead,
// off the state's dependency chain, and are fetched with ds_bpermute after the
// ballot.  Chunks stored RAW are rebuilt in a separate loop.
template <int DT>
__device__ inline uint32_t bload_sm(rsrc_t r, uint32_t off) {
    if (Fmt<DT>::R == 0) return 0u;
    if (Fmt<DT>::R == 1) return bld8(r, off);
    return bld8(r, off) | (bld8(r, off + 1) << 8) | (bld8(r, off + 2) << 16);
}

// fp16 and fp8: the raw field of the value whose bits start at bit position
// bit of the raw region behind r (one unaligned dword: the field's 11, 4 or 3
// bits start at most 7 bits into it)
template <int DT>
__device__ inline uint32_t raw_field(rsrc_t r, uint32_t bit) {
    return (bld32(r, bit >> 3) >> (bit & 7u)) & ((1u << Fmt<DT>::RB) - 1u);
}

// 16 values rebuilt from 16 symbol bytes E and their 16 R raw bytes S, stored
// as 16 EB bytes at `off` of r (an out-of-range offset drops the stores)
template <int DT>
__device__ inline void store_unit(rsrc_t r, uint32_t off, const uint4 &E, const uint4 *S) {
    const uint32_t e[4] = {E.x, E.y, E.z, E.w};
    if (DT == 4) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{E.x, E.y, E.z, E.w}, r, (int)off, 0, 0);
    } else if (DT == 1 || DT == 3) {
        const uint32_t sv[4] = {S[0].x, S[0].y, S[0].z, S[0].w};
        uint32_t o[8];
#pragma unroll
        for (uint32_t d = 0; d < 4; ++d) {
            // low and high byte of four values at once, then interleaved
            uint32_t lo = sv[d], hi = e[d];
            if (DT == 1) {
                lo = (sv[d] & 0x7F7F7F7Fu) | ((e[d] & 0x01010101u) << 7);
                hi = (sv[d] & 0x80808080u) | ((e[d] >> 1) & 0x7F7F7F7Fu);
            }
            o[2 * d] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            o[2 * d + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, r, (int)off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[4], o[5], o[6], o[7]}, r, (int)(off + 16), 0, 0);
    } else {
        const uint32_t w[12] = {S[0].x, S[0].y, S[0].z, S[0].w, S[1].x, S[1].y,
                                S[1].z, S[1].w, S[2].x, S[2].y, S[2].z, S[2].w};
        uint32_t o[16];
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            // raw field k: bytes 3k .. 3k + 2 of w
            const uint32_t b = 3 * k, d = b >> 2;
            const uint32_t sm = __builtin_amdgcn_alignbyte(w[d + 1 < 12 ? d + 1 : 11], w[d], b & 3) & 0xFFFFFFu;
            o[k] = join_value<2>((e[k >> 2] >> (8 * (k & 3))) & 0xFFu, sm);
        }
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]}, r,
                                                   (int)(off + 16 * q), 0, 0);
    }
}

// S: the variant for frames with sampled tables (record mode 2).  Both are
// launched for every call; each leaves at once unless a valid buffer of its
// kind is present, and skips the buffers of the other kind.
template <int DT, bool S>
__global__ __launch_bounds__(64) void k_decode(DecodeParams p) {
    constexpr uint32_t EB = Fmt<DT>::EB;
    constexpr uint32_t R = Fmt<DT>::R;
    // bf16: 2-byte values with one raw byte (raw bytes by dword and
    // bpermute, two steps per store in the main loop below)
    constexpr bool kB16 = DT == 1;
    constexpr uint32_t RB = Fmt<DT>::RB, SB = Fmt<DT>::SB;
    // refills found stale by the scalar refill masks and reloaded in a rare
    // branch (bf16, fp16, fp8); fp32 also loads the pair 64 words further
    constexpr bool kScalarStale = DT != 2;
    // one LDS array, so that the slot table sits at address 0 and a slot's
    // address is a single and-or of the state
    // fp32 (about one wave per SIMD, so each step's latency is exposed) looks
    // up its entry in one read of a direct slot table, kTableSize u32 per
    // chunk (32 KiB per workgroup); the others read the slot's rank byte,
    // then the rank's entry (10 KiB per workgroup, more waves per CU)
    constexpr bool kDirect = DT == 2;
    constexpr uint32_t kSlotWords = kDirect ? 2 * kTableSize : 2 * kTableSize / 4;
    __shared__ __align__(16) uint32_t s_dec[kSlotWords + 2 * 256];
    uint8_t(*s_sym)[kTableSize] = reinterpret_cast<uint8_t(*)[kTableSize]>(s_dec);
    uint32_t(*s_slot)[kTableSize] = reinterpret_cast<uint32_t(*)[kTableSize]>(s_dec);
    uint32_t(*s_rk)[256] = reinterpret_cast<uint32_t(*)[256]>(s_dec + kSlotWords);

    const uint32_t lane = threadIdx.x;
    const uint32_t h = lane >> 5, lj = lane & 31;
    if ((uniform_u32(gload<uint32_t>(p.kinds)) & (S ? 2u : 1u)) == 0) return;
    const uint64_t PT = uniform_u64(gload<uint64_t>(p.pair_first + p.nbuf));

    for (uint64_t q = blockIdx.x; q < PT; q += gridDim.x) {
        // ---- the pair: buffer, chunks, index entries (wave-uniform) ----
        const uint32_t b = p.nbuf == 1 ? 0u : uniform_u32(find_dec_buffer(p.pair_first, p.nbuf, q));
        const DecDesc d = p.nbuf == 1 ? p.single : load_dec_desc(p.descs + b);
        if (uniform_u32(gload<uint32_t>(p.status + b)) != 0) continue;
        if (((uniform_u32((uint32_t)gload<uint64_t>(&p.info[b].flags)) & 1u) != 0) != S) continue;
        const uint64_t ce = uniform_u64(gload<uint64_t>(&p.info[b].chunk_elems));
        const uint64_t C = uniform_u64(gload<uint64_t>(&p.info[b].chunks));
        const uint64_t sm_off = uniform_u64(gload<uint64_t>(&p.info[b].sm_off));
        const uint64_t exp_off = uniform_u64(gload<uint64_t>(&p.info[b].exp_off));
        const uint64_t total = uniform_u64(gload<uint64_t>(&p.info[b].total));
        const uint64_t n = uniform_u64(d.n);
        const uint64_t c0 = 2 * (q - uniform_u64(gload<uint64_t>(p.pair_first + b)));
        const uint32_t nch = C - c0 >= 2 ? 2u : 1u;
        const uint32_t vals0 = (uint32_t)min<uint64_t>(ce, n - c0 * ce);
        const uint32_t vals1 = nch == 2 ? (uint32_t)min<uint64_t>(ce, n - (c0 + 1) * ce) : 0u;
        const uint8_t *ix = d.in + kHeaderBytes + 8 * c0;
        const uint64_t a0 = uniform_u64(gload<uint64_t>(ix));
        const uint64_t a1 = uniform_u64(gload<uint64_t>(ix + 8));
        const uint64_t a2 = nch == 2 ? uniform_u64(gload<uint64_t>(ix + 16)) : a1;
        const uint64_t rawmax = raw_record_bytes(ce, SB);
        // V5 for the pair's index entries: aligned, ordered, inside the records,
        // and no record longer than a full chunk's RAW record (a coarse bound
        // that keeps the 32-bit resource sizes below valid; each record is then
        // held to its own chunk's RAW size below)
        const bool pair_ok = ((a0 | a1 | a2) & 15u) == 0 && a0 <= a1 && a1 <= a2 && a2 <= total - exp_off &&
                             a1 - a0 <= rawmax && a2 - a1 <= rawmax;
        if (!pair_ok) {
            if (lane == 0) gstore<uint32_t>(p.status + b, 3u);
            continue;
        }
        const rsrc_t rrec = make_rsrc(d.in + exp_off + a0, (uint32_t)(a2 - a0));

        // ---- this half's record (V6) ----
        bool ok = h < nch;
        const uint32_t ni = h ? vals1 : vals0;
        const uint32_t rel = h ? (uint32_t)(a1 - a0) : 0u;  // record start inside rrec
        const uint32_t len = h ? (uint32_t)(a2 - a1) : (uint32_t)(a1 - a0);
        uint32_t mode = 1, nsym = 0, nw = 0, nesc = 0;
        // coded records: mode 0 in frames with full tables, mode 2 with sampled ones
        constexpr uint32_t kCoded = S ? 2u : 0u;
        ok = ok && len >= 16;
        {
            const uint4 rh = bld128(rrec, ok ? rel : kOutOfRange);
            mode = rh.x & 0xFFu;
            nsym = rh.x >> 16;
            nw = rh.y;
            ok = ok && (mode == 1 || mode == kCoded) && rh.z == ni && rh.w == len;
            if (ok && mode == 1) ok = nsym == 0 && nw == 0 && len == raw_record_bytes(ni, SB);
            // a coded record is strictly smaller than the chunk's RAW record
            // (it would have been stored RAW otherwise); a longer one is corrupt
            if (ok && mode == kCoded) ok = nsym >= 1 && nsym <= 256 && len < raw_record_bytes(ni, SB);
            if (S && ok && mode == kCoded) {
                ok = len >= words_offset_sampled(nsym);
                nesc = bld32(rrec, ok ? rel + (uint32_t)esc_count_offset(nsym) : kOutOfRange);
                ok = ok && nesc <= ni && len == align16(words_offset_sampled(nsym) + 2ull * nw + nesc);
            } else if (ok && mode == kCoded) {
                ok = len == align16(words_offset(nsym) + 2ull * nw);
            }
        }
        const bool coded = ok && mode == kCoded;

        // ---- table: presence bitmap byte lj covers symbols 8lj..8lj+7 (V7) ----
        const uint32_t pb = bld8(rrec, coded ? rel + kRecHeaderBytes + lj : kOutOfRange);
        const uint32_t np = __popc(pb);
        const uint32_t pre = half_excl_scan(np, lj);
        uint32_t fk[8], lsum = 0, cpre[8];
        // (a table names only symbols below 2^SB, the exponent field's range)
        bool fok = SB == 8 || 8 * lj < (1u << SB) || pb == 0;
        {
            uint32_t k2 = pre;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                fk[k] = 0;
                if ((pb >> k) & 1u) {
                    fk[k] = bld16(rrec, k2 < nsym ? rel + 48 + 2 * k2 : kOutOfRange);
                    if (fk[k] == 0 || fk[k] > kTableSize) fok = false;
                    ++k2;
                }
                cpre[k] = lsum;
                lsum += fk[k];
            }
        }
        const uint32_t tot = half_sum(lsum);
        const uint32_t cbase = half_excl_scan(lsum, lj);
        const uint32_t seen = half_sum(np);
        const bool fbad = half_mask(__ballot(!fok), h) != 0;
        // (a sampled table leaves its last slot to the escape symbol)
        if (coded) ok = seen == nsym && !fbad && tot == kTableSize - (S ? 1u : 0u);
        const bool coded_ok = ok && mode == kCoded;
        if (coded_ok) {
            uint32_t k2 = pre;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (fk[k]) s_rk[h][k2++] = (kTableSize - fk[k]) | ((cbase + cpre[k]) << 12) | ((lj * 8 + k) << 24);
            }
        }
        // the escape symbol: rank nsym, f = 1, slot 4095 (no owner when all 256
        // symbols are sampled: a stream reaching it is corrupt, found below)
        if (S && coded_ok && lj == 0 && nsym < 256) s_rk[h][nsym] = (kTableSize - 1u) | (kEscSlot << 12);
        __syncthreads();
        if (coded_ok) {
            for (uint32_t m = 0; m < nsym + (S && nsym < 256 ? 1u : 0u); ++m) {
                const uint32_t em = s_rk[h][m];
                const uint32_t fs = kTableSize - (em & 0xFFFu), c0s = (em >> 12) & 0xFFFu;
                if (kDirect) {
                    for (uint32_t k = lj; k < fs; k += 32) s_slot[h][c0s + k] = em;
                } else {
                    for (uint32_t k = lj; k < fs; k += 32) s_sym[h][c0s + k] = (uint8_t)m;
                }
            }
        }
        __syncthreads();

        // ---- states (V8) ----
        uint32_t x = bld32(rrec, coded_ok ? rel + (uint32_t)(S ? states_offset_sampled(nsym) : states_offset(nsym)) + 4 * lj
                                          : kOutOfRange);
        if (!coded_ok) x = kStateLow;
        const bool sbad = half_mask(__ballot(coded_ok && x < kStateLow), h) != 0;
        ok = ok && !sbad;
        const bool rans_run = ok && mode == kCoded;
        const bool raw_run = ok && mode == 1;

        // ---- rANS decode (V9: end state L on every lane, every word consumed) ----
        // Word window of a half: words [base, base + 64), two blocks of 32
        // words, each held by 16 lanes of the half as adjacent word pairs (lane
        // i of a group: words 2i and 2i + 1 of its block, one dword in P); base
        // is a multiple of 32.  Word k of the stream lives in lane (k >> 1) mod
        // 32 of the half, half-word k & 1.  The bookkeeping is per lane, in
        // vector registers: offv = words consumed by the lane's half, lim = the
        // count at which the lane's block is used up (the end of its block);
        // the lane then takes the pair 64 words further, loaded ahead into NX.
        // Loads past the pair's records read zero, and words past n_words are
        // never consumed by a valid stream (a stream that tries fails the end
        // check offv == n_words).
        const uint32_t pair_vals = vals0 + vals1;
        // (fp16, fp8: the pair's packed raw fields, and the 3 bytes after them
        // that a field's dword load may touch, inside the readable buffer)
        const uint64_t rsm_at = sm_off + c0 * ce * RB / 8;
        const rsrc_t rsm = make_rsrc(d.in + rsm_at, R > 0 ? pair_vals * R
                                                          : (uint32_t)min<uint64_t>(packed_bytes(pair_vals, RB) + 3,
                                                                                    d.in_bytes - rsm_at));
        const uint32_t lanebit = ((h ? vals0 : 0u) + lj) * RB;  // fp16, fp8: bit of the lane's step-0 raw field
        const rsrc_t rout = make_rsrc(d.out + c0 * ce * EB, pair_vals * EB);
        const uint32_t sm_lane = (h ? vals0 : 0u) * R + lj * R;
        const uint32_t out_lane = rans_run ? (h ? vals0 : 0u) * EB + lj * EB : kOutOfRange;
        // wave-uniform view of the two halves
        const uint64_t runm = __builtin_amdgcn_ballot_w64(rans_run);
        const bool run0 = (uint32_t)runm != 0, run1 = (runm >> 32) != 0;
        const uint32_t ni0 = uniform_u32(__shfl((int)ni, 0, 64)), ni1 = uniform_u32(__shfl((int)ni, 32, 64));
        const uint32_t T0 = run0 ? (ni0 + 31) / 32 : 0u, T1 = run1 ? (ni1 + 31) / 32 : 0u;
        const uint32_t Tw = max(T0, T1);
        // steps in which every lane of each running half holds a value
        const uint32_t F0 = run0 ? ni0 / 32 : 0xFFFFFFFFu, F1 = run1 ? ni1 / 32 : 0xFFFFFFFFu;
        // (sampled tables: a half with more escapes than its registers hold
        // is decoded by the tail loop alone, whose escape path may load)
        const uint32_t nesc_w = S ? max(uniform_u32(__shfl((int)nesc, 0, 64)), uniform_u32(__shfl((int)nesc, 32, 64))) : 0u;
        const uint32_t Tmain = S && nesc_w > 256 ? 0u : min(min(F0, F1), Tw) & ~7u;
        const uint32_t Tmain16 = Tmain & ~15u;  // bf16 main loop: 16 steps per iteration
        // The main loop takes four steps at a time, and lane j the raw fields of
        // positions 4j .. 4j + 3 of a group (4 R bytes, or 4 RB bits starting at
        // bit gsh of byte gbyte; see the main loop); groups 0 and 1 are loaded
        // here, before the word window, so that many memory operations lie
        // between these loads and their first use
        using SmGroup = std::conditional_t<DT == 2, u32x3, std::conditional_t<DT == 3, u32x2, uint32_t>>;
        const uint32_t smg = ((h ? vals0 : 0u) + 4 * lj) * R;  // the lane's bytes of group 0
        const uint32_t gbit = ((h ? vals0 : 0u) + 4 * lj) * RB, gbyte = gbit >> 3, gsh = gbit & 7u;
        auto load_group = [&](uint32_t g) __attribute__((always_inline)) {
            if constexpr (DT == 2) {
                return __builtin_amdgcn_raw_buffer_load_b96(rsm, (int)(smg + 128 * R * g), 0, 0);
            } else if constexpr (DT == 1) {
                return bld32(rsm, smg + 128 * R * g);
            } else if constexpr (DT == 3) {
                // 44 bits from bit gsh (0 or 4) of an unaligned byte: two dwords
                return u32x2{bld32(rsm, gbyte + 16 * RB * g), bld32(rsm, gbyte + 16 * RB * g + 4)};
            } else {
                return bld32(rsm, gbyte + 16 * RB * g);  // (a group's fields: 128 RB bits)
            }
        };
        const SmGroup G0first = load_group(0), G1first = load_group(1);
        // Refill: at every step, after its own refill decision, each lane loads
        // the pair it takes at its next refill (block end lim, 32 words past
        // it, pair position 2i) into NX[t mod 4]; the load is consumed four
        // steps later.  Waiting for a load also waits for every older store
        // (one counter covers both), so the distance keeps the output stores
        // off the critical path.  A lane refills at most once every two steps
        // (a refill takes 64 words, a step at most 32); one that refills again
        // two or three steps after its last refill (more than 16 words per
        // step: near-uniform exponents only) finds in NX a pair loaded before
        // that refill.  bf16, fp16 and fp8 detect this from the refill masks
        // of the last three steps (scalar) and then reload synchronously;
        // fp32, whose waves are too few to hide a branch, also loads the pair
        // 64 words further (NB), which is the right one exactly in that case.
        const uint32_t wstart = rel + (uint32_t)(S ? words_offset_sampled(nsym) : words_offset(nsym));  // byte offset of word 0
        uint32_t P = bld32(rrec, wstart + 4 * lj);                    // words 2lj, 2lj + 1
        uint32_t lim = 32 + 32 * (lj >> 4);                           // end of the lane's block
        const uint32_t rbase = wstart + 64 + 4 * (lj & 15u);          // byte offset of its next pair = 2 lim + rbase
        uint32_t NX[4], NB[4];
        NX[0] = NX[1] = NX[2] = NX[3] = bld32(rrec, 2 * lim + rbase); // words 64 + 2lj, 65 + 2lj
        NB[0] = NB[1] = NB[2] = NB[3] = kScalarStale ? 0u : bld32(rrec, 2 * lim + rbase + 128);
        uint64_t R1 = 0, R2 = 0, R3 = 0;  // refill masks of the last three steps (kScalarStale)
        uint32_t age = 4;                  // fp32: steps since the lane's last refill
        const uint32_t lanebits = (h << 5) << 2;
        const uint32_t hsym = h << kProbBits, hrk = h << 8;  // this half's table rows
        const uint32_t selbase = 0x05040100u, selkeep = 0x07060504u;
        uint32_t offv = 0;  // words consumed by this half
        // the current state's slot index and its first table read (the direct
        // entry, or the rank), carried from step to step
        uint32_t slot_c, first_c;
        const uint32_t lstate = rans_run ? kStateLow : 0u;  // main-loop renormalisation bound (0: no words)
        const uint8_t *s_symf = &s_sym[0][0];
        const uint32_t *s_rkf = &s_rk[0][0];
        const uint32_t *s_slotf = &s_slot[0][0];
        // Escapes (sampled tables): the value whose slot is 4095 takes its
        // exponent from the record's escape list, in value order; a half's
        // first 256 escaped bytes are held four to a lane in two registers
        // (fetched by bpermute), later ones are loaded.  The byte must not be
        // a sampled symbol, and the list must be used exactly.
        const uint32_t escat = rel + (uint32_t)words_offset_sampled(nsym) + 2 * nw;  // byte offset of the list
        uint32_t escw = 0, escw1 = 0;  // list bytes [4j, 4j + 4) and [128 + 4j, 132 + 4j) of lane j of the half
        if (S) {
            const uint32_t ea = (escat & ~3u) + 4 * lj;
            escw = __builtin_amdgcn_alignbyte(bld32(rrec, rans_run ? ea + 4 : kOutOfRange),
                                              bld32(rrec, rans_run ? ea : kOutOfRange), escat & 3u);
            escw1 = __builtin_amdgcn_alignbyte(bld32(rrec, rans_run ? ea + 132 : kOutOfRange),
                                               bld32(rrec, rans_run ? ea + 128 : kOutOfRange), escat & 3u);
        }
        const uint32_t escaddr = kEscSlot | hsym;
        uint32_t escv = 0;  // escapes used by this half
        bool escbad = false;
        if (S) {
            // the held list bytes are checked here, once: none may be a sampled
            // symbol (lane e >> 3 of the half holds the bitmap byte of e's group)
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                const uint32_t e = ((k < 4 ? escw : escw1) >> (8 * (k & 3u))) & 0xFFu;
                const uint32_t idx = (k < 4 ? 0u : 128u) + 4 * lj + (k & 3u);
                const uint32_t pbe = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((e >> 3) | (h << 5)) << 2), (int)pb);
                escbad = escbad || (rans_run && idx < nesc && ((pbe >> (e & 7u)) & 1u));
            }
        }
        // (called once a step's table entry em is read; returns it with the
        // escaped exponent in place of the symbol, in the top byte, for the
        // escaping lanes)
        auto escape_sym = [&](uint64_t escm, uint32_t em, bool tail) __attribute__((always_inline)) {
            const uint32_t elo = __builtin_popcount((uint32_t)escm), ehi = __builtin_popcount((uint32_t)(escm >> 32));
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(escm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)escm, 0u));
            const uint32_t idx = escv + below - (h ? elo : 0u);
            const bool mine = (escm >> lane) & 1u;
            const int src = (int)((((idx >> 2) & 31u) | (h << 5)) << 2);
            const uint32_t ew0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)escw);
            const uint32_t ew1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)escw1);
            uint32_t e = ((idx >= 128 ? ew1 : ew0) >> (8 * (idx & 3u))) & 0xFFu;
            bool bad = idx >= nesc || nsym == 256 || (SB < 8 && e >= (1u << SB));
            if (tail && idx >= 256) {
                // past the held bytes: load it, and check here that it is no sampled
                // symbol (the bitmap byte of e's group is held by lane e >> 3 of the half)
                e = bld8(rrec, mine && idx < nesc ? escat + idx : kOutOfRange);
                const uint32_t pbe = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((e >> 3) | (h << 5)) << 2), (int)pb);
                bad = bad || ((pbe >> (e & 7u)) & 1u) || (SB < 8 && e >= (1u << SB));
            }
            escbad = escbad || (mine && bad);
            escv += h ? ehi : elo;
            return mine ? (em & 0x00FFFFFFu) | (e << 24) : em;
        };
        // One step of both half-waves.  act = lanes holding a value this step
        // (TAIL steps only: in the main loop every lane of a running half
        // holds one, and lanes of a half that is not running never reach the
        // output or the checks); par = step mod 4 (selects the refill
        // register).  With the table entry em = g | c0 << 12 | sym << 24,
        // g = 4096 - f, the decode step f * (x >> 12) + (x & 4095) - c0 is
        // x - (g * (x >> 12) + c0).
        // sp: the value's sign+mantissa, for bf16 as the byte in bytes 0 and 1.
        // Returns the entry (escapes in place) and stores nothing unless
        // `store` (the main loop builds and stores four steps' values at once).
        auto step = [&](uint32_t t, uint64_t act, bool tail, uint32_t sp, int par, bool store) __attribute__((always_inline)) {
            // (x & 4095) | this half's row, and its first table read (the direct
            // entry, or the rank), both issued at the end of the step before
            const uint32_t slot_addr = slot_c;
            // (sampled tables: the lanes at the escape slot; their exponent is
            // patched into the entry in a rare branch)
            const uint64_t escm = S ? lanes_eq(slot_addr, escaddr) & act : 0ull;
            const uint32_t em = kDirect ? first_c : s_rkf[first_c | hrk];
            const uint32_t xd = x - (__umul24(em & 0xFFFu, x >> kProbBits) + ((em >> 12) & 0xFFFu));
            // The lanes that take a word.  In the main loop every lane of a
            // running half is active, and a half that is not running compares
            // against 0 (lstate) and takes none, so the compare's own mask serves,
            // with no scalar instruction on the state's dependent path; only
            // compiler-placed instructions read it there, since the hardware
            // needs spacing between a vector compare writing scalar registers and
            // a vector read of them, which the compiler cannot see through inline
            // asm.  Tail steps mask it with act on the scalar unit, and the asm
            // selects below may read that copy.
            const bool need = xd < lstate;
            const uint64_t m = tail ? lanes_lt(xd, kStateLow) & act : __builtin_amdgcn_ballot_w64(need);
            const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
            // the lane's word: stream position offv + rank inside the half (one mbcnt per half)
            const uint32_t kk = vsel(kHighHalf, __builtin_amdgcn_mbcnt_lo(lo, offv), __builtin_amdgcn_mbcnt_hi(hi, offv));
            // lane (kk >> 1) mod 32 of this half
            const uint32_t wv = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((kk << 1) & 124u) | lanebits), (int)P);
            __builtin_amdgcn_sched_barrier(0);  // (the permute issues before the bookkeeping below)
            // bookkeeping in vector registers, split around the state's update so
            // that the next step's table read follows that update at once: here,
            // in the permute's shadow, the half's consumed count; after the read,
            // the lanes whose block is used up take the pairs loaded four steps
            // ago (the permute above has read P)
            offv = vsel(kHighHalf, offv + __builtin_popcount(lo), offv + __builtin_popcount(hi));
            // (plain selects: the mask comes from a vector compare, and the
            // compiler spaces its reads as the hardware requires)
            const bool used_up = offv >= lim;
            // x' = (xd << 16) | word: bytes 0-1 (kk even) or 2-3 of wv below bytes
            // 0-1 of xd; lanes without a word keep xd (bytes 4-7)
            uint32_t selw;
            asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(selw) : "v"(kk & 1u), "s"(0x0202u), "v"(selbase));
            const uint32_t sel = tail ? vsel(m, selkeep, selw) : (need ? selw : selkeep);
            // The state's update, the next slot and its first table read issue
            // back to back: the scheduling barriers keep everything above (the
            // consumed count and the word select, in the permute's shadow) before
            // them and everything below (the refill, the step's value, the
            // group's packing) after them, in the read's shadow.  With one or two
            // waves per SIMD (fp32, fp8) nothing else fills those shadows.
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t xn = __builtin_amdgcn_perm(xd, wv, sel);
            x = tail ? vsel(act, x, xn) : xn;
            asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(slot_c) : "v"(x), "s"(kTableSize - 1), "v"(hsym));
            first_c = kDirect ? s_slotf[slot_c] : (uint32_t)s_symf[slot_c];
            __builtin_amdgcn_sched_barrier(0);
            // the refill, in the read's shadow (the next step's permute reads P)
            if (kScalarStale) {
                const uint64_t um = __builtin_amdgcn_ballot_w64(used_up);
                const uint64_t stale = um & (R2 | R3);
                R3 = R2;
                R2 = R1;
                R1 = um;
                if (stale) {
                    // (the asm copy makes the wait for the fresh pair happen
                    // inside the branch, so no load is pending where the paths meet)
                    uint32_t fresh;
                    asm volatile("v_mov_b32 %0, %1" : "=v"(fresh) : "v"(bld32(rrec, 2 * lim + rbase)));
                    P = used_up ? fresh : P;
                } else {
                    P = used_up ? NX[par] : P;
                }
            } else {
                P = used_up ? (age < 4u ? NB[par] : NX[par]) : P;
                age = used_up ? 1u : age + 1u;
            }
            lim += used_up ? 64u : 0u;
            NX[par] = bld32(rrec, 2 * lim + rbase);
            if (!kScalarStale) NB[par] = bld32(rrec, 2 * lim + rbase + 128);
            const uint32_t emx = S && __builtin_expect(escm != 0, 0) ? escape_sym(escm, em, tail) : em;
            if (DT == 1) {
                // sign (bit 7 of sm, copied to bit 15) and mantissa bits 0-6
                // from sp, exponent (emx bits 24-31) to bits 7-14; the store
                // keeps the low 16 bits
                if (store) {
                    uint32_t v;
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v) : "s"(0x807Fu), "v"(sp), "v"(emx >> 17));
                    bst16(rout, out_lane + t * 32 * EB, v);
                }
                return emx;
            } else if constexpr (DT != 2) {
                // fp16, fp8: sign (the raw field's top bit, copied to the value's
                // top bit) and mantissa from sp, the exponent (emx bits 24-31) to
                // bit SYM; the store keeps the value's EB bytes
                constexpr uint32_t SYM = Fmt<DT>::SYM, top = 8 * EB - 1;
                constexpr uint32_t keep = (1u << top) | ((1u << (RB - 1)) - 1u);
                if (store) {
                    const uint32_t spx = sp | ((sp >> (RB - 1)) << top);
                    uint32_t v;
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v) : "s"(keep), "v"(spx), "v"(emx >> (24 - SYM)));
                    bst_value<DT>(rout, out_lane + t * 32 * EB, v);
                }
                return emx;
            } else if (DT == 2) {
                // sign (bit 23 of sm) to bit 31, mantissa bits 0-22, exponent to bits 23-30
                if (store) {
                    const uint32_t sx = sp | ((sp & 0x800000u) << 8), ex = emx >> 1;
                    bst32(rout, out_lane + t * 32 * EB, (sx & 0x807FFFFFu) | (ex & ~0x807FFFFFu));
                }
                return emx;
            }
            return 0u;
        };
        asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(slot_c) : "v"(x), "s"(kTableSize - 1), "v"(hsym));
        first_c = kDirect ? s_slotf[slot_c] : (uint32_t)s_symf[slot_c];
        uint32_t t = 0;
        {
            // Four steps at a time.  A group of four steps holds 128 values of
            // each half; lane j takes positions 4j .. 4j + 3 of them, that is
            // step j >> 3 of lanes 4 (j & 7) .. 4 (j & 7) + 3: their raw fields
            // (one 32-bit load for bf16 and fp8, 96 bits for fp32, two unaligned
            // dwords for fp16; two groups ahead) and their one store of 4 EB
            // bytes.
            // Their exponents reach it in three moves: each lane packs its four
            // steps' symbols into the bytes of one dword (entry byte 3 of each
            // step, by v_perm); each quad of lanes transposes its 4 x 4 bytes
            // (three DPP quad permutes and three v_perm), after which lane
            // 4m + q holds the symbols of step q for lanes 4m .. 4m + 3; and one
            // ds_bpermute fetches that dword from lane 4 (j & 7) + (j >> 3).
            const uint32_t q4 = lj & 3u;
            // transposition: from the own dword (A) and those of lanes q ^ 1 (B),
            // q ^ 2 (C), q ^ 3 (D), lane q takes byte q of A, B, C, D in the
            // order of their lanes; selT picks the two bytes of a pair (A, B) or
            // (C, D), selW places the pairs
            const uint32_t selT = q4 == 0 ? 0x0C0C0400u : q4 == 1 ? 0x0C0C0105u : q4 == 2 ? 0x0C0C0602u : 0x0C0C0307u;
            const uint32_t selW = q4 < 2 ? 0x05040100u : 0x01000504u;
            const int xsrc = (int)(((4 * (lj & 7u) + (lj >> 3)) | (h << 5)) << 2);
            const uint32_t outg = rans_run ? ((h ? vals0 : 0u) + 4 * lj) * EB : kOutOfRange;
            auto group4 = [&](uint32_t t0, SmGroup S4) __attribute__((always_inline)) {
                uint32_t e[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) e[u] = step(t0 + u, runm, false, 0u, u, false);
                const uint32_t E = __builtin_amdgcn_perm(__builtin_amdgcn_perm(e[3], e[2], 0x0C0C0703u),
                                                         __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0703u), 0x05040100u);
                const uint32_t B = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)E, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
                const uint32_t C = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)E, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
                const uint32_t D = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)E, 0x1B, 0xF, 0xF, true);  // quad_perm [3,2,1,0]
                const uint32_t T = __builtin_amdgcn_perm(__builtin_amdgcn_perm(D, C, selT), __builtin_amdgcn_perm(B, E, selT), selW);
                const uint32_t X = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)T);
                if constexpr (DT == 1) {
                    // bytewise: low bytes (the exponent's bit 0 under the mantissa),
                    // high bytes (the sign over the exponent's bits 1-7), interleaved
                    uint32_t lo, hi;
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(lo) : "s"(0x7F7F7F7Fu), "v"(S4), "v"(X << 7));
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(hi) : "s"(0x80808080u), "v"(S4), "v"(X >> 1));
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)},
                        rout, (int)(outg + t0 * 32 * EB), 0, 0);
                } else if constexpr (DT == 2) {
                    // value k's raw field is bytes 3k .. 3k + 2 of the 12; one v_perm
                    // takes them with the top one twice (the sign lands in bit 31),
                    // and one v_bfi puts exponent byte k into bits 23-30
                    uint32_t v0, v1, v2, v3;
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v0) : "s"(0x807FFFFFu), "v"(__builtin_amdgcn_perm(S4.y, S4.x, 0x02020100u)), "v"(X << 23));
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v1) : "s"(0x807FFFFFu), "v"(__builtin_amdgcn_perm(S4.y, S4.x, 0x05050403u)), "v"(X << 15));
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v2) : "s"(0x807FFFFFu), "v"(__builtin_amdgcn_perm(S4.z, S4.y, 0x04040302u)), "v"(X << 7));
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v3) : "s"(0x807FFFFFu), "v"(__builtin_amdgcn_perm(S4.z, S4.z, 0x03030201u)), "v"(X >> 1));
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v0, v1, v2, v3}, rout, (int)(outg + t0 * 32 * EB), 0, 0);
                } else if constexpr (DT == 3) {
                    // fp16: two fields a dword (f0 in bits 0-10, f1 in 16-26), then
                    // the mantissas kept, the exponent bytes of X moved to bits 10-14
                    // and 26-30, and the fields' top bits (the signs) to bits 15, 31
                    const uint32_t a01 = __builtin_amdgcn_alignbit(S4.y, S4.x, gsh);
                    const uint32_t a23 = __builtin_amdgcn_alignbit(S4.y, S4.x, gsh + 22);
                    uint32_t w[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uint32_t a = k ? a23 : a01;
                        uint32_t F, P, Wk;
                        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(F) : "s"(0x7FFu), "v"(a), "v"(a << 5));
                        const uint32_t E = __builtin_amdgcn_perm(0u, X, k ? 0x030C020Cu : 0x010C000Cu) << 2;
                        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(P) : "s"(0x03FF03FFu), "v"(F), "v"(E));
                        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(Wk) : "s"(0x80008000u), "v"(F << 5), "v"(P));
                        w[k] = Wk;
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rout, (int)(outg + t0 * 32 * EB), 0, 0);
                } else {
                    // fp8: the four RB-bit fields spread to bytes, then per byte the
                    // mantissa from the field, the exponent at bit SYM and the
                    // field's top bit (the sign) to bit 7; one 32-bit store
                    constexpr uint32_t SYM = Fmt<DT>::SYM;
                    constexpr uint32_t mant4 = ((1u << (RB - 1)) - 1u) * 0x01010101u;
                    const uint32_t F = S4 >> gsh;
                    uint32_t Bf;
                    if constexpr (RB == 4) {
                        Bf = __builtin_amdgcn_perm((F >> 4) & 0x0F0Fu, F & 0x0F0Fu, 0x05010400u);
                    } else {
                        Bf = (F & 7u) | (((F >> 3) & 7u) << 8) | (((F >> 6) & 7u) << 16) | (((F >> 9) & 7u) << 24);
                    }
                    uint32_t V, W;
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(V) : "s"(mant4), "v"(Bf), "v"(X << SYM));
                    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(W) : "s"(0x80808080u), "v"(Bf << (8 - RB)), "v"(V));
                    bst32(rout, outg + t0 * 32 * EB, W);
                }
            };
            SmGroup G0 = G0first, G1 = G1first;
            for (; t < Tmain16; t += 16) {
                const SmGroup N0 = load_group(t / 4 + 2), N1 = load_group(t / 4 + 3);
                group4(t, G0);
                group4(t + 4, G1);
                G0 = load_group(t / 4 + 4);
                G1 = load_group(t / 4 + 5);
                group4(t + 8, N0);
                group4(t + 12, N1);
            }
        }
        // tail: the last steps of the shorter chunk and the ragged end, value by value
        for (; t < Tw; t += 8) {
            uint32_t smt[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                smt[u] = R > 0 ? bload_sm<DT>(rsm, sm_lane + (t + u) * 32 * R) : raw_field<DT>(rsm, lanebit + (t + u) * 32 * RB);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t tt = t + u;
                const uint64_t act = (run0 && ni0 > 32 * tt ? half_prefix_mask(ni0 - 32 * tt, 0) : 0ull) |
                                     (run1 && ni1 > 32 * tt ? half_prefix_mask(ni1 - 32 * tt, 1) : 0ull);
                step(tt, act, true, DT == 1 ? __umul24(smt[u], 0x101u) : smt[u], u & 3, true);  // (bf16: sign byte in bits 8-15 too)
            }
        }
        const bool endbad =
            half_mask(__ballot(rans_run && (x != kStateLow || offv != nw || (S && (escbad || escv != nesc)))), h) != 0;
        ok = ok && !endbad;
        // ---- chunks stored RAW: exponent bytes straight from the record ----
        if (R == 0 && raw_run) {
            // fp16, fp8: the chunk's symbols (packed at SB bits after the record
            // header) and raw fields (packed at RB bits).  A lane takes whole
            // groups of 32 values (SB and RB aligned dwords in, 8 EB dwords of
            // values out); the ragged last group value by value.
            const uint32_t ob = (h ? vals0 : 0u) * EB, eo = rel + kRecHeaderBytes, vb = (h ? vals0 : 0u) * RB;
            const uint32_t ng = ni / 32;
            for (uint32_t g = lj; g < ng; g += 32) {
                uint32_t sy[SB], rw[RB], w[8 * EB];
                load_dwords<SB>(rrec, eo + 4 * SB * g, sy);
                load_dwords<RB>(rsm, vb / 8 + 4 * RB * g, rw);
#pragma unroll
                for (uint32_t k = 0; k < 8 * EB; ++k) w[k] = 0;
#pragma unroll
                for (uint32_t i = 0; i < 32; ++i)
                    w[i * EB / 4] |= join_value<DT>(field32<SB>(sy, i), field32<RB>(rw, i)) << (8 * EB * (i % (4 / EB)));
                store_dwords<8 * EB>(rout, ob + 32 * EB * g, w);
            }
            for (uint32_t i = 32 * ng + lj; i < ni; i += 32) {
                const uint32_t sym = packed_field(rrec, eo, i * SB, SB);
                bst_value<DT>(rout, ob + i * EB, join_value<DT>(sym, raw_field<DT>(rsm, vb + i * RB)));
            }
        } else if (raw_run) {
            // units of 16 values: 16 exponent bytes and 16 R raw bytes in,
            // 16 EB bytes out, all 128-bit; four units per lane in flight
            const uint32_t ob = (h ? vals0 : 0u) * EB, sb = (h ? vals0 : 0u) * R, eo = rel + kRecHeaderBytes;
            const uint32_t nu = ni / 16;
            constexpr uint32_t U = 4, RS = R > 0 ? R : 1;
            for (uint32_t u0 = lj; u0 < nu; u0 += 32 * U) {
                uint4 E[U], SV[U][RS];
#pragma unroll
                for (uint32_t k = 0; k < U; ++k) {
                    const uint32_t u = u0 + 32 * k;
                    E[k] = bld128(rrec, u < nu ? eo + 16 * u : kOutOfRange);
#pragma unroll
                    for (uint32_t r = 0; r < R; ++r) SV[k][r] = bld128(rsm, u < nu ? sb + 16 * R * u + 16 * r : kOutOfRange);
                }
#pragma unroll
                for (uint32_t k = 0; k < U; ++k) {
                    const uint32_t u = u0 + 32 * k;
                    store_unit<DT>(rout, u < nu ? ob + 16 * EB * u : kOutOfRange, E[k], SV[k]);
                }
            }
            for (uint32_t i = 16 * nu + lj; i < ni; i += 32) {  // the chunk's last values
                const uint32_t v = join_value<DT>(bld8(rrec, eo + i), bload_sm<DT>(rsm, sb + i * R));
                bst_value<DT>(rout, ob + i * EB, v);
            }
        }
        if (h < nch && !ok && lj == 0) gstore<uint32_t>(p.status + b, 3u);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// scratch of uzip_compress_noalloc: the compress workspace for callers that
// cannot allocate device memory.  One array per device (each device that
// loads the library holds its own copy until the process ends).  Host code
// never names the array except in hipGetSymbolAddress: the name is a host-side
// stand-in, not a device address.  Its device address is looked up once per
// device, with that device current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[UZIP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// (the kernel template parameter is the dtype code, 1 to 5)
static int kernel_format(int dtype) { return dtype; }

hipError_t launch_compress(const EncParams &ep, hipStream_t stream, const ProfileEvents *ev) {
    uint64_t threads = ep.total_pairs > ep.nbuf ? ep.total_pairs : ep.nbuf;
    if (ep.plans != nullptr) {
        switch (kernel_format(ep.dtype)) {
        case 1: k_plan<1><<<dim3(ep.nbuf), dim3(256), 0, stream>>>(ep); break;
        case 2: k_plan<2><<<dim3(ep.nbuf), dim3(256), 0, stream>>>(ep); break;
        case 3: k_plan<3><<<dim3(ep.nbuf), dim3(256), 0, stream>>>(ep); break;
        case 4: k_plan<4><<<dim3(ep.nbuf), dim3(256), 0, stream>>>(ep); break;
        default: k_plan<5><<<dim3(ep.nbuf), dim3(256), 0, stream>>>(ep); break;
        }
    }
    k_prepare<<<dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, stream>>>(ep);
    if (ep.total_pairs > 0) {
        const dim3 grid((uint32_t)ep.total_pairs);
        if (ev != nullptr) (void)hipEventRecord(ev->start, stream);
        const int kf = kernel_format(ep.dtype) + (ep.sampled ? 8 : 0);
        switch (kf) {
        case 1: k_encode<1, false><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 2: k_encode<2, false><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 3: k_encode<3, false><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 4: k_encode<4, false><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 5: k_encode<5, false><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 9: k_encode<1, true><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 10: k_encode<2, true><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 11: k_encode<3, true><<<grid, dim3(64), 0, stream>>>(ep); break;
        case 12: k_encode<4, true><<<grid, dim3(64), 0, stream>>>(ep); break;
        default: k_encode<5, true><<<grid, dim3(64), 0, stream>>>(ep); break;
        }
        if (ev != nullptr) (void)hipEventRecord(ev->stop, stream);
        if (ep.plans != nullptr) {
            const dim3 rgrid((uint32_t)(ep.total_chunks < 2048 ? ep.total_chunks : 2048));
            switch (kernel_format(ep.dtype)) {
            case 1: k_raw_frame<1><<<rgrid, dim3(256), 0, stream>>>(ep); break;
            case 2: k_raw_frame<2><<<rgrid, dim3(256), 0, stream>>>(ep); break;
            case 3: k_raw_frame<3><<<rgrid, dim3(256), 0, stream>>>(ep); break;
            case 4: k_raw_frame<4><<<rgrid, dim3(256), 0, stream>>>(ep); break;
            default: k_raw_frame<5><<<rgrid, dim3(256), 0, stream>>>(ep); break;
            }
        }
        const dim3 cgrid((uint32_t)((ep.total_pairs + kCompactPairs - 1) / kCompactPairs));
        switch (kernel_format(ep.dtype)) {
        case 1: k_compact<1><<<cgrid, dim3(128 * kCompactPairs), 0, stream>>>(ep); break;
        case 2: k_compact<2><<<cgrid, dim3(128 * kCompactPairs), 0, stream>>>(ep); break;
        case 3: k_compact<3><<<cgrid, dim3(128 * kCompactPairs), 0, stream>>>(ep); break;
        case 4: k_compact<4><<<cgrid, dim3(128 * kCompactPairs), 0, stream>>>(ep); break;
        default: k_compact<5><<<cgrid, dim3(128 * kCompactPairs), 0, stream>>>(ep); break;
        }
        if (ep.plans != nullptr) {
            // the realised frames' gain check, then the RAW frame of each buffer that failed it
            const dim3 agrid((ep.nbuf + 255) / 256);
            EncParams rp = ep;
            rp.raw_pass = 1;
            const dim3 rgrid((uint32_t)(ep.total_chunks < 2048 ? ep.total_chunks : 2048));
            switch (kernel_format(ep.dtype)) {
            case 1: k_accept<1><<<agrid, dim3(256), 0, stream>>>(ep); k_raw_frame<1><<<rgrid, dim3(256), 0, stream>>>(rp); break;
            case 2: k_accept<2><<<agrid, dim3(256), 0, stream>>>(ep); k_raw_frame<2><<<rgrid, dim3(256), 0, stream>>>(rp); break;
            case 3: k_accept<3><<<agrid, dim3(256), 0, stream>>>(ep); k_raw_frame<3><<<rgrid, dim3(256), 0, stream>>>(rp); break;
            case 4: k_accept<4><<<agrid, dim3(256), 0, stream>>>(ep); k_raw_frame<4><<<rgrid, dim3(256), 0, stream>>>(rp); break;
            default: k_accept<5><<<agrid, dim3(256), 0, stream>>>(ep); k_raw_frame<5><<<rgrid, dim3(256), 0, stream>>>(rp); break;
            }
        }
    }
    return hipGetLastError();
}

hipError_t launch_decompress(const DecParams &vp, const DecodeParams &dp, int dtype, uint64_t max_chunks,
                             hipStream_t stream, const ProfileEvents *ev) {
    k_dec_validate<<<(vp.nbuf + 255) / 256, 256, 0, stream>>>(vp);
    if (vp.nbuf > 1) k_dec_scan<<<1, 1024, 0, stream>>>(vp);
    if (max_chunks > 0) {
        const uint64_t pairs = (max_chunks + 1) / 2 + vp.nbuf;  // upper bound of the chunk pairs
        const uint64_t grid = pairs < 8192 ? pairs : 8192;
        if (ev != nullptr) (void)hipEventRecord(ev->start, stream);
        // full-table frames, then sampled-table frames (each kernel leaves at
        // once when the call holds no valid buffer of its kind)
        switch (kernel_format(dtype)) {
        case 1: k_decode<1, false><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 2: k_decode<2, false><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 3: k_decode<3, false><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 4: k_decode<4, false><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        default: k_decode<5, false><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        }
        switch (kernel_format(dtype)) {
        case 1: k_decode<1, true><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 2: k_decode<2, true><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 3: k_decode<3, true><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        case 4: k_decode<4, true><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        default: k_decode<5, true><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp); break;
        }
        if (ev != nullptr) (void)hipEventRecord(ev->stop, stream);
    }
    return hipGetLastError();
}

}  // namespace uzip
