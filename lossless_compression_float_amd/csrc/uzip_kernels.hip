// uzip_kernels.hip -- gfx950 kernels of the lossless bf16/fp32 codec.
//
// Compression of one chunk (UCCL-Zip, Figure 2: split the exponent field
// from the sign and fraction bits and entropy-code only the exponents;
// Figure 5(b): every block builds its own local table, so there is no global
// pass and no cross-block synchronisation):
//   k_encode     one half-wave (32 lanes) per chunk, two chunks per wave:
//                pass 1 streams the chunk forward with 128-bit loads, writes
//                the sign+mantissa bytes straight to their final place in the
//                output and counts the exponents in an LDS histogram; the
//                half-wave then normalises the counts to a 2^12 table and runs
//                the 32-lane rANS encoder backward over the chunk (re-reading
//                the input), placing each step's renormalisation words by wave
//                ballot + popcount rank.  The record goes to a workspace slot.
//   k_tile_reduce, k_scan_u64
//                exclusive scan of the record sizes (two levels: tiles of
//                1024 chunks, then one workgroup over the tile sums).
//   k_compact    moves every record to its final offset, writes the record
//                index and, for the last chunk of a buffer, the header and the
//                compressed size (NCCLZ Sec. IV-D2: self-describing frames).
// Decompression (NCCLZ Algorithm 2: validate the header, then decode):
//   k_dec_validate  one thread per buffer checks the buffer header.
//   k_decode        one half-wave per chunk: validates the record, builds the
//                   slot->symbol table in LDS, runs the rANS decoder forward
//                   and merges each exponent with its sign+mantissa bytes.
//
// Nothing here is a dense contraction: all arithmetic is 32-bit integer and
// bit manipulation on the vector ALU, and the kernels are bounded by HBM
// bandwidth and VALU issue, not by the matrix cores.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "uzip_common.hpp"
#include "uzip_kernels.hpp"

namespace uzip {

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

// the buffer holding global chunk g: the largest b with chunk_first[b] <= g
// (buffers without chunks share their successor's chunk_first and are skipped)
__device__ inline uint32_t find_enc_buffer(const EncDesc *d, uint32_t nbuf, uint64_t g) {
    uint32_t lo = 0, hi = nbuf - 1;
    while (lo < hi) {
        uint32_t mid = (lo + hi + 1) >> 1;
        if (d[mid].chunk_first <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ inline uint32_t find_dec_buffer(const uint64_t *chunk_first, uint32_t nbuf, uint64_t g) {
    uint32_t lo = 0, hi = nbuf - 1;
    while (lo < hi) {
        uint32_t mid = (lo + hi + 1) >> 1;
        if (chunk_first[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int DT>
__device__ inline uint32_t load_value(const uint8_t *in, uint32_t i) {
    if (DT == 1) return *(const uint16_t *)(in + 2ull * i);
    return *(const uint32_t *)(in + 4ull * i);
}

template <int DT>
__device__ inline uint32_t exponent_of(uint32_t v) {
    return DT == 1 ? (v >> 7) & 0xFFu : (v >> 23) & 0xFFu;
}

// ---------------------------------------------------------------------------
// k_encode: split + histogram + normalise + interleaved rANS, per chunk
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(64) void k_encode(EncParams p) {
    constexpr uint32_t EB = DT == 1 ? 2 : 4;  // bytes per value
    constexpr uint32_t R = DT == 1 ? 1 : 3;   // raw sign+mantissa bytes per value
    constexpr uint32_t VPL = 16 / EB;         // values per lane per 128-bit load
    constexpr uint32_t VPI = 32 * VPL;        // values per half-wave per pass-1 step

    __shared__ uint32_t s_hist[2][256];
    __shared__ uint32_t s_tab[2][256];   // f | c0 << 16
    __shared__ uint32_t s_keys[2][256];  // remainder << 8 | (255 - symbol), present symbols

    const uint32_t lane = threadIdx.x;
    const uint32_t h = lane >> 5, lj = lane & 31;
    const uint64_t g = uint64_t(blockIdx.x) * 2 + h;
    const bool valid = g < p.total_chunks;
    const uint64_t gq = valid ? g : p.total_chunks - 1;

    const EncDesc d = p.nbuf == 1 ? p.single : p.descs[find_enc_buffer(p.descs, p.nbuf, gq)];
    const uint64_t ci = gq - d.chunk_first;
    const uint64_t v0 = ci * p.chunk_elems;
    const uint32_t ni = valid ? (uint32_t)min<uint64_t>(p.chunk_elems, d.n - v0) : 0u;
    const uint8_t *in = d.in + v0 * EB;
    uint8_t *sm_out = d.out + d.sm_off + v0 * R;
    uint8_t *slot = p.slots + gq * p.slot_stride;

    for (uint32_t k = lj; k < 256; k += 32) s_hist[h][k] = 0;
    __syncthreads();

    // ---- pass 1: split, sign+mantissa bytes to the output, LDS histogram ----
    const uint32_t iters = (ni + VPI - 1) / VPI;
    const uint32_t iters_w = max(iters, (uint32_t)__shfl_xor(iters, 32, 64));
    for (uint32_t it = 0; it < iters_w; ++it) {
        const uint32_t i0 = it * VPI + lj * VPL;
        if (i0 >= ni) continue;
        uint32_t w[4];
        const bool full = i0 + VPL <= ni;
        if (full) {
            const uint4 q = *(const uint4 *)(in + uint64_t(i0) * EB);
            w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        } else {
            for (int k = 0; k < 4; ++k) w[k] = 0;
            for (uint32_t k = 0; k < VPL; ++k) {
                if (i0 + k < ni) {
                    const uint32_t v = load_value<DT>(in, i0 + k);
                    if (DT == 1) w[k >> 1] |= v << (16 * (k & 1));
                    else w[k] = v;
                }
            }
        }
        if (DT == 1) {
            uint32_t smw[2] = {0, 0};
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                const uint32_t v = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                const uint32_t sm = ((v >> 8) & 0x80u) | (v & 0x7Fu);
                smw[k >> 2] |= sm << (8 * (k & 3));
                if (full || i0 + k < ni) atomicAdd(&s_hist[h][(v >> 7) & 0xFFu], 1u);
            }
            if (full) {
                *(uint2 *)(sm_out + i0) = make_uint2(smw[0], smw[1]);
            } else {
                for (uint32_t k = 0; k < 8; ++k)
                    if (i0 + k < ni) sm_out[i0 + k] = (uint8_t)(smw[k >> 2] >> (8 * (k & 3)));
            }
        } else {
            uint32_t sm[4];
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t v = w[k];
                sm[k] = ((v >> 8) & 0x800000u) | (v & 0x7FFFFFu);
                if (full || i0 + k < ni) atomicAdd(&s_hist[h][(v >> 23) & 0xFFu], 1u);
            }
            if (full) {
                uint32_t *o = (uint32_t *)(sm_out + 3ull * i0);
                o[0] = sm[0] | (sm[1] << 24);
                o[1] = (sm[1] >> 8) | (sm[2] << 16);
                o[2] = (sm[2] >> 16) | (sm[3] << 8);
            } else {
                for (uint32_t k = 0; k < 4; ++k) {
                    if (i0 + k < ni) {
                        uint8_t *o = sm_out + 3ull * (i0 + k);
                        o[0] = (uint8_t)sm[k];
                        o[1] = (uint8_t)(sm[k] >> 8);
                        o[2] = (uint8_t)(sm[k] >> 16);
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- normalise the counts to a table of 4096 (lane lj owns symbols 8lj..8lj+7) ----
    // Reserve one slot per present symbol, share R = 4096 - nsym slots by the
    // floor of each quota, give the leftover slots to the largest remainders
    // (lower symbol first on equal remainders).
    uint32_t c[8], pm = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        c[k] = s_hist[h][lj * 8 + k];
        if (c[k]) pm |= 1u << k;
    }
    const uint32_t np = __popc(pm);
    const uint32_t nsym = half_sum(np);
    const uint32_t pre = half_excl_scan(np, lj);
    const uint32_t Rr = kTableSize - nsym;
    uint32_t fl[8], key[8], given = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        fl[k] = 0;
        key[k] = 0;
        if (c[k]) {
            const uint32_t q = c[k] * Rr;  // < 2^32: c <= 2^20, R < 2^12
            fl[k] = q / ni;
            key[k] = ((q - fl[k] * ni) << 8) | (255u - (lj * 8 + k));
            given += fl[k];
        }
    }
    given = half_sum(given);
    const uint32_t left = Rr - given;
    {
        uint32_t k2 = pre;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (c[k]) s_keys[h][k2++] = key[k];
    }
    __syncthreads();
    uint32_t above[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint32_t nsym_w = max(nsym, (uint32_t)__shfl_xor(nsym, 32, 64));
    const uint32_t left_w = max(left * (ni > 0), (uint32_t)__shfl_xor(left * (ni > 0), 32, 64));
    if (left_w > 0) {
        for (uint32_t m = 0; m < nsym_w; ++m) {
            const uint32_t km = s_keys[h][m & 255];
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
    for (int k = 0; k < 8; ++k) s_tab[h][lj * 8 + k] = f[k] | ((cbase + cpre[k]) << 16);

    // record prefix: presence bitmap, frequencies (ascending symbols), pad
    if (valid) {
        slot[kRecHeaderBytes + lj] = (uint8_t)pm;
        uint32_t k2 = pre;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (c[k]) *(uint16_t *)(slot + 48 + 2 * (k2++)) = (uint16_t)f[k];
        if (lj == 0 && (nsym & 1)) *(uint16_t *)(slot + 48 + 2 * nsym) = 0;
    }
    __syncthreads();

    // ---- pass 2: 32-lane interleaved rANS, steps from the last down to 0 ----
    // Words of one step are placed, lanes ascending, right before the words of
    // the following step, filling the slot from its end.
    const uint64_t raw_i = raw_record_bytes(ni);
    const uint64_t wofs = words_offset(nsym);
    uint32_t x = kStateLow;
    uint32_t nw = 0;
    bool dead = !valid;  // set when the words outgrow the RAW size: the chunk goes RAW
    const uint32_t T = (ni + 31) / 32;
    const uint32_t Tw = max(T, (uint32_t)__shfl_xor(T, 32, 64));
    const uint32_t nblk = (Tw + 7) / 8;
    uint32_t cur[8], nxt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t i = ((nblk - 1) * 8 + k) * 32 + lj;
        cur[k] = (nblk > 0 && i < ni) ? load_value<DT>(in, i) : 0u;
    }
    for (int32_t b = (int32_t)nblk - 1; b >= 0; --b) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t i = ((uint32_t)(b - 1) * 8 + k) * 32 + lj;
            nxt[k] = (b > 0 && i < ni) ? load_value<DT>(in, i) : 0u;
        }
#pragma unroll
        for (int k = 7; k >= 0; --k) {
            const uint32_t i = ((uint32_t)b * 8 + k) * 32 + lj;
            const bool act = !dead && i < ni;
            const uint32_t ft = s_tab[h][exponent_of<DT>(cur[k])];
            const uint32_t fs = ft & 0xFFFFu, c0 = ft >> 16;
            const bool need = act && (x >> 20) >= fs;  // x >= f * 2^20
            const uint32_t hm = half_mask(__ballot(need), h);
            const uint32_t cnt = __popc(hm);
            const uint32_t rank = __popc(hm & ((1u << lj) - 1u));
            if (!dead && wofs + 2ull * (nw + cnt) > raw_i) dead = true;
            if (need && !dead) {
                *(uint16_t *)(slot + raw_i - 2ull * (nw + cnt) + 2ull * rank) = (uint16_t)(x & 0xFFFFu);
                x >>= 16;
            }
            nw += cnt;
            if (act && !dead) {
                const uint32_t q = x / fs;
                x = q * kTableSize + (x - q * fs) + c0;
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) cur[k] = nxt[k];
    }

    const uint64_t rans_bytes = align16(wofs + 2ull * nw);
    const bool rans = valid && !dead && rans_bytes < raw_i;
    if (valid) {
        if (rans) {
            *(uint32_t *)(slot + states_offset(nsym) + 4 * lj) = x;
            if (lj == 0) {
                *(uint4 *)slot = make_uint4(nsym << 16, nw, ni, (uint32_t)rans_bytes);
                p.rec_sizes[g] = (uint32_t)rans_bytes;
            }
        } else {
            if (lj == 0) {
                *(uint4 *)slot = make_uint4(1u, 0u, ni, (uint32_t)raw_i);
                p.rec_sizes[g] = (uint32_t)raw_i;
            }
            for (uint32_t k = lj; k + kRecHeaderBytes < raw_i; k += 32)
                slot[kRecHeaderBytes + k] = k < ni ? (uint8_t)exponent_of<DT>(load_value<DT>(in, k)) : 0;
        }
    }
}

// ---------------------------------------------------------------------------
// scan of the record sizes
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tile_reduce(const uint32_t *sizes, uint64_t total_chunks, uint64_t *tile_sums) {
    __shared__ uint64_t s[256];
    const uint64_t t0 = uint64_t(blockIdx.x) * kTile;
    uint64_t acc = 0;
    for (uint64_t k = t0 + threadIdx.x; k < t0 + kTile && k < total_chunks; k += 256) acc += sizes[k];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = s[0];
}

// exclusive scan of n values into out[0..n] (out[n] = total); in may equal out
__global__ __launch_bounds__(1024) void k_scan_u64(const uint64_t *in, uint64_t *out, uint64_t n) {
    __shared__ uint64_t s[1024];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < n; base += 1024) {
        const uint64_t i = base + threadIdx.x;
        const uint64_t v = i < n ? in[i] : 0;
        s[threadIdx.x] = v;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const uint64_t t = (int)threadIdx.x >= o ? s[threadIdx.x - o] : 0;
            __syncthreads();
            s[threadIdx.x] += t;
            __syncthreads();
        }
        if (i < n) out[i] = carry + s[threadIdx.x] - v;
        carry += s[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[n] = carry;
}

// global exclusive offset of chunk g (whole wave of 64 lanes participates)
__device__ inline uint64_t chunk_offset(const uint32_t *sizes, const uint64_t *tile_offs, uint64_t g, uint32_t lane) {
    const uint64_t t0 = (g / kTile) * kTile;
    uint64_t s = 0;
    for (uint64_t k = t0 + lane; k < g; k += 64) s += sizes[k];
    return tile_offs[g / kTile] + wave_sum_u64(s);
}

// ---------------------------------------------------------------------------
// k_compact: records to their final offsets, index, header, size
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_compact(CompactParams p) {
    const uint64_t g = blockIdx.x;
    const uint32_t lane = threadIdx.x;
    const EncDesc d = p.nbuf == 1 ? p.single : p.descs[find_enc_buffer(p.descs, p.nbuf, g)];
    const uint64_t ci = g - d.chunk_first;
    const uint32_t size = p.rec_sizes[g];
    const uint64_t off_g = chunk_offset(p.rec_sizes, p.tile_offs, g, lane);
    const uint64_t off_first = ci == 0 ? off_g : chunk_offset(p.rec_sizes, p.tile_offs, d.chunk_first, lane);
    const uint64_t rec_off = off_g - off_first;
    uint8_t *out = d.out;
    if (lane == 0) *(uint64_t *)(out + kHeaderBytes + 8 * ci) = rec_off;
    if (ci + 1 == d.chunks) {
        const uint64_t total = d.exp_off + rec_off + size;
        if (lane == 0) {
            *(uint64_t *)(out + kHeaderBytes + 8 * d.chunks) = rec_off + size;
            *d.out_size = total;
        }
        if (lane < 16) {
            uint32_t wv = 0;
            switch (lane) {
                case 0: wv = kMagic; break;
                case 1: wv = kVersion | (uint32_t(p.dtype) << 16) | (kProbBits << 24); break;
                case 2: wv = kLanes | (raw_bytes_per_value(p.dtype) << 8); break;
                case 3: wv = p.chunk_elems; break;
                case 4: wv = (uint32_t)d.n; break;
                case 5: wv = (uint32_t)(d.n >> 32); break;
                case 6: wv = (uint32_t)d.chunks; break;
                case 7: wv = (uint32_t)(d.chunks >> 32); break;
                case 8: wv = (uint32_t)d.sm_off; break;
                case 9: wv = (uint32_t)(d.sm_off >> 32); break;
                case 10: wv = (uint32_t)d.exp_off; break;
                case 11: wv = (uint32_t)(d.exp_off >> 32); break;
                case 12: wv = (uint32_t)total; break;
                case 13: wv = (uint32_t)(total >> 32); break;
                default: wv = 0; break;
            }
            ((uint32_t *)out)[lane] = wv;
        }
        // zero the gaps after the index and after the sign+mantissa region
        const uint64_t gap0 = kHeaderBytes + 8 * (d.chunks + 1);
        for (uint64_t k = gap0 + lane; k < d.sm_off; k += 64) out[k] = 0;
        const uint64_t gap1 = d.sm_off + uint64_t(raw_bytes_per_value(p.dtype)) * d.n;
        for (uint64_t k = gap1 + lane; k < d.exp_off; k += 64) out[k] = 0;
    }
    // copy the record
    const uint8_t *src = p.slots + g * p.slot_stride;
    uint8_t *dst = out + d.exp_off + rec_off;
    const uint32_t mode = src[0];
    if (mode == 0) {
        const uint32_t nsym = *(const uint16_t *)(src + 2);
        const uint32_t nw = *(const uint32_t *)(src + 4);
        const uint32_t ni = *(const uint32_t *)(src + 8);
        const uint32_t wofs = (uint32_t)words_offset(nsym);
        for (uint32_t k = lane; k < wofs / 4; k += 64) ((uint32_t *)dst)[k] = ((const uint32_t *)src)[k];
        const uint16_t *wsrc = (const uint16_t *)(src + raw_record_bytes(ni) - 2ull * nw);
        uint16_t *wdst = (uint16_t *)(dst + wofs);
        for (uint32_t k = lane; k < nw; k += 64) wdst[k] = wsrc[k];
        for (uint32_t k = wofs + 2 * nw + lane; k < size; k += 64) dst[k] = 0;
    } else {
        for (uint32_t k = lane; k < size / 16; k += 64) ((uint4 *)dst)[k] = ((const uint4 *)src)[k];
    }
}

// header of an empty buffer (N = 0): 64-byte header, one index entry, pad
__global__ void k_empty_headers(const EncDesc *descs, EncDesc single, uint32_t nbuf, int dtype, uint32_t chunk_elems) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nbuf) return;
    const EncDesc d = nbuf == 1 ? single : descs[b];
    if (d.n != 0) return;
    uint32_t *o = (uint32_t *)d.out;
    const uint32_t hdr[20] = {kMagic, kVersion | (uint32_t(dtype) << 16) | (kProbBits << 24),
                              kLanes | (raw_bytes_per_value(dtype) << 8), chunk_elems, 0, 0, 0, 0, 80, 0, 80, 0,
                              80, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < 20; ++k) o[k] = hdr[k];
    *d.out_size = 80;
}

// ---------------------------------------------------------------------------
// decompression
// ---------------------------------------------------------------------------
__global__ void k_dec_validate(DecParams p) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= p.nbuf) return;
    const DecDesc d = p.nbuf == 1 ? p.single : p.descs[b];
    bool ok = d.in_bytes >= kHeaderBytes;
    DecInfo inf = {};
    if (ok) {
        const uint4 h0 = ((const uint4 *)d.in)[0], h1 = ((const uint4 *)d.in)[1];
        const uint4 h2 = ((const uint4 *)d.in)[2], h3 = ((const uint4 *)d.in)[3];
        const uint32_t r = raw_bytes_per_value(p.dtype);
        // V1 magic, version, fixed coder parameters; V2 dtype and count
        ok = h0.x == kMagic && (h0.y & 0xFFFFu) == kVersion && ((h0.y >> 16) & 0xFFu) == (uint32_t)p.dtype &&
             (h0.y >> 24) == kProbBits && (h0.z & 0xFFu) == kLanes && ((h0.z >> 8) & 0xFFu) == r;
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
                const uint64_t first = *(const uint64_t *)(d.in + kHeaderBytes);
                const uint64_t last = *(const uint64_t *)(d.in + kHeaderBytes + 8 * C);
                ok = first == 0 && last == total - exp_off;
            }
            inf.chunks = ok ? C : 0;
            inf.chunk_elems = ce;
            inf.sm_off = sm_off;
            inf.exp_off = exp_off;
            inf.total = total;
        }
    }
    if (!ok) inf.chunks = 0;
    p.info[b] = inf;
    p.status[b] = ok ? 0u : 3u;
    if (p.nbuf == 1) {
        p.chunk_first[0] = 0;
        p.chunk_first[1] = inf.chunks;
    } else {
        p.chunk_first[b] = inf.chunks;  // counts; scanned in place afterwards
    }
}

template <int DT>
__global__ __launch_bounds__(64) void k_decode(DecodeParams p) {
    constexpr uint32_t EB = DT == 1 ? 2 : 4;
    constexpr uint32_t R = DT == 1 ? 1 : 3;
    __shared__ uint8_t s_sym[2][kTableSize];
    __shared__ uint32_t s_ft[2][256];  // f | c0 << 16
    __shared__ uint8_t s_plist[2][256];

    const uint32_t lane = threadIdx.x;
    const uint32_t h = lane >> 5, lj = lane & 31;
    const uint64_t G = p.chunk_first[p.nbuf];

    for (uint64_t pair = blockIdx.x; pair * 2 < G; pair += gridDim.x) {
        const uint64_t g = pair * 2 + h;
        bool ok = g < G;
        const uint64_t gq = ok ? g : G - 1;
        const uint32_t b = p.nbuf == 1 ? 0u : find_dec_buffer(p.chunk_first, p.nbuf, gq);
        const DecDesc d = p.nbuf == 1 ? p.single : p.descs[b];
        const DecInfo inf = p.info[b];
        ok = ok && p.status[b] == 0;
        const bool real = ok;
        const uint64_t ci = gq - p.chunk_first[b];
        const uint64_t ce = inf.chunk_elems;
        const uint64_t v0 = ci * ce;
        const uint32_t ni = ok ? (uint32_t)min<uint64_t>(ce, d.n - v0) : 0u;

        // record bounds from the index (V5) and record header (V6)
        uint64_t a = 0, e = 0;
        if (ok) {
            a = *(const uint64_t *)(d.in + kHeaderBytes + 8 * ci);
            e = *(const uint64_t *)(d.in + kHeaderBytes + 8 * (ci + 1));
            ok = (a & 15u) == 0 && (e & 15u) == 0 && a <= e && e <= inf.total - inf.exp_off && e - a >= 16;
        }
        const uint8_t *rec = d.in + inf.exp_off + a;
        const uint64_t len = e - a;
        uint32_t mode = 1, nsym = 0, nw = 0;
        if (ok) {
            const uint4 rh = *(const uint4 *)rec;
            mode = rh.x & 0xFFu;
            nsym = rh.x >> 16;
            nw = rh.y;
            ok = mode <= 1 && rh.z == ni && rh.w == len;
            if (ok && mode == 1) ok = nsym == 0 && nw == 0 && len == raw_record_bytes(ni);
            if (ok && mode == 0) ok = nsym >= 1 && nsym <= 256 && len == align16(words_offset(nsym) + 2ull * nw);
        }
        const bool coded = ok && mode == 0;

        // table: presence bitmap byte lj covers symbols 8lj..8lj+7 (V7)
        uint32_t pb = coded ? rec[kRecHeaderBytes + lj] : 0u;
        const uint32_t np = __popc(pb);
        const uint32_t pre = half_excl_scan(np, lj);
        uint32_t fk[8], lsum = 0, cpre[8];
        bool fok = true;
        {
            uint32_t k2 = pre;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                fk[k] = 0;
                if ((pb >> k) & 1u) {
                    fk[k] = (k2 < nsym) ? *(const uint16_t *)(rec + 48 + 2 * k2) : 0u;
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
        if (coded) ok = seen == nsym && !fbad && tot == kTableSize;
        const bool coded_ok = ok && mode == 0;
        if (coded_ok) {
            uint32_t k2 = pre;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                s_ft[h][lj * 8 + k] = fk[k] | ((cbase + cpre[k]) << 16);
                if (fk[k]) s_plist[h][k2++] = (uint8_t)(lj * 8 + k);
            }
        }
        __syncthreads();
        if (coded_ok) {
            for (uint32_t m = 0; m < nsym; ++m) {
                const uint32_t s = s_plist[h][m];
                const uint32_t ft = s_ft[h][s];
                const uint32_t fs = ft & 0xFFFFu, c0 = ft >> 16;
                for (uint32_t k = lj; k < fs; k += 32) s_sym[h][c0 + k] = (uint8_t)s;
            }
        }
        __syncthreads();

        // states (V8)
        uint32_t x = kStateLow;
        const uint8_t *words = rec + words_offset(nsym);
        if (coded_ok) x = *(const uint32_t *)(rec + states_offset(nsym) + 4 * lj);
        const bool sbad = half_mask(__ballot(coded_ok && x < kStateLow), h) != 0;
        ok = ok && !sbad;

        // decode (V9: never read past n_words; end state L on every lane)
        const uint8_t *sm = d.in + inf.sm_off + v0 * R;
        uint8_t *outp = d.out + v0 * EB;
        const uint32_t T = ok ? (ni + 31) / 32 : 0u;
        const uint32_t Tw = max(T, (uint32_t)__shfl_xor(T, 32, 64));
        uint32_t pos = 0;
        for (uint32_t t = 0; t < Tw; ++t) {
            const uint32_t i = t * 32 + lj;
            const bool act = ok && i < ni;
            const uint32_t wpre = (ok && mode == 0 && pos + lj < nw) ? *(const uint16_t *)(words + 2ull * (pos + lj)) : 0u;
            uint32_t ex = 0;
            bool need = false;
            if (act) {
                if (mode == 0) {
                    const uint32_t slot = x & (kTableSize - 1);
                    const uint32_t s = s_sym[h][slot];
                    const uint32_t ft = s_ft[h][s];
                    x = (ft & 0xFFFFu) * (x >> kProbBits) + slot - (ft >> 16);
                    need = x < kStateLow;
                    ex = s;
                } else {
                    ex = rec[kRecHeaderBytes + i];
                }
            }
            const uint32_t hm = half_mask(__ballot(need), h);
            const uint32_t cnt = __popc(hm);
            const uint32_t rank = __popc(hm & ((1u << lj) - 1u));
            const uint32_t w = (uint32_t)__shfl((int)wpre, (int)rank, 32);
            if (ok && pos + cnt > nw) ok = false;
            if (need && ok) x = (x << 16) | w;
            pos += cnt;
            if (act && ok) {
                if (DT == 1) {
                    const uint32_t smb = sm[i];
                    ((uint16_t *)outp)[i] = (uint16_t)(((smb & 0x80u) << 8) | (ex << 7) | (smb & 0x7Fu));
                } else {
                    const uint8_t *q = sm + 3ull * i;
                    const uint32_t s24 = uint32_t(q[0]) | (uint32_t(q[1]) << 8) | (uint32_t(q[2]) << 16);
                    ((uint32_t *)outp)[i] = ((s24 & 0x800000u) << 8) | (ex << 23) | (s24 & 0x7FFFFFu);
                }
            }
        }
        const bool endbad = half_mask(__ballot(ok && mode == 0 && (x != kStateLow || pos != nw)), h) != 0;
        ok = ok && !endbad;
        if (real && !ok && lj == 0) p.status[b] = 3u;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
thread_local ProfileEvents g_profile;

hipError_t launch_compress(const EncParams &ep, const CompactParams &cp, uint64_t *tile_sums, uint64_t *tile_offs,
                           uint64_t ntiles, bool any_empty, hipStream_t stream) {
    if (any_empty) {
        const uint32_t nb = ep.nbuf;
        k_empty_headers<<<(nb + 255) / 256, 256, 0, stream>>>(ep.descs, ep.single, nb, ep.dtype, ep.chunk_elems);
    }
    if (ep.total_chunks > 0) {
        const uint64_t grid = (ep.total_chunks + 1) / 2;
        if (g_profile.start) (void)hipEventRecord(g_profile.start, stream);
        if (ep.dtype == 1) k_encode<1><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(ep);
        else k_encode<2><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(ep);
        if (g_profile.stop) (void)hipEventRecord(g_profile.stop, stream);
        k_tile_reduce<<<dim3((uint32_t)ntiles), dim3(256), 0, stream>>>(ep.rec_sizes, ep.total_chunks, tile_sums);
        k_scan_u64<<<1, 1024, 0, stream>>>(tile_sums, tile_offs, ntiles);
        k_compact<<<dim3((uint32_t)ep.total_chunks), dim3(64), 0, stream>>>(cp);
    }
    return hipGetLastError();
}

hipError_t launch_decompress(const DecParams &vp, const DecodeParams &dp, int dtype, uint64_t max_chunks,
                             hipStream_t stream) {
    k_dec_validate<<<(vp.nbuf + 255) / 256, 256, 0, stream>>>(vp);
    if (vp.nbuf > 1) k_scan_u64<<<1, 1024, 0, stream>>>(vp.chunk_first, vp.chunk_first, vp.nbuf);
    if (max_chunks > 0) {
        const uint64_t half = (max_chunks + 1) / 2;
        const uint64_t grid = half < 8192 ? half : 8192;
        if (g_profile.start) (void)hipEventRecord(g_profile.start, stream);
        if (dtype == 1) k_decode<1><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp);
        else k_decode<2><<<dim3((uint32_t)grid), dim3(64), 0, stream>>>(dp);
        if (g_profile.stop) (void)hipEventRecord(g_profile.stop, stream);
    }
    return hipGetLastError();
}

}  // namespace uzip
