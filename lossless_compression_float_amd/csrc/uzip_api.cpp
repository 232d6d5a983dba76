// uzip_api.cpp -- the C ABI declared in include/uzip.h: argument checks,
// layout and workspace carving, descriptor upload, and launches on the
// caller's stream.  Nothing here synchronises the stream.  Device memory is
// never allocated; the batched calls stage their descriptors in a small
// pinned host area per calling thread (see DescStage).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include <hip/hip_runtime.h>

#include "uzip.h"
#include "uzip_common.hpp"
#include "uzip_kernels.hpp"

using namespace uzip;

namespace {

constexpr uint64_t kWsAlign = 256;

uint64_t al(uint64_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool dtype_ok(uzip_dtype d) { return d >= UZIP_BF16 && d <= UZIP_FP8_E5M2; }

// chunk_elems of a call, or 0 when the chunk size is invalid: the chunk must
// hold a multiple of 32 values (whole rANS steps) and at most 2^20 values
// (so that count * (4096 - nsym) fits 32 bits in the normalisation).
uint64_t chunk_elems_of(uzip_dtype dtype, size_t chunk_bytes) {
    if (!dtype_ok(dtype)) return 0;
    const uint64_t eb = elem_bytes(dtype);
    if (chunk_bytes == 0) chunk_bytes = dtype == UZIP_FP32 ? 262144 : 65536;
    if (chunk_bytes % (32 * eb) != 0) return 0;
    const uint64_t ce = chunk_bytes / eb;
    return (ce == 0 || ce > kMaxChunkElems) ? 0 : ce;
}

// Limits of one compress call, checked on the host before any size is
// computed or anything launched: a buffer holds fewer than 2^44 values (so
// that every byte count below is exact in 64 bits), and a call has at most
// kMaxPairs chunk pairs, so that each launch grid (k_compact's: 1024 threads
// per kCompactPairs = 8 pairs) stays within the 2^32 - 1 work-items of one
// grid dimension.  The arbitrated batched calls also launch a 256-thread
// workgroup per buffer, hence kMaxPlanBuffers.
constexpr uint64_t kMaxElems = 1ull << 44;
constexpr uint64_t kMaxPairs = (1ull << 25) - 8;
constexpr uint64_t kMaxPlanBuffers = (1ull << 24) - 1;

uint64_t pairs_of(uint64_t n, uint64_t ce) { return ((n + ce - 1) / ce + 1) / 2; }

bool count_ok(uint64_t n, uint64_t ce) { return n < kMaxElems && pairs_of(n, ce) <= kMaxPairs; }

struct EncWs {
    uint64_t descs, sizes, flags, ticket, slots, slot_stride, bytes;
};

// Compress workspace: descriptors (batched calls), record size per chunk,
// one look-back word per chunk pair (at most one pair per chunk), the
// compaction's ticket counter, and one slot per chunk, where the encoder
// builds the record before its offset is known.  A slot holds the chunk's RAW
// record, and at least the largest RANS prefix (header, bitmap, 256
// frequencies, states), which the encoder writes before it knows whether the
// chunk will be stored RAW.
EncWs enc_ws(uzip_dtype dtype, uint64_t nbuf, uint64_t chunks, uint64_t ce) {
    EncWs w{};
    uint64_t o = 0;
    w.descs = o;
    o += al(nbuf > 1 ? nbuf * sizeof(EncDesc) : 0);
    w.sizes = o;
    o += al(chunks * 4);
    w.flags = o;
    o += al(chunks * 8);
    w.ticket = o;
    o += al(8);
    w.slot_stride = std::max<uint64_t>(raw_record_bytes(ce, sym_bits(dtype)), align16(words_offset_sampled(256)));
    w.slots = o;
    o += chunks * w.slot_stride;
    w.bytes = o + kWsAlign;  // slack: the caller's pointer need only be 16-byte aligned
    return w;
}

struct DecWs {
    uint64_t descs, info, pair_first, kinds, bytes;
};

DecWs dec_ws(uint64_t nbuf) {
    DecWs w{};
    uint64_t o = 0;
    w.descs = o;
    o += al(nbuf > 1 ? nbuf * sizeof(DecDesc) : 0);
    w.info = o;
    o += al(nbuf * sizeof(DecInfo));
    w.pair_first = o;
    o += al((nbuf + 1) * 8);
    w.kinds = o;
    o += al(4);
    w.bytes = o + kWsAlign;
    return w;
}

uint8_t *ws_base(void *ws) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(ws);
    return reinterpret_cast<uint8_t *>((p + kWsAlign - 1) & ~uintptr_t(kWsAlign - 1));
}

uint64_t max_size(uzip_dtype dtype, uint64_t n, uint64_t ce) {
    const Layout l = layout_of(dtype, n, ce);
    if (l.chunks == 0) return l.exp_off;
    const uint64_t last = n - (l.chunks - 1) * ce;
    const uint32_t sb = sym_bits(dtype);
    return l.exp_off + (l.chunks - 1) * raw_record_bytes(ce, sb) + raw_record_bytes(last, sb);
}

static_assert(sizeof(uzip_policy) == 56 && sizeof(uzip_plan) == 32, "arbitration structs as uzip.h lays them out");

// Host staging of the batched calls' descriptors.  A host-to-device copy from
// pageable memory does not return before the stream has reached it, so it
// would hold the caller behind every kernel already queued; the descriptors
// are written to pinned host memory instead and copied asynchronously.  Each
// host thread keeps, per device, a ring of kStageSlots pinned buffers, each
// with an event recorded after its copy: a slot is reused once its event has
// completed, so the caller waits only when it runs kStageSlots batched calls
// ahead of the device.  The buffers are allocated on a thread's first batched
// call on a device (and grown when a call needs more), and kept until the
// process ends.
constexpr int kStageSlots = 8;
constexpr int kStageDevices = 16;

struct StageSlot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
};

struct DescStage {
    StageSlot slot[kStageDevices][kStageSlots];
    int next[kStageDevices] = {};
};

thread_local DescStage t_stage;

// Copies `bytes` of `src` to the device at `dst` on `stream` without waiting
// for the stream.  Returns false on a HIP error.
bool stage_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (dev < 0 || dev >= kStageDevices)  // beyond the staged devices: a plain (blocking) copy
        return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, stream) == hipSuccess;
    int &next = t_stage.next[dev];
    StageSlot &sl = t_stage.slot[dev][next];
    next = (next + 1) % kStageSlots;
    if (sl.pending) {
        if (hipEventSynchronize(sl.done) != hipSuccess) return false;
        sl.pending = false;
    }
    if (sl.done == nullptr && hipEventCreateWithFlags(&sl.done, hipEventDisableTiming) != hipSuccess) {
        sl.done = nullptr;
        return false;
    }
    if (sl.cap < bytes) {
        if (sl.host != nullptr) (void)hipHostFree(sl.host);
        sl.host = nullptr;
        sl.cap = 0;
        const size_t cap = std::max<size_t>(bytes, 64 << 10);
        if (hipHostMalloc(&sl.host, cap, hipHostMallocDefault) != hipSuccess) {
            sl.host = nullptr;
            return false;
        }
        sl.cap = cap;
    }
    memcpy(sl.host, src, bytes);
    if (hipMemcpyAsync(dst, sl.host, bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return false;
    if (hipEventRecord(sl.done, stream) != hipSuccess) return false;
    sl.pending = true;
    return true;
}

// The cost model's inputs must be usable as the header states: positive
// rates, per-mille fields at most 1000, reserved zero.
bool policy_ok(const uzip_policy *p) {
    return p != nullptr && p->link_bytes_per_us > 0 && p->encode_bytes_per_us > 0 && p->decode_bytes_per_us > 0 &&
           p->exposed_encode_permil <= 1000 && p->exposed_decode_permil <= 1000 && p->min_gain_permil <= 1000 &&
           p->reserved == 0;
}

// Shared body of the single and batched compress calls (plans non-null: the
// arbitrated forms).
uzip_status compress_impl(uzip_dtype dtype, uint64_t ce, EncDesc *descs, uint32_t nbuf, uint64_t chunks,
                          void *d_workspace, size_t workspace_bytes, hipStream_t stream,
                          uzip_plan *plans = nullptr, const uzip_policy *policy = nullptr, bool sampled = false,
                          const ProfileEvents *ev = nullptr) {
    const EncWs w = enc_ws(dtype, nbuf, chunks, ce);
    if (d_workspace == nullptr || workspace_bytes < w.bytes || !aligned(d_workspace, 16))
        return UZIP_ERR_INVALID_ARGUMENT;
    uint8_t *base = ws_base(d_workspace);
    EncParams ep{};
    ep.nbuf = nbuf;
    ep.chunk_elems = (uint32_t)ce;
    ep.total_chunks = chunks;
    ep.total_pairs = 0;
    uint64_t tiles = 0;
    for (uint32_t b = 0; b < nbuf; ++b) {
        EncDesc &d = descs[b];
        const uint64_t pairs = (d.chunks + 1) / 2;
        d.pair_first = ep.total_pairs;
        d.tile_first = tiles;
        ep.total_pairs += pairs;
        tiles += (pairs + kPairTile - 1) / kPairTile;
    }
    ep.slots = base + w.slots;
    ep.slot_stride = w.slot_stride;
    ep.rec_sizes = reinterpret_cast<uint32_t *>(base + w.sizes);
    ep.flags = reinterpret_cast<uint64_t *>(base + w.flags);
    ep.ticket = reinterpret_cast<uint32_t *>(base + w.ticket);
    ep.dtype = dtype;
    ep.sampled = sampled ? 1u : 0u;
    ep.plans = plans;
    if (policy) ep.policy = *policy;
    if (nbuf == 1) {
        ep.single = descs[0];
        ep.descs = nullptr;
    } else {
        EncDesc *dd = reinterpret_cast<EncDesc *>(base + w.descs);
        if (!stage_copy(dd, descs, nbuf * sizeof(EncDesc), stream)) return UZIP_ERR_DEVICE;
        ep.descs = dd;
    }
    const hipError_t e = launch_compress(ep, stream, ev);
    return e == hipSuccess ? UZIP_OK : UZIP_ERR_DEVICE;
}

// Body of uzip_compress and uzip_compress_arbitrated (policy null: no arbitration).
uzip_status compress_single(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                            const uzip_policy *policy, void *d_out, size_t out_capacity, uint64_t *d_out_size,
                            uzip_plan *d_plan, void *d_workspace, size_t workspace_bytes, hipStream_t stream,
                            bool sampled = false) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    if (!ce || !count_ok(num_elements, ce)) return UZIP_ERR_INVALID_ARGUMENT;
    if (num_elements > 0 && (d_in == nullptr || !aligned(d_in, 16))) return UZIP_ERR_INVALID_ARGUMENT;
    if (d_out == nullptr || !aligned(d_out, 16) || d_out_size == nullptr || !aligned(d_out_size, 8))
        return UZIP_ERR_INVALID_ARGUMENT;
    if (out_capacity < max_size(dtype, num_elements, ce)) return UZIP_ERR_CAPACITY;
    const Layout l = layout_of(dtype, num_elements, ce);
    EncDesc desc{static_cast<const uint8_t *>(d_in), static_cast<uint8_t *>(d_out), d_out_size, num_elements,
                 0, l.sm_off, l.exp_off, l.chunks, 0, 0};
    return compress_impl(dtype, ce, &desc, 1, l.chunks, d_workspace, workspace_bytes, stream,
                         policy ? d_plan : nullptr, policy, sampled);
}

// Body of uzip_compress_batched and its arbitrated form (policy null: no arbitration).
uzip_status compress_batched(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                             const size_t *h_num_elements, size_t chunk_bytes, const uzip_policy *policy,
                             void *const *h_out, const size_t *h_out_capacity, uint64_t *d_out_sizes,
                             uzip_plan *d_plans, void *d_workspace, size_t workspace_bytes, hipStream_t stream,
                             bool sampled = false, const ProfileEvents *ev = nullptr) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    if (!ce || num_buffers == 0 || num_buffers > 0xFFFFFFFFull) return UZIP_ERR_INVALID_ARGUMENT;
    if (policy != nullptr && num_buffers > kMaxPlanBuffers) return UZIP_ERR_INVALID_ARGUMENT;
    if (!h_in || !h_num_elements || !h_out || !h_out_capacity || !d_out_sizes || !aligned(d_out_sizes, 8))
        return UZIP_ERR_INVALID_ARGUMENT;
    // (kept per thread across calls: no heap allocation once it has grown)
    thread_local std::vector<EncDesc> descs;
    if (descs.size() < num_buffers) descs.resize(num_buffers);
    uint64_t chunks = 0, pairs = 0;
    for (size_t b = 0; b < num_buffers; ++b) {
        const uint64_t n = h_num_elements[b];
        if (n >= kMaxElems) return UZIP_ERR_INVALID_ARGUMENT;
        pairs += pairs_of(n, ce);
        if (pairs > kMaxPairs) return UZIP_ERR_INVALID_ARGUMENT;
        if (n > 0 && (h_in[b] == nullptr || !aligned(h_in[b], 16))) return UZIP_ERR_INVALID_ARGUMENT;
        if (h_out[b] == nullptr || !aligned(h_out[b], 16)) return UZIP_ERR_INVALID_ARGUMENT;
        if (h_out_capacity[b] < max_size(dtype, n, ce)) return UZIP_ERR_CAPACITY;
        const Layout l = layout_of(dtype, n, ce);
        descs[b] = EncDesc{static_cast<const uint8_t *>(h_in[b]), static_cast<uint8_t *>(h_out[b]), d_out_sizes + b, n,
                           chunks, l.sm_off, l.exp_off, l.chunks, 0, 0};
        chunks += l.chunks;
    }
    return compress_impl(dtype, ce, descs.data(), (uint32_t)num_buffers, chunks, d_workspace, workspace_bytes, stream,
                         policy ? d_plans : nullptr, policy, sampled, ev);
}

uzip_status decompress_impl(uzip_dtype dtype, const DecDesc *descs, uint32_t nbuf, uint32_t *d_status,
                            void *d_workspace, size_t workspace_bytes, hipStream_t stream,
                            const ProfileEvents *ev = nullptr) {
    const DecWs w = dec_ws(nbuf);
    if (d_workspace == nullptr || workspace_bytes < w.bytes || !aligned(d_workspace, 16))
        return UZIP_ERR_INVALID_ARGUMENT;
    uint8_t *base = ws_base(d_workspace);
    uint64_t max_chunks = 0;
    for (uint32_t b = 0; b < nbuf; ++b) max_chunks += (descs[b].n + 31) / 32;  // chunks hold >= 32 values
    DecParams vp{};
    vp.nbuf = nbuf;
    vp.dtype = dtype;
    vp.info = reinterpret_cast<DecInfo *>(base + w.info);
    vp.pair_first = reinterpret_cast<uint64_t *>(base + w.pair_first);
    vp.status = d_status;
    vp.kinds = reinterpret_cast<uint32_t *>(base + w.kinds);
    if (nbuf == 1) {
        vp.single = descs[0];
    } else {
        DecDesc *dd = reinterpret_cast<DecDesc *>(base + w.descs);
        if (!stage_copy(dd, descs, nbuf * sizeof(DecDesc), stream)) return UZIP_ERR_DEVICE;
        vp.descs = dd;
    }
    DecodeParams dp{};
    dp.descs = vp.descs;
    dp.single = vp.single;
    dp.nbuf = nbuf;
    dp.info = vp.info;
    dp.pair_first = vp.pair_first;
    dp.status = d_status;
    dp.kinds = vp.kinds;
    const hipError_t e = launch_decompress(vp, dp, dtype, max_chunks, stream, ev);
    return e == hipSuccess ? UZIP_OK : UZIP_ERR_DEVICE;
}

}  // namespace

extern "C" {

size_t uzip_max_compressed_size(uzip_dtype dtype, size_t num_elements, size_t chunk_bytes) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    return ce && count_ok(num_elements, ce) ? (size_t)max_size(dtype, num_elements, ce) : 0;
}

size_t uzip_workspace_size(uzip_dtype dtype, size_t num_elements, size_t chunk_bytes) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    if (!ce || !count_ok(num_elements, ce)) return 0;
    const uint64_t chunks = (num_elements + ce - 1) / ce;
    return (size_t)std::max(enc_ws(dtype, 1, chunks, ce).bytes, dec_ws(1).bytes);
}

size_t uzip_workspace_size_batched(uzip_dtype dtype, size_t num_buffers, const size_t *h_num_elements,
                                   size_t chunk_bytes) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    if (!ce || num_buffers == 0 || num_buffers > 0xFFFFFFFFull || h_num_elements == nullptr) return 0;
    uint64_t chunks = 0, pairs = 0;
    for (size_t b = 0; b < num_buffers; ++b) {
        if (h_num_elements[b] >= kMaxElems) return 0;
        chunks += (h_num_elements[b] + ce - 1) / ce;
        pairs += pairs_of(h_num_elements[b], ce);
        if (pairs > kMaxPairs) return 0;
    }
    return (size_t)std::max(enc_ws(dtype, num_buffers, chunks, ce).bytes, dec_ws(num_buffers).bytes);
}

uzip_status uzip_compress(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes, void *d_out,
                          size_t out_capacity, uint64_t *d_out_size, void *d_workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return compress_single(dtype, d_in, num_elements, chunk_bytes, nullptr, d_out, out_capacity, d_out_size, nullptr,
                           d_workspace, workspace_bytes, stream);
}

uzip_status uzip_compress_noalloc(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                  void *d_out, size_t out_capacity, uint64_t *d_out_size, hipStream_t stream) {
    const uint64_t ce = chunk_elems_of(dtype, chunk_bytes);
    if (!ce || !count_ok(num_elements, ce)) return UZIP_ERR_INVALID_ARGUMENT;
    const uint64_t chunks = (num_elements + ce - 1) / ce;
    if (enc_ws(dtype, 1, chunks, ce).bytes > UZIP_NOALLOC_SCRATCH_BYTES) return UZIP_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return UZIP_ERR_DEVICE;
    return compress_single(dtype, d_in, num_elements, chunk_bytes, nullptr, d_out, out_capacity, d_out_size, nullptr,
                           ws, UZIP_NOALLOC_SCRATCH_BYTES, stream);
}

uzip_status uzip_compress_sampled(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                  void *d_out, size_t out_capacity, uint64_t *d_out_size, void *d_workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return compress_single(dtype, d_in, num_elements, chunk_bytes, nullptr, d_out, out_capacity, d_out_size, nullptr,
                           d_workspace, workspace_bytes, stream, true);
}

uzip_status uzip_compress_arbitrated(uzip_dtype dtype, const void *d_in, size_t num_elements, size_t chunk_bytes,
                                     const uzip_policy *policy, void *d_out, size_t out_capacity,
                                     uint64_t *d_out_size, uzip_plan *d_plan, void *d_workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    if (!policy_ok(policy) || d_plan == nullptr || !aligned(d_plan, 8) || num_elements >= (1ull << 44))
        return UZIP_ERR_INVALID_ARGUMENT;
    return compress_single(dtype, d_in, num_elements, chunk_bytes, policy, d_out, out_capacity, d_out_size, d_plan,
                           d_workspace, workspace_bytes, stream);
}

uzip_status uzip_decompress(const void *d_in, size_t in_bytes, uzip_dtype dtype, size_t num_elements, void *d_out,
                            uint32_t *d_status, void *d_workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return UZIP_ERR_INVALID_ARGUMENT;
    if (in_bytes > 0 && (d_in == nullptr || !aligned(d_in, 16))) return UZIP_ERR_INVALID_ARGUMENT;
    if (num_elements > 0 && (d_out == nullptr || !aligned(d_out, 16))) return UZIP_ERR_INVALID_ARGUMENT;
    if (d_status == nullptr || !aligned(d_status, 4)) return UZIP_ERR_INVALID_ARGUMENT;
    const DecDesc desc{static_cast<const uint8_t *>(d_in), static_cast<uint8_t *>(d_out), in_bytes, num_elements};
    return decompress_impl(dtype, &desc, 1, d_status, d_workspace, workspace_bytes, stream);
}

uzip_status uzip_compress_batched(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                  const size_t *h_num_elements, size_t chunk_bytes, void *const *h_out,
                                  const size_t *h_out_capacity, uint64_t *d_out_sizes, void *d_workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return compress_batched(dtype, num_buffers, h_in, h_num_elements, chunk_bytes, nullptr, h_out, h_out_capacity,
                            d_out_sizes, nullptr, d_workspace, workspace_bytes, stream);
}

uzip_status uzip_compress_batched_sampled(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                          const size_t *h_num_elements, size_t chunk_bytes, void *const *h_out,
                                          const size_t *h_out_capacity, uint64_t *d_out_sizes, void *d_workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    return compress_batched(dtype, num_buffers, h_in, h_num_elements, chunk_bytes, nullptr, h_out, h_out_capacity,
                            d_out_sizes, nullptr, d_workspace, workspace_bytes, stream, true);
}

uzip_status uzip_compress_batched_arbitrated(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                             const size_t *h_num_elements, size_t chunk_bytes,
                                             const uzip_policy *policy, void *const *h_out,
                                             const size_t *h_out_capacity, uint64_t *d_out_sizes,
                                             uzip_plan *d_plans, void *d_workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
    if (!policy_ok(policy) || d_plans == nullptr || !aligned(d_plans, 8)) return UZIP_ERR_INVALID_ARGUMENT;
    return compress_batched(dtype, num_buffers, h_in, h_num_elements, chunk_bytes, policy, h_out, h_out_capacity,
                            d_out_sizes, d_plans, d_workspace, workspace_bytes, stream);
}

uzip_status uzip_decompress_batched(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                    const size_t *h_in_bytes, const size_t *h_num_elements, void *const *h_out,
                                    uint32_t *d_status, void *d_workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    return uzip_decompress_batched_timed(dtype, num_buffers, h_in, h_in_bytes, h_num_elements, h_out, d_status,
                                         d_workspace, workspace_bytes, stream, nullptr, nullptr);
}

uzip_status uzip_decompress_batched_timed(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                          const size_t *h_in_bytes, const size_t *h_num_elements,
                                          void *const *h_out, uint32_t *d_status, void *d_workspace,
                                          size_t workspace_bytes, hipStream_t stream, hipEvent_t main_start,
                                          hipEvent_t main_stop) {
    if (!dtype_ok(dtype) || num_buffers == 0 || num_buffers > 0xFFFFFFFFull) return UZIP_ERR_INVALID_ARGUMENT;
    if ((main_start == nullptr) != (main_stop == nullptr)) return UZIP_ERR_INVALID_ARGUMENT;
    if (!h_in || !h_in_bytes || !h_num_elements || !h_out || !d_status || !aligned(d_status, 4))
        return UZIP_ERR_INVALID_ARGUMENT;
    thread_local std::vector<DecDesc> descs;  // (kept per thread across calls)
    if (descs.size() < num_buffers) descs.resize(num_buffers);
    for (size_t b = 0; b < num_buffers; ++b) {
        if (h_in_bytes[b] > 0 && (h_in[b] == nullptr || !aligned(h_in[b], 16))) return UZIP_ERR_INVALID_ARGUMENT;
        if (h_num_elements[b] > 0 && (h_out[b] == nullptr || !aligned(h_out[b], 16)))
            return UZIP_ERR_INVALID_ARGUMENT;
        descs[b] = DecDesc{static_cast<const uint8_t *>(h_in[b]), static_cast<uint8_t *>(h_out[b]), h_in_bytes[b],
                           h_num_elements[b]};
    }
    const ProfileEvents ev{main_start, main_stop};
    return decompress_impl(dtype, descs.data(), (uint32_t)num_buffers, d_status, d_workspace, workspace_bytes, stream,
                           main_start != nullptr ? &ev : nullptr);
}

uzip_status uzip_compress_batched_timed(uzip_dtype dtype, size_t num_buffers, const void *const *h_in,
                                        const size_t *h_num_elements, size_t chunk_bytes, uint32_t sampled,
                                        const uzip_policy *policy, void *const *h_out, const size_t *h_out_capacity,
                                        uint64_t *d_out_sizes, uzip_plan *d_plans, void *d_workspace,
                                        size_t workspace_bytes, hipStream_t stream, hipEvent_t main_start,
                                        hipEvent_t main_stop) {
    if ((main_start == nullptr) != (main_stop == nullptr) || sampled > 1) return UZIP_ERR_INVALID_ARGUMENT;
    if (policy != nullptr && (sampled || !policy_ok(policy) || d_plans == nullptr || !aligned(d_plans, 8)))
        return UZIP_ERR_INVALID_ARGUMENT;
    const ProfileEvents ev{main_start, main_stop};
    return compress_batched(dtype, num_buffers, h_in, h_num_elements, chunk_bytes, policy, h_out, h_out_capacity,
                            d_out_sizes, d_plans, d_workspace, workspace_bytes, stream, sampled != 0,
                            main_start != nullptr ? &ev : nullptr);
}

const char *uzip_status_string(uzip_status s) {
    switch (s) {
        case UZIP_OK: return "ok";
        case UZIP_ERR_INVALID_ARGUMENT: return "invalid argument";
        case UZIP_ERR_CAPACITY: return "output capacity below uzip_max_compressed_size";
        case UZIP_ERR_CORRUPT_INPUT: return "corrupt compressed input";
        case UZIP_ERR_DEVICE: return "HIP launch or copy failed";
        case UZIP_ERR_UNSUPPORTED: return "unsupported";
        case UZIP_ERR_SCRATCH_LIMIT: return "input too large for the no-allocation scratch (UZIP_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

}  // extern "C"
