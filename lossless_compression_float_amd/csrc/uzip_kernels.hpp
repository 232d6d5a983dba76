// uzip_kernels.hpp -- kernel parameter blocks and launchers (internal).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "uzip.h"
#include "uzip_common.hpp"

namespace uzip {

struct EncParams {
    const EncDesc *descs;  // device array, used when nbuf > 1
    EncDesc single;        // used when nbuf == 1
    uint32_t nbuf;
    uint32_t chunk_elems;
    uint64_t total_chunks;  // chunks over all buffers
    uint64_t total_pairs;   // chunk pairs (two consecutive chunks of one buffer) over all buffers
    uint8_t *slots;         // one slot of slot_stride bytes per chunk: record prefix, words filled from the end
    uint64_t slot_stride;
    uint32_t *rec_sizes;    // record bytes per chunk
    uint64_t *flags;        // one look-back word per chunk pair (zeroed before compaction)
    uint32_t *ticket;       // chunk-pair ticket counter of the compaction (zeroed before it)
    int dtype;
    uint32_t sampled;       // 1: tables from each chunk's sample (header flag bit 0, record mode 2)
    uzip_plan *plans;       // per-call arbitration: one plan per buffer (null: every buffer is coded)
    uzip_policy policy;     // the cost model's inputs when plans is set
    uint32_t raw_pass;      // k_raw_frame: 0 writes the buffers planned RAW, 1 those whose realised frame failed
};

struct DecParams {
    const DecDesc *descs;
    DecDesc single;
    uint32_t nbuf;
    int dtype;
    DecInfo *info;
    uint64_t *pair_first;  // nbuf + 1 entries: exclusive prefix of the chunk-pair counts
    uint32_t *status;
    uint32_t *kinds;       // written after validation: which decoders have work (see DecodeParams)
};

struct DecodeParams {
    const DecDesc *descs;
    DecDesc single;
    uint32_t nbuf;
    const DecInfo *info;
    const uint64_t *pair_first;
    uint32_t *status;
    const uint32_t *kinds;  // bit 0: some valid buffer has full tables, bit 1: some has sampled ones
};

// events the caller asks to have recorded around the main coding kernel
// (benchmark instrumentation; passed per call, never kept)
struct ProfileEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

hipError_t launch_compress(const EncParams &ep, hipStream_t stream, const ProfileEvents *ev = nullptr);
// device address of the current device's no-allocation scratch (looked up on
// the first call on each device, then kept)
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_decompress(const DecParams &vp, const DecodeParams &dp, int dtype, uint64_t max_chunks,
                             hipStream_t stream, const ProfileEvents *ev = nullptr);

}  // namespace uzip
