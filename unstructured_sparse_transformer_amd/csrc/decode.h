// decode.h -- workspace layout and limits of the decode-shaped path (host and
// device side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace twell {

constexpr int DEC_MAX_T = 64;           // rows per decode call
constexpr int DEC_BASE_CHUNKS = 1024;   // gather chunks aimed for at most (plus one per row)
constexpr int DEC_MIN_E = 8;            // entries per gather chunk: 8 * 2^m ...
constexpr int DEC_MAX_E = 1024;         // ... up to this
constexpr int DEC_GATHER_WGS = 256;     // gather workgroups (4 waves, one chunk per wave at a time)
constexpr int DEC_MAX_NB = 512;         // tiles per row (F / tile_w) the gather holds in LDS
// T * F bound that keeps the chunk count within DEC_BASE_CHUNKS + T
constexpr int64_t DEC_MAX_TF = (int64_t)DEC_BASE_CHUNKS * DEC_MAX_E;

struct DecodeWs {
    float *z;            // [T][F] gate pre-activations (fp32)
    int32_t *counter;    // packing workgroups finished (cleared by the gate kernel)
    int32_t *chunk_e;    // entries per gather chunk
    int32_t *row_e;      // [T] active neurons of each row (sum of its tiles' true counts)
    int32_t *row_o;      // [T] nonzero iff some tile of the row holds more than cap
    int32_t *chunk0;     // [T + 1] first chunk of each row; chunk0[T] = number of chunks
    float *part;         // [max_chunks][d] partial y row of each chunk
    int max_chunks;
    size_t bytes;        // total size from `base`
};

// Carve the workspace at `base` (256-byte aligned sections).  With base ==
// nullptr only `bytes` is meaningful.
DecodeWs decode_ws_layout(void *base, int T, int F, int tile_w, int d);

// Size of the static scratch array behind twell_ffn_decode_noalloc.  Every
// decode shape with d <= 2048 fits: z is at most 2^20 floats (4 MiB) and the
// partial rows (DEC_BASE_CHUNKS + T) x d floats (8.5 MiB at d = 2048).
constexpr size_t DEC_STATIC_BYTES = (size_t)16 << 20;

// Device address of the static scratch's copy on the current device, looked
// up once per device (no allocation) and kept for later calls.
hipError_t decode_static_workspace(void **ptr);

}  // namespace twell
