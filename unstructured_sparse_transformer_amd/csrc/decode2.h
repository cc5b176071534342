// decode2.h -- the two-kernel decode step (gate_gather_kernel,
// reduce_pack_kernel in decode.hip): its workspace and launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "decode.h"

namespace twell {

constexpr int DEC_MAX_G = DEC_MAX_NB * 256 / 32;  // gate workgroups (F / 32) at most
// Rows up to which twell_ffn_decode takes the two-kernel path: measured at the
// 2B-like shape, 20.6 / 25.6 us at T = 1 / 8 against 22.0 / 29.9 us for the
// four-kernel path, but 47.9 against 42.3 us at T = 64, where the partial rows
// per (row, gate workgroup) outnumber the four-kernel path's chunks ~8 times.
constexpr int DEC2_MAX_T = 16;

// z, the packing blocks' completion counter, and per (row, gate workgroup of
// 32 neurons) a flag and a partial y row.
struct DecodeWs2 {
    float *z;          // [T][F] gate pre-activations (fp32)
    int32_t *counter;  // packing blocks finished (cleared by the gate kernel)
    int32_t *flag;     // [T][F / 32]: 1 iff the partial row below was written
    float *part;       // [T][F / 32][d] partial y rows
    size_t bytes;      // total size from `base`
};

// Carve the workspace at `base` (256-byte aligned sections); with base ==
// nullptr only `bytes` is meaningful.
DecodeWs2 decode_ws2_layout(void *base, int T, int F, int d);

// The decode-shaped layer (T <= DEC_MAX_T, bf16) in two kernels: the gate with
// each workgroup's gather of its own neurons, then the per-row reduction
// beside the TwELL packing and the per-row results.
hipError_t launch_decode2(const void *x, const void *wg_t, const void *wu_t, const void *wd, int T, int d, int F,
                          int tile_w, int cap, void *val, uint8_t *idx, int32_t *cnt, int32_t *row_ovf,
                          int32_t *ovf_rows, int32_t *n_ovf, int32_t *order, int max_ovf, void *dense, float *y,
                          const DecodeWs2 &w, hipStream_t s);

}  // namespace twell
