// backward.h -- arguments, workspace layout and limits of the backward pass
// (host and device side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twell {

constexpr int BW_CE = 64;       // entries per token-major chunk
constexpr int BW_RC = 32;       // rows per block of the neuron regrouping
constexpr int BW_WGS = 1024;    // workgroups of the grid-stride kernels (4 waves each)
constexpr int BW_MAX_NB = 512;  // tiles per row held in LDS
constexpr int BW_MAX_D = 2048;  // model width: x, dy and three accumulators per lane in registers

struct BwWs {
    int32_t *status;     // [0] entries, [1] 1 if entries > max_entries (nothing computed)
    int32_t *row_e;      // [T] entries per row
    int32_t *row_src;    // [T] -1 fitting row, i >= 0 dense row i of an overflow row, -2 not held
    int32_t *row_ptr;    // [T + 1]
    int32_t *chunk0;     // [T + 1] first token-major chunk of each row
    int32_t *chunk_row;  // [chunks] row of each chunk
    int32_t *ent_j;      // [E] neuron of each entry (row-major, ascending j in a row)
    float *ent_h, *ent_du, *ent_dz, *ent_hu;  // [E]
    float *part;         // [chunks][d] partial dx rows
    int32_t *cnt_rc;     // [n_rc][F] per-block neuron counts, then bases, then counters
    int32_t *col_ptr;    // [F + 1]
    int32_t *csc_t, *csc_e;  // [E] row and entry of each neuron-major entry
    size_t bytes;
};

struct BwArgs {
    int T, F, tile_w, cap, n_b, d, nchunks, n_rc, max_entries, max_ovf;
    const int32_t *cnt;
    const __bf16 *val;
    const uint8_t *idx;
    const int32_t *row_ovf, *ovf_rows, *n_ovf;
    const __bf16 *dense;
    const __bf16 *x, *wg_t, *wu_t, *wd;
    const float *dy;
    float *dx, *dwg, *dwu, *dwd;
    BwWs ws;
};

BwWs bw_ws_layout(void *base, int T, int F, int d, int max_entries);

}  // namespace twell
