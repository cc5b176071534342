// launch.h -- internal launchers behind the C ABI (host side).  Every
// launcher assumes the C-ABI layer has validated its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward.h"
#include "decode.h"

namespace twell {

// Gate GEMM + TwELL epilogue over all T rows.
hipError_t launch_gate_twell(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w,
                             int cap, void *val, uint8_t *idx, int32_t *cnt, hipStream_t s);

// The same, plus per-neuron active-row counts (added to neuron_cnt [F]) and
// per (row, tile) sums of the positive gate values (l1 [T][F / tile_w]).
hipError_t launch_gate_twell_stats(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w,
                                   int cap, void *val, uint8_t *idx, int32_t *cnt, int32_t *neuron_cnt, float *l1,
                                   hipStream_t s);

// The gate GEMM with a plain epilogue: h [T][F] = ReLU(x . W_g) stored
// densely in the element type.
hipError_t launch_gate_dense(int vdtype, const void *x, const void *wg_t, int T, int d, int F, void *h,
                             hipStream_t s);

// row_ovf[t] = any tile of row t has cnt > cap; work[t] = stored entries of
// row t (0 for an overflow row).
hipError_t launch_row_flags(const int32_t *cnt, int T, int n_b, int cap, int32_t *row_ovf, int32_t *work,
                            hipStream_t s);

// Ascending list of flagged rows (first max_ovf of them) and their total
// count; `order` holds the work values on entry and the work order on return.
// With order_e: also the work value of the row at each work position.
hipError_t launch_compact_rows(const int32_t *row_ovf, int T, int max_ovf, int32_t *ovf_rows, int32_t *n_ovf,
                               int32_t *order, hipStream_t s, int32_t *order_e = nullptr);

// dense[i][:] = ReLU(x[ovf_rows[i]] . W_g) for i < min(*n_ovf, max_ovf).
hipError_t launch_dense_gate(int vdtype, const void *x, int T, const void *wg_t, const int32_t *ovf_rows,
                             const int32_t *n_ovf, int max_ovf, int d, int F, void *dense, hipStream_t s);

// p[i][:] = round(dense[i][:] * (x[ovf_rows[i]] . W_u)) for i < min(*n_ovf, max_ovf).
hipError_t launch_gated_up(int vdtype, const void *x, int T, const void *wu_t, const int32_t *ovf_rows,
                           const int32_t *n_ovf, int max_ovf, int d, int F, const void *dense, void *p,
                           hipStream_t s);

// Both of the above in one GEMM (one pass over the gathered x rows):
// dense[i][:] = ReLU(x[ovf_rows[i]] . W_g) and p[i][:] = round(dense[i][:] *
// (x[ovf_rows[i]] . W_u)) for i < min(*n_ovf, max_ovf); the same values.
hipError_t launch_dense_gate_up(int vdtype, const void *x, int T, const void *wg_t, const void *wu_t,
                                const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf, int d, int F, void *dense,
                                void *p, hipStream_t s);

// y[ovf_rows[i]][:] = p[i][:] . W_d for i < min(*n_ovf, max_ovf); split-K with
// `splits` fp32 partial slabs in `part` ([splits][max_ovf][d]) when splits > 1.
hipError_t launch_down(int vdtype, const void *p, const void *wd, const int32_t *ovf_rows, const int32_t *n_ovf,
                       int max_ovf, int F, int d, float *y, float *part, int splits, hipStream_t s);

// Workspace of the fused step (256-byte aligned sections).
struct FusedWs {
    int32_t *row_e;    // [T] stored entries of each row (0 for an overflow row)
    int32_t *order_e;  // [T] the same in work order (one-call path: written by the compaction)
    int2 *ent;       // [T][n_b cap] each row's entries (neuron, gate value bits), packed first
    float *p;        // [nch][T n_b cap] partial dot products of u over d's column slices
    int64_t pstride; // T n_b cap: distance between two column slices' partials
    int nch;
    size_t bytes;
};
FusedWs fused_ws_layout(void *base, int T, int F, int tile_w, int cap, int d, int esz);

// Width of the fused step's column slices of d for element size esz.
int fused_slice_cols(int d, int esz);

// Fused up/down from TwELL for every row (overflow rows -> 0), rows started
// in `order` (ascending when null): the entries kernel, an up pass writing
// each stored entry's partial dot products, a down pass writing y.
hipError_t launch_ffn_fused(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, const int32_t *order,
                            int T, int F, int tile_w, int cap, const void *x, const void *wu_t, const void *wd, int d,
                            float *y, void *ws, hipStream_t s);

// The fused step in two parts, for the one-call path: the entries kernel,
// which also writes row_ovf[t] (some tile of row t has cnt > cap) and
// work[t] (stored entries of row t, 0 for an overflow row) as the partition's
// flag step does; then, after the compaction, the two passes.
hipError_t launch_ffn_entries(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                              int tile_w, int cap, int d, void *ws, int32_t *row_ovf, int32_t *work, hipStream_t s);
// use_order_e: the compaction wrote the entry counts in work order (FusedWs order_e).
hipError_t launch_ffn_passes(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx,
                             const int32_t *order, int T, int F, int tile_w, int cap, const void *x, const void *wu_t,
                             const void *wd, int d, float *y, void *ws, bool use_order_e, hipStream_t s);

// Decode-shaped calls (T <= DEC_MAX_T, bf16): gate into w.z, TwELL, overflow
// flags / list / count, work order, and the gather's chunking.
hipError_t launch_decode_gate_pack(const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                                   void *val, uint8_t *idx, int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows,
                                   int32_t *n_ovf, int32_t *order, int max_ovf, const DecodeWs &w, hipStream_t s);

// Decode-shaped FFN from the results of launch_decode_gate_pack: every row of
// y (overflow rows included), and the dense backup of the first
// min(n_ovf, max_ovf) overflow rows.
hipError_t launch_ffn_decode(const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F, int tile_w,
                             int cap, const void *x, const void *wu_t, const void *wd, int d, const int32_t *row_ovf,
                             const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf, void *dense, float *y,
                             const DecodeWs &w, hipStream_t s);

// Dense activations h [T][F] -> hybrid: TwELL (active iff h > 0), overflow
// flags / list / count, work order, dense backup rows max(h, 0).
hipError_t launch_dense_to_hybrid(int vdtype, const void *h, int T, int F, int tile_w, int cap, void *val,
                                  uint8_t *idx, int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows, int32_t *n_ovf,
                                  int32_t *order, int max_ovf, void *dense, hipStream_t s);

// Hybrid -> dense out [T][F]: every row from its TwELL slots, then the first
// min(n_ovf, max_ovf) overflow rows from the dense backup.
hipError_t launch_hybrid_to_dense(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                                  int tile_w, int cap, const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf,
                                  const void *dense, void *out, hipStream_t s);

// Compact form of the hybrid into buf (layout and header as in twell.h).
hipError_t launch_compact_hybrid(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx,
                                 const int32_t *row_ovf, const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf,
                                 const void *dense, int T, int F, int tile_w, int cap, void *buf, int64_t buf_bytes,
                                 hipStream_t s);

// Dense [T][F] from a compact buffer.
hipError_t launch_compact_to_dense(int vdtype, const void *buf, int T, int F, void *out, hipStream_t s);

// y[t] = sum of row t's partial rows part[c] (c in [chunk0[t], chunk0[t+1])),
// in chunk order.
hipError_t launch_chunk_reduce(const float *part, const int32_t *chunk0, int T, int d, float *y, hipStream_t s);

// Backward pass of the sparse FFN on the hybrid (arguments in backward.h).
hipError_t launch_ffn_backward(const BwArgs &a, hipStream_t s);

// Number of split-K slabs the hybrid down projection uses for these sizes.
int down_splits(int max_ovf, int F, int d);

}  // namespace twell
