/*
 * twell.h -- C ABI of libtwell: the ReLU-sparse gated FFN on MI355X
 * (gfx950), with its activations held in TwELL (tile-wise ELLPACK).
 *
 * Source of the method: "Sparser, Faster, Lighter Transformer Language Models"
 * (gist.science summary page).  Section 2.1 defines TwELL and its production
 * in the gate matmul's epilogue; section 2.2 the fused up/down inference
 * kernel; section 2.3 the hybrid ELL + dense-backup format for rows whose
 * nonzeros do not fit; section 2.4 the training side (conversions between the
 * hybrid and dense activations, the L1 penalty on the activations).  The page
 * gives no API; the calls below are this library's own:
 *   inference   twell_ffn_forward (the whole layer in one call),
 *               twell_ffn_from_gate (the layer after twell_pack_gate[_stats]),
 *               twell_pack_gate, twell_partition_overflow, twell_pack_gate_hybrid,
 *               twell_gate_dense (the gate with a plain dense epilogue),
 *               twell_ffn_fused, twell_ffn_overflow, twell_ffn_hybrid,
 *               twell_ffn_decode (T <= 64), twell_ffn_decode_noalloc
 *   statistics  twell_pack_gate_stats
 *   training    twell_dense_to_hybrid, twell_hybrid_to_dense,
 *               twell_compact_hybrid, twell_compact_to_dense, twell_ffn_backward
 *
 * Notation: T tokens (rows), d model width, F hidden width (d_ff), w tile
 * width, n_b = F / w tiles per row, cap = slots per (row, tile).
 *   z = x . W_g  (fp32 accumulation),  h_g = ReLU(z),  u = x . W_u,
 *   y = (h_g * u) . W_d                                  (y in fp32)
 *
 * Conventions shared by every call
 *   - Every pointer argument inside the structs and every x / weight / y
 *     pointer is DEVICE memory owned by the caller; the struct itself lives in
 *     host memory and is read during the call only.  The library never
 *     allocates, frees or synchronises: work is queued on `stream` (a
 *     hipStream_t; NULL = the default stream) and the call returns at once.
 *   - Layouts are row-major.  Weights come as W_g^T, W_u^T and W_d, each
 *     [F][d]: the three weight vectors of hidden neuron j are contiguous rows
 *     of d elements.  x is [T][d], y is [T][d] float.
 *   - Element type (vdtype) of x, the weights, TwELL values and the dense
 *     backup: TWELL_BF16 (bf16 inputs, fp32 accumulation) or TWELL_F32.
 *   - A gate value is active iff its fp32 accumulator is > 0 (0, -0 and NaN
 *     are inactive).  Inside a tile, entries appear in ascending column order.
 *     cnt holds the TRUE number of actives of a (row, tile), which may exceed
 *     cap; only the cap lowest columns are stored.  Slots at or past
 *     min(cnt, cap) hold value 0 and index 0.
 *   - Inputs must be finite, except that the bias column of W_g^T may hold
 *     -inf (a dead neuron: never active).
 *   - Errors the host can see return a negative status BEFORE anything is
 *     queued: NULL pointer, pointer not 16-byte aligned, bad shape, unsupported
 *     tile width / capacity / dtype, workspace too small.  A failed launch
 *     returns TWELL_E_HIP.  Overflow is data, not an error.
 *   - No C++ exception crosses this interface.  The library keeps no mutable
 *     global state, except the static scratch array of
 *     twell_ffn_decode_noalloc and its per-device address.  Concurrent calls
 *     on different streams are safe when their output and workspace buffers
 *     do not overlap (twell_ffn_decode_noalloc: see its own note).
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define TWELL_API __attribute__((visibility("default")))
#else
#define TWELL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum twell_status {
    TWELL_OK = 0,
    TWELL_E_NULL = -1,        /* a required pointer is NULL */
    TWELL_E_ALIGN = -2,       /* a device pointer is not 16-byte aligned */
    TWELL_E_SHAPE = -3,       /* T < 0, T*n_b too large, d % 64 != 0, F % tile_w != 0, ... */
    TWELL_E_UNSUPPORTED = -4, /* tile_w not in {32,64,128,256}, cap not in [1, tile_w], dtype */
    TWELL_E_HIP = -5,         /* the HIP runtime refused a launch */
    TWELL_E_WORKSPACE = -6,   /* workspace pointer NULL or smaller than required */
    TWELL_E_SCRATCH = -7      /* the call needs more than the static scratch array holds */
};

enum twell_dtype { TWELL_F32 = 0, TWELL_BF16 = 1 };

/* TwELL activations (section 2.1 of the page: per (row, tile) a count, packed
 * values and tile-local indices). */
typedef struct twell_t {
    int32_t T;      /* rows (tokens), >= 0 */
    int32_t F;      /* columns (hidden width), multiple of tile_w */
    int32_t tile_w; /* tile width w: 32, 64, 128 or 256 */
    int32_t cap;    /* slots per (row, tile): 1 <= cap <= tile_w */
    int32_t vdtype; /* enum twell_dtype of val (and of x and the weights) */
    int32_t reserved;
    void *val;      /* device [T][n_b][cap] activation values h_g, vdtype */
    uint8_t *idx;   /* device [T][n_b][cap] tile-local column 0..w-1 */
    int32_t *cnt;   /* device [T][n_b] true active count per (row, tile) */
} twell_t;

/* Hybrid ELL + dense backup (section 2.3 of the page).  A row is an overflow
 * row iff some tile of it has cnt > cap; such rows are listed in ascending
 * token order and their full h_g rows are kept densely. */
typedef struct twell_hybrid_t {
    twell_t ell;       /* TwELL of all rows */
    int32_t max_ovf;   /* rows available in ovf_rows / dense, >= 0 */
    int32_t reserved;
    int32_t *row_ovf;  /* device [T]: 1 for an overflow row, else 0 */
    int32_t *ovf_rows; /* device [max_ovf]: overflow rows, ascending */
    int32_t *n_ovf;    /* device [1]: number of overflow rows (may exceed max_ovf) */
    void *dense;       /* device [max_ovf][F] vdtype: h_g rows of the overflow tokens */
    int32_t *order;    /* device [T]: a permutation of the rows, the fused step's work
                          order (rows with more stored entries first) */
} twell_hybrid_t;

/* Gate GEMM with the TwELL epilogue (section 2.1 of the page: x . W_g, ReLU
 * and packing into TwELL done in the matmul's epilogue, with no separate
 * conversion pass).
 *   x    : device [h->T][d], vdtype h->vdtype
 *   wg_t : device [h->F][d], vdtype h->vdtype (column d-1 may hold -inf)
 *   d    : model width, multiple of 64
 *   h    : output TwELL; writes every element of h->cnt, h->val, h->idx.
 * Returns TWELL_OK or a negative twell_status. */
TWELL_API int twell_pack_gate(const void *x, const void *wg_t, int32_t d, const twell_t *h, void *stream);

/* The gate GEMM without the TwELL epilogue (section 2.1 of the page: the
 * gate activation ReLU(x . W_g) that TwELL encodes, here stored densely):
 *   h : device [T][F], vdtype, every element written with
 *       ReLU(z) rounded to nearest even (z the fp32 accumulator; the same
 *       values the dense backup holds), element-aligned.
 * The same GEMM core and tiles as twell_pack_gate, with a plain store
 * epilogue, so the difference between the two prices the TwELL packing; its
 * output is the dense activation twell_dense_to_hybrid takes.
 *   x : device [T][d], wg_t : device [F][d] (16-byte aligned), vdtype as
 *   enum twell_dtype; d and F multiples of 64.
 * Returns TWELL_OK or a negative twell_status. */
TWELL_API int twell_gate_dense(const void *x, const void *wg_t, int32_t d, int32_t T, int32_t F, int32_t vdtype,
                               void *h, void *stream);

/* twell_pack_gate plus activation statistics taken in the same epilogue
 * (section 2.4 of the page: the L1 penalty on the activations that training
 * adds, and the neurons it leaves dead).  Writes the same TwELL, and:
 *   neuron_cnt : device [h->F] int32, ADDED TO with atomics: per neuron j,
 *                the number of rows t with (x . W_g)[t][j] > 0.  Zero it
 *                before the first call; calls accumulate, so a neuron still at
 *                0 after a set of calls is dead on all their rows.  The caller
 *                keeps the accumulated rows under 2^31.
 *   l1         : device [h->T][h->F / h->tile_w] float, overwritten: per
 *                (row, tile), the sum of the positive gate values of the tile
 *                (fp32 accumulators, before rounding to vdtype), added in a
 *                fixed order, so repeated calls give the same bits.  The L1
 *                term of a row is the sum of its tiles.
 * Both 4-byte aligned.  Returns TWELL_OK or a negative twell_status. */
TWELL_API int twell_pack_gate_stats(const void *x, const void *wg_t, int32_t d, const twell_t *h,
                                    int32_t *neuron_cnt, float *l1, void *stream);

/* Overflow partition and dense backup (section 2.3 of the page): from
 * hy->ell.cnt (written by twell_pack_gate) computes row_ovf, the ascending
 * ovf_rows list and n_ovf, then recomputes ReLU(x . W_g) for the first
 * min(n_ovf, max_ovf) overflow rows into hy->dense.  Rows past max_ovf are
 * counted in n_ovf but get no dense row: the caller checks n_ovf <= max_ovf
 * after synchronising and retries with larger buffers otherwise.
 * Also writes hy->order: the rows grouped by their number of stored entries
 * e = sum over tiles of min(cnt, cap) (e = 0 for overflow rows) into the
 * classes e >= 256, 192..255, 128..191, 64..127, 32..63, 16..31, 1..15, 0,
 * heaviest class first and ascending rows inside a class (per chunk of
 * 16384 rows).  It is a schedule only: no result depends on it. */
TWELL_API int twell_partition_overflow(const void *x, const void *wg_t, int32_t d,
                             const twell_hybrid_t *hy, void *stream);

/* The hybrid ELL + dense-backup activation in one call (sections 2.1 and
 * 2.3 of the page: TwELL packed in the gate's epilogue, then the rows whose
 * tiles overflow the capacity moved to a dense backup): twell_pack_gate on
 * hy->ell followed by twell_partition_overflow, with their arguments, checks
 * and outputs.  Needs no workspace: every output is one of hy's arrays. */
TWELL_API int twell_pack_gate_hybrid(const void *x, const void *wg_t, int32_t d,
                           const twell_hybrid_t *hy, void *stream);

/* Fused up/down projection from TwELL (section 2.2 of the page): for every
 * row and every stored entry (b, s), j = b*w + idx:  u = x[t] . W_u^T[j]
 * (fp32), y[t] += (val * u) * W_d[j] (fp32).  Only the kept rows of W_u^T
 * and W_d are read.  Rows with some cnt > cap (overflow rows) get y = 0;
 * rows without actives get y = 0.
 *   x, wu_t, wd : device, vdtype h->vdtype;  y : device [h->T][d] float.
 *   order : optional device [h->T] permutation of 0..T-1 (as written by
 *           twell_partition_overflow): rows are started in that order, so the
 *           heavy ones do not trail at the end; NULL = ascending rows.  Each
 *           row's result is the same bits for any order; a non-permutation
 *           leaves some rows unwritten (entries are range-checked).
 *   workspace : device, >= twell_workspace_bytes(T, F, tile_w, cap, 0, d,
 *           vdtype) (it holds each stored entry's partial dot products
 *           x[t] . W_u^T[j] over 8 column slices of d, from the up pass to
 *           the down pass), 256-byte aligned, content ignored on entry. */
TWELL_API int twell_ffn_fused(const twell_t *h, const int32_t *order, const void *x, const void *wu_t,
                              const void *wd, int32_t d, float *y, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Bytes of device workspace that twell_ffn_fused (with max_ovf = 0),
 * twell_ffn_overflow, twell_ffn_hybrid, twell_ffn_forward and
 * twell_ffn_from_gate need for these sizes: T * (F / tile_w) * cap * nch
 * floats for the fused step's partial dot products (nch = 8 column slices
 * of d when d is a multiple of 512 (bf16) or 256 (fp32); d / 64 when d is
 * smaller; more for other widths), plus, when max_ovf > 0, the overflow
 * rows' gated products and split-K partial sums.  One workspace of
 * this size serves every one of these calls.  Returns 0 for invalid sizes. */
TWELL_API size_t twell_workspace_bytes(int32_t T, int32_t F, int32_t tile_w, int32_t cap, int32_t max_ovf,
                                       int32_t d, int32_t vdtype);

/* Dense part of the hybrid FFN (section 2.3 of the page): for the first
 * min(n_ovf, max_ovf) overflow rows r = ovf_rows[i], writes
 * y[r] = (dense[i] * (x[r] . W_u)) . W_d, the gated product rounded to
 * vdtype before the down projection (fp32 accumulation).  Other y rows are
 * not touched.  Expects hy filled by twell_pack_gate_hybrid on the same
 * stream.  workspace: device, >= twell_workspace_bytes(T, F, tile_w, cap,
 * max_ovf, d, vdtype), 256-byte aligned, content ignored on entry. */
TWELL_API int twell_ffn_overflow(const twell_hybrid_t *hy, const void *x, const void *wu_t, const void *wd,
                       int32_t d, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* Hybrid FFN (sections 2.2 and 2.3 of the page: the fused up/down step over
 * the sparse part, the dense FFN over the dense backup's rows):
 * twell_ffn_fused for all rows in hy->order (overflow rows get 0), then
 * twell_ffn_overflow for the overflow rows; every row of y is the full FFN
 * output when n_ovf <= max_ovf.  Expects hy filled by twell_pack_gate_hybrid
 * on the same stream.  workspace: as twell_ffn_overflow's (it serves both
 * steps); y : device [T][d] float. */
TWELL_API int twell_ffn_hybrid(const twell_hybrid_t *hy, const void *x, const void *wu_t, const void *wd,
                     int32_t d, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* The whole layer in one call (sections 2.1-2.3 of the page): the hybrid of
 * the gate activation (as twell_pack_gate_hybrid writes it: TwELL, row_ovf,
 * ovf_rows, n_ovf, order, dense backup) and y (as twell_ffn_hybrid writes it),
 * bit for bit the same as those two calls.  The dense backup and the
 * overflow rows' up projection come from one GEMM over the gathered x rows
 * (W_g^T and W_u^T tiles side by side) instead of two.
 *   x, wg_t, wu_t, wd : device, vdtype hy->ell.vdtype, 16-byte aligned;
 *   y : device [T][d] float; workspace: device, >=
 *   twell_workspace_bytes(T, F, tile_w, cap, max_ovf, d, vdtype), 256-byte
 *   aligned, content ignored on entry.
 *   Every check is made before the first launch. */
TWELL_API int twell_ffn_forward(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                      const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes,
                      void *stream);

/* twell_ffn_forward without its first step: hy->ell holds the TwELL of
 * x . W_g already (twell_pack_gate or twell_pack_gate_stats on the same
 * stream); writes the rest of the hybrid and y.  Same arguments and checks;
 * twell_ffn_forward = twell_pack_gate + twell_ffn_from_gate. */
TWELL_API int twell_ffn_from_gate(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                        const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Dense activations to the hybrid (section 2.4 of the page: the conversion
 * kernels training uses in the forward and backward passes).  h : device
 * [T][F], vdtype hy->ell.vdtype, row-major, 16-byte aligned.  Writes the
 * TwELL of h (an entry is active iff h > 0: 0, -0, negatives and NaN are not;
 * the same packing rules as twell_pack_gate), row_ovf, ovf_rows, n_ovf,
 * order (as twell_partition_overflow), and dense[i] = max(h[ovf_rows[i]], 0)
 * for the first min(n_ovf, max_ovf) overflow rows.  The hybrid of a
 * non-negative h with every overflow row served holds h exactly. */
TWELL_API int twell_dense_to_hybrid(const void *h, const twell_hybrid_t *hy, void *stream);

/* The hybrid to dense activations (section 2.4 of the page).  out : device
 * [T][F], vdtype hy->ell.vdtype, 16-byte aligned, every element written: each
 * row holds its kept TwELL entries and zeros elsewhere, except the first
 * min(n_ovf, max_ovf) overflow rows, which are their dense backup rows
 * (later overflow rows keep only their TwELL entries: the hybrid holds
 * nothing more of them).  Expects hy as written by twell_dense_to_hybrid,
 * twell_pack_gate_hybrid or twell_ffn_decode. */
TWELL_API int twell_hybrid_to_dense(const twell_hybrid_t *hy, void *out, void *stream);

/* Compacted hybrid storage (section 2.3 of the page: the rows with few
 * nonzeros kept in a compact sparse part, the overflow rows densely, memory
 * sized by what the rows need).  TwELL pads every tile to cap slots; the
 * compact form keeps exactly the entries of the rows that fit.  It lives in
 * one device buffer laid out as
 *   [0, 256)                  twell_compact_header_t
 *   off_row_ptr               int32 [T + 1]: row t's entries are [row_ptr[t], row_ptr[t+1])
 *   off_col                   uint16 [n_entries]: global column, ascending within a row
 *   off_val                   vdtype [n_entries]
 *   off_ovf                   int32 [n_dense]: ids of the overflow rows held densely
 *   off_dense                 vdtype [n_dense][F]
 * (sections 256-byte aligned).  Overflow rows have no compact entries; the
 * first n_dense = min(n_ovf, max_ovf) of them are held densely.  The layout
 * depends on counts only the device knows, so the header is written on the
 * device: read it after the call to learn `bytes`. */
typedef struct twell_compact_header_t {
    int32_t T, F, tile_w, vdtype;
    int32_t n_entries;  /* entries of the rows that fit */
    int32_t n_ovf;      /* overflow rows */
    int32_t n_dense;    /* overflow rows held densely = min(n_ovf, max_ovf) */
    int32_t fits;       /* 1: the buffer held everything; 0: only the header and row_ptr were written */
    int64_t off_row_ptr, off_col, off_val, off_ovf, off_dense;
    int64_t bytes;      /* bytes the compact form needs */
} twell_compact_header_t;

/* Bytes every compact buffer needs before its variable part: the header and
 * the row offsets (written even when the rest does not fit). */
TWELL_API size_t twell_compact_min_bytes(int32_t T);

/* Write the compact form of a hybrid (as written by twell_pack_gate_hybrid,
 * twell_dense_to_hybrid or twell_ffn_decode) into buf (device, 256-byte
 * aligned, buf_bytes >= twell_compact_min_bytes(T)).  When buf_bytes is
 * smaller than the header's `bytes`, fits = 0 and only the header and the row
 * offsets are written: call again with a buffer of `bytes`.  Requires
 * F <= 65536 and F / tile_w <= 512. */
TWELL_API int twell_compact_hybrid(const twell_hybrid_t *hy, void *buf, size_t buf_bytes, void *stream);

/* Dense activations from a compact buffer: out : device [T][F] vdtype,
 * 16-byte aligned, every element written (zeros where nothing is held; all
 * zeros when the header says fits = 0 or its T, F differ from the
 * arguments). */
TWELL_API int twell_compact_to_dense(const void *buf, int32_t T, int32_t F, int32_t vdtype, void *out, void *stream);

/* Bytes of device workspace twell_ffn_decode needs for these sizes (0 when
 * the sizes are outside its range).  For T <= 16 it holds a partial y row
 * per (row, group of 32 neurons): T * (F / 32) * d floats, plus z. */
TWELL_API size_t twell_ffn_decode_workspace_bytes(int32_t T, int32_t F, int32_t d, int32_t tile_w);

/* The whole FFN for decode-shaped calls, T <= 64 rows, bf16 (sections
 * 2.1-2.3 of the page: the same gate, TwELL, overflow partition and fused
 * up/down, organised for a few tokens: the gate spread over F/32
 * workgroups).  For T <= 16 each gate workgroup does the up/down work of its
 * own 32 neurons as soon as their gate values are known, and a second kernel
 * adds the partial rows while it packs TwELL; for larger T every row's
 * entries are cut into chunks shared out over the GPU.  Writes everything
 * twell_pack_gate_hybrid writes (TwELL, row_ovf, ovf_rows, n_ovf, the dense
 * backup of the first min(n_ovf, max_ovf) overflow rows, order) and every row
 * of y, overflow rows included (whatever max_ovf is): y[t] = sum over t's
 * active neurons j of (h * (x[t] . W_u^T[j])) * W_d[j], h the stored bf16
 * gate value, in fp32, summed in a fixed order (which depends on T).  Same
 * bits for repeated calls.
 *   x : device [T][d] bf16; wg_t, wu_t, wd : device [F][d] bf16; y : [T][d] float.
 *   hy : T <= 64, vdtype TWELL_BF16, T * F <= 2^20, F / tile_w <= 512.
 *   workspace : device, >= twell_ffn_decode_workspace_bytes(T, F, d, tile_w),
 *               256-byte aligned, content ignored on entry.
 * Returns TWELL_OK, TWELL_E_UNSUPPORTED outside that range, or another
 * negative twell_status. */
TWELL_API int twell_ffn_decode(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                               const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes,
                               void *stream);

/* twell_ffn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus the workspace) and
 * checks as twell_ffn_decode, and the same kernels when their scratch fits:
 * for T <= 16 the two-kernel organisation if its T * F / 32 partial rows of
 * d floats fit, else (and for T > 16) the chunked kernels.  TwELL, the
 * partition, the order and the dense backup are always the same bits as
 * twell_ffn_decode's; y too when both take the same kernels, else the same
 * sums in another order.
 * Its scratch is a 16 MiB array in the library's device code: each GPU the
 * library runs on holds one copy from the first call on it until the process
 * ends.  The first call on a device looks up that copy's address
 * (hipGetSymbolAddress) and keeps it; no call allocates or frees anything.
 * Every call on one GPU uses the same copy and finds there whatever the last
 * call left; what must start at zero is cleared by the call's own kernels.
 * Calls that overlap in time on one GPU (e.g. on two streams) race on the
 * scratch: serialise them.
 * Limit: one of the two scratch layouts must fit 16 MiB: for T <= 16,
 * T * F fp32 values of z plus T * F / 32 partial rows of d floats (and
 * T * F / 32 flags), or for any T, T * F values of z plus (1024 + T) partial
 * rows of d floats (and a few KiB of tables).  The second holds every shape
 * twell_ffn_decode accepts with d <= 2048; when neither fits the call returns
 * TWELL_E_SCRATCH before anything is queued. */
TWELL_API int twell_ffn_decode_noalloc(const void *x, const void *wg_t, const void *wu_t, const void *wd,
                                       int32_t d, const twell_hybrid_t *hy, float *y, void *stream);

/* Bytes of device workspace twell_ffn_backward needs for these sizes (0 when
 * they are invalid). */
TWELL_API size_t twell_ffn_backward_workspace_bytes(int32_t T, int32_t F, int32_t d, int32_t max_entries);

/* Backward pass of the sparse FFN on its hybrid (section 2.4 of the page: the
 * forward and backward passes of training run on the hybrid).  For
 * y = sum over the active neurons j of row t of h (x[t] . W_u^T[j]) W_d[j],
 * with h the stored gate value and ReLU's derivative 1 on active entries,
 * given dy = dL/dy it writes
 *   dx [T][d], dwg = dL/dW_g^T, dwu = dL/dW_u^T, dwd = dL/dW_d ([F][d]),
 * all float, overwritten (neurons without entries get zero rows).  The active
 * entries are a fitting row's TwELL entries and a held overflow row's nonzero
 * dense-backup values; an overflow row past max_ovf has no dense row and
 * contributes nothing (its dx row is 0).  Per entry: u = x . W_u^T[j],
 * g = dy . W_d[j] (fp32), du = g h, dz = g u; every sum in a fixed order, so
 * repeated calls give the same bits.
 *   hy : as written by twell_pack_gate_hybrid / twell_dense_to_hybrid /
 *        twell_ffn_decode, vdtype TWELL_BF16, d <= 2048, F / tile_w <= 512;
 *   x, wg_t, wu_t, wd : the forward's inputs (bf16); dy : device [T][d] float;
 *   max_entries : bound on the active entries the workspace holds;
 *   workspace : >= twell_ffn_backward_workspace_bytes(T, F, d, max_entries),
 *               256-byte aligned.  Its first 8 bytes hold, after the call,
 *               int32 entries and int32 too_many: when entries > max_entries
 *               nothing is computed and every output is zero.
 * Returns TWELL_OK or a negative twell_status. */
TWELL_API int twell_ffn_backward(const twell_hybrid_t *hy, const void *x, const void *wg_t, const void *wu_t,
                                 const void *wd, int32_t d, const float *dy, float *dx, float *dwg, float *dwu,
                                 float *dwd, int32_t max_entries, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Static text for a status code. */
TWELL_API const char *twell_status_str(int status);

/* Library ABI version (major * 100 + minor). */
TWELL_API int twell_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
