// ffn_fused.hip -- fused up/down projection straight from TwELL.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.2: with the gate activation h_g in TwELL, the up and
// down projections become one step that, for each nonzero h_g[j], reads
// only the weights it needs (column j of W_u, row j of W_d), takes a dot
// product and a scalar product, and accumulates -- DRAM traffic is the point.
//
// gfx950 mapping (batch path): two passes, each arranged so that one XCD
// gathers only weight rows that fit its L2 (see "batch path" below); every
// weight row, x row and partial sum is moved with 16-byte-per-lane coalesced
// loads, dot products are reduced with DPP, and all sums run in a fixed order
// (no atomics), so the result does not depend on timing.  The decode path
// (T <= 64) keeps one wave per chunk of a row's entries, with both weight
// rows of an entry in registers (group_load / group_apply below).
#include <algorithm>

#include "decode.h"
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

namespace twell {

// The token's x row as this lane's chunks in fp32 registers.
template <typename TI, int NC> struct XRow {
    float f[NC][Elt<TI>::PER_CHUNK];
    __device__ __forceinline__ void set(int c, const u32x4 &v)
    {
#pragma unroll
        for (int e = 0; e < Elt<TI>::PER_CHUNK; ++e)
            f[c][e] = chunk_elem<TI>(v, e);
    }
    __device__ __forceinline__ float get(int c, int e) const { return f[c][e]; }
};

template <typename TI> struct FusedArgs {
    const int32_t *cnt;
    const TI *val;
    const uint8_t *idx;
    const int32_t *order;  // row of workgroup i (null: row i)
    int T, n_b, tile_w, cap, F;
    const TI *x, *wu_t, *wd;
    int d, nchunks;  // nchunks = 16-byte chunks per row
    float *y;
};

// Weight rows of G list entries in registers.
template <typename TI, int NC, int G> struct Group {
    u32x4 wu[G][NC], wv[G][NC];
    float h[G];
};

// Request the W_u^T and W_d rows of entries e0 .. e0+G-1.
template <typename TI, int NC, int G>
__device__ __forceinline__ void group_load(const FusedArgs<TI> &a, const int2 *list, int e0, int lane,
                                           int64_t row_bytes, Group<TI, NC, G> &g)
{
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const int2 en = list[e0 + k];
        const int j = __builtin_amdgcn_readfirstlane(en.x);
        g.h[k] = __int_as_float(__builtin_amdgcn_readfirstlane(en.y));
        const char *pu = (const char *)a.wu_t + (int64_t)j * row_bytes;
        const char *pd = (const char *)a.wd + (int64_t)j * row_bytes;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = lane + 64 * c;
            const bool ok = ch < a.nchunks;
            g.wu[k][c] = ok ? ldg16(pu + ch * 16) : u32x4{0, 0, 0, 0};
            g.wv[k][c] = ok ? ldg16(pd + ch * 16) : u32x4{0, 0, 0, 0};
        }
    }
}

// y += (h * (x . W_u^T[j])) * W_d[j] for the entries of a loaded group.
// Each dot product sums over chunks, then elements, in order.
template <typename TI, int NC, int G>
__device__ __forceinline__ void group_apply(const Group<TI, NC, G> &g, const XRow<TI, NC> &xr,
                                            float (&yacc)[NC][Elt<TI>::PER_CHUNK])
{
    constexpr int E = Elt<TI>::PER_CHUNK;
    float part[G];
#pragma unroll
    for (int k = 0; k < G; ++k)
        part[k] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < G; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                part[k] = fmaf(xr.get(c, e), chunk_elem<TI>(g.wu[k][c], e), part[k]);
#pragma unroll
    for (int k = 0; k < G; ++k)
        part[k] = wave_sum(part[k]);
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const float sc = g.h[k] * part[k];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < E; ++e)
                yacc[c][e] = fmaf(sc, chunk_elem<TI>(g.wv[k][c], e), yacc[c][e]);
    }
}

// This wave's groups q = q0, q0 + step, ... < ngroups, in order, with the next
// group's rows requested before the current group is reduced.
template <typename TI, int NC, int G>
__device__ __forceinline__ void group_stream(const FusedArgs<TI> &a, const int2 *list, int q0, int step, int ngroups,
                                             int lane, int64_t row_bytes, const XRow<TI, NC> &xf,
                                             float (&yacc)[NC][Elt<TI>::PER_CHUNK])
{
    Group<TI, NC, G> ga, gb;
    int q = q0;
    if (q < ngroups)
        group_load<TI, NC, G>(a, list, q * G, lane, row_bytes, ga);
    while (q < ngroups) {
        if (q + step < ngroups)
            group_load<TI, NC, G>(a, list, (q + step) * G, lane, row_bytes, gb);
        group_apply<TI, NC, G>(ga, xf, yacc);
        q += step;
        if (q >= ngroups)
            break;
        if (q + step < ngroups)
            group_load<TI, NC, G>(a, list, (q + step) * G, lane, row_bytes, ga);
        group_apply<TI, NC, G>(gb, xf, yacc);
        q += step;
    }
}

// ------------------------------------------------------------------ batch path
// Three kernels.
//
// Entries (ffn_entries_kernel), one wave per row t: the row's stored entries
// (j, h) in ascending (tile, slot) order, packed at the start of the row's own
// range of TwELL slots (ent[t n_b cap + k], k < e_t), and e_t (0 for an
// overflow row), so that the passes below need one round of dependent loads
// per row instead of reading counts, then indices and values, per column
// slice.  In the one-call path it also writes the overflow flag and work value
// (row_ovf, work) the partition's compaction reads.
//
// Up and down passes (ffn_pass_kernel), split over the columns of d: a
// workgroup serves one column slice [c cw, (c + 1) cw) (cw = d / nch, nch = 8
// column slices at the usual widths), and workgroups are handed to the 8 XCDs
// round-robin (workgroup g runs on XCD g % 8), so XCD c only ever reads
// column slice c of x, W_u^T and W_d: the live rows' slices of one weight
// matrix (3.4 MB at the 2B shape) stay in its 4 MB L2.  A wave takes
// PASS_ROWS rows at work positions strided across the work order (w, w + W,
// ...: the heaviest rows, which lead the order, land in different waves),
// learns their entry counts in one round of loads, skips the empty ones and
// runs the others in turn, requesting the next row's entries before the
// current row's weight stream.  A row slice is LPE 16-byte pieces: the lanes
// take 64 / LPE entries per step, LPE lanes per entry and one piece per lane.
// The up pass keeps the lane's piece of x[t] in registers and writes, per
// entry, the partial dot product of x[t] and W_u^T[j] over the slice (bf16:
// v_dot2_f32_bf16, two products per instruction; DPP reduction over the
// entry's lanes) to p[c][slot] (fp32; slice-major, so one
// XCD's writes for consecutive entries share cache lines).  The down pass
// forms s = h * (p[0][slot] + ... + p[nch - 1][slot]) (fixed order) and
// accumulates y[t][slice] += s * W_d[j] in the lanes' registers, each lane its
// entries in ascending order, the lane groups then added by a fixed
// butterfly.  Every value comes from one wave in a fixed order, so the result
// does not depend on timing.  Overflow rows, and rows without entries, get
// y = 0 (the dense path writes the overflow rows afterwards).
template <typename TI> struct PassArgs {
    const int32_t *cnt;
    const TI *val;
    const uint8_t *idx;
    const int32_t *order;  // row of work position i (null: row i)
    int T, n_b, tile_w, cap, F;
    const TI *x, *wu_t, *wd;
    int d;
    FusedWs w;
    float *y;
    int cw;                   // width of a column slice (d = w.nch * cw)
    int32_t *row_ovf, *work;  // optional (one-call path): overflow flag, work value
    const int32_t *order_e;   // optional: entry counts in work order (else row_e[order[i]])
};

constexpr int PASS_WAVES = 4;
#ifndef PASS_STEPS
#define PASS_STEPS 8
#endif
#ifndef PASS_PREFETCH
#define PASS_PREFETCH 1
#endif
constexpr int PASS_U = PASS_STEPS;  // entry steps in flight per lane

template <typename TI>
__global__ __launch_bounds__(64 * PASS_WAVES) void ffn_entries_kernel(PassArgs<TI> a)
{
    constexpr int E = Elt<TI>::PER_CHUNK;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * PASS_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T)
        return;
    const int32_t *crow = a.cnt + (int64_t)t * a.n_b;
    bool ovf = false;
    for (int b0 = 0; b0 < a.n_b; b0 += 64) {
        const int b = b0 + lane;
        ovf |= __ballot(b < a.n_b && crow[b] > a.cap) != 0ull;
    }
    const int64_t rbase = (int64_t)t * a.n_b * a.cap;
    int2 *erow = a.w.ent + rbase;
    int run = 0;
    if (!ovf) {
        const bool vec = a.cap % 16 == 0 && (reinterpret_cast<uintptr_t>(a.idx) & 15u) == 0 &&
                         (reinterpret_cast<uintptr_t>(a.val) & 15u) == 0;
        for (int b0 = 0; b0 < a.n_b; b0 += 64) {
            const int b = b0 + lane;
            int c = b < a.n_b ? crow[b] : 0;
            c = c < a.cap ? c : a.cap;
            const int incl = wave_incl_scan(c, lane);
            const int excl = run + incl - c;
            run += __shfl(incl, 63, 64);
            const int64_t slot0 = rbase + (int64_t)b * a.cap;
            if (vec) {
                for (int s0 = 0; s0 < c; s0 += 16) {
                    const u32x4 iw = ldg16(a.idx + slot0 + s0);
                    u32x4 vw[16 / E];
#pragma unroll
                    for (int q = 0; q < 16 / E; ++q)
                        vw[q] = ldg16(a.val + slot0 + s0 + q * E);
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        if (s0 + k < c) {
                            int j = b * a.tile_w + (int)((iw[k >> 2] >> (8 * (k & 3))) & 0xFFu);
                            j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
                            erow[excl + s0 + k] = make_int2(j, __float_as_int(chunk_elem<TI>(vw[k / E], k % E)));
                        }
                    }
                }
            } else {
                for (int s = 0; s < c; ++s) {
                    int j = b * a.tile_w + a.idx[slot0 + s];
                    j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
                    erow[excl + s] = make_int2(j, __float_as_int(load_elem(a.val + slot0 + s)));
                }
            }
        }
    }
    if (lane == 0) {
        a.w.row_e[t] = run;
        if (a.row_ovf) {
            a.row_ovf[t] = ovf;
            a.work[t] = run;
        }
    }
}

// x . w over the 8 bf16 elements of two 16-byte pieces, two products and the
// running sum per v_dot2_f32_bf16, pairs in ascending element order.  (The
// pairs are taken by shuffles of the whole piece: bit-casting a subscripted
// element of the 4 x u32 vector made the compiler read element 0 for all four.)
__device__ __forceinline__ float dot8_bf16(const u32x4 &x, const u32x4 &w)
{
    const bf16x8 xb = __builtin_bit_cast(bf16x8, x), wb = __builtin_bit_cast(bf16x8, w);
    float p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(xb, xb, 0, 1),
                                              __builtin_shufflevector(wb, wb, 0, 1), 0.f, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(xb, xb, 2, 3), __builtin_shufflevector(wb, wb, 2, 3), p,
                                        false);
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(xb, xb, 4, 5), __builtin_shufflevector(wb, wb, 4, 5), p,
                                        false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(xb, xb, 6, 7),
                                           __builtin_shufflevector(wb, wb, 6, 7), p, false);
}

// Sum of v over each aligned group of L lanes (L = 8, 16, 32, 64), left in
// the group's last lane (DPP row shifts, then row broadcasts).
template <int L> __device__ __forceinline__ float group_sum_last(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
    if (L >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
    if (L >= 32)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
    if (L >= 64)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return v;
}

// One row's window of up to 64 entries (k = w0 + lane), as (j, payload):
// up pass payload = slot; down pass payload = s = h * (sum of the entry's
// partial dot products).  x piece: the up pass's lane piece of x[t].
template <typename TI, bool DOWN> struct RowWin {
    int2 en;
    uint32_t off;  // byte offset of entry k's weight row, j * d * sizeof(TI) (< 2^32 by the host checks)
    float pv[DOWN ? 8 : 1];
    u32x4 xv;
};

template <typename TI, bool DOWN>
__device__ __forceinline__ void row_win_load(const PassArgs<TI> &a, int t, int e, int w0, int lane, int64_t col_off,
                                             RowWin<TI, DOWN> &r)
{
    const int slots = a.n_b * a.cap;
    const int64_t rbase = (int64_t)t * slots;
    const int k = w0 + lane;
    const bool ok = k < e;
    r.en = ok ? a.w.ent[rbase + k] : make_int2(0, 0);
    r.off = (uint32_t)r.en.x * (uint32_t)(a.d * Elt<TI>::SIZE);
    if (DOWN) {
        if (a.w.nch == 8) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                r.pv[c] = ok ? a.w.p[c * a.w.pstride + rbase + k] : 0.f;
        }
    } else if (w0 == 0) {
        r.xv = ldg16((const char *)a.x + (int64_t)t * a.d * Elt<TI>::SIZE + col_off);
    }
}

#ifndef PASS_NROWS
#define PASS_NROWS 2
#endif
constexpr int PASS_ROWS = PASS_NROWS;  // consecutive work positions per wave

template <typename TI, int LPE, bool DOWN>
__global__ __launch_bounds__(64 * PASS_WAVES) void ffn_pass_kernel(PassArgs<TI> a)
{
    constexpr int E = Elt<TI>::PER_CHUNK;  // elements per 16-byte piece
    constexpr int EPI = 64 / LPE;          // entries per step
    constexpr bool BF16 = sizeof(TI) == 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = a.w.nch;
    const int csl = blockIdx.x % nch;
    // the wave's rows: work positions w, w + W, w + 2 W, ... (W waves per
    // slice), so that the heaviest rows, which lead the work order, land in
    // different waves; lane r < PASS_ROWS holds row r and its entry count
    const int nwv = (a.T + PASS_ROWS - 1) / PASS_ROWS;
    const int wv0 = (blockIdx.x / nch) * PASS_WAVES + wave;
    if (wv0 >= nwv)
        return;
    const int ip = wv0 + lane * nwv;
    int tv = -1, ev = 0;
    if (lane < PASS_ROWS && ip < a.T) {
        tv = a.order ? a.order[ip] : ip;
        if (a.order_e)
            ev = a.order_e[ip];  // the same round of loads as the row
        tv = (unsigned)tv < (unsigned)a.T ? tv : -1;  // not a permutation: not ours to write
    }
    if (tv >= 0 && !a.order_e)
        ev = a.w.row_e[tv];
    // row r of the wave: tr(r), er(r) (scalar reads of lane r)
#define tr(r) __builtin_amdgcn_readlane(tv, (r))
#define er(r) __builtin_amdgcn_readlane(ev, (r))
    const int q = lane / LPE, pc = lane % LPE;  // entry of the step, 16-byte piece of the row slice
    const int64_t col_off = (int64_t)(csl * a.cw + pc * E) * Elt<TI>::SIZE;
    // weight rows: a base uniform over the workgroup (its slice) plus a 32-bit
    // per-lane offset (entry row + the lane's piece), one VGPR add per load
    const char *wbase = (const char *)(DOWN ? a.wd : a.wu_t) + (int64_t)csl * a.cw * Elt<TI>::SIZE;
    const uint32_t piece_off = (uint32_t)(pc * 16);
    const int slots = a.n_b * a.cap;
    // first row with entries, its first window requested at once
    int r = 0;
    while (r < PASS_ROWS && (tr(r) < 0 || er(r) == 0)) {
        if (DOWN && tr(r) >= 0 && er(r) == 0) {
            float *yrow = a.y + (int64_t)tr(r) * a.d + csl * a.cw;
            for (int k = lane * 4; k < a.cw; k += 256)
                *reinterpret_cast<float4 *>(yrow + k) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        ++r;
    }
    if (r == PASS_ROWS)
        return;
    RowWin<TI, DOWN> cur;
    row_win_load<TI, DOWN>(a, tr(r), er(r), 0, lane, col_off, cur);
    while (r < PASS_ROWS) {
        const int t = tr(r), e = er(r);
        const int64_t rbase = (int64_t)t * slots;
        float xf[E], acc[E];
        const u32x4 xr = cur.xv;  // bf16: x pairs for the packed dot products
        if (!DOWN && !BF16) {
#pragma unroll
            for (int e2 = 0; e2 < E; ++e2)
                xf[e2] = chunk_elem<TI>(cur.xv, e2);
        }
#pragma unroll
        for (int e2 = 0; e2 < E; ++e2)
            acc[e2] = 0.f;
        // the next row with entries (zero-filling the empty ones on the way, down pass)
        int rn = r + 1;
        while (rn < PASS_ROWS && (tr(rn) < 0 || er(rn) == 0)) {
            if (DOWN && tr(rn) >= 0 && er(rn) == 0) {
                float *yrow = a.y + (int64_t)tr(rn) * a.d + csl * a.cw;
                for (int k = lane * 4; k < a.cw; k += 256)
                    *reinterpret_cast<float4 *>(yrow + k) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            ++rn;
        }
        for (int w0 = 0; w0 < e; w0 += 64) {
            if (w0 > 0)
                row_win_load<TI, DOWN>(a, t, e, w0, lane, col_off, cur);
            float sv = 0.f;
            if (DOWN) {
                float u = 0.f;
                if (nch == 8) {
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        u += cur.pv[c];
                } else if (w0 + lane < e) {
                    for (int c = 0; c < nch; ++c)
                        u += a.w.p[c * a.w.pstride + rbase + w0 + lane];
                }
                sv = __int_as_float(cur.en.y) * u;
            }
            const int n = e - w0 < 64 ? e - w0 : 64;
            // the next row's first window, requested before this window's weight stream
            RowWin<TI, DOWN> nxt;
            if (PASS_PREFETCH && w0 + 64 >= e && rn < PASS_ROWS)
                row_win_load<TI, DOWN>(a, tr(rn), er(rn), 0, lane, col_off, nxt);
            for (int k0 = 0; k0 < n; k0 += EPI * PASS_U) {
                // (a fresh zero for lanes past the window's end: keeping the
                // registers across steps and skipping those loads instead was
                // 25% slower, the steps' loads then waiting on each other)
                u32x4 wv[PASS_U];
                float sc[PASS_U];
#pragma unroll
                for (int u = 0; u < PASS_U; ++u) {
                    const int kk = k0 + u * EPI + q;
                    const uint32_t oj = (uint32_t)__shfl((int)cur.off, kk, 64);
                    sc[u] = DOWN ? __shfl(sv, kk, 64) : 0.f;
                    wv[u] = kk < n ? ldg16(wbase + (oj + piece_off)) : u32x4{0, 0, 0, 0};
                }
                if (DOWN) {
#pragma unroll
                    for (int u = 0; u < PASS_U; ++u) {
                        if (k0 + u * EPI + q < n) {
#pragma unroll
                            for (int e2 = 0; e2 < E; ++e2)
                                acc[e2] = fmaf(sc[u], chunk_elem<TI>(wv[u], e2), acc[e2]);
                        }
                    }
                } else {
                    float part[PASS_U];
#pragma unroll
                    for (int u = 0; u < PASS_U; ++u) {
                        part[u] = 0.f;
                        if constexpr (BF16) {
                            part[u] = dot8_bf16(xr, wv[u]);
                        } else {
#pragma unroll
                            for (int e2 = 0; e2 < E; ++e2)
                                part[u] = fmaf(xf[e2], chunk_elem<TI>(wv[u], e2), part[u]);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < PASS_U; ++u)
                        part[u] = group_sum_last<LPE>(part[u]);
                    if (pc == LPE - 1) {
#pragma unroll
                        for (int u = 0; u < PASS_U; ++u) {
                            const int kk = k0 + u * EPI + q;
                            if (kk < n)
                                a.w.p[csl * a.w.pstride + rbase + w0 + kk] = part[u];
                        }
                    }
                }
            }
            if (PASS_PREFETCH && w0 + 64 >= e && rn < PASS_ROWS)
                cur = nxt;
        }
        if (DOWN) {
            // the EPI lane groups hold partial sums of the same columns: fixed butterfly
#pragma unroll
            for (int m = LPE; m < 64; m <<= 1)
#pragma unroll
                for (int e2 = 0; e2 < E; ++e2)
                    acc[e2] += __shfl_xor(acc[e2], m, 64);
            if (q == 0) {
                float *yp = a.y + (int64_t)t * a.d + csl * a.cw + pc * E;
#pragma unroll
                for (int e4 = 0; e4 < E; e4 += 4)
                    *reinterpret_cast<float4 *>(yp + e4) = make_float4(acc[e4], acc[e4 + 1], acc[e4 + 2], acc[e4 + 3]);
            }
        }
        r = rn;
        if (!PASS_PREFETCH && r < PASS_ROWS)
            row_win_load<TI, DOWN>(a, tr(r), er(r), 0, lane, col_off, cur);
    }
#undef tr
#undef er
}

// Column slices: the widest cw = 64 * 2^k with at most 64 16-byte pieces per
// row slice and d / cw >= 8 slices, else cw = 64.
int fused_slice_cols(int d, int esz)
{
    const int max_cw = esz == 2 ? 512 : 256;
    for (int cw = max_cw; cw >= 64; cw >>= 1)
        if (d % cw == 0 && d / cw >= 8)
            return cw;
    return 64;
}

FusedWs fused_ws_layout(void *base, int T, int F, int tile_w, int cap, int d, int esz)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    FusedWs w{};
    w.nch = d / fused_slice_cols(d, esz);
    if (T == 0)
        return w;  // nothing to hold (bytes = 0)
    const size_t slots = (size_t)T * (size_t)(F / tile_w) * (size_t)cap;
    const size_t o_row = 0;
    const size_t o_ord = o_row + up((size_t)T * 4);
    const size_t o_ent = o_ord + up((size_t)T * 4);
    const size_t o_p = o_ent + up(slots * sizeof(int2));
    w.bytes = o_p + up(slots * (size_t)w.nch * sizeof(float));
    w.pstride = (int64_t)slots;
    if (base) {
        char *b = static_cast<char *>(base);
        w.row_e = reinterpret_cast<int32_t *>(b + o_row);
        w.order_e = reinterpret_cast<int32_t *>(b + o_ord);
        w.ent = reinterpret_cast<int2 *>(b + o_ent);
        w.p = reinterpret_cast<float *>(b + o_p);
    }
    return w;
}

template <typename TI, int LPE>
static hipError_t passes_go(const PassArgs<TI> &a, hipStream_t s)
{
    const int groups = (a.T + PASS_WAVES * PASS_ROWS - 1) / (PASS_WAVES * PASS_ROWS);
    ffn_pass_kernel<TI, LPE, false><<<dim3(groups * a.w.nch), dim3(64 * PASS_WAVES), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    ffn_pass_kernel<TI, LPE, true><<<dim3(groups * a.w.nch), dim3(64 * PASS_WAVES), 0, s>>>(a);
    return hipGetLastError();
}

// stage 0: the entries kernel (with row_ovf / work when given); stage 1: the
// two passes; stage 2: both.
template <typename TI>
static hipError_t fused_dispatch(int stage, const int32_t *cnt, const void *val, const uint8_t *idx,
                                 const int32_t *order, int T, int F, int tile_w, int cap, const void *x,
                                 const void *wu_t, const void *wd, int d, float *y, void *ws, int32_t *row_ovf,
                                 int32_t *work, bool use_order_e, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    constexpr int SZ = Elt<TI>::SIZE;
    const FusedWs w = fused_ws_layout(ws, T, F, tile_w, cap, d, SZ);
    PassArgs<TI> a{cnt, static_cast<const TI *>(val), idx, order, T, F / tile_w, tile_w, cap, F,
                   static_cast<const TI *>(x), static_cast<const TI *>(wu_t), static_cast<const TI *>(wd), d,
                   w, y, d / w.nch, row_ovf, work, use_order_e ? w.order_e : nullptr};
    if (stage != 1) {
        ffn_entries_kernel<TI><<<dim3((T + PASS_WAVES - 1) / PASS_WAVES), dim3(64 * PASS_WAVES), 0, s>>>(a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || stage == 0)
            return e;
    }
    const int lpe = a.cw * SZ / 16;  // 16-byte pieces per row slice (a power of two, 8..64)
    if (lpe == 8)
        return passes_go<TI, 8>(a, s);
    if (lpe == 16)
        return passes_go<TI, 16>(a, s);
    if (lpe == 32)
        return passes_go<TI, 32>(a, s);
    return passes_go<TI, 64>(a, s);
}

hipError_t launch_ffn_entries(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                              int tile_w, int cap, int d, void *ws, int32_t *row_ovf, int32_t *work, hipStream_t s)
{
    if (vdtype == 1)
        return fused_dispatch<__bf16>(0, cnt, val, idx, nullptr, T, F, tile_w, cap, nullptr, nullptr, nullptr, d,
                                      nullptr, ws, row_ovf, work, false, s);
    return fused_dispatch<float>(0, cnt, val, idx, nullptr, T, F, tile_w, cap, nullptr, nullptr, nullptr, d, nullptr,
                                 ws, row_ovf, work, false, s);
}

hipError_t launch_ffn_passes(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx,
                             const int32_t *order, int T, int F, int tile_w, int cap, const void *x, const void *wu_t,
                             const void *wd, int d, float *y, void *ws, bool use_order_e, hipStream_t s)
{
    if (vdtype == 1)
        return fused_dispatch<__bf16>(1, cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, ws, nullptr,
                                      nullptr, use_order_e, s);
    return fused_dispatch<float>(1, cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, ws, nullptr, nullptr,
                                 use_order_e, s);
}

hipError_t launch_ffn_fused(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, const int32_t *order,
                            int T, int F, int tile_w, int cap, const void *x, const void *wu_t, const void *wd, int d,
                            float *y, void *ws, hipStream_t s)
{
    if (vdtype == 1)
        return fused_dispatch<__bf16>(2, cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, ws, nullptr,
                                      nullptr, false, s);
    return fused_dispatch<float>(2, cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, ws, nullptr, nullptr,
                                 false, s);
}

// ------------------------------------------------------------------ decode-shaped calls
// The same per-entry work for T <= 64, cut into chunks of CE consecutive
// entries of a row (row order: tiles ascending, slots ascending; a row's
// entries are all its active neurons, CE from the packing kernel), so that a
// heavy row is spread over many waves instead of trailing in one workgroup.
// One wave per chunk: it lists the chunk's (j, h) in LDS -- from the TwELL
// slots for a row that fits (binary search of each entry's tile in the row's
// tile prefix), from z for an overflow row (one pass per tile the chunk
// touches, values rounded to bf16 as the dense backup stores them) -- streams
// the entries as the batch kernel does and writes its partial y row.  The
// partial rows of a row are added in chunk order by chunk_reduce_kernel.
struct ChunkArgs {
    FusedArgs<__bf16> f;        // x, wu_t, wd, d, nchunks, T, F, tile_w, n_b, cap, cnt, val, idx
    const float *z;             // [T][F]
    const int32_t *row_ovf, *row_e, *chunk0, *chunk_e;
    float *part;                // [chunks][d]
};

template <int NC>
__global__ __launch_bounds__(256) void ffn_chunks_kernel(ChunkArgs a)
{
    constexpr int E = Elt<__bf16>::PER_CHUNK;
    constexpr int PMAX = DEC_MAX_NB + 1;  // tile prefix entries held in LDS
    __shared__ int2 clist[4][DEC_MAX_E];
    __shared__ int spre[4][PMAX];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.f.T, n_b = a.f.n_b, w = a.f.tile_w, cap = a.f.cap;
    const int n_chunks = a.chunk0[T];
    const int CE = *a.chunk_e;
    const int64_t row_bytes = (int64_t)a.f.d * Elt<__bf16>::SIZE;
    int2 *list = clist[wave];
    int *sp = spre[wave];
    for (int c = blockIdx.x * 4 + wave; c < n_chunks; c += gridDim.x * 4) {
        // the chunk's row: rows whose first chunk is <= c, minus one (chunk0 ascends)
        const int le = __popcll(__ballot(lane < T && a.chunk0[lane] <= c));
        const int t = __builtin_amdgcn_readfirstlane(le - 1);
        // exclusive prefix of the row's tile counts: sp[b] = entries before tile b
        const int32_t *crow = a.f.cnt + (int64_t)t * n_b;
        int run = 0;
        for (int b0 = 0; b0 < n_b; b0 += 64) {
            const int b = b0 + lane;
            const int v = b < n_b ? crow[b] : 0;
            const int incl = wave_incl_scan(v, lane);
            if (b < n_b)
                sp[b] = run + incl - v;
            run += __shfl(incl, 63, 64);
        }
        if (lane == 0)
            sp[n_b] = run;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const int e_t = sp[n_b];
        const int k0 = (c - a.chunk0[t]) * CE;
        const int n = CE < e_t - k0 ? CE : e_t - k0;
        if (!a.row_ovf[t]) {
            // every entry is a TwELL slot: entry k sits in the last tile b with sp[b] <= k
            for (int p = lane; p < n; p += 64) {
                const int k = k0 + p;
                int lo = 0, hi = n_b - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (sp[mid] <= k)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                const int64_t slot = ((int64_t)t * n_b + lo) * cap + (k - sp[lo]);
                int j = lo * w + a.f.idx[slot];
                j = j < a.f.F ? j : a.f.F - 1;  // memory safety for a corrupt index
                list[p] = make_int2(j, __float_as_int(load_elem(a.f.val + slot)));
            }
        } else {
            // an overflow row: its entries are all active columns, taken from z
            int b = 0;
            {
                int lo = 0, hi = n_b - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (sp[mid] <= k0)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                b = lo;
            }
            for (; b < n_b && sp[b] < k0 + n; ++b) {
                const float *zt = a.z + (int64_t)t * a.f.F + (int64_t)b * w;
                int base = sp[b];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int col = lane + 64 * jj;
                    const float v = col < w ? zt[col] : 0.f;
                    const uint64_t bal = __ballot(col < w && v > 0.f);
                    const int k = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                    if (((bal >> lane) & 1ull) && k >= k0 && k < k0 + n)
                        list[k - k0] = make_int2(b * w + col, __float_as_int((float)(__bf16)v));
                    base += __popcll(bal);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's list stores are done
        __builtin_amdgcn_wave_barrier();

        XRow<__bf16, NC> xf;
        float yacc[NC][E];
        const char *xrow = (const char *)a.f.x + (int64_t)t * row_bytes;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const int ch = lane + 64 * cc;
            xf.set(cc, ch < a.f.nchunks ? ldg16(xrow + ch * 16) : u32x4{0, 0, 0, 0});
#pragma unroll
            for (int e = 0; e < E; ++e)
                yacc[cc][e] = 0.f;
        }
        constexpr int DG = 2;  // entries per group
        const int ngroups = n / DG;
        group_stream<__bf16, NC, DG>(a.f, list, 0, 1, ngroups, lane, row_bytes, xf, yacc);
        for (int e0 = ngroups * DG; e0 < n; ++e0) {
            Group<__bf16, NC, 1> g1;
            group_load<__bf16, NC, 1>(a.f, list, e0, lane, row_bytes, g1);
            group_apply<__bf16, NC, 1>(g1, xf, yacc);
        }
        float *pr = a.part + (int64_t)c * a.f.d;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const int ch = lane + 64 * cc;
            if (ch < a.f.nchunks) {
                *reinterpret_cast<float4 *>(pr + ch * E) =
                    make_float4(yacc[cc][0], yacc[cc][1], yacc[cc][2], yacc[cc][3]);
                *reinterpret_cast<float4 *>(pr + ch * E + 4) =
                    make_float4(yacc[cc][4], yacc[cc][5], yacc[cc][6], yacc[cc][7]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // list and prefix reads done before the next chunk's stores
    }
}

// y[t] = sum of row t's partial rows (0 for a row without entries), in a
// fixed order: one workgroup per (row, 256 columns); its 4 waves each add every
// 4th chunk in chunk order, two loads in flight, and the 4 sums meet in LDS in
// wave order.  Blocks past the rows write the dense backup rows ReLU(z) (bf16)
// of the first min(n_ovf, max_ovf) overflow rows.
__global__ __launch_bounds__(256) void chunk_reduce_kernel(const float *part, const int32_t *chunk0, int T, int d,
                                                           float *y, const float *z, int F, const int32_t *ovf_rows,
                                                           const int32_t *n_ovf, int max_ovf, __bf16 *dense)
{
    __shared__ float4 sred[4][64];
    const int cpr = (d + 255) / 256;  // column slices per row (d is a multiple of 64)
    const int r = blockIdx.x / cpr;
    if (r < T) {
        const int tid = threadIdx.x, g = tid >> 6, l = tid & 63;
        const int col = (blockIdx.x - r * cpr) * 256 + 4 * l;
        const int c0 = chunk0[r];
        const int c1 = col < d ? chunk0[r + 1] : c0;  // columns past d: nothing to add
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        int c = c0 + g;
        for (; c + 4 < c1; c += 8) {
            const float4 p = *reinterpret_cast<const float4 *>(part + (int64_t)c * d + col);
            const float4 q = *reinterpret_cast<const float4 *>(part + (int64_t)(c + 4) * d + col);
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
            s.x += q.x; s.y += q.y; s.z += q.z; s.w += q.w;
        }
        if (c < c1) {
            const float4 p = *reinterpret_cast<const float4 *>(part + (int64_t)c * d + col);
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        sred[g][l] = s;
        __syncthreads();
        if (g == 0 && col < d) {
            float4 o = sred[0][l];
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const float4 p = sred[k][l];
                o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
            }
            *reinterpret_cast<float4 *>(y + (int64_t)r * d + col) = o;
        }
        return;
    }
    const int i = blockIdx.x - T * cpr;
    const int nv = *n_ovf < max_ovf ? *n_ovf : max_ovf;
    if (i >= nv)
        return;
    // 8 elements per thread and step (F is a multiple of 64; z rows and dense
    // rows are 16-byte aligned), so a thread's loads are all in flight together
    const float *zr = z + (int64_t)ovf_rows[i] * F;
    __bf16 *dr = dense + (int64_t)i * F;
#pragma unroll 4
    for (int j = threadIdx.x * 8; j < F; j += 256 * 8) {
        const float4 p = *reinterpret_cast<const float4 *>(zr + j);
        const float4 q = *reinterpret_cast<const float4 *>(zr + j + 4);
        const float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            h[e] = __builtin_bit_cast(uint16_t, (__bf16)(v[e] > 0.f ? v[e] : 0.f));
        *reinterpret_cast<u32x4 *>(dr + j) =
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
}

hipError_t launch_ffn_decode(const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F, int tile_w,
                             int cap, const void *x, const void *wu_t, const void *wd, int d, const int32_t *row_ovf,
                             const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf, void *dense, float *y,
                             const DecodeWs &w, hipStream_t s)
{
    ChunkArgs a{};
    a.f = FusedArgs<__bf16>{cnt, static_cast<const __bf16 *>(val), idx, nullptr, T, F / tile_w, tile_w, cap, F,
                            static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(wu_t),
                            static_cast<const __bf16 *>(wd), d, d * 2 / 16, y};
    a.z = w.z;
    a.row_ovf = row_ovf;
    a.row_e = w.row_e;
    a.chunk0 = w.chunk0;
    a.chunk_e = w.chunk_e;
    a.part = w.part;
    const dim3 grid(DEC_GATHER_WGS), block(256);
    const int nch = a.f.nchunks;
    if (nch <= 64)
        ffn_chunks_kernel<1><<<grid, block, 0, s>>>(a);
    else if (nch <= 128)
        ffn_chunks_kernel<2><<<grid, block, 0, s>>>(a);
    else if (nch <= 256)
        ffn_chunks_kernel<4><<<grid, block, 0, s>>>(a);
    else
        ffn_chunks_kernel<8><<<grid, block, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int dense_blocks = T < max_ovf ? T : max_ovf;
    chunk_reduce_kernel<<<dim3(T * ((d + 255) / 256) + dense_blocks), dim3(256), 0, s>>>(
        w.part, w.chunk0, T, d, y, w.z, F, ovf_rows, n_ovf, max_ovf, static_cast<__bf16 *>(dense));
    return hipGetLastError();
}

hipError_t launch_chunk_reduce(const float *part, const int32_t *chunk0, int T, int d, float *y, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    chunk_reduce_kernel<<<dim3(T * ((d + 255) / 256)), dim3(256), 0, s>>>(part, chunk0, T, d, y, nullptr, 0, nullptr,
                                                                          nullptr, 0, nullptr);
    return hipGetLastError();
}

}  // namespace twell
