// convert.hip -- conversions between a dense activation matrix and the
// ELL + dense-backup hybrid.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.4: training keeps the activations in the hybrid format
// and needs kernels that turn a dense matrix into the hybrid and back, in the
// forward and the backward pass.  Both directions are streaming kernels bound
// by HBM (the dense side is T x F elements):
//   dense -> hybrid: one workgroup per row, 16 bytes of the row per lane; the
//     TwELL rules are the gate epilogue's (active iff h > 0, ascending
//     columns, true count kept, first cap values stored, zero padding), with
//     slots from a segmented scan over each tile's lanes, and the row's
//     overflow flag and work value written by its workgroup; the ascending
//     overflow list and work order then come from the batch path's compaction
//     kernel, and the dense backup rows are the overflow rows' max(h, 0).
//   hybrid -> dense: one workgroup per row; each wave expands whole tiles
//     through a per-wave LDS row (zeros, then the kept slots scattered by
//     column) and writes it with 16-byte stores; a second kernel overwrites
//     the first min(n_ovf, max_ovf) overflow rows with their dense backup
//     rows.
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

namespace twell {

template <typename TI> struct ConvArgs {
    TI *dense;  // [T][F]: input of dense -> hybrid, output of hybrid -> dense
    int T, F, tile_w, cap, n_b;
    TI *val;
    uint8_t *idx;
    int32_t *cnt;
    int32_t *row_ovf, *work;  // dense -> hybrid: per-row flag and stored entries (0 if flagged)
};

// Row t; lane l of a wave pass owns CPL = 16 / sizeof(TI) consecutive columns
// (one 16-byte load), so a pass covers 64 * CPL columns = 64 * CPL / w whole
// tiles, each spread over L = w / CPL consecutive lanes.  A lane's activity
// bits give its count; a segmented scan over the L lanes of its tile gives the
// count before it, so every active column's slot is known in ascending column
// order.  Wave w takes passes w, w + NW, ...; up to 4 passes' loads are
// requested together (NW = 4: a 16 KiB row is one batch of 4 loads per lane;
// 8 waves of 2 loads each measured 46 vs 42 us at the 2B-like layer).  The
// row's overflow flag and stored-entry count (the work order's input) are
// gathered with LDS atomics and written at the end.
#ifndef CONV_NW
#define CONV_NW 4
#endif
template <typename TI, int NW>
__global__ __launch_bounds__(NW * 64) void dense_pack_kernel(ConvArgs<TI> a)
{
    constexpr int BATCH = 4, CPL = 16 / (int)sizeof(TI);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w, cap = a.cap;
    const int L = w / CPL;                    // lanes per tile (power of two, 4..64)
    const int gl = lane & (L - 1);            // lane within its tile
    const int F16 = a.F / CPL;                // 16-byte chunks per row
    const char *hr = reinterpret_cast<const char *>(a.dense + (int64_t)t * a.F);
    __shared__ int s_stored, s_ovf;
    if (threadIdx.x == 0) {
        s_stored = 0;
        s_ovf = 0;
    }
    __syncthreads();
    for (int p0 = wave; p0 * 64 < F16; p0 += NW * BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int ch = (p0 + u * NW) * 64 + lane;
            v[u] = ch < F16 ? ldg16(hr + (int64_t)ch * 16) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int ch = (p0 + u * NW) * 64 + lane;  // this lane's chunk
            if ((p0 + u * NW) * 64 >= F16)
                break;
            const bool live = ch < F16;
            float x[CPL];
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                x[k] = chunk_elem<TI>(v[u], k);
                m |= (live && x[k] > 0.f) ? (1u << k) : 0u;
            }
            const int cntl = __popc(m);
            // segmented inclusive scan over the tile's L lanes
            const int incl = seg_incl_scan(cntl, gl, L);
            const int total = __shfl(incl, (lane | (L - 1)), 64);
            const int col0 = ch * CPL;                 // first column of the lane in the row
            const int b = col0 / w;                    // its tile
            const int64_t slot0 = ((int64_t)t * a.n_b + b) * cap;
            if (live) {
                int slot = incl - cntl;
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    if ((m >> k) & 1u) {
                        if (slot < cap) {
                            store_elem(a.val + slot0 + slot, x[k]);
                            a.idx[slot0 + slot] = (uint8_t)(gl * CPL + k);
                        }
                        ++slot;
                    }
                }
                const int kept = total < cap ? total : cap;
                for (int s2 = kept + gl; s2 < cap; s2 += L) {
                    store_elem(a.val + slot0 + s2, 0.f);
                    a.idx[slot0 + s2] = 0;
                }
                if (gl == 0) {
                    a.cnt[(int64_t)t * a.n_b + b] = total;
                    if (kept)
                        atomicAdd(&s_stored, kept);
                    if (total > cap)
                        atomicOr(&s_ovf, 1);
                }
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a.row_ovf[t] = s_ovf;
        a.work[t] = s_ovf ? 0 : s_stored;
    }
}

// dense[i][:] = max(h[ovf_rows[i]][:], 0) (NaN -> 0) for i < min(n_ovf, max_ovf).
template <typename TI>
__global__ __launch_bounds__(256) void relu_rows_kernel(const TI *h, int F, const int32_t *ovf_rows,
                                                        const int32_t *n_ovf, int max_ovf, TI *dense)
{
    const int i = blockIdx.x;
    const int nv = *n_ovf < max_ovf ? *n_ovf : max_ovf;
    if (i >= nv)
        return;
    constexpr int CPL = 16 / (int)sizeof(TI);
    const char *src = reinterpret_cast<const char *>(h + (int64_t)ovf_rows[i] * F);
    char *dst = reinterpret_cast<char *>(dense + (int64_t)i * F);
    for (int c = threadIdx.x; c < F / CPL; c += 256) {
        const u32x4 v = ldg16(src + (int64_t)c * 16);
        u32x4 o = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            if (chunk_elem<TI>(v, e) > 0.f) {  // keep the element's bits; 0, negatives and NaN -> +0
                if constexpr (sizeof(TI) == 2)
                    o[e >> 1] |= v[e >> 1] & ((e & 1) ? 0xFFFF0000u : 0x0000FFFFu);
                else
                    o[e] = v[e];
            }
        }
        *reinterpret_cast<u32x4 *>(dst + (int64_t)c * 16) = o;
    }
}

// Row t of the dense matrix from its TwELL tiles (kept slots only).  A wave
// pass covers 64 * CPL columns (whole tiles): the pass is zeroed in a per-wave
// LDS row, the tiles' kept slots are scattered into it by column, and each
// lane writes its CPL columns with one 16-byte store.
template <typename TI>
__global__ __launch_bounds__(512) void twell_expand_kernel(ConvArgs<TI> a)
{
    constexpr int NW = 8, CPL = 16 / (int)sizeof(TI), PW = 64 * CPL;  // columns per wave pass
    __shared__ __attribute__((aligned(16))) TI srow[NW][PW];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w, cap = a.cap;
    TI *sr = srow[wave];
    char *orow = reinterpret_cast<char *>(a.dense + (int64_t)t * a.F);
    const int F16 = a.F / CPL;
    for (int p = wave; p * 64 < F16; p += NW) {
        const int c0 = p * PW;                                // first column of the pass
        const int ncol = a.F - c0 < PW ? a.F - c0 : PW;       // multiple of w
        const int nt = ncol / w, b0 = c0 / w;
        *reinterpret_cast<u32x4 *>(sr + lane * CPL) = u32x4{0, 0, 0, 0};
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        for (int i = lane; i < nt * cap; i += 64) {
            const int tl = i / cap, sl = i - tl * cap;
            const int64_t tb = (int64_t)t * a.n_b + b0 + tl;
            int kept = a.cnt[tb];
            kept = kept < cap ? kept : cap;
            if (sl < kept) {
                const int c = a.idx[tb * cap + sl];
                if (c < w)  // memory safety for a corrupt index
                    sr[tl * w + c] = a.val[tb * cap + sl];
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        const int ch = p * 64 + lane;
        if (ch < F16)
            *reinterpret_cast<u32x4 *>(orow + (int64_t)ch * 16) = *reinterpret_cast<const u32x4 *>(sr + lane * CPL);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();  // LDS reads done before the next pass's zeros
    }
}

// out[ovf_rows[i]][:] = dense[i][:] for i < min(n_ovf, max_ovf).
template <typename TI>
__global__ __launch_bounds__(256) void dense_rows_kernel(const TI *dense, int F, const int32_t *ovf_rows,
                                                         const int32_t *n_ovf, int max_ovf, TI *out)
{
    const int i = blockIdx.x;
    const int nv = *n_ovf < max_ovf ? *n_ovf : max_ovf;
    if (i >= nv)
        return;
    const int nch = F * (int)sizeof(TI) / 16;  // F * size is a multiple of 128 bytes
    const char *src = reinterpret_cast<const char *>(dense + (int64_t)i * F);
    char *dst = reinterpret_cast<char *>(out + (int64_t)ovf_rows[i] * F);
    for (int c = threadIdx.x; c < nch; c += 256)
        *reinterpret_cast<u32x4 *>(dst + c * 16) = ldg16(src + c * 16);
}

template <typename TI>
static hipError_t dense_to_hybrid_go(const void *h, int T, int F, int tile_w, int cap, void *val, uint8_t *idx,
                                     int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows, int32_t *n_ovf,
                                     int32_t *order, int max_ovf, void *dense, hipStream_t s)
{
    ConvArgs<TI> a{const_cast<TI *>(static_cast<const TI *>(h)), T, F, tile_w, cap, F / tile_w,
                   static_cast<TI *>(val), idx, cnt, row_ovf, order};
    dense_pack_kernel<TI, CONV_NW><<<dim3(T), dim3(CONV_NW * 64), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if ((e = launch_compact_rows(row_ovf, T, max_ovf, ovf_rows, n_ovf, order, s)) != hipSuccess)
        return e;
    if (max_ovf > 0)
        relu_rows_kernel<TI><<<dim3(max_ovf), dim3(256), 0, s>>>(static_cast<const TI *>(h), F, ovf_rows, n_ovf,
                                                                 max_ovf, static_cast<TI *>(dense));
    return hipGetLastError();
}

hipError_t launch_dense_to_hybrid(int vdtype, const void *h, int T, int F, int tile_w, int cap, void *val,
                                  uint8_t *idx, int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows, int32_t *n_ovf,
                                  int32_t *order, int max_ovf, void *dense, hipStream_t s)
{
    if (vdtype == 1)
        return dense_to_hybrid_go<__bf16>(h, T, F, tile_w, cap, val, idx, cnt, row_ovf, ovf_rows, n_ovf, order,
                                          max_ovf, dense, s);
    return dense_to_hybrid_go<float>(h, T, F, tile_w, cap, val, idx, cnt, row_ovf, ovf_rows, n_ovf, order, max_ovf,
                                     dense, s);
}

template <typename TI>
static hipError_t hybrid_to_dense_go(const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                                     int tile_w, int cap, const int32_t *ovf_rows, const int32_t *n_ovf,
                                     int max_ovf, const void *dense, void *out, hipStream_t s)
{
    ConvArgs<TI> a{static_cast<TI *>(out), T, F, tile_w, cap, F / tile_w,
                   const_cast<TI *>(static_cast<const TI *>(val)), const_cast<uint8_t *>(idx),
                   const_cast<int32_t *>(cnt), nullptr, nullptr};
    twell_expand_kernel<TI><<<dim3(T), dim3(512), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_ovf == 0)
        return e;
    dense_rows_kernel<TI><<<dim3(max_ovf), dim3(256), 0, s>>>(static_cast<const TI *>(dense), F, ovf_rows, n_ovf,
                                                              max_ovf, static_cast<TI *>(out));
    return hipGetLastError();
}

hipError_t launch_hybrid_to_dense(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                                  int tile_w, int cap, const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf,
                                  const void *dense, void *out, hipStream_t s)
{
    if (vdtype == 1)
        return hybrid_to_dense_go<__bf16>(cnt, val, idx, T, F, tile_w, cap, ovf_rows, n_ovf, max_ovf, dense, out, s);
    return hybrid_to_dense_go<float>(cnt, val, idx, T, F, tile_w, cap, ovf_rows, n_ovf, max_ovf, dense, out, s);
}

}  // namespace twell
