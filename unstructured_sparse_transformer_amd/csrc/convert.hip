// convert.hip -- conversions between a dense activation matrix and the
// ELL + dense-backup hybrid.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.4: training keeps the activations in the hybrid format
// and needs kernels that turn a dense matrix into the hybrid and back, in the
// forward and the backward pass.  Both directions are streaming kernels bound
// by HBM (the dense side is T x F elements):
//   dense -> hybrid: one workgroup per row; each wave packs TwELL tiles with
//     the same ballot / mbcnt rules as the gate epilogue (active iff h > 0,
//     ascending columns, true count kept, first cap values stored, zero
//     padding); the overflow flags, list and work order then come from the
//     batch path's partition kernels, and the dense backup rows are the
//     overflow rows' max(h, 0).
//   hybrid -> dense: one workgroup per row; each wave expands a tile through a
//     per-wave LDS row (zeros, then the kept slots scattered by column) and
//     writes it with coalesced stores; a second kernel overwrites the first
//     min(n_ovf, max_ovf) overflow rows with their dense backup rows.
#include "launch.h"
#include "twell_device.h"

namespace twell {

template <typename TI> struct ConvArgs {
    TI *dense;  // [T][F]: input of dense -> hybrid, output of hybrid -> dense
    int T, F, tile_w, cap, n_b;
    TI *val;
    uint8_t *idx;
    int32_t *cnt;
};

// Tiles of row t, wave-strided: wave w handles tiles w, w + 8, ...; the
// values of up to 4 tiles are requested together.
template <typename TI>
__global__ __launch_bounds__(512) void dense_pack_kernel(ConvArgs<TI> a)
{
    constexpr int NW = 8, BATCH = 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w, cap = a.cap;
    const TI *hr = a.dense + (int64_t)t * a.F;
    for (int b0 = wave; b0 < a.n_b; b0 += NW * BATCH) {
        float v[BATCH][4];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = lane + 64 * j;
                v[u][j] = (b < a.n_b && c < w) ? load_elem(hr + (int64_t)b * w + c) : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
            if (b >= a.n_b)
                continue;
            uint64_t bal[4];
            int total = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bal[j] = __ballot(lane + 64 * j < w && v[u][j] > 0.f);
                total += __popcll(bal[j]);
            }
            const int64_t slot0 = ((int64_t)t * a.n_b + b) * cap;
            int base = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
                if (((bal[j] >> lane) & 1ull) && slot < cap) {
                    store_elem(a.val + slot0 + slot, v[u][j]);
                    a.idx[slot0 + slot] = (uint8_t)(lane + 64 * j);
                }
                base += __popcll(bal[j]);
            }
            const int kept = total < cap ? total : cap;
            for (int s = kept + lane; s < cap; s += 64) {
                store_elem(a.val + slot0 + s, 0.f);
                a.idx[slot0 + s] = 0;
            }
            if (lane == 0)
                a.cnt[(int64_t)t * a.n_b + b] = total;
        }
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
    const TI *src = h + (int64_t)ovf_rows[i] * F;
    TI *dst = dense + (int64_t)i * F;
    for (int j = threadIdx.x; j < F; j += 256) {
        const float v = load_elem(src + j);
        store_elem(dst + j, v > 0.f ? v : 0.f);
    }
}

// Row t of the dense matrix from its TwELL tiles (kept slots only).
template <typename TI>
__global__ __launch_bounds__(512) void twell_expand_kernel(ConvArgs<TI> a)
{
    constexpr int NW = 8;
    __shared__ float srow[NW][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w, cap = a.cap;
    float *sr = srow[wave];
    TI *orow = a.dense + (int64_t)t * a.F;
    for (int b = wave; b < a.n_b; b += NW) {
        const int64_t slot0 = ((int64_t)t * a.n_b + b) * cap;
        int kept = a.cnt[(int64_t)t * a.n_b + b];
        kept = kept < cap ? kept : cap;
        kept = kept > 0 ? kept : 0;
        for (int c = lane; c < w; c += 64)
            sr[c] = 0.f;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        for (int s = lane; s < kept; s += 64) {
            const int c = a.idx[slot0 + s];
            if (c < w)  // memory safety for a corrupt index
                sr[c] = load_elem(a.val + slot0 + s);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        for (int c = lane; c < w; c += 64)
            store_elem(orow + (int64_t)b * w + c, sr[c]);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();  // LDS reads done before the next tile's zeros
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
                   static_cast<TI *>(val), idx, cnt};
    dense_pack_kernel<TI><<<dim3(T), dim3(512), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if ((e = launch_row_flags(cnt, T, F / tile_w, cap, row_ovf, order, s)) != hipSuccess)
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
                   const_cast<int32_t *>(cnt)};
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
