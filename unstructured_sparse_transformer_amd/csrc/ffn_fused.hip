// ffn_fused.hip -- fused up/down projection straight from TwELL.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.2: with the gate activation h_g in TwELL, the up and
// down projections become one kernel that, for each nonzero h_g[j], reads
// only the weights it needs (column j of W_u, row j of W_d), takes a dot
// product and a scalar product, and accumulates -- DRAM traffic is the point.
//
// gfx950 mapping: one wave64 per token.  The token's x row and y accumulator
// live in registers (chunk c of lane l covers elements (l + 64c)*E .. +E, so
// every weight-row read is one fully coalesced 16-byte-per-lane sweep).  The
// token's TwELL entries are first compacted into an LDS list of (j, h) in
// ascending j (wave prefix sum over the per-tile counts), then consumed G at a
// time: 2*G weight rows are in flight per wave, the G dot products are reduced
// across the wave with butterflies (every lane ends with the same bits), and
// y += (h*u) * W_d[j] runs in fp32 in ascending j.  No atomics: each y row has
// one owner, so the result is deterministic.
#include "launch.h"
#include "twell_device.h"

namespace twell {

constexpr int LIST_MAX = 512;  // entries staged per pass (8 bytes each)

template <typename TI> struct FusedArgs {
    const int32_t *cnt;
    const TI *val;
    const uint8_t *idx;
    int T, n_b, tile_w, cap, F;
    const TI *x, *wu_t, *wd;
    int d, nchunks;  // nchunks = 16-byte chunks per row
    float *y;
};

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ int wave_isum(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o)
            v += u;
    }
    return v;
}

template <typename TI, int NC, int G>
__global__ __launch_bounds__(64) void ffn_fused_kernel(FusedArgs<TI> a)
{
    constexpr int E = Elt<TI>::PER_CHUNK;
    __shared__ int2 list[LIST_MAX];
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const int64_t row_bytes = (int64_t)a.d * Elt<TI>::SIZE;
    float *yrow = a.y + (int64_t)t * a.d;

    // Overflow rows (some tile count > cap) and the number of kept entries.
    const int32_t *crow = a.cnt + (int64_t)t * a.n_b;
    bool ovf = false;
    int total = 0;
    for (int b0 = 0; b0 < a.n_b; b0 += 64) {
        const int b = b0 + lane;
        const int c = b < a.n_b ? crow[b] : 0;
        ovf |= __ballot(c > a.cap) != 0ull;
        total += wave_isum(c < a.cap ? c : a.cap);
    }

    float yacc[NC][E];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
            yacc[c][e] = 0.f;

    if (!ovf && total > 0) {
        float xf[NC][E];
        const char *xrow = (const char *)a.x + (int64_t)t * row_bytes;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = lane + 64 * c;
            const u32x4 v = ch < a.nchunks ? ldg16(xrow + ch * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < E; ++e)
                xf[c][e] = chunk_elem<TI>(v, e);
        }
        for (int win = 0; win < total; win += LIST_MAX) {
            // Stage entries [win, win + LIST_MAX) in ascending (tile, slot) order.
            int base = 0;
            for (int b0 = 0; b0 < a.n_b; b0 += 64) {
                const int b = b0 + lane;
                int c = b < a.n_b ? crow[b] : 0;
                c = c < a.cap ? c : a.cap;
                const int incl = wave_incl_scan(c, lane);
                const int excl = base + incl - c;
                const int64_t slot0 = ((int64_t)t * a.n_b + b) * a.cap;
                for (int s = 0; s < c; ++s) {
                    const int pos = excl + s - win;
                    if (pos >= 0 && pos < LIST_MAX) {
                        int j = b * a.tile_w + a.idx[slot0 + s];
                        j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
                        list[pos] = make_int2(j, __float_as_int(load_elem(a.val + slot0 + s)));
                    }
                }
                base += __shfl(incl, 63, 64);
            }
            __syncthreads();
            const int n = total - win < LIST_MAX ? total - win : LIST_MAX;
            int e0 = 0;
            for (; e0 + G <= n; e0 += G) {
                int j[G];
                float h[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int2 en = list[e0 + g];
                    j[g] = __builtin_amdgcn_readfirstlane(en.x);
                    h[g] = __int_as_float(__builtin_amdgcn_readfirstlane(en.y));
                }
                u32x4 wu[G][NC], wv[G][NC];
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const int ch = lane + 64 * c;
                        const bool ok = ch < a.nchunks;
                        wu[g][c] = ok ? ldg16((const char *)a.wu_t + (int64_t)j[g] * row_bytes + ch * 16)
                                      : u32x4{0, 0, 0, 0};
                        wv[g][c] = ok ? ldg16((const char *)a.wd + (int64_t)j[g] * row_bytes + ch * 16)
                                      : u32x4{0, 0, 0, 0};
                    }
                float part[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            s = fmaf(xf[c][e], chunk_elem<TI>(wu[g][c], e), s);
                    part[g] = s;
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
                    part[g] = wave_sum(part[g]);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float sc = h[g] * part[g];
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            yacc[c][e] = fmaf(sc, chunk_elem<TI>(wv[g][c], e), yacc[c][e]);
                }
            }
            for (; e0 < n; ++e0) {
                const int2 en = list[e0];
                const int j = __builtin_amdgcn_readfirstlane(en.x);
                const float h = __int_as_float(__builtin_amdgcn_readfirstlane(en.y));
                u32x4 wu[NC], wv[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ch = lane + 64 * c;
                    const bool ok = ch < a.nchunks;
                    wu[c] = ok ? ldg16((const char *)a.wu_t + (int64_t)j * row_bytes + ch * 16) : u32x4{0, 0, 0, 0};
                    wv[c] = ok ? ldg16((const char *)a.wd + (int64_t)j * row_bytes + ch * 16) : u32x4{0, 0, 0, 0};
                }
                float s = 0.f;
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        s = fmaf(xf[c][e], chunk_elem<TI>(wu[c], e), s);
                const float sc = h * wave_sum(s);
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        yacc[c][e] = fmaf(sc, chunk_elem<TI>(wv[c], e), yacc[c][e]);
            }
            __syncthreads();
        }
    }

    // y row: lane's chunk c covers y elements (lane + 64c)*E .. +E.
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < a.nchunks) {
            float4 *dst = reinterpret_cast<float4 *>(yrow + (int64_t)ch * E);
#pragma unroll
            for (int q = 0; q < E / 4; ++q)
                dst[q] = make_float4(yacc[c][4 * q], yacc[c][4 * q + 1], yacc[c][4 * q + 2], yacc[c][4 * q + 3]);
        }
    }
}

template <typename TI, int NC>
static hipError_t fused_go(const FusedArgs<TI> &a, hipStream_t s)
{
    if (a.T == 0)
        return hipSuccess;
    ffn_fused_kernel<TI, NC, 4><<<dim3(a.T), dim3(64), 0, s>>>(a);
    return hipGetLastError();
}

template <typename TI>
static hipError_t fused_dispatch(const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F, int tile_w,
                                 int cap, const void *x, const void *wu_t, const void *wd, int d, float *y,
                                 hipStream_t s)
{
    FusedArgs<TI> a{cnt, static_cast<const TI *>(val), idx, T, F / tile_w, tile_w, cap, F,
                    static_cast<const TI *>(x), static_cast<const TI *>(wu_t), static_cast<const TI *>(wd),
                    d, (int)((int64_t)d * Elt<TI>::SIZE / 16), y};
    const int nch = a.nchunks;
    if (nch <= 64)
        return fused_go<TI, 1>(a, s);
    if (nch <= 128)
        return fused_go<TI, 2>(a, s);
    if (nch <= 256)
        return fused_go<TI, 4>(a, s);
    return fused_go<TI, 8>(a, s);
}

hipError_t launch_ffn_fused(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, int T, int F,
                            int tile_w, int cap, const void *x, const void *wu_t, const void *wd, int d, float *y,
                            hipStream_t s)
{
    if (vdtype == 1)
        return fused_dispatch<__bf16>(cnt, val, idx, T, F, tile_w, cap, x, wu_t, wd, d, y, s);
    return fused_dispatch<float>(cnt, val, idx, T, F, tile_w, cap, x, wu_t, wd, d, y, s);
}

}  // namespace twell
