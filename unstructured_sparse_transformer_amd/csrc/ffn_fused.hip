// ffn_fused.hip -- fused up/down projection straight from TwELL.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.2: with the gate activation h_g in TwELL, the up and
// down projections become one kernel that, for each nonzero h_g[j], reads
// only the weights it needs (column j of W_u, row j of W_d), takes a dot
// product and a scalar product, and accumulates -- DRAM traffic is the point.
//
// gfx950 mapping: one workgroup of 4 waves per token.  Each wave keeps the
// token's x row and a partial y row in registers (chunk c of lane l covers
// elements (l + 64c)*E .. +E, so every weight-row read is one fully coalesced
// 16-byte-per-lane sweep).  The token's TwELL entries are compacted into an LDS
// list of (j, h) in ascending j (wave prefix sum over the per-tile counts) and
// dealt to the waves G at a time, so heavy tokens (hundreds of entries) run 4
// latency chains in parallel; 2*G weight rows are in flight per wave, the G
// dot products are reduced with DPP, and y += (h*u) * W_d[j] runs in fp32.
// The partial rows are added in LDS in a fixed order: no atomics, and the
// result does not depend on timing.
#include "launch.h"
#include "twell_device.h"

namespace twell {

constexpr int LIST_MAX = 512;  // entries staged per pass (8 bytes each)
constexpr int NWV = 4;         // waves per token

template <typename TI> struct FusedArgs {
    const int32_t *cnt;
    const TI *val;
    const uint8_t *idx;
    int T, n_b, tile_w, cap, F;
    const TI *x, *wu_t, *wd;
    int d, nchunks;  // nchunks = 16-byte chunks per row
    float *y;
};

// Sum over the 64 lanes with DPP row shifts and row broadcasts (an inclusive
// scan whose last lane holds the total), returned as a wave-uniform value.
// The order of the additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

// G entries (j, h) of the list at `e0`: y += (h * (x . W_u^T[j])) * W_d[j].
template <typename TI, int NC, int G>
__device__ __forceinline__ void fused_group(const FusedArgs<TI> &a, const int2 *list, int e0, int lane,
                                            int64_t row_bytes, const float (&xf)[NC][Elt<TI>::PER_CHUNK],
                                            float (&yacc)[NC][Elt<TI>::PER_CHUNK])
{
    constexpr int E = Elt<TI>::PER_CHUNK;
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
            wu[g][c] = ok ? ldg16((const char *)a.wu_t + (int64_t)j[g] * row_bytes + ch * 16) : u32x4{0, 0, 0, 0};
            wv[g][c] = ok ? ldg16((const char *)a.wd + (int64_t)j[g] * row_bytes + ch * 16) : u32x4{0, 0, 0, 0};
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

// One workgroup of NWV waves per token.  Wave 0 stages the token's entries
// (ascending j) into LDS; wave w then takes the groups of G entries numbered
// w, w + NWV, w + 2 NWV, ...; the NWV partial y rows meet in LDS and are added
// in wave order.  Tokens without entries, and overflow rows, get y = 0.
template <typename TI, int NC, int G>
__global__ __launch_bounds__(64 * NWV) void ffn_fused_kernel(FusedArgs<TI> a)
{
    constexpr int E = Elt<TI>::PER_CHUNK;
    constexpr int YW = NC * 64 * E;  // floats of one partial y row (>= d)
    __shared__ int2 list[LIST_MAX];
    __shared__ __attribute__((aligned(16))) float part[NWV - 1][YW];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x;
    const int64_t row_bytes = (int64_t)a.d * Elt<TI>::SIZE;
    float *yrow = a.y + (int64_t)t * a.d;

    // Overflow test and number of kept entries (every wave, same values).
    const int32_t *crow = a.cnt + (int64_t)t * a.n_b;
    bool ovf = false;
    int total = 0;
    for (int b0 = 0; b0 < a.n_b; b0 += 64) {
        const int b = b0 + lane;
        const int c = b < a.n_b ? crow[b] : 0;
        ovf |= __ballot(c > a.cap) != 0ull;
        total += wave_isum(c < a.cap ? c : a.cap);
    }
    if (ovf || total == 0) {
        for (int i = tid * 4; i < a.d; i += 64 * NWV * 4)
            *reinterpret_cast<float4 *>(yrow + i) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }

    float xf[NC][E], yacc[NC][E];
    const char *xrow = (const char *)a.x + (int64_t)t * row_bytes;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        const u32x4 v = ch < a.nchunks ? ldg16(xrow + ch * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < E; ++e) {
            xf[c][e] = chunk_elem<TI>(v, e);
            yacc[c][e] = 0.f;
        }
    }
    for (int win = 0; win < total; win += LIST_MAX) {
        if (wave == 0) {
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
        }
        __syncthreads();
        const int n = total - win < LIST_MAX ? total - win : LIST_MAX;
        const int ngroups = n / G;
        for (int q = wave; q < ngroups; q += NWV)
            fused_group<TI, NC, G>(a, list, q * G, lane, row_bytes, xf, yacc);
        // the tail entries (n % G), one at a time, on the wave whose turn is next
        for (int e0 = ngroups * G; e0 < n; ++e0)
            if (wave == (ngroups + (e0 - ngroups * G)) % NWV)
                fused_group<TI, NC, 1>(a, list, e0, lane, row_bytes, xf, yacc);
        __syncthreads();
    }

    // Partial rows of waves 1.. meet wave 0's in LDS; y = ((p0 + p1) + p2) + p3.
    if (wave > 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int q = 0; q < E / 4; ++q)
                *reinterpret_cast<float4 *>(&part[wave - 1][((lane + 64 * c) * E) + 4 * q]) =
                    make_float4(yacc[c][4 * q], yacc[c][4 * q + 1], yacc[c][4 * q + 2], yacc[c][4 * q + 3]);
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = lane + 64 * c;
            if (ch < a.nchunks) {
                float4 *dst = reinterpret_cast<float4 *>(yrow + (int64_t)ch * E);
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    float4 acc4 = make_float4(yacc[c][4 * q], yacc[c][4 * q + 1], yacc[c][4 * q + 2],
                                              yacc[c][4 * q + 3]);
#pragma unroll
                    for (int w = 0; w < NWV - 1; ++w) {
                        const float4 p4 = *reinterpret_cast<const float4 *>(&part[w][ch * E + 4 * q]);
                        acc4.x += p4.x;
                        acc4.y += p4.y;
                        acc4.z += p4.z;
                        acc4.w += p4.w;
                    }
                    dst[q] = acc4;
                }
            }
        }
    }
}

template <typename TI, int NC>
static hipError_t fused_go(const FusedArgs<TI> &a, hipStream_t s)
{
    if (a.T == 0)
        return hipSuccess;
    ffn_fused_kernel<TI, NC, 4><<<dim3(a.T), dim3(64 * NWV), 0, s>>>(a);
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
