// ffn_fused.hip -- fused up/down projection straight from TwELL.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.2: with the gate activation h_g in TwELL, the up and
// down projections become one kernel that, for each nonzero h_g[j], reads
// only the weights it needs (column j of W_u, row j of W_d), takes a dot
// product and a scalar product, and accumulates -- DRAM traffic is the point.
//
// gfx950 mapping: one workgroup of 4 waves per token, started in a given
// work order (tokens with the most entries first, so that they do not trail
// at the end of the launch while the light ones have long finished).  Each wave keeps the
// token's x row and a partial y row in registers (chunk c of lane l covers
// elements (l + 64c)*E .. +E, so every weight-row read is one fully coalesced
// 16-byte-per-lane sweep).  The token's TwELL entries are compacted into an LDS
// list of (j, h) in ascending j (wave prefix sum over the per-tile counts) and
// dealt to the waves G at a time (G = 1), so heavy tokens (hundreds of
// entries) run 4 latency chains in parallel; the next group's 2*G weight rows
// are in flight while a wave reduces the current one, the dot products are
// reduced with DPP, and y += (h*u) * W_d[j] runs in fp32.
// The partial rows are added in LDS in a fixed order: no atomics, and the
// result does not depend on timing.
#include "decode.h"
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

// Entries per group (G).  One entry per group keeps the 2B-shaped kernel at
// 166 VGPRs: three waves per SIMD, three tokens per CU in flight (two at
// G = 2, 234 VGPRs), which the latency-bound light and empty rows need.
#ifndef FUSED_G
#define FUSED_G 1
#endif

namespace twell {

#ifndef FUSED_WAVES
#define FUSED_WAVES 4
#endif
constexpr int NWV = FUSED_WAVES;  // waves per token

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

// One workgroup of NWV waves per token.  Wave w owns the TwELL tiles
// b = w, w + NWV, w + 2 NWV, ...: it reads their counts, indices and values
// itself, compacts its entries (ascending tile, then slot) into a private LDS
// list of at most WLIST entries at a time, and streams them G at a time.  No
// barrier is needed until the NWV partial y rows meet in LDS, where every wave
// adds a quarter of the columns in wave order.  Tokens without entries and
// overflow rows get y = 0.
constexpr int WLIST = 128;  // entries per wave per pass

template <typename TI, int NC, int G>
__global__ __launch_bounds__(64 * NWV) void ffn_fused_kernel(FusedArgs<TI> a)
{
    constexpr int E = Elt<TI>::PER_CHUNK;
    constexpr int YW = NC * 64 * E;  // floats of one partial y row (>= d)
    __shared__ int2 wlist[NWV][WLIST];
    __shared__ __attribute__((aligned(16))) float part[NWV][YW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int t = blockIdx.x;
    if (a.order) {
        t = a.order[t];
        if ((unsigned)t >= (unsigned)a.T)
            return;  // not a permutation: this row is not ours to write
    }
    const int64_t row_bytes = (int64_t)a.d * Elt<TI>::SIZE;
    float *yrow = a.y + (int64_t)t * a.d;

    // Overflow test over the whole row (every wave, same answer).
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

    XRow<TI, NC> xf;
    float yacc[NC][E];
    const char *xrow = (const char *)a.x + (int64_t)t * row_bytes;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
            yacc[c][e] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        xf.set(c, ch < a.nchunks ? ldg16(xrow + ch * 16) : u32x4{0, 0, 0, 0});
    }

    // This wave's tiles: b = wave + NWV * l for l = 0, 1, ...; lane l holds tile l.
    const int my_tiles = (a.n_b - wave + NWV - 1) / NWV;
    const bool vec = a.cap % 16 == 0 && (reinterpret_cast<uintptr_t>(a.idx) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.val) & 15u) == 0;
    int2 *list = wlist[wave];
    for (int l0 = 0; l0 < my_tiles; l0 += 64) {
        const int l = l0 + lane;
        const int b = wave + NWV * l;
        int c = l < my_tiles ? crow[b] : 0;
        c = c < a.cap ? c : a.cap;
        const int incl = wave_incl_scan(c, lane);
        const int ctot = __shfl(incl, 63, 64);
        const int64_t slot0 = ((int64_t)t * a.n_b + b) * a.cap;
        for (int win = 0; win < ctot; win += WLIST) {
            const int excl = incl - c - win;  // position of this tile's first entry in the window
            if (vec) {
                for (int s0 = 0; s0 < c; s0 += 16) {
                    if (excl + s0 >= WLIST || excl + s0 + 16 <= 0)
                        continue;
                    const u32x4 iw = ldg16(a.idx + slot0 + s0);
                    u32x4 vw[16 / E];
#pragma unroll
                    for (int q = 0; q < 16 / E; ++q)
                        vw[q] = ldg16(a.val + slot0 + s0 + q * E);
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const int pos = excl + s0 + k;
                        if (s0 + k < c && pos >= 0 && pos < WLIST) {
                            int j = b * a.tile_w + (int)((iw[k >> 2] >> (8 * (k & 3))) & 0xFFu);
                            j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
                            list[pos] = make_int2(j, __float_as_int(chunk_elem<TI>(vw[k / E], k % E)));
                        }
                    }
                }
            } else {
                for (int s = 0; s < c; ++s) {
                    const int pos = excl + s;
                    if (pos >= 0 && pos < WLIST) {
                        int j = b * a.tile_w + a.idx[slot0 + s];
                        j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
                        list[pos] = make_int2(j, __float_as_int(load_elem(a.val + slot0 + s)));
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's list stores are done
            __builtin_amdgcn_wave_barrier();
            const int n = ctot - win < WLIST ? ctot - win : WLIST;
            const int ngroups = n / G;
            group_stream<TI, NC, G>(a, list, 0, 1, ngroups, lane, row_bytes, xf, yacc);
            for (int e0 = ngroups * G; e0 < n; ++e0) {
                Group<TI, NC, 1> g1;
                group_load<TI, NC, 1>(a, list, e0, lane, row_bytes, g1);
                group_apply<TI, NC, 1>(g1, xf, yacc);
            }
            __builtin_amdgcn_wave_barrier();  // list reads done before the next window's stores
        }
    }

    // The NWV partial rows meet in LDS; wave w adds columns [w d/NWV, (w+1) d/NWV)
    // as ((p0 + p1) + p2) + p3.
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < E / 4; ++q)
            *reinterpret_cast<float4 *>(&part[wave][((lane + 64 * c) * E) + 4 * q]) =
                make_float4(yacc[c][4 * q], yacc[c][4 * q + 1], yacc[c][4 * q + 2], yacc[c][4 * q + 3]);
    __syncthreads();
    for (int i = tid * 4; i < a.d; i += 64 * NWV * 4) {
        float4 acc4 = *reinterpret_cast<const float4 *>(&part[0][i]);
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            const float4 p4 = *reinterpret_cast<const float4 *>(&part[w][i]);
            acc4.x += p4.x;
            acc4.y += p4.y;
            acc4.z += p4.z;
            acc4.w += p4.w;
        }
        *reinterpret_cast<float4 *>(yrow + i) = acc4;
    }
}

template <typename TI, int NC>
static hipError_t fused_go(const FusedArgs<TI> &a, hipStream_t s)
{
    if (a.T == 0)
        return hipSuccess;
    ffn_fused_kernel<TI, NC, FUSED_G><<<dim3(a.T), dim3(64 * NWV), 0, s>>>(a);
    return hipGetLastError();
}

template <typename TI>
static hipError_t fused_dispatch(const int32_t *cnt, const void *val, const uint8_t *idx, const int32_t *order,
                                 int T, int F, int tile_w, int cap, const void *x, const void *wu_t, const void *wd,
                                 int d, float *y, hipStream_t s)
{
    FusedArgs<TI> a{cnt, static_cast<const TI *>(val), idx, order, T, F / tile_w, tile_w, cap, F,
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

hipError_t launch_ffn_fused(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx, const int32_t *order,
                            int T, int F, int tile_w, int cap, const void *x, const void *wu_t, const void *wd, int d,
                            float *y, hipStream_t s)
{
    if (vdtype == 1)
        return fused_dispatch<__bf16>(cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, s);
    return fused_dispatch<float>(cnt, val, idx, order, T, F, tile_w, cap, x, wu_t, wd, d, y, s);
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
