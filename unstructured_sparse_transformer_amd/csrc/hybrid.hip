// hybrid.hip -- the ELL + dense-backup hybrid ("Sparser, Faster, Lighter
// Transformer Language Models", gist.science summary, section 2.3): rows whose
// nonzeros overflow the fixed ELL capacity are moved to a dense backup matrix,
// the rest stay in the compact ELL part; the partition is dynamic.
//
// Steps on the device, all on the caller's stream with no host round trip:
//   row_flags     row_ovf[t] = some tile of row t has cnt > cap
//   compact_rows  one workgroup turns the flags into the ascending overflow-row
//                 list and its length (workgroup prefix sum, no atomics), and
//                 the rows' entry counts into the fused step's work order
//   dense_gate    ReLU(x . W_g) for the listed rows  -> dense backup
//   gated_up      round(dense * (x . W_u))  for the listed rows -> workspace
//   down          (gated product) . W_d     -> y rows of the listed tokens
// The three GEMMs run with M = min(n_ovf, max_ovf) read on the device:
// workgroups past it return at once.
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

namespace twell {

// ------------------------------------------------------------------ partition
// One thread per row; VEC: the row's counts are read as 16-byte vectors.
// work[t] = stored entries of row t, sum over tiles of min(cnt, cap), or 0
// for an overflow row (its fused-step work is a row of zeros).
template <bool VEC>
__global__ __launch_bounds__(256) void row_flags_kernel(const int32_t *__restrict__ cnt, int T, int n_b, int cap,
                                                        int32_t *__restrict__ row_ovf, int32_t *__restrict__ work)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T)
        return;
    const int32_t *c = cnt + (int64_t)t * n_b;
    int f = 0, e = 0;
    if constexpr (VEC) {
        for (int b = 0; b < n_b; b += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(c + b);
            f |= (v.x > cap) | (v.y > cap) | (v.z > cap) | (v.w > cap);
            e += min(v.x, cap) + min(v.y, cap) + min(v.z, cap) + min(v.w, cap);
        }
    } else {
        for (int b = 0; b < n_b; ++b) {
            f |= c[b] > cap;
            e += min(c[b], cap);
        }
    }
    row_ovf[t] = f;
    work[t] = f ? 0 : e;
}

// Work classes of the fused step's schedule, heaviest = 7.
__device__ __forceinline__ int work_class(int e)
{
    return e == 0 ? 0 : e < 16 ? 1 : e < 32 ? 2 : e < 64 ? 3 : e < 128 ? 4 : e < 192 ? 5 : e < 256 ? 6 : 7;
}

// One workgroup, per chunk of 16384 rows: thread i owns rows [ROWS i, ROWS i +
// ROWS) of the chunk and reads their flags and work values with one batch of
// loads (16-byte vectors when VEC).  ROWS = 16 makes a pass one chunk; when
// all rows fit in 8192, ROWS = 8 covers them in one pass (the same single
// chunk) with half of each thread's serial work (layer_2b: 7.9 -> 6.5 us).  Nine per-thread counts (flagged rows;
// rows of each work class) go through one workgroup exclusive scan (DPP
// wave scans + 16 wave totals in LDS); each thread writes its flagged rows to
// the ascending overflow list and its rows to their places in the chunk's
// work order (classes from the heaviest, ascending rows inside a class),
// staged in LDS and written out coalesced.  `order` holds the rows' work
// values on entry; each chunk reads all of its values before the first
// barrier and writes only its own positions after it.  n_ovf is the true
// number of flagged rows.  WE: also order_e[i] = the work value of the row at
// work position i (staged in LDS beside the order), so that the fused step
// learns a row and its entry count in one load.
constexpr int CR_THREADS = 1024, CR_NC = 8, CR_CHUNK = 16384;  // rows per work-order chunk

template <bool VEC, int ROWS, bool WE>
__global__ __launch_bounds__(CR_THREADS) void compact_rows_kernel(const int32_t *__restrict__ row_ovf, int T,
                                                                  int max_ovf, int32_t *__restrict__ ovf_rows,
                                                                  int32_t *__restrict__ n_ovf, int32_t *order,
                                                                  int32_t *__restrict__ order_e)
{
    constexpr int NV = CR_NC + 1;  // scanned values: classes 0..7, flagged rows
    constexpr int NW = CR_THREADS / 64;
    constexpr int PASS = CR_THREADS * ROWS;  // rows per pass: a whole chunk, or (ROWS = 8) all T <= 8192 rows
    static_assert(PASS == CR_CHUNK || PASS * 2 == CR_CHUNK, "a pass is a chunk, or half of one used for T <= PASS");
    __shared__ int wave_tot[NW][NV];
    __shared__ int wave_off[NW + 1][NV];  // exclusive prefix over waves; row NW = totals
    __shared__ int sord[PASS];        // the chunk's work order
    __shared__ int swork[WE ? PASS : 1];  // the work values in that order
    const int tid = threadIdx.x, wave = tid >> 6;
    int base = 0;
    for (int t0 = 0; t0 < T; t0 += PASS) {
        const int nrows = T - t0 < PASS ? T - t0 : PASS;
        const int i0 = tid * ROWS;
        int fl[ROWS], wk[ROWS];
        if (VEC && i0 + ROWS <= nrows) {
#pragma unroll
            for (int q = 0; q < ROWS / 4; ++q) {
                const int4 f4 = *reinterpret_cast<const int4 *>(row_ovf + t0 + i0 + 4 * q);
                const int4 w4 = *reinterpret_cast<const int4 *>(order + t0 + i0 + 4 * q);
                fl[4 * q] = f4.x, fl[4 * q + 1] = f4.y, fl[4 * q + 2] = f4.z, fl[4 * q + 3] = f4.w;
                wk[4 * q] = w4.x, wk[4 * q + 1] = w4.y, wk[4 * q + 2] = w4.z, wk[4 * q + 3] = w4.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < ROWS; ++k) {
                const bool in = i0 + k < nrows;
                fl[k] = in ? row_ovf[t0 + i0 + k] : 0;
                wk[k] = in ? order[t0 + i0 + k] : 0;
            }
        }
        uint32_t bits = 0;
        uint64_t cls = 0;   // 4 bits per row: its work class
        uint64_t ccnt = 0;  // 8 bits per class: rows of this thread in it
#pragma unroll
        for (int k = 0; k < ROWS; ++k) {
            if (i0 + k < nrows) {
                bits |= fl[k] != 0 ? (1u << k) : 0u;
                const uint32_t c = (uint32_t)work_class(wk[k]);
                cls |= (uint64_t)c << (4 * k);
                ccnt += 1ull << (8 * c);
            }
        }
        int mine[NV], incl[NV];
#pragma unroll
        for (int v = 0; v < CR_NC; ++v)
            mine[v] = (int)((ccnt >> (8 * v)) & 0xFFu);
        mine[CR_NC] = __popc(bits);
#pragma unroll
        for (int v = 0; v < NV; ++v)
            incl[v] = wave_incl_scan_dpp(mine[v]);
        if ((tid & 63) == 63) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                wave_tot[wave][v] = incl[v];
        }
        __syncthreads();
        if (tid < NW * NV) {
            const int w = tid / NV, v = tid - w * NV;
            int off = 0;
            for (int q = 0; q < w; ++q)
                off += wave_tot[q][v];
            wave_off[w][v] = off;
            if (w == NW - 1)
                wave_off[NW][v] = off + wave_tot[w][v];
        }
        __syncthreads();
        int start[NV], tot[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            start[v] = wave_off[wave][v] + incl[v] - mine[v];  // this thread's first position inside value v
            tot[v] = wave_off[NW][v];
        }
        // overflow list
        int pos = base + start[CR_NC];
        uint32_t bb = bits;
        while (bb) {
            const int k = __ffs(bb) - 1;
            bb &= bb - 1;
            if (pos < max_ovf)
                ovf_rows[pos] = t0 + i0 + k;
            ++pos;
        }
        // work order: class c starts after all rows of the heavier classes
        int cpos[CR_NC];
        int above = 0;
#pragma unroll
        for (int c = CR_NC - 1; c >= 0; --c) {
            cpos[c] = above + start[c];
            above += tot[c];
        }
        uint64_t used = 0;  // 8 bits per class: rows placed so far
#pragma unroll
        for (int k = 0; k < ROWS; ++k) {
            if (i0 + k < nrows) {
                const int c = (int)((cls >> (4 * k)) & 0xFu);
                int p = 0;
#pragma unroll
                for (int q = 0; q < CR_NC; ++q)
                    p = c == q ? cpos[q] : p;
                sord[p + (int)((used >> (8 * c)) & 0xFFu)] = t0 + i0 + k;
                if (WE)
                    swork[p + (int)((used >> (8 * c)) & 0xFFu)] = wk[k];
                used += 1ull << (8 * c);
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < ROWS; ++k) {
            const int i = k * CR_THREADS + tid;
            if (i < nrows) {
                order[t0 + i] = sord[i];
                if (WE)
                    order_e[t0 + i] = swork[i];
            }
        }
        base += tot[CR_NC];
        __syncthreads();
    }
    if (tid == 0)
        n_ovf[0] = base;
}

hipError_t launch_row_flags(const int32_t *cnt, int T, int n_b, int cap, int32_t *row_ovf, int32_t *work,
                            hipStream_t s)
{
    const bool vec = (n_b % 4 == 0) && ((reinterpret_cast<uintptr_t>(cnt) & 15u) == 0);
    if (vec)
        row_flags_kernel<true><<<dim3((T + 255) / 256), dim3(256), 0, s>>>(cnt, T, n_b, cap, row_ovf, work);
    else
        row_flags_kernel<false><<<dim3((T + 255) / 256), dim3(256), 0, s>>>(cnt, T, n_b, cap, row_ovf, work);
    return hipGetLastError();
}

template <bool WE>
static void compact_rows_go(bool vec, bool one_pass8, const int32_t *row_ovf, int T, int max_ovf, int32_t *ovf_rows,
                            int32_t *n_ovf, int32_t *order, int32_t *order_e, hipStream_t s)
{
    const dim3 g(1), b(CR_THREADS);
    if (vec && one_pass8)
        compact_rows_kernel<true, 8, WE><<<g, b, 0, s>>>(row_ovf, T, max_ovf, ovf_rows, n_ovf, order, order_e);
    else if (vec)
        compact_rows_kernel<true, 16, WE><<<g, b, 0, s>>>(row_ovf, T, max_ovf, ovf_rows, n_ovf, order, order_e);
    else if (one_pass8)
        compact_rows_kernel<false, 8, WE><<<g, b, 0, s>>>(row_ovf, T, max_ovf, ovf_rows, n_ovf, order, order_e);
    else
        compact_rows_kernel<false, 16, WE><<<g, b, 0, s>>>(row_ovf, T, max_ovf, ovf_rows, n_ovf, order, order_e);
}

hipError_t launch_compact_rows(const int32_t *row_ovf, int T, int max_ovf, int32_t *ovf_rows, int32_t *n_ovf,
                               int32_t *order, hipStream_t s, int32_t *order_e)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(row_ovf) | reinterpret_cast<uintptr_t>(order)) & 15u) == 0;
    const bool one_pass8 = T <= CR_THREADS * 8;  // ROWS = 8 only where its single pass is the single chunk
    if (order_e)
        compact_rows_go<true>(vec, one_pass8, row_ovf, T, max_ovf, ovf_rows, n_ovf, order, order_e, s);
    else
        compact_rows_go<false>(vec, one_pass8, row_ovf, T, max_ovf, ovf_rows, n_ovf, order, nullptr, s);
    return hipGetLastError();
}

// Compile-time tuning knobs of the small-M GEMMs (-D on the compiler line),
// defaults as measured best at the 2B-like layer: HB_* the separate gate and
// up GEMMs, DU_* the dual gate/up GEMM, DN_* the down GEMM (N tile width,
// stage width in bytes, ring depth, workgroups per CU, wave tile width, most
// K splits; DU_DB the W_g / W_u block height, DU_BN the B tile's rows).
// Shapes the knobs do not cover are the constants further down.
#ifndef HB_BN
#define HB_BN 128
#endif
#ifndef HB_WN
#define HB_WN 64
#endif
#ifndef HB_KB
#define HB_KB 128
#endif
#ifndef HB_STAGES
#define HB_STAGES 3
#endif
#ifndef HB_PER_CU
#define HB_PER_CU 2
#endif
#ifndef DN_PER_CU
#define DN_PER_CU 3
#endif
#ifndef DU_STAGES
#define DU_STAGES 4
#endif
#ifndef DU_PER_CU
#define DU_PER_CU 1
#endif
#ifndef DN_KB
#define DN_KB 128
#endif
#ifndef DN_STAGES
#define DN_STAGES 2
#endif
#ifndef DN_WN
#define DN_WN 64
#endif
#ifndef DN_BN
#define DN_BN 128
#endif
#ifndef DN_MAX_SPLITS
#define DN_MAX_SPLITS 16
#endif
#ifndef DN_TARGET_WGS
#define DN_TARGET_WGS 512
#endif
#ifndef DN_ROWS_HINT
#define DN_ROWS_HINT 256
#endif
#ifndef DN_PART_MB
#define DN_PART_MB 256
#endif
#ifndef DU_BM
#define DU_BM 128
#endif
#ifndef DU_DB
#define DU_DB 32
#endif
#ifndef DU_BN
#define DU_BN 128
#endif

// ------------------------------------------------------------------ dense GEMMs
template <typename TI> struct DenseOut {
    TI *out;            // [max_ovf][N]
    const TI *gate;     // MODE 1: dense backup [max_ovf][N]
};

__device__ __forceinline__ int rows_used(const GemmArgs &p)
{
    const int n = *p.m_count;
    return n < p.M ? n : p.M;
}

// MODE 0: out = ReLU(acc) (dense backup).  MODE 1: out = round(gate * acc).
// The grid is at most one workgroup per CU; workgroup g takes output tiles
// t = g, g + gridDim.x, ... of the tiles that cover the rows in use (M tiles
// slowest), so no workgroup is launched for rows past n_ovf.  With the grid
// and the N-tile count multiples of 8, every tile of one N column (one B
// tile) lands on the same XCD.
template <typename TI, int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void dense_epi_kernel(GemmArgs p, DenseOut<TI> o)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, false, HB_KB, HB_STAGES>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    const int m_used = rows_used(p);
    const int ntiles = (m_used + BM - 1) / BM * p.NT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Core::NWN, wn = wave % Core::NWN;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int nt = t % p.NT, mt = t / p.NT;
        const int m0 = mt * BM, n0 = nt * BN;
        Core core;
        f32x16 acc[Core::FM][Core::FN];
        core.run(p, smem, m0, n0, m_used, p.k_begin, p.k_len, tid, acc);
#pragma unroll
        for (int fm = 0; fm < Core::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Core::FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + fm * 32 + acc_row(i, lane);
                    const int n = n0 + wn * WN + fn * 32 + (lane & 31);
                    if (m < m_used && n < p.N) {
                        const int64_t off = (int64_t)m * p.N + n;
                        const float v = acc[fm][fn][i];
                        if (MODE == 0)
                            store_elem(o.out + off, v > 0.f ? v : 0.f);
                        else
                            store_elem(o.out + off, load_elem(o.gate + off) * v);
                    }
                }
    }
}

// Dense backup and gated up product of the overflow rows in one GEMM: the
// workgroup's B tile interleaves DB-row blocks of W_g^T and W_u^T (the core's
// dual mode), so for each of its BN/2 output columns a lane holds both
// z = x . W_g and u = x . W_u.  Writes dense = round(ReLU(z)) and
// prod = round(dense * u): the values of dense_epi_kernel's two modes, with
// the same accumulation order, from one pass over A.  Same tile loop.
template <typename TI> struct DualOut {
    TI *dense;  // [max_ovf][N]
    TI *prod;   // [max_ovf][N]
};

template <typename TI, int BM, int BN, int WM, int DB>
__global__ __launch_bounds__((BM / WM) * (BN / (2 * DB)) * 64) void dual_epi_kernel(GemmArgs p, DualOut<TI> o)
{
    using Core = GemmCore<TI, BM, BN, WM, 2 * DB, false, HB_KB, DU_STAGES, DB>;
    constexpr int ZB = DB / 32;  // 32-column blocks of each product per wave
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    const int m_used = rows_used(p);
    const int ntiles = (m_used + BM - 1) / BM * p.NT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Core::NWN, wn = wave % Core::NWN;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int nt = t % p.NT, mt = t / p.NT;
        const int m0 = mt * BM, n0 = nt * (BN / 2);
        Core core;
        f32x16 acc[Core::FM][Core::FN];
        core.run(p, smem, m0, n0, m_used, p.k_begin, p.k_len, tid, acc);
#pragma unroll
        for (int fm = 0; fm < Core::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < ZB; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + fm * 32 + acc_row(i, lane);
                    const int n = n0 + wn * DB + fn * 32 + (lane & 31);
                    if (m < m_used && n < p.N) {
                        const int64_t off = (int64_t)m * p.N + n;
                        const float z = acc[fm][fn][i];
                        const TI hv = (TI)(z > 0.f ? z : 0.f);
                        o.dense[off] = hv;
                        store_elem(o.prod + off, (float)hv * acc[fm][fn + ZB][i]);
                    }
                }
    }
}

template <typename TI> struct DownOut {
    float *part;           // [splits][M][N] when splits > 1
    float *y;              // [*][N]
    const int32_t *rows;   // output row of local row m
    int splits;
};

// Same tile loop as dense_epi_kernel over (M tile, split, N tile), N tile fastest.
template <typename TI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void down_kernel(GemmArgs p, DownOut<TI> o)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, true, DN_KB, DN_STAGES>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    const int m_used = rows_used(p);
    const int per_m = p.NT * o.splits;
    const int ntiles = (m_used + BM - 1) / BM * per_m;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Core::NWN, wn = wave % Core::NWN;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int mt = t / per_m, u = t - mt * per_m;
        const int sidx = u / p.NT, nt = u - sidx * p.NT;
        const int m0 = mt * BM, n0 = nt * BN;
        Core core;
        f32x16 acc[Core::FM][Core::FN];
        core.run(p, smem, m0, n0, m_used, p.k_begin + sidx * p.k_split_len, p.k_split_len, tid, acc);
#pragma unroll
        for (int fm = 0; fm < Core::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Core::FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + fm * 32 + acc_row(i, lane);
                    const int n = n0 + wn * WN + fn * 32 + (lane & 31);
                    if (m < m_used && n < p.N) {
                        if (o.splits == 1)
                            o.y[(int64_t)o.rows[m] * p.N + n] = acc[fm][fn][i];
                        else
                            o.part[((int64_t)sidx * p.M + m) * p.N + n] = acc[fm][fn][i];
                    }
                }
    }
}

// y[rows[m]][n] = sum over splits s (in order) of part[s][m][n].
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ part, int splits, int M_cap,
                                                           const int32_t *__restrict__ m_count, int N,
                                                           const int32_t *__restrict__ rows, float *__restrict__ y)
{
    const int mc = *m_count;
    const int m_used = mc < M_cap ? mc : M_cap;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N)
        return;
    for (int m = blockIdx.y; m < m_used; m += gridDim.y) {
        // every slab's loads first (at most DN_MAX_SPLITS), then the sum in slab order
        float4 v[DN_MAX_SPLITS];
#pragma unroll
        for (int s = 0; s < DN_MAX_SPLITS; ++s)
            v[s] = s < splits ? *reinterpret_cast<const float4 *>(part + ((int64_t)s * M_cap + m) * N + n)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 acc = v[0];
#pragma unroll
        for (int s = 1; s < DN_MAX_SPLITS; ++s) {
            if (s < splits) {
                acc.x += v[s].x;
                acc.y += v[s].y;
                acc.z += v[s].z;
                acc.w += v[s].w;
            }
        }
        *reinterpret_cast<float4 *>(y + (int64_t)rows[m] * N + n) = acc;
    }
}

// Small-M tile shapes for the hybrid GEMMs (M = overflow rows, a few hundred;
// they stream whole weight matrices, so each workgroup keeps several K stages
// of copies in flight): gate / up: 64 x 128 per workgroup, 4 waves, 3-deep
// ring of 128-byte K stages (72 KiB), two workgroups per CU; down: 64 x 128,
// 4 waves of 32 x 64, 2-deep ring of raw W_d stages (bf16: read with
// transposing LDS reads, 48 KiB; fp32: transposed in LDS, 64 KiB), split
// over K, three workgroups per CU where they fit (a 3-deep ring with two per
// CU measured no faster).
constexpr int HB_BM = 64, HB_WM = 32;
#ifndef DN_BM
#define DN_BM 64
#endif
#ifndef DN_WM
#define DN_WM 32
#endif
// Dual gate / up GEMM: 128 rows x 64 output columns per workgroup (a
// 128-row B tile of 32-row W_g / W_u blocks), 4 waves of 64 x 64, 4-deep
// ring of 32 KiB stages (128 KiB), one workgroup per CU.  Against 64-row
// tiles (two 72 KiB workgroups per CU) it moves a third fewer L2->LDS bytes
// for a few hundred rows: measured 1-2 us faster per call at 211 and 328
// overflow rows, no slower at 1.
#ifndef DU_WM
#define DU_WM 64
#endif

// Workgroups for a tile loop: one per CU, at most `tiles`, rounded down to a
// multiple of 8 when that many (keeps N columns on one XCD).
static int loop_grid(long tiles, int per_cu = 1)
{
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const long slots = (long)ncu * per_cu;
    long g = tiles < slots ? tiles : slots;
    if (g >= 8)
        g &= ~7L;
    return (int)(g > 0 ? g : 1);
}

template <typename TI, int MODE>
static hipError_t dense_go(const void *x, int T, const void *w_t, const int32_t *ovf_rows, const int32_t *n_ovf,
                           int max_ovf, int d, int F, const void *gate, void *out, hipStream_t s)
{
    if (max_ovf == 0)
        return hipSuccess;
    GemmArgs p{};
    p.A = x;
    p.lda = d;
    p.a_rows = ovf_rows;
    p.M = max_ovf;
    p.m_count = n_ovf;
    p.B = w_t;
    p.ldb = d;
    p.N = F;
    p.k_begin = 0;
    p.k_len = d;
    p.MT = (max_ovf + HB_BM - 1) / HB_BM;
    p.NT = (F + HB_BN - 1) / HB_BN;
    p.a_bytes = (uint32_t)((int64_t)T * d * sizeof(TI));
    p.b_bytes = (uint32_t)((int64_t)F * d * sizeof(TI));
    DenseOut<TI> o{static_cast<TI *>(out), static_cast<const TI *>(gate)};
    dense_epi_kernel<TI, HB_BM, HB_BN, HB_WM, HB_WN, MODE>
        <<<dim3(loop_grid((long)p.MT * p.NT, HB_PER_CU)), dim3((HB_BM / HB_WM) * (HB_BN / HB_WN) * 64), 0, s>>>(p, o);
    return hipGetLastError();
}

hipError_t launch_dense_gate(int vdtype, const void *x, int T, const void *wg_t, const int32_t *ovf_rows,
                             const int32_t *n_ovf, int max_ovf, int d, int F, void *dense, hipStream_t s)
{
    if (vdtype == 1)
        return dense_go<__bf16, 0>(x, T, wg_t, ovf_rows, n_ovf, max_ovf, d, F, nullptr, dense, s);
    return dense_go<float, 0>(x, T, wg_t, ovf_rows, n_ovf, max_ovf, d, F, nullptr, dense, s);
}

hipError_t launch_gated_up(int vdtype, const void *x, int T, const void *wu_t, const int32_t *ovf_rows,
                           const int32_t *n_ovf, int max_ovf, int d, int F, const void *dense, void *pbuf,
                           hipStream_t s)
{
    if (vdtype == 1)
        return dense_go<__bf16, 1>(x, T, wu_t, ovf_rows, n_ovf, max_ovf, d, F, dense, pbuf, s);
    return dense_go<float, 1>(x, T, wu_t, ovf_rows, n_ovf, max_ovf, d, F, dense, pbuf, s);
}

template <typename TI>
static hipError_t dual_go(const void *x, int T, const void *wg_t, const void *wu_t, const int32_t *ovf_rows,
                          const int32_t *n_ovf, int max_ovf, int d, int F, void *dense, void *prod, hipStream_t s)
{
    if (max_ovf == 0)
        return hipSuccess;
    GemmArgs p{};
    p.A = x;
    p.lda = d;
    p.a_rows = ovf_rows;
    p.M = max_ovf;
    p.m_count = n_ovf;
    p.B = wg_t;
    p.B2 = wu_t;
    p.ldb = d;
    p.N = F;
    p.k_begin = 0;
    p.k_len = d;
    p.MT = (max_ovf + DU_BM - 1) / DU_BM;
    p.NT = (F + DU_BN / 2 - 1) / (DU_BN / 2);
    p.a_bytes = (uint32_t)((int64_t)T * d * sizeof(TI));
    p.b_bytes = (uint32_t)((int64_t)F * d * sizeof(TI));
    DualOut<TI> o{static_cast<TI *>(dense), static_cast<TI *>(prod)};
    dual_epi_kernel<TI, DU_BM, DU_BN, DU_WM, DU_DB>
        <<<dim3(loop_grid((long)p.MT * p.NT, DU_PER_CU)), dim3((DU_BM / DU_WM) * (DU_BN / (2 * DU_DB)) * 64), 0, s>>>(p, o);
    return hipGetLastError();
}

hipError_t launch_dense_gate_up(int vdtype, const void *x, int T, const void *wg_t, const void *wu_t,
                                const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf, int d, int F, void *dense,
                                void *pbuf, hipStream_t s)
{
    if (vdtype == 1)
        return dual_go<__bf16>(x, T, wg_t, wu_t, ovf_rows, n_ovf, max_ovf, d, F, dense, pbuf, s);
    return dual_go<float>(x, T, wg_t, wu_t, ovf_rows, n_ovf, max_ovf, d, F, dense, pbuf, s);
}

int down_splits(int max_ovf, int F, int d)
{
    // The rows in use (n_ovf) are known only on the device; size the split for
    // about DN_ROWS_HINT of them (a few hundred overflow rows is the usual
    // case): about two (tile, split) pairs per CU, K slices whole multiples of
    // 64, and the partial slabs ([splits][max_ovf][d] fp32) at most DN_PART_MB
    // of workspace.  At the 2B-like layer (211 rows) that is 8 splits of 1024
    // K elements: 18 us for the down GEMM, against 26 us with 4 splits (K
    // chains twice as long) and 25 us with 16 (twice the partial traffic).
    const long tiles = (long)((DN_ROWS_HINT + DN_BM - 1) / DN_BM) * ((d + DN_BN - 1) / DN_BN);
    const long slab = (long)max_ovf * d * 4;
    int s = 1;
    while (s < DN_MAX_SPLITS && tiles * s < DN_TARGET_WGS && F % (s * 2 * 64) == 0 &&
           slab * s * 2 <= ((long)DN_PART_MB << 20))
        s *= 2;
    return s;
}

template <typename TI>
static hipError_t down_go(const void *pbuf, const void *wd, const int32_t *ovf_rows, const int32_t *n_ovf,
                          int max_ovf, int F, int d, float *y, float *part, int splits, hipStream_t s)
{
    if (max_ovf == 0)
        return hipSuccess;
    GemmArgs p{};
    p.A = pbuf;
    p.lda = F;
    p.M = max_ovf;
    p.m_count = n_ovf;
    p.B = wd;
    p.ldb = d;
    p.N = d;
    p.k_begin = 0;
    p.k_len = F;
    p.k_split_len = F / splits;
    p.MT = (max_ovf + DN_BM - 1) / DN_BM;
    p.NT = (d + DN_BN - 1) / DN_BN;
    p.a_bytes = (uint32_t)((int64_t)max_ovf * F * sizeof(TI));
    p.b_bytes = (uint32_t)((int64_t)F * d * sizeof(TI));
    DownOut<TI> o{part, y, ovf_rows, splits};
    down_kernel<TI, DN_BM, DN_BN, DN_WM, DN_WN>
        <<<dim3(loop_grid((long)p.MT * p.NT * splits, DN_PER_CU)), dim3((DN_BM / DN_WM) * (DN_BN / DN_WN) * 64), 0, s>>>(p, o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    split_reduce_kernel<<<dim3((d / 4 + 255) / 256, max_ovf < 512 ? max_ovf : 512), dim3(256), 0, s>>>(part, splits, max_ovf, n_ovf, d,
                                                                             ovf_rows, y);
    return hipGetLastError();
}

hipError_t launch_down(int vdtype, const void *pbuf, const void *wd, const int32_t *ovf_rows, const int32_t *n_ovf,
                       int max_ovf, int F, int d, float *y, float *part, int splits, hipStream_t s)
{
    if (vdtype == 1)
        return down_go<__bf16>(pbuf, wd, ovf_rows, n_ovf, max_ovf, F, d, y, part, splits, s);
    return down_go<float>(pbuf, wd, ovf_rows, n_ovf, max_ovf, F, d, y, part, splits, s);
}

}  // namespace twell
