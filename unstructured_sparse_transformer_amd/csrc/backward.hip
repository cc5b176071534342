// backward.hip -- backward pass of the ReLU-sparse gated FFN on the hybrid.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.4: training runs the sparse FFN forward and backward on
// the ELL + dense-backup hybrid.  With y = sum over active j of
// h_j (x . W_u^T[j]) W_d[j] and dy given, every gradient term lives on an
// active (row, neuron) entry (ReLU's derivative is 0 elsewhere):
//   u = x_t . W_u^T[j],  g = dy_t . W_d[j],  du = g h,  dz = g u,
//   dx_t += du W_u^T[j] + dz W_g^T[j],
//   dW_d[j] += (h u) dy_t,  dW_u^T[j] += du x_t,  dW_g^T[j] += dz x_t.
// The work is organised twice over the same entry list:
//   token-major (dx): a row's entries cut into chunks of BW_CE, one wave per
//     chunk, three weight rows per entry streamed with the next entry's rows
//     requested early; the chunk writes its entries' du, dz, h u and a
//     partial dx row, added per row in chunk order;
//   neuron-major (dW): the entries regrouped by neuron in ascending row order
//     (a stable counting sort: per block of BW_RC rows a histogram, per neuron
//     a scan over the blocks, then each block places its rows' entries in row
//     order -- a row holds a neuron once, so no two entries of a row collide),
//     one wave per neuron summing x and dy rows into its three gradient rows.
// Every sum runs in a fixed order: the results do not depend on timing.
// Entry list: a fitting row's TwELL entries (ascending column), a held
// overflow row's nonzero dense-backup values; an overflow row without a dense
// row (past max_ovf) has none.
#include "backward.h"
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

namespace twell {

// ------------------------------------------------------------------ counts
// One wave per row: its entries and where they come from.  Also clears the
// per-block neuron histogram (grid-stride).
__global__ __launch_bounds__(256) void bw_count_kernel(BwArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < (int64_t)a.n_rc * a.F;
         i += (int64_t)gridDim.x * 256)
        a.ws.cnt_rc[i] = 0;
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T)
        return;
    int e = 0, src = -1;  // src: dense row index of a held overflow row, -1 fitting, -2 not held
    if (!a.row_ovf[t]) {
        const int32_t *crow = a.cnt + (int64_t)t * a.n_b;
        for (int b0 = 0; b0 < a.n_b; b0 += 64)
            e += wave_isum(b0 + lane < a.n_b ? crow[b0 + lane] : 0);
    } else {
        const int nd = *a.n_ovf < a.max_ovf ? *a.n_ovf : a.max_ovf;
        int lo = 0, hi = nd - 1;
        src = -2;
        while (lo <= hi) {  // ovf_rows ascends
            const int mid = (lo + hi) >> 1;
            const int r = a.ovf_rows[mid];
            if (r == t) {
                src = mid;
                break;
            }
            if (r < t)
                lo = mid + 1;
            else
                hi = mid - 1;
        }
        if (src >= 0) {  // nonzeros of the dense row, 8 columns (16 bytes) per lane
            const char *dr = reinterpret_cast<const char *>(a.dense + (int64_t)src * a.F);
            const int nch = a.F / 8;
            int mine = 0;
            for (int c = lane; c < nch; c += 64) {
                const u32x4 v = ldg16(dr + (int64_t)c * 16);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    mine += chunk_elem<__bf16>(v, q) > 0.f ? 1 : 0;
            }
            e = wave_isum(mine);
        }
    }
    if (lane == 0) {
        a.ws.row_e[t] = e;
        a.ws.row_src[t] = src;
    }
}

// One workgroup: row_ptr and chunk0 (exclusive scans over the rows), the
// entry total and the status word.
__global__ __launch_bounds__(1024) void bw_scan_kernel(BwArgs a)
{
    constexpr int NWV = 16;
    __shared__ int wt[2][NWV];
    __shared__ int carry[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry[0] = carry[1] = 0;
    }
    __syncthreads();
    for (int base = 0; base < a.T; base += 1024) {
        const int t = base + tid;
        const int e = t < a.T ? a.ws.row_e[t] : 0;
        const int c = (e + BW_CE - 1) / BW_CE;
        const int ie = wave_incl_scan(e, lane), ic = wave_incl_scan(c, lane);
        if (lane == 63) {
            wt[0][wave] = ie;
            wt[1][wave] = ic;
        }
        __syncthreads();
        int be = carry[0], bc = carry[1];
        for (int w = 0; w < wave; ++w) {
            be += wt[0][w];
            bc += wt[1][w];
        }
        if (t < a.T) {
            a.ws.row_ptr[t] = be + ie - e;
            a.ws.chunk0[t] = bc + ic - c;
        }
        __syncthreads();
        if (tid == 1023) {
            carry[0] = be + ie;
            carry[1] = bc + ic;
        }
        __syncthreads();
    }
    const bool too_many = carry[0] > a.max_entries;
    if (tid == 0) {
        a.ws.row_ptr[a.T] = carry[0];
        a.ws.chunk0[a.T] = too_many ? 0 : carry[1];
        a.ws.status[0] = carry[0];
        a.ws.status[1] = too_many ? 1 : 0;
    }
    if (too_many)  // no chunks: dx comes out as zeros
        for (int t = tid; t < a.T; t += 1024)
            a.ws.chunk0[t] = 0;
}

// chunk -> row map (one thread per row)
__global__ __launch_bounds__(256) void bw_chunk_rows_kernel(BwArgs a)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= a.T || a.ws.status[1])
        return;
    for (int c = a.ws.chunk0[t]; c < a.ws.chunk0[t + 1]; ++c)
        a.ws.chunk_row[c] = t;
}

// ------------------------------------------------------------------ entry list
// One wave per row: (j, h) of its entries in ascending j at row_ptr[t].
__global__ __launch_bounds__(256) void bw_entries_kernel(BwArgs a)
{
    __shared__ int spre[4][BW_MAX_NB + 1];
    if (a.ws.status[1])
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T)
        return;
    const int src = a.ws.row_src[t];
    const int p0 = a.ws.row_ptr[t];
    if (src == -1) {
        int *sp = spre[wave];
        const int32_t *crow = a.cnt + (int64_t)t * a.n_b;
        int run = 0;
        for (int b0 = 0; b0 < a.n_b; b0 += 64) {
            const int b = b0 + lane;
            const int c = b < a.n_b ? crow[b] : 0;
            const int incl = wave_incl_scan(c, lane);
            if (b < a.n_b)
                sp[b] = run + incl - c;
            run += __shfl(incl, 63, 64);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        for (int k = lane; k < run; k += 64) {
            int lo = 0, hi = a.n_b - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sp[mid] <= k)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int64_t slot = ((int64_t)t * a.n_b + lo) * a.cap + (k - sp[lo]);
            int j = lo * a.tile_w + a.idx[slot];
            j = j < a.F ? j : a.F - 1;  // memory safety for a corrupt index
            a.ws.ent_j[p0 + k] = j;
            a.ws.ent_h[p0 + k] = (float)a.val[slot];
        }
    } else if (src >= 0) {
        // nonzeros of the dense row in ascending column: 8 columns per lane,
        // a wave scan of the lanes' counts places them
        const char *dr = reinterpret_cast<const char *>(a.dense + (int64_t)src * a.F);
        const int nch = a.F / 8;
        int base = p0;
        for (int c0 = 0; c0 < nch; c0 += 64) {
            const int c = c0 + lane;
            const u32x4 v = c < nch ? ldg16(dr + (int64_t)c * 16) : u32x4{0, 0, 0, 0};
            int mine = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                mine += chunk_elem<__bf16>(v, q) > 0.f ? 1 : 0;
            const int incl = wave_incl_scan(mine, lane);
            int pos = base + incl - mine;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float h = chunk_elem<__bf16>(v, q);
                if (h > 0.f) {
                    a.ws.ent_j[pos] = c * 8 + q;
                    a.ws.ent_h[pos] = h;
                    ++pos;
                }
            }
            base += __shfl(incl, 63, 64);
        }
    }
}

// ------------------------------------------------------------------ token-major: dx
// Three weight rows of one entry in registers (lane l, chunk c: elements
// (l + 64 c) * 8 .. +8).
template <int NC> struct BwRows {
    u32x4 wu[NC], wd[NC], wg[NC];
};

template <int NC>
__device__ __forceinline__ void bw_load_rows(const BwArgs &a, int j, int lane, BwRows<NC> &r)
{
    const int64_t rb = (int64_t)a.d * 2;
    const char *pu = (const char *)a.wu_t + (int64_t)j * rb;
    const char *pd = (const char *)a.wd + (int64_t)j * rb;
    const char *pg = (const char *)a.wg_t + (int64_t)j * rb;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        const bool ok = ch < a.nchunks;
        r.wu[c] = ok ? ldg16(pu + ch * 16) : u32x4{0, 0, 0, 0};
        r.wd[c] = ok ? ldg16(pd + ch * 16) : u32x4{0, 0, 0, 0};
        r.wg[c] = ok ? ldg16(pg + ch * 16) : u32x4{0, 0, 0, 0};
    }
}

template <int NC>
__device__ __forceinline__ void bw_apply(const BwArgs &a, const BwRows<NC> &r, int k, float h,
                                         const float (&xf)[NC][8], const float (&gf)[NC][8], float (&dxa)[NC][8],
                                         int lane)
{
    float su = 0.f, sg = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            su = fmaf(xf[c][e], chunk_elem<__bf16>(r.wu[c], e), su);
            sg = fmaf(gf[c][e], chunk_elem<__bf16>(r.wd[c], e), sg);
        }
    const float u = wave_sum(su), g = wave_sum(sg);
    const float du = g * h, dz = g * u;
    if (lane == 0) {
        a.ws.ent_du[k] = du;
        a.ws.ent_dz[k] = dz;
        a.ws.ent_hu[k] = h * u;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            dxa[c][e] = fmaf(dz, chunk_elem<__bf16>(r.wg[c], e), fmaf(du, chunk_elem<__bf16>(r.wu[c], e), dxa[c][e]));
}

template <int NC>
__global__ __launch_bounds__(256) void bw_token_kernel(BwArgs a)
{
    if (a.ws.status[1])
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_chunks = a.ws.chunk0[a.T];
    const int64_t xb = (int64_t)a.d * 2;
    for (int c = blockIdx.x * 4 + wave; c < n_chunks; c += gridDim.x * 4) {
        const int t = a.ws.chunk_row[c];
        const int k0 = a.ws.row_ptr[t] + (c - a.ws.chunk0[t]) * BW_CE;
        const int kend = a.ws.row_ptr[t + 1];
        const int n = kend - k0 < BW_CE ? kend - k0 : BW_CE;
        float xf[NC][8], gf[NC][8], dxa[NC][8];
        const char *xr = (const char *)a.x + (int64_t)t * xb;
        const float *gr = a.dy + (int64_t)t * a.d;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const int ch = lane + 64 * cc;
            const bool ok = ch < a.nchunks;
            const u32x4 v = ok ? ldg16(xr + ch * 16) : u32x4{0, 0, 0, 0};
            const float4 g0 = ok ? *reinterpret_cast<const float4 *>(gr + ch * 8) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 g1 = ok ? *reinterpret_cast<const float4 *>(gr + ch * 8 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xf[cc][e] = chunk_elem<__bf16>(v, e);
                dxa[cc][e] = 0.f;
            }
            gf[cc][0] = g0.x; gf[cc][1] = g0.y; gf[cc][2] = g0.z; gf[cc][3] = g0.w;
            gf[cc][4] = g1.x; gf[cc][5] = g1.y; gf[cc][6] = g1.z; gf[cc][7] = g1.w;
        }
        BwRows<NC> ra, rb;
        if (n > 0)
            bw_load_rows<NC>(a, a.ws.ent_j[k0], lane, ra);
        for (int q = 0; q < n; q += 2) {
            if (q + 1 < n)
                bw_load_rows<NC>(a, a.ws.ent_j[k0 + q + 1], lane, rb);
            bw_apply<NC>(a, ra, k0 + q, a.ws.ent_h[k0 + q], xf, gf, dxa, lane);
            if (q + 1 >= n)
                break;
            if (q + 2 < n)
                bw_load_rows<NC>(a, a.ws.ent_j[k0 + q + 2], lane, ra);
            bw_apply<NC>(a, rb, k0 + q + 1, a.ws.ent_h[k0 + q + 1], xf, gf, dxa, lane);
        }
        float *pr = a.ws.part + (int64_t)c * a.d;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const int ch = lane + 64 * cc;
            if (ch < a.nchunks) {
                *reinterpret_cast<float4 *>(pr + ch * 8) = make_float4(dxa[cc][0], dxa[cc][1], dxa[cc][2], dxa[cc][3]);
                *reinterpret_cast<float4 *>(pr + ch * 8 + 4) =
                    make_float4(dxa[cc][4], dxa[cc][5], dxa[cc][6], dxa[cc][7]);
            }
        }
    }
}

// ------------------------------------------------------------------ regroup by neuron
// Histogram of the entries' neurons per block of BW_RC rows (one wave per row).
__global__ __launch_bounds__(256) void bw_hist_kernel(BwArgs a)
{
    if (a.ws.status[1])
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T)
        return;
    int32_t *h = a.ws.cnt_rc + (int64_t)(t / BW_RC) * a.F;
    for (int k = a.ws.row_ptr[t] + lane; k < a.ws.row_ptr[t + 1]; k += 64)
        atomicAdd(h + a.ws.ent_j[k], 1);
}

// Per neuron: exclusive scan of its block counts (in place) and its total.
__global__ __launch_bounds__(256) void bw_colbase_kernel(BwArgs a)
{
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= a.F || a.ws.status[1])
        return;
    int run = 0;
    int32_t *col = a.ws.cnt_rc + j;
    for (int r0 = 0; r0 < a.n_rc; r0 += 16) {  // 16 loads in flight, then the stores
        int v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
            v[q] = r0 + q < a.n_rc ? col[(int64_t)(r0 + q) * a.F] : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (r0 + q < a.n_rc)
                col[(int64_t)(r0 + q) * a.F] = run;
            run += v[q];
        }
    }
    a.ws.col_ptr[j + 1] = run;
}

// col_ptr[0] = 0, col_ptr[1..F] scanned in place (one workgroup).
__global__ __launch_bounds__(1024) void bw_colscan_kernel(BwArgs a)
{
    constexpr int NWV = 16;
    __shared__ int wt[NWV];
    __shared__ int carry;
    if (a.ws.status[1])
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry = 0;
        a.ws.col_ptr[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < a.F; base += 1024) {
        const int j = base + tid;
        const int v = j < a.F ? a.ws.col_ptr[j + 1] : 0;
        const int incl = wave_incl_scan(v, lane);
        if (lane == 63)
            wt[wave] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w)
            before += wt[w];
        if (j < a.F)
            a.ws.col_ptr[j + 1] = before + incl;
        __syncthreads();
        if (tid == 1023)
            carry = before + incl;
        __syncthreads();
    }
}

// One workgroup per block of BW_RC rows, rows in order: entry (t, j) goes to
// col_ptr[j] + (entries of j in earlier rows).  The block's counter for j
// starts at the entries of j in earlier blocks.
__global__ __launch_bounds__(256) void bw_csc_fill_kernel(BwArgs a)
{
    if (a.ws.status[1])
        return;
    const int rc = blockIdx.x;
    int32_t *ctr = a.ws.cnt_rc + (int64_t)rc * a.F;
    const int t1 = (rc + 1) * BW_RC < a.T ? (rc + 1) * BW_RC : a.T;
    for (int t = rc * BW_RC; t < t1; ++t) {
        for (int k = a.ws.row_ptr[t] + threadIdx.x; k < a.ws.row_ptr[t + 1]; k += 256) {
            const int j = a.ws.ent_j[k];  // distinct within a row
            const int pos = a.ws.col_ptr[j] + ctr[j];
            ctr[j] += 1;
            a.ws.csc_t[pos] = t;
            a.ws.csc_e[pos] = k;
        }
        __syncthreads();  // this row's counter updates before the next row's reads
    }
}

// ------------------------------------------------------------------ neuron-major: dW
// One wave per neuron: its entries in ascending row order; the x and dy rows
// of the next entry are requested before the current one is added.
template <int NC>
__global__ __launch_bounds__(256) void bw_weight_kernel(BwArgs a)
{
    const bool none = a.ws.status[1] != 0;  // too many entries: zero gradients
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t xb = (int64_t)a.d * 2;
    for (int j = blockIdx.x * 4 + wave; j < a.F; j += gridDim.x * 4) {
        float ad[NC][8], au[NC][8], ag[NC][8];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ad[c][e] = au[c][e] = ag[c][e] = 0.f;
        const int p0 = none ? 0 : a.ws.col_ptr[j], p1 = none ? 0 : a.ws.col_ptr[j + 1];
        u32x4 xv[2][NC];
        float4 gv[2][NC][2];
        auto load = [&](int p, int s) {
            const int t = a.ws.csc_t[p];
            const char *xr = (const char *)a.x + (int64_t)t * xb;
            const float *gr = a.dy + (int64_t)t * a.d;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ch = lane + 64 * c;
                const bool ok = ch < a.nchunks;
                xv[s][c] = ok ? ldg16(xr + ch * 16) : u32x4{0, 0, 0, 0};
                gv[s][c][0] = ok ? *reinterpret_cast<const float4 *>(gr + ch * 8) : make_float4(0.f, 0.f, 0.f, 0.f);
                gv[s][c][1] = ok ? *reinterpret_cast<const float4 *>(gr + ch * 8 + 4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        auto add = [&](int p, int s) {
            const int k = a.ws.csc_e[p];
            const float du = a.ws.ent_du[k], dz = a.ws.ent_dz[k], hu = a.ws.ent_hu[k];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float g[8] = {gv[s][c][0].x, gv[s][c][0].y, gv[s][c][0].z, gv[s][c][0].w,
                                    gv[s][c][1].x, gv[s][c][1].y, gv[s][c][1].z, gv[s][c][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xe = chunk_elem<__bf16>(xv[s][c], e);
                    ad[c][e] = fmaf(hu, g[e], ad[c][e]);
                    au[c][e] = fmaf(du, xe, au[c][e]);
                    ag[c][e] = fmaf(dz, xe, ag[c][e]);
                }
            }
        };
        if (p0 < p1)
            load(p0, 0);
        for (int p = p0; p < p1; p += 2) {
            if (p + 1 < p1)
                load(p + 1, 1);
            add(p, 0);
            if (p + 1 >= p1)
                break;
            if (p + 2 < p1)
                load(p + 2, 0);
            add(p + 1, 1);
        }
        float *od = a.dwd + (int64_t)j * a.d, *ou = a.dwu + (int64_t)j * a.d, *og = a.dwg + (int64_t)j * a.d;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = lane + 64 * c;
            if (ch < a.nchunks) {
                *reinterpret_cast<float4 *>(od + ch * 8) = make_float4(ad[c][0], ad[c][1], ad[c][2], ad[c][3]);
                *reinterpret_cast<float4 *>(od + ch * 8 + 4) = make_float4(ad[c][4], ad[c][5], ad[c][6], ad[c][7]);
                *reinterpret_cast<float4 *>(ou + ch * 8) = make_float4(au[c][0], au[c][1], au[c][2], au[c][3]);
                *reinterpret_cast<float4 *>(ou + ch * 8 + 4) = make_float4(au[c][4], au[c][5], au[c][6], au[c][7]);
                *reinterpret_cast<float4 *>(og + ch * 8) = make_float4(ag[c][0], ag[c][1], ag[c][2], ag[c][3]);
                *reinterpret_cast<float4 *>(og + ch * 8 + 4) = make_float4(ag[c][4], ag[c][5], ag[c][6], ag[c][7]);
            }
        }
    }
}

// ------------------------------------------------------------------ launch
BwWs bw_ws_layout(void *base, int T, int F, int d, int max_entries)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t E = (size_t)max_entries;
    const size_t n_rc = (size_t)((T + BW_RC - 1) / BW_RC);
    const size_t max_chunks = E / BW_CE + (size_t)T + 1;
    size_t off = 0;
    size_t o_status = off;
    off += 256;
    size_t o_row_e = off;
    off += up((size_t)T * 4);
    size_t o_row_src = off;
    off += up((size_t)T * 4);
    size_t o_row_ptr = off;
    off += up((size_t)(T + 1) * 4);
    size_t o_chunk0 = off;
    off += up((size_t)(T + 1) * 4);
    size_t o_chunk_row = off;
    off += up(max_chunks * 4);
    size_t o_ent_j = off;
    off += up(E * 4);
    size_t o_ent_h = off;
    off += up(E * 4);
    size_t o_ent_du = off;
    off += up(E * 4);
    size_t o_ent_dz = off;
    off += up(E * 4);
    size_t o_ent_hu = off;
    off += up(E * 4);
    size_t o_part = off;
    off += up(max_chunks * (size_t)d * 4);
    size_t o_cnt_rc = off;
    off += up(n_rc * (size_t)F * 4);
    size_t o_col_ptr = off;
    off += up((size_t)(F + 1) * 4);
    size_t o_csc_t = off;
    off += up(E * 4);
    size_t o_csc_e = off;
    off += up(E * 4);
    BwWs w{};
    w.bytes = off;
    if (base) {
        char *p = static_cast<char *>(base);
        w.status = reinterpret_cast<int32_t *>(p + o_status);
        w.row_e = reinterpret_cast<int32_t *>(p + o_row_e);
        w.row_src = reinterpret_cast<int32_t *>(p + o_row_src);
        w.row_ptr = reinterpret_cast<int32_t *>(p + o_row_ptr);
        w.chunk0 = reinterpret_cast<int32_t *>(p + o_chunk0);
        w.chunk_row = reinterpret_cast<int32_t *>(p + o_chunk_row);
        w.ent_j = reinterpret_cast<int32_t *>(p + o_ent_j);
        w.ent_h = reinterpret_cast<float *>(p + o_ent_h);
        w.ent_du = reinterpret_cast<float *>(p + o_ent_du);
        w.ent_dz = reinterpret_cast<float *>(p + o_ent_dz);
        w.ent_hu = reinterpret_cast<float *>(p + o_ent_hu);
        w.part = reinterpret_cast<float *>(p + o_part);
        w.cnt_rc = reinterpret_cast<int32_t *>(p + o_cnt_rc);
        w.col_ptr = reinterpret_cast<int32_t *>(p + o_col_ptr);
        w.csc_t = reinterpret_cast<int32_t *>(p + o_csc_t);
        w.csc_e = reinterpret_cast<int32_t *>(p + o_csc_e);
    }
    return w;
}

template <int NC>
static hipError_t bw_go(const BwArgs &a, hipStream_t s)
{
    const int rows4 = (a.T + 3) / 4;
    if (a.T > 0)
        bw_count_kernel<<<dim3(rows4), dim3(256), 0, s>>>(a);
    bw_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(a);
    if (a.T > 0) {
        bw_chunk_rows_kernel<<<dim3((a.T + 255) / 256), dim3(256), 0, s>>>(a);
        bw_entries_kernel<<<dim3(rows4), dim3(256), 0, s>>>(a);
        bw_token_kernel<NC><<<dim3(BW_WGS), dim3(256), 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if ((e = launch_chunk_reduce(a.ws.part, a.ws.chunk0, a.T, a.d, a.dx, s)) != hipSuccess)
            return e;
        bw_hist_kernel<<<dim3(rows4), dim3(256), 0, s>>>(a);
    }
    bw_colbase_kernel<<<dim3((a.F + 255) / 256), dim3(256), 0, s>>>(a);
    bw_colscan_kernel<<<dim3(1), dim3(1024), 0, s>>>(a);
    if (a.n_rc > 0)
        bw_csc_fill_kernel<<<dim3(a.n_rc), dim3(256), 0, s>>>(a);
    bw_weight_kernel<NC><<<dim3(BW_WGS), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_ffn_backward(const BwArgs &a, hipStream_t s)
{
    if (a.nchunks <= 64)
        return bw_go<1>(a, s);
    if (a.nchunks <= 128)
        return bw_go<2>(a, s);
    return bw_go<4>(a, s);  // nchunks <= 256: d <= BW_MAX_D
}

}  // namespace twell
