// compact.hip -- compacted storage of the ELL + dense-backup hybrid.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.3: the hybrid keeps the rows with few nonzeros in a
// compact sparse part and the overflow rows in a dense part, and its dynamic
// partitioning keeps memory (training saves these activations for the
// backward pass) small.  TwELL pads every tile to `cap` slots; this compact
// form keeps exactly the entries of the rows that fit, row after row in
// ascending column order (row offsets, 16-bit global columns, values), and the
// overflow rows' ids and dense rows, in one caller buffer whose layout depends
// on the entry and overflow counts, so it is written on the device into a
// header (see twell.h).  Kernels:
//   compact_rows_count_kernel: one thread per row, its entries (0 for an
//     overflow row) into row_ptr[t + 1];
//   compact_scan_kernel: one workgroup, row_ptr scanned in place, the header;
//   compact_scatter_kernel: one wave per row, each entry placed by a binary
//     search of the row's tile prefix (in LDS), if the buffer is large enough;
//   compact_dense_kernel: the overflow ids and held dense rows.
// Back to dense: compact_expand_kernel (zeros, then the entries of a row, one
// workgroup per row) and compact_expand_dense_kernel (the dense rows).
#include "launch.h"
#include "twell.h"
#include "twell_device.h"

namespace twell {

using CompactHdr = twell_compact_header_t;
constexpr int CP_SCAN_THREADS = 1024;

__device__ __forceinline__ int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

__global__ __launch_bounds__(256) void compact_rows_count_kernel(const int32_t *cnt, const int32_t *row_ovf, int T,
                                                                 int n_b, int32_t *row_ptr)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T)
        return;
    int e = 0;
    if (!row_ovf[t]) {
        const int32_t *c = cnt + (int64_t)t * n_b;
        for (int b = 0; b < n_b; ++b)
            e += c[b];
    }
    row_ptr[t + 1] = e;
}

// row_ptr[0] = 0 and row_ptr[1..T] scanned in place (T entries per pass of
// CP_SCAN_THREADS * 8), then the header.
__global__ __launch_bounds__(CP_SCAN_THREADS) void compact_scan_kernel(char *buf, int64_t buf_bytes, int T, int F,
                                                                       int tile_w, int vdtype, const int32_t *n_ovf,
                                                                       int max_ovf)
{
    constexpr int PER = 8, NWV = CP_SCAN_THREADS / 64;
    __shared__ int wtot[NWV];
    __shared__ int carry_s;
    int32_t *row_ptr = reinterpret_cast<int32_t *>(buf + 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry_s = 0;
        row_ptr[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < T; base += CP_SCAN_THREADS * PER) {
        int v[PER], s = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int t = base + tid * PER + k;
            v[k] = t < T ? row_ptr[t + 1] : 0;
            s += v[k];
        }
        int incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o)
                incl += y;
        }
        if (lane == 63)
            wtot[wave] = incl;
        __syncthreads();
        int before = carry_s;
        for (int w = 0; w < wave; ++w)
            before += wtot[w];
        int run = before + incl - s;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int t = base + tid * PER + k;
            run += v[k];
            if (t < T)
                row_ptr[t + 1] = run;
        }
        __syncthreads();
        if (tid == CP_SCAN_THREADS - 1)
            carry_s = run;
        __syncthreads();
    }
    if (tid == 0) {
        const int esz = vdtype == 1 ? 2 : 4;
        const int n_entries = carry_s;
        const int n = T > 0 ? *n_ovf : 0;  // with no rows the hybrid's pointers may be NULL
        const int nd = n < max_ovf ? n : max_ovf;
        CompactHdr h{};
        h.T = T;
        h.F = F;
        h.tile_w = tile_w;
        h.vdtype = vdtype;
        h.n_entries = n_entries;
        h.n_ovf = n;
        h.n_dense = nd;
        h.off_row_ptr = 256;
        h.off_col = h.off_row_ptr + align256((int64_t)(T + 1) * 4);
        h.off_val = h.off_col + align256((int64_t)n_entries * 2);
        h.off_ovf = h.off_val + align256((int64_t)n_entries * esz);
        h.off_dense = h.off_ovf + align256((int64_t)nd * 4);
        h.bytes = h.off_dense + (int64_t)nd * F * esz;
        h.fits = h.bytes <= buf_bytes ? 1 : 0;
        *reinterpret_cast<CompactHdr *>(buf) = h;
    }
}

// One wave per row that fits: entry k of the row is slot k - pre[b] of the
// last tile b with pre[b] <= k (pre = the row's tile prefix, in LDS).
template <typename TI>
__global__ __launch_bounds__(256) void compact_scatter_kernel(const int32_t *cnt, const TI *val, const uint8_t *idx,
                                                              const int32_t *row_ovf, int T, int n_b, int tile_w,
                                                              int cap, char *buf)
{
    __shared__ int spre[4][DEC_MAX_NB + 1];
    const CompactHdr &h = *reinterpret_cast<const CompactHdr *>(buf);
    if (!h.fits)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wave;
    if (t >= T || row_ovf[t])
        return;
    const int32_t *row_ptr = reinterpret_cast<const int32_t *>(buf + h.off_row_ptr);
    uint16_t *col = reinterpret_cast<uint16_t *>(buf + h.off_col);
    TI *vout = reinterpret_cast<TI *>(buf + h.off_val);
    int *sp = spre[wave];
    const int32_t *crow = cnt + (int64_t)t * n_b;
    int run = 0;
    for (int b0 = 0; b0 < n_b; b0 += 64) {
        const int b = b0 + lane;
        int c = b < n_b ? crow[b] : 0;
        c = c < cap ? c : cap;
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o)
                incl += y;
        }
        if (b < n_b)
            sp[b] = run + incl - c;
        run += __shfl(incl, 63, 64);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int p0 = row_ptr[t];
    for (int k = lane; k < run; k += 64) {
        int lo = 0, hi = n_b - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sp[mid] <= k)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int64_t slot = ((int64_t)t * n_b + lo) * cap + (k - sp[lo]);
        col[p0 + k] = (uint16_t)(lo * tile_w + idx[slot]);
        vout[p0 + k] = val[slot];
    }
}

// Block i < n_dense: dense row i; block 0 also writes the n_dense ids.
template <typename TI>
__global__ __launch_bounds__(256) void compact_dense_kernel(const TI *dense, const int32_t *ovf_rows, int max_ovf,
                                                            int F, char *buf)
{
    const CompactHdr &h = *reinterpret_cast<const CompactHdr *>(buf);
    if (!h.fits)
        return;
    const int i = blockIdx.x;
    if (i == 0) {
        int32_t *ids = reinterpret_cast<int32_t *>(buf + h.off_ovf);
        for (int k = threadIdx.x; k < h.n_dense; k += 256)
            ids[k] = ovf_rows[k];
    }
    if (i >= h.n_dense)
        return;
    const int nch = F * (int)sizeof(TI) / 16;
    const char *src = reinterpret_cast<const char *>(dense + (int64_t)i * F);
    char *dst = buf + h.off_dense + (int64_t)i * F * (int64_t)sizeof(TI);
    for (int c = threadIdx.x; c < nch; c += 256)
        *reinterpret_cast<u32x4 *>(dst + c * 16) = ldg16(src + c * 16);
}

// Row t of `out`: zeros, then the row's compact entries.
template <typename TI>
__global__ __launch_bounds__(256) void compact_expand_kernel(const char *buf, int T, int F, TI *out)
{
    const CompactHdr &h = *reinterpret_cast<const CompactHdr *>(buf);
    const int t = blockIdx.x;
    const int nch = F * (int)sizeof(TI) / 16;
    char *orow = reinterpret_cast<char *>(out + (int64_t)t * F);
    for (int c = threadIdx.x; c < nch; c += 256)
        *reinterpret_cast<u32x4 *>(orow + c * 16) = u32x4{0, 0, 0, 0};
    __syncthreads();  // the zeros before the entries (same addresses, other threads)
    if (!h.fits || h.T != T || h.F != F)
        return;
    const int32_t *row_ptr = reinterpret_cast<const int32_t *>(buf + h.off_row_ptr);
    const uint16_t *col = reinterpret_cast<const uint16_t *>(buf + h.off_col);
    const TI *v = reinterpret_cast<const TI *>(buf + h.off_val);
    const int a = row_ptr[t], b = row_ptr[t + 1];
    for (int k = a + threadIdx.x; k < b; k += 256) {
        const int c = col[k];
        if (c < F)  // memory safety for a corrupt column
            out[(int64_t)t * F + c] = v[k];
    }
}

// The held dense rows into their rows of `out`.
template <typename TI>
__global__ __launch_bounds__(256) void compact_expand_dense_kernel(const char *buf, int T, int F, int max_rows, TI *out)
{
    const CompactHdr &h = *reinterpret_cast<const CompactHdr *>(buf);
    const int i = blockIdx.x;
    if (!h.fits || h.T != T || h.F != F || i >= h.n_dense || i >= max_rows)
        return;
    const int32_t *ids = reinterpret_cast<const int32_t *>(buf + h.off_ovf);
    const int t = ids[i];
    if (t < 0 || t >= T)
        return;
    const int nch = F * (int)sizeof(TI) / 16;
    const char *src = buf + h.off_dense + (int64_t)i * F * (int64_t)sizeof(TI);
    char *dst = reinterpret_cast<char *>(out + (int64_t)t * F);
    for (int c = threadIdx.x; c < nch; c += 256)
        *reinterpret_cast<u32x4 *>(dst + c * 16) = ldg16(src + c * 16);
}

template <typename TI>
static hipError_t compact_go(const int32_t *cnt, const void *val, const uint8_t *idx, const int32_t *row_ovf,
                             const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf, const void *dense, int T,
                             int F, int tile_w, int cap, int vdtype, void *buf, int64_t buf_bytes, hipStream_t s)
{
    const int n_b = F / tile_w;
    char *b = static_cast<char *>(buf);
    if (T > 0)
        compact_rows_count_kernel<<<dim3((T + 255) / 256), dim3(256), 0, s>>>(cnt, row_ovf, T, n_b,
                                                                             reinterpret_cast<int32_t *>(b + 256));
    compact_scan_kernel<<<dim3(1), dim3(CP_SCAN_THREADS), 0, s>>>(b, buf_bytes, T, F, tile_w, vdtype, n_ovf, max_ovf);
    if (T > 0)
        compact_scatter_kernel<TI><<<dim3((T + 3) / 4), dim3(256), 0, s>>>(cnt, static_cast<const TI *>(val), idx,
                                                                           row_ovf, T, n_b, tile_w, cap, b);
    compact_dense_kernel<TI><<<dim3(max_ovf > 0 ? max_ovf : 1), dim3(256), 0, s>>>(static_cast<const TI *>(dense),
                                                                                  ovf_rows, max_ovf, F, b);
    return hipGetLastError();
}

hipError_t launch_compact_hybrid(int vdtype, const int32_t *cnt, const void *val, const uint8_t *idx,
                                 const int32_t *row_ovf, const int32_t *ovf_rows, const int32_t *n_ovf, int max_ovf,
                                 const void *dense, int T, int F, int tile_w, int cap, void *buf, int64_t buf_bytes,
                                 hipStream_t s)
{
    if (vdtype == 1)
        return compact_go<__bf16>(cnt, val, idx, row_ovf, ovf_rows, n_ovf, max_ovf, dense, T, F, tile_w, cap, vdtype,
                                  buf, buf_bytes, s);
    return compact_go<float>(cnt, val, idx, row_ovf, ovf_rows, n_ovf, max_ovf, dense, T, F, tile_w, cap, vdtype, buf,
                             buf_bytes, s);
}

hipError_t launch_compact_to_dense(int vdtype, const void *buf, int T, int F, void *out, hipStream_t s)
{
    const char *b = static_cast<const char *>(buf);
    if (vdtype == 1) {
        compact_expand_kernel<__bf16><<<dim3(T), dim3(256), 0, s>>>(b, T, F, static_cast<__bf16 *>(out));
        compact_expand_dense_kernel<__bf16><<<dim3(T), dim3(256), 0, s>>>(b, T, F, T, static_cast<__bf16 *>(out));
    } else {
        compact_expand_kernel<float><<<dim3(T), dim3(256), 0, s>>>(b, T, F, static_cast<float *>(out));
        compact_expand_dense_kernel<float><<<dim3(T), dim3(256), 0, s>>>(b, T, F, T, static_cast<float *>(out));
    }
    return hipGetLastError();
}

}  // namespace twell
