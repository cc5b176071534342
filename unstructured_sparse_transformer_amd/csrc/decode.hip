// decode.hip -- gate and TwELL packing for decode-shaped calls (T <= 64).
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), sections 2.1-2.3: the same gate, TwELL packing and overflow
// partition as the batch path, organised for a handful of tokens.  With
// T <= 64 the gate is a skinny GEMM bound by reading W_g once (d x F bf16);
// the batch kernel's 256 x 256 tiles would give only F / 256 workgroups, so
// here every workgroup owns 32 neurons (F / 32 workgroups) and its 8 waves
// split the K dimension.  z goes to an fp32 workspace; a second kernel packs
// it into TwELL, one workgroup per row, and its last workgroup derives the
// per-row results (overflow flags and list, work order, tile prefixes and the
// chunking of the rows' entries for the gather in ffn_fused.hip).
#include <mutex>

#include "decode.h"
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

// Workspace of twell_ffn_decode_noalloc, for callers that cannot allocate
// (graph capture, serving loops).  A device array of the code object: every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends.  On the host the array's name is only a stand-in, never a
// device address: host code uses the address hipGetSymbolAddress returns for
// the current device (decode_static_workspace), kept per device.  Calls on
// one GPU share the copy, so calls that overlap in time on one GPU race.
static __device__ __align__(256) char scratch[twell::DEC_STATIC_BYTES];

namespace twell {

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES];
}  // namespace

hipError_t decode_static_workspace(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

// ------------------------------------------------------------------ gate
// z[m][n0 + n] for the workgroup's 32 neurons n, all rows m < T (MB blocks of
// 32 rows).  The workgroup's 32 rows of W_g (a contiguous d x 64-byte block)
// stream into LDS with global->LDS copies, a stage of up to DEC_KS K elements
// at a time, so the whole stage is in flight at once and no VGPRs hold it;
// the x operands of the wave's K chunks are requested before the copies
// (x is small and shared by all workgroups through L2).  LDS rows hold the
// stage's 16-byte chunks with the chunk index XORed with the row (inside
// groups of 16 chunks; rows padded to a multiple of 256 bytes), so the 16 rows
// one ds_read_b128 phase touches hit 16 distinct bank groups.  K is cut into
// 64-element chunks dealt to the 8 waves round-robin; in a chunk, lane half h
// supplies elements [32 h, 32 h + 32) of its row as four 8-element MFMA
// operands (A and B in the same element order).  The 8 partial 32 x 32 blocks
// are added in LDS in wave order (deterministic).  Block 0 also clears the
// packing kernel's completion counter.
constexpr int DEC_KS = 2048;  // K elements per LDS stage (32 rows x 4 KiB)

__device__ __forceinline__ int skinny_slot(int ch, int n) { return (ch & ~15) | ((ch ^ n) & 15); }

template <int MB>
__global__ __launch_bounds__(512) void gate_skinny_kernel(const __bf16 *x, const __bf16 *wg_t, int T, int d,
                                                          int F, float *z, int32_t *counter)
{
    constexpr int NW = 8, KCW = DEC_KS / 64 / NW;  // K chunks per wave per stage
    static_assert(MB * NW * 16 * 64 * 4 <= 32 * DEC_KS * 2, "reduction fits the stage buffer");
    __shared__ __attribute__((aligned(16))) char sb[32 * DEC_KS * 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 32;
    if (blockIdx.x == 0 && tid == 0)
        *counter = 0;
    const int n = lane & 31, h = lane >> 5;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wg_t + (int64_t)n0 * d, (uint32_t)(32 * d * 2));
    const char *arow[MB];
    bool aok[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 32 + n;
        aok[mb] = m < T;
        arow[mb] = reinterpret_cast<const char *>(x + (int64_t)(aok[mb] ? m : 0) * d);
    }
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[mb][i] = 0.f;
    for (int k0 = 0; k0 < d; k0 += DEC_KS) {
        const int ks = d - k0 < DEC_KS ? d - k0 : DEC_KS;  // multiple of 64
        const int cpr = ks / 8;                              // 16-byte chunks per row
        const int spr = (cpr + 15) & ~15;                    // LDS slots per row
        const int nkc = ks / 64;
        // this wave's x operands for the stage
        u32x4 a[KCW][MB][4];
#pragma unroll
        for (int u = 0; u < KCW; ++u) {
            const int kc = wave + u * NW;
            const int off = (k0 + kc * 64 + 32 * h) * 2;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[u][mb][q] = (kc < nkc && aok[mb]) ? ldg16(arow[mb] + off + 16 * q) : u32x4{0, 0, 0, 0};
        }
        // the stage of W_g: 64 slots (1 KiB) per wave instruction
        for (int s0 = wave * 64; s0 < 32 * spr; s0 += NW * 64) {
            const int slot = s0 + lane;
            const int r = slot / spr, sl = slot - r * spr;
            const int ch = skinny_slot(sl, r);
            const int voff = (r * d + k0) * 2 + (ch < cpr ? ch : 0) * 16;  // padding slots re-read chunk 0
            dma16(rw, sb + s0 * 16, voff, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // copies and x loads complete
        wg_barrier();
#pragma unroll
        for (int u = 0; u < KCW; ++u) {
            const int kc = wave + u * NW;
            if (kc < nkc) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ch = kc * 8 + 4 * h + q;
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(sb + (n * spr + skinny_slot(ch, n)) * 16);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        mfma_chunk(__bf16{}, a[u][mb][q], b, acc[mb]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
        wg_barrier();                        // before the next stage (or the reduction) overwrites sb
    }
    float *red = reinterpret_cast<float *>(sb);  // [wave][block][register][lane]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            red[((wave * MB + mb) * 16 + i) * 64 + lane] = acc[mb][i];
    __syncthreads();
    // element (row r, column c) of block mb sits in register i of lane l
    for (int e = tid; e < MB * 1024; e += 512) {
        const int mb = e >> 10, r = (e >> 5) & 31, c = e & 31;
        const int m = mb * 32 + r;
        if (m >= T)
            continue;
        const int l = c + 32 * ((r >> 2) & 1), i = ((r >> 3) << 2) + (r & 3);
        float s = red[((0 * MB + mb) * 16 + i) * 64 + l];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            s += red[((w * MB + mb) * 16 + i) * 64 + l];
        z[(int64_t)m * F + n0 + c] = s;
    }
}

// ------------------------------------------------------------------ packing
// One workgroup of 8 waves per row t; wave w packs tiles w, w + 8, ... (the
// z values of up to 4 tiles are requested together).  Per tile, lane l holds
// columns l + 64 j; one ballot per j gives the activity (z > 0) and each
// active column's slot (earlier j's counts plus the active lanes below it):
// ascending columns.  Values are rounded to bf16 (nearest even); slots past
// min(count, cap) are zero.  The row's total and overflow flag are summed in
// LDS.  The workgroup that finishes last (completion counter, device-scope
// fences) then derives every per-row result, one lane per row.
struct PackArgs {
    const float *z;
    int T, F, tile_w, cap, n_b;
    __bf16 *val;
    uint8_t *idx;
    int32_t *cnt;
    int32_t *row_ovf, *ovf_rows, *n_ovf, *order;
    int max_ovf;
    int32_t *counter, *row_e, *row_o, *chunk0, *chunk_e;
};

// Entries per gather chunk: the smallest DEC_MIN_E * 2^m with total <=
// DEC_BASE_CHUNKS chunks of that size (at most DEC_MAX_E).
__device__ __forceinline__ int chunk_entries(int total)
{
    int e = DEC_MIN_E;
    while (e < DEC_MAX_E && (int64_t)e * DEC_BASE_CHUNKS < total)
        e <<= 1;
    return e;
}

// Work class of a row with e stored entries (0: heaviest), as in the batch
// path's order: e >= 256, 192..255, 128..191, 64..127, 32..63, 16..31, 1..15, 0.
__device__ __forceinline__ int work_class_of(int e)
{
    return e >= 256 ? 0 : e >= 192 ? 1 : e >= 128 ? 2 : e >= 64 ? 3 : e >= 32 ? 4 : e >= 16 ? 5 : e >= 1 ? 6 : 7;
}

// Pack tile b of row t (all lanes of the wave); returns its true count.
__device__ __forceinline__ int pack_tile(const PackArgs &a, int t, int b, const float (&v)[4], int lane)
{
    const int w = a.tile_w, cap = a.cap;
    uint64_t bal[4];
    int total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bal[j] = __ballot(lane + 64 * j < w && v[j] > 0.f);
        total += __popcll(bal[j]);
    }
    const int64_t slot0 = ((int64_t)t * a.n_b + b) * cap;
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
        if (((bal[j] >> lane) & 1ull) && slot < cap) {
            store_elem(a.val + slot0 + slot, v[j]);
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
    return total;
}

__global__ __launch_bounds__(512) void pack_rows_kernel(PackArgs a)
{
    constexpr int NW = 8, BATCH = 4;
    __shared__ int s_last, s_e[NW], s_o[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w;
    const float *zr = a.z + (int64_t)t * a.F;
    int e = 0, o = 0;
    for (int b0 = wave; b0 < a.n_b; b0 += NW * BATCH) {
        float v[BATCH][4];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = lane + 64 * j;
                v[u][j] = (b < a.n_b && c < w) ? zr[(int64_t)b * w + c] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
            if (b < a.n_b) {
                const int tot = pack_tile(a, t, b, v[u], lane);
                e += tot;
                o |= tot > a.cap;
            }
        }
    }
    if (lane == 0) {
        s_e[wave] = e;
        s_o[wave] = o;
    }
    __syncthreads();
    if (tid == 0) {
        int se = 0, so = 0;
        for (int k = 0; k < NW; ++k) {
            se += s_e[k];
            so |= s_o[k];
        }
        a.row_e[t] = se;
        a.row_o[t] = so;
        if (gridDim.x == 1) {
            s_last = 1;  // a single row: this workgroup is the last, no fences needed
        } else {
            __threadfence();
            s_last = atomicAdd(a.counter, 1) == (int)gridDim.x - 1;
        }
    }
    __syncthreads();
    if (!s_last)
        return;
    if (gridDim.x > 1)
        __threadfence();
    if (wave != 0)
        return;
    // one lane per row (T <= 64)
    const bool live = lane < a.T;
    const int re = live ? a.row_e[lane] : 0;
    const int ovf = live ? (a.row_o[lane] != 0) : 0;
    if (live)
        a.row_ovf[lane] = ovf;
    int sum_e;
    (void)wave_excl_scan(re, lane, sum_e);
    const int E = chunk_entries(sum_e);
    const int nch = (re + E - 1) / E;
    int n_chunks;
    const int c0 = wave_excl_scan(nch, lane, n_chunks);
    if (live)
        a.chunk0[lane] = c0;
    if (lane == 0) {
        a.chunk0[a.T] = n_chunks;
        *a.chunk_e = E;
    }
    // ascending overflow list (first max_ovf rows) and its true length
    const uint64_t om = __ballot(live && ovf);
    const int opos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(om >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)om, 0u));
    if (live && ovf && opos < a.max_ovf)
        a.ovf_rows[opos] = lane;
    if (lane == 0)
        *a.n_ovf = __popcll(om);
    // work order: classes of stored entries (0 for overflow rows), heaviest first
    const int cls = work_class_of(ovf ? 0 : re);
    int base = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint64_t m = __ballot(live && cls == k);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (live && cls == k)
            a.order[pos] = lane;
        base += __popcll(m);
    }
}

// ------------------------------------------------------------------ launchers
DecodeWs decode_ws_layout(void *base, int T, int F, int tile_w, int d)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    (void)tile_w;
    const size_t o_z = 0;
    const size_t o_ctr = o_z + up((size_t)T * F * 4);
    const size_t o_rows = o_ctr + 256;
    const size_t o_c0 = o_rows + up((size_t)T * 8);
    const size_t o_part = o_c0 + up((size_t)(T + 1) * 4);
    DecodeWs w{};
    w.max_chunks = DEC_BASE_CHUNKS + T;
    w.bytes = o_part + up((size_t)w.max_chunks * d * 4);
    if (base) {
        char *p = static_cast<char *>(base);
        w.z = reinterpret_cast<float *>(p + o_z);
        w.counter = reinterpret_cast<int32_t *>(p + o_ctr);
        w.chunk_e = w.counter + 1;
        w.row_e = reinterpret_cast<int32_t *>(p + o_rows);
        w.row_o = w.row_e + T;
        w.chunk0 = reinterpret_cast<int32_t *>(p + o_c0);
        w.part = reinterpret_cast<float *>(p + o_part);
    }
    return w;
}

hipError_t launch_decode_gate_pack(const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                                   void *val, uint8_t *idx, int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows,
                                   int32_t *n_ovf, int32_t *order, int max_ovf, const DecodeWs &w, hipStream_t s)
{
    const __bf16 *xb = static_cast<const __bf16 *>(x);
    const __bf16 *wb = static_cast<const __bf16 *>(wg_t);
    if (T <= 32)
        gate_skinny_kernel<1><<<dim3(F / 32), dim3(512), 0, s>>>(xb, wb, T, d, F, w.z, w.counter);
    else
        gate_skinny_kernel<2><<<dim3(F / 32), dim3(512), 0, s>>>(xb, wb, T, d, F, w.z, w.counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    PackArgs a{w.z, T, F, tile_w, cap, F / tile_w, static_cast<__bf16 *>(val), idx, cnt,
               row_ovf, ovf_rows, n_ovf, order, max_ovf, w.counter, w.row_e, w.row_o, w.chunk0, w.chunk_e};
    pack_rows_kernel<<<dim3(T), dim3(512), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace twell
